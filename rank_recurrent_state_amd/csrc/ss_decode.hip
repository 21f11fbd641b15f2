// ss_decode.hip -- decode step and read-only readout.
//
// Factored states (SinkState 4.2 "(i) Buffering", 4.4 "Kernel fusion"): one
// 64-lane wavefront per state.  The factors are streamed once: every
// component of the active region, every component of the frozen region and
// every filled pad slot is a pair (x in R^{d_k}, y in R^{d_v}) with a weight,
// and the three lists are walked as one list, so a chunk of G * UN pairs is
// in flight whatever region its pairs come from.  Lanes are split into 64/P
// groups of P lanes (P = next power of two >= max(d_k, d_v) / 4); a group
// reads one pair per step as float4 lanes, reduces <x, q> with DPP inside
// the group and keeps a float4 slice of the d_v-vector accumulator.  The
// decay is applied through Gamma (accumulated since the last compaction), so
// the factors are never rewritten; only the new pad slot, o and the 16-byte
// record are written.  With fp16 factors (SEED 6 "Lower precision composes")
// a lane reads four fp16 elements (8 bytes) per vector; the components then
// stream as one list and the fp32 pad as a second one.
//
//   p_q = S_{t-1}^T q,  p_k = S_{t-1}^T k  (delta rule only)
//   w   = v (scalar rule)  or  beta (v - alpha p_k)  (Gated DeltaNet, SEED eq. (2))
//   o   = alpha p_q + <k, q> w            (= S_t^T q, read after the update)
//   pad slot n <- (k, w, 1 / (alpha Gamma)),  Gamma <- alpha Gamma
//
// Dense states (SinkState 4.4 dense region) are stored transposed, H = S^T,
// row-major [d_v][d_k]: row j of H is column j of S, and everything a step
// does to it depends on that row alone.  The dense region is buffered the
// way the factors are (SinkState 4.4 keeps the buffer apart so that a step
// does not write the state back): a dense state is
//   S = Gamma (H^T + sum_{j<n} c_j k_j w_j^T),
// a step reads H and the pad and appends one slot, and only the step that
// fills the pad rewrites H (the pad folded in, Gamma reset).  Per row j:
//   p_q,j = Gamma (<H_j, q> + sum_i c_i <k_i, q> w_i,j)   (p_k likewise)
//   w_j   = v_j or beta (v_j - alpha p_k,j),  o_j = alpha p_q,j + <k, q> w_j
//   fold:  H_j <- alpha Gamma (H_j + sum_i c_i w_i,j k_i) + w_j k.
// One wavefront per state streams batches of rows (P lanes per row, float4
// per lane) and reduces each row inside its lane group; the pad's w rows and
// its contribution vectors sit in LDS, and so do the pad keys.  The plain
// kernel (the dense baseline: the recurrence the dense Mamba-2 / GDN kernels
// run) reads and writes every row every step: H_j <- alpha H_j + w_j k.
#include <type_traits>

#include "ss_internal.h"
#include "ss_wave.h"

namespace ss {

namespace {

// ---------------------------------------------------------------------------
// factored states
// ---------------------------------------------------------------------------
__device__ __forceinline__ float4 mul4(float4 a, float4 b) { return make_float4(a.x * b.x, a.y * b.y, a.z * b.z, a.w * b.w); }
__device__ __forceinline__ float4 div4(float4 a, float4 b) { return make_float4(a.x / b.x, a.y / b.y, a.z / b.z, a.w / b.w); }
__device__ __forceinline__ float4 one4() { return make_float4(1.f, 1.f, 1.f, 1.f); }

// DIAG: per-channel decay (Kimi Delta Attention, SEED appendix B.1 eq. (6)).  The decay is
// accumulated per key channel in gamma (d_k values per state, reset by a compaction), so
//   S = diag(gamma) (sum sigma_i u_i v_i^T + sum_j k~_j w_j^T),  k~_j = k_j / gamma_j (at insertion),
// and a step with decays lambda reads the stored parts with q~ = gamma' q and k~ = gamma' k,
// gamma' = gamma lambda:  p_q = stored^T q~,  w = beta (v - stored^T k~) (delta) or v,
// o = p_q + <k, q> w;  the new slot is (k / gamma', w, 1).
// A state's pairs lie in up to five contiguous runs: its active components (two runs when they
// wrap around the ring's end), its frozen components (likewise) and its pad.  The stream walks
// them in chunks of at most G * UN pairs that never cross a run, so a chunk is a wave-uniform
// base address per vector plus a small per-lane offset (the pair's place in the run times d).
#ifndef SS_FACT_WAVES
#define SS_FACT_WAVES 4
#endif
constexpr int kFactWaves = SS_FACT_WAVES;  // wavefronts (states) per workgroup of the factored decode

template <int P, int UN, bool RO, bool ANYDELTA, typename F, bool DIAG>
__global__ __launch_bounds__(64 * kFactWaves) void k_decode_factored(DecodeArgs a) {
  constexpr int G = 64 / P, C = G * UN;
  const int lane = threadIdx.x & 63;
  const uint32_t li = blockIdx.x * (uint32_t)kFactWaves + (uint32_t)uniform(threadIdx.x >> 6);
  const uint32_t cnt = *a.fact_count;
  if (li >= cnt) return;
  // a list of every state is a permutation of them: wave li takes state li, one dependent load less
  const int64_t s = cnt == (uint32_t)a.n_states ? (int64_t)li : uniform(a.fact_ids[li]);
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 2), vin = col < (dv >> 2);
  const int colk = kin ? col : (dk >> 2) - 1, colv = vin ? col : (dv >> 2) - 1;  // clamped: loads stay in bounds
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const uint32_t flags = meta_flags(packed);
  if (flags & FLAG_DENSE) return;  // the dense-region kernel serves this state
  const int ra = meta_ra(packed), rf = meta_rf(packed), n = meta_n(packed);
  const int off_a = uniform(m.off_a), off_f = uniform(m.off_f);
  const float gamma = uniformf(m.gamma);
  if (!RO && n >= K) {  // the caller skipped a compaction: record it and leave the state alone
    if (lane == 0) {
      __hip_atomic_fetch_add(&a.counters[C_ERR_PAD], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *a.hflag = 1u;
    }
    return;
  }
  const int rr = ra + rf;
  // the inputs are issued before the pair stream
  const float4 q4 = sel4(kin, ld4nt(a.q + s * dk + 4 * colk));
  const float4 k4 = RO ? zero4() : sel4(kin, ld4nt(a.k + s * dk + 4 * colk));
  const float4 v4 = RO ? zero4() : sel4(vin, ld4nt(a.v + s * dv + 4 * colv));
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
  const float al = (RO || DIAG) ? 1.f : uniformf(a.alpha[s]);
  const float be = delta ? uniformf(a.beta[s]) : 0.f;
  float4 gn4 = one4();  // DIAG: the accumulated decays after this step (readout: as they are)
  if constexpr (DIAG) {
    const float4 g4 = ld4(a.gam + s * dk + 4 * colk);  // clamped lanes: q4 = k4 = 0 and nothing is stored
    gn4 = RO ? g4 : mul4(g4, ld4nt(a.alpha + s * dk + 4 * colk));
  }
  const float4 qs = DIAG ? mul4(gn4, q4) : q4;  // what the stored parts are read with
  const float4 ks = DIAG ? mul4(gn4, k4) : k4;
  float4 acc = zero4(), acck = zero4();

  // the runs, in list order: active (up to the ring's end, then from its start), frozen (likewise),
  // pad; each by its first component's position in its arena (the pad: its first slot)
  const int64_t capA = a.act.cap, capF = a.frz.cap;
  const int na0 = (int)((int64_t)off_a + ra <= capA ? ra : capA - off_a);
  const int nf0 = (int)((int64_t)off_f + rf <= capF ? rf : capF - off_f);
  const int rn0 = na0, rn1 = ra - na0, rn2 = nf0, rn3 = rf - nf0, rn4 = n;
  const int64_t padc = s * (int64_t)K;
  // chunk cursor (wave-uniform): run index and pairs of that run already taken
  int ri = 0, rp = 0;
  struct Chunk {
    const F *xf, *yf;        // component runs
    const float *xp, *yp;    // the pad run
    const float *w;
    int cnt, pad;
    int sh;                  // lane group of the chunk's first pair: its index in the whole list, mod G
  };
  auto run_len = [&](int r) { return r == 0 ? rn0 : r == 1 ? rn1 : r == 2 ? rn2 : r == 3 ? rn3 : rn4; };
  auto next = [&](Chunk &c) -> bool {
    while (ri < 5 && rp >= run_len(ri)) {
      ++ri;
      rp = 0;
    }
    if (ri >= 5) return false;
    const int len = run_len(ri);
    const int cnt = len - rp < C ? len - rp : C;
    const bool isa = ri < 2;
    const int64_t c0 = (ri == 0 ? (int64_t)off_a : ri == 1 ? 0 : ri == 2 ? (int64_t)off_f : ri == 3 ? 0 : padc) + rp;
    const Arena &ar = isa ? a.act : a.frz;
    c.xf = ar.U<F>() + c0 * dk;
    c.yf = ar.V<F>() + c0 * dv;
    c.xp = a.pk + c0 * dk;
    c.yp = a.pw + c0 * dv;
    c.w = ri == 4 ? a.pc + c0 : ar.s + c0;
    c.cnt = cnt;
    c.pad = ri == 4;
    const int gs = (ri == 0 ? 0 : ri == 1 ? na0 : ri == 2 ? ra : ri == 3 ? ra + nf0 : rr) + rp;
    c.sh = gs & (G - 1);
    rp += cnt;
    return true;
  };
  // Pair i of the whole list is always reduced by lane group i mod G, in list order, whatever the
  // runs: each group's sum, and so the result, does not depend on where the ring wraps.  In a
  // chunk starting at list index gs, group g takes the chunk's pairs p = u * G + ((g - gs) mod G).
  auto slot = [&](const Chunk &c, int u) -> uint32_t { return (uint32_t)(u * G + ((grp - c.sh) & (G - 1))); };
  // the pair of unroll slot u, clamped into the chunk's run; the chunk's weights in one load (lane l
  // holds the weight of pair l mod C), handed to the lane groups by a cross-lane permute
  auto load = [&](const Chunk &c, float4 (&x)[UN], float4 (&y)[UN], float &wl) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const uint32_t pc = min(slot(c, u), (uint32_t)(c.cnt - 1));
      const uint32_t ox = pc * (uint32_t)dk + 4u * (uint32_t)colk, oy = pc * (uint32_t)dv + 4u * (uint32_t)colv;
      if (std::is_same<F, float>::value) {
        const float *xb = c.pad ? c.xp : reinterpret_cast<const float *>(c.xf);
        const float *yb = c.pad ? c.yp : reinterpret_cast<const float *>(c.yf);
        x[u] = ld4nt(xb + ox);
        y[u] = ld4nt(yb + oy);
      } else if (c.pad) {
        x[u] = ld4nt(c.xp + ox);
        y[u] = ld4nt(c.yp + oy);
      } else {
        x[u] = ldf4nt(c.xf + ox);
        y[u] = ldf4nt(c.yf + oy);
      }
    }
    wl = ldnt(c.w + min((uint32_t)(lane % C), (uint32_t)(c.cnt - 1)));
  };
  auto reduce = [&](const Chunk &c, const float4 (&x)[UN], const float4 (&y)[UN], float wl) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const float wp = __shfl(wl, (int)slot(c, u));
      const float wu = (slot(c, u) < (uint32_t)c.cnt) ? wp : 0.f;  // the clamped pairs weigh nothing
      const float cq = group_sum<P>(dot4(x[u], qs)) * wu;
      acc = fma4(cq, y[u], acc);
      if (delta) {
        const float ck = group_sum<P>(dot4(x[u], ks)) * wu;
        acck = fma4(ck, y[u], acck);
      }
    }
  };
  // double-buffered: the next chunk's loads are in flight while the current one is reduced
  {
    float4 xA[UN], yA[UN], xB[UN], yB[UN];
    float wA, wB;
    Chunk cA, cB;
    bool hA = next(cA);
    if (hA) load(cA, xA, yA, wA);
    while (hA) {
      const bool hB = next(cB);
      if (hB) load(cB, xB, yB, wB);
      reduce(cA, xA, yA, wA);
      if (!hB) break;
      hA = next(cA);
      if (hA) load(cA, xA, yA, wA);
      reduce(cB, xB, yB, wB);
    }
  }
  acc = cross_group_sum4<P>(acc);
  const float4 pq = DIAG ? acc : scale4(gamma, acc);
  if constexpr (RO) {
    if (grp == 0 && vin) st4(a.o + s * dv + 4 * col, pq);
    return;
  } else {
    float4 w4 = v4;
    if (delta) {
      acck = cross_group_sum4<P>(acck);
      w4 = scale4(be, sub4(v4, DIAG ? acck : scale4(al * gamma, acck)));
    }
    const float kq = group_sum<P>(dot4(k4, q4));
    const float4 o4 = add4(scale4(al, pq), scale4(kq, w4));
    const float gnew = al * gamma;  // DIAG: stays 1 (the decays live in gam)
    if (grp == 0) {
      if (kin) {
        st4nt(a.pk + (s * (int64_t)K + n) * dk + 4 * col, DIAG ? div4(k4, gn4) : k4);
        if constexpr (DIAG) st4(a.gam + s * dk + 4 * col, gn4);
      }
      if (vin) {
        st4nt(a.pw + (s * (int64_t)K + n) * dv + 4 * col, w4);
        st4(a.o + s * dv + 4 * col, o4);
      }
    }
    if (lane == 0) {
      a.pc[s * (int64_t)K + n] = 1.0f / gnew;
      Meta nm;
      nm.off_a = off_a;
      nm.off_f = off_f;
      nm.gamma = gnew;
      nm.packed = meta_pack(ra, rf, n + 1, flags);
      a.meta[s] = nm;
      const unsigned long long b = decode_bytes(dk, dv, K, rr, n, delta, KIND_FACTORED, (int)sizeof(F), DIAG);
      __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// factored states with fp16 factors, d_k and d_v multiples of 8: eight elements per lane, so a
// component vector is one 16-byte load per lane (an fp32 pad vector two float4 loads), and
// P = next power of two >= max(d_k, d_v) / 8 lanes serve a pair: twice the pairs of the fp32
// kernel per wavefront instruction.  Same arithmetic and writes as k_decode_factored.
// ---------------------------------------------------------------------------
struct f8 {
  float4 a, b;
};
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f8 zero8() { return {zero4(), zero4()}; }
__device__ __forceinline__ f8 ld8nt(const float *p) { return {ld4nt(p), ld4nt(p + 4)}; }
__device__ __forceinline__ f8 ldh8nt(const _Float16 *p) {
  const half8_t h = __builtin_nontemporal_load(reinterpret_cast<const half8_t *>(p));
  return {make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]),
          make_float4((float)h[4], (float)h[5], (float)h[6], (float)h[7])};
}
__device__ __forceinline__ f8 sel8(bool ok, f8 x) { return {sel4(ok, x.a), sel4(ok, x.b)}; }
__device__ __forceinline__ float dot8(f8 x, f8 y) { return dot4(x.a, y.a) + dot4(x.b, y.b); }
__device__ __forceinline__ f8 fma8(float s, f8 x, f8 c) { return {fma4(s, x.a, c.a), fma4(s, x.b, c.b)}; }
__device__ __forceinline__ f8 scale8(float s, f8 x) { return {scale4(s, x.a), scale4(s, x.b)}; }
__device__ __forceinline__ f8 add8(f8 x, f8 y) { return {add4(x.a, y.a), add4(x.b, y.b)}; }
__device__ __forceinline__ f8 sub8(f8 x, f8 y) { return {sub4(x.a, y.a), sub4(x.b, y.b)}; }
__device__ __forceinline__ void st8(float *p, f8 x) {
  st4(p, x.a);
  st4(p + 4, x.b);
}
__device__ __forceinline__ void st8nt(float *p, f8 x) {
  st4nt(p, x.a);
  st4nt(p + 4, x.b);
}
template <int P>
__device__ __forceinline__ f8 cross_group_sum8(f8 x) {
  return {cross_group_sum4<P>(x.a), cross_group_sum4<P>(x.b)};
}
__device__ __forceinline__ f8 mul8(f8 x, f8 y) { return {mul4(x.a, y.a), mul4(x.b, y.b)}; }
__device__ __forceinline__ f8 div8(f8 x, f8 y) { return {div4(x.a, y.a), div4(x.b, y.b)}; }
__device__ __forceinline__ f8 ld8(const float *p) { return {ld4(p), ld4(p + 4)}; }

// DIAG: per-channel decay, as in k_decode_factored.
template <int P, int UN, bool RO, bool ANYDELTA, bool DIAG>
__global__ __launch_bounds__(256) void k_decode_factored_h8(DecodeArgs a) {
  constexpr int G = 64 / P;
  const int lane = threadIdx.x & 63;
  const uint32_t li = blockIdx.x * 4u + (uint32_t)uniform(threadIdx.x >> 6);
  const uint32_t cnt = *a.fact_count;
  if (li >= cnt) return;
  // a list of every state is a permutation of them: wave li takes state li, one dependent load less
  const int64_t s = cnt == (uint32_t)a.n_states ? (int64_t)li : uniform(a.fact_ids[li]);
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 3), vin = col < (dv >> 3);
  const int colk = kin ? col : (dk >> 3) - 1, colv = vin ? col : (dv >> 3) - 1;  // clamped: loads stay in bounds
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const uint32_t flags = meta_flags(packed);
  if (flags & FLAG_DENSE) return;
  const int ra = meta_ra(packed), rf = meta_rf(packed), n = meta_n(packed);
  const int off_a = uniform(m.off_a), off_f = uniform(m.off_f);
  const float gamma = uniformf(m.gamma);
  if (!RO && n >= K) {
    if (lane == 0) {
      __hip_atomic_fetch_add(&a.counters[C_ERR_PAD], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *a.hflag = 1u;
    }
    return;
  }
  const int rr = ra + rf, T = rr + n;
  const int64_t pad0 = s * (int64_t)K - rr;
  const f8 q8 = sel8(kin, ld8nt(a.q + s * dk + 8 * colk));
  const f8 k8 = RO ? zero8() : sel8(kin, ld8nt(a.k + s * dk + 8 * colk));
  const f8 v8 = RO ? zero8() : sel8(vin, ld8nt(a.v + s * dv + 8 * colv));
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
  const float al = (RO || DIAG) ? 1.f : uniformf(a.alpha[s]);
  const float be = delta ? uniformf(a.beta[s]) : 0.f;
  f8 gn8 = {one4(), one4()};  // DIAG: the accumulated decays after this step (readout: as they are)
  if constexpr (DIAG) {
    const f8 g8 = ld8(a.gam + s * dk + 8 * colk);  // clamped lanes: q8 = k8 = 0 and nothing is stored
    gn8 = RO ? g8 : mul8(g8, ld8nt(a.alpha + s * dk + 8 * colk));
  }
  const f8 qs = DIAG ? mul8(gn8, q8) : q8;
  const f8 ks = DIAG ? mul8(gn8, k8) : k8;
  // per-channel decay: q, k and the decays are held apart from the scaled qs and ks, so k.q, the
  // new pad key (slot n, which the stream does not read) and the decays are taken before the
  // stream, which frees their registers (four waves per SIMD instead of three on the delta rule)
  float kq = 0.f;
  if constexpr (!RO && DIAG) {
    kq = group_sum<P>(dot8(k8, q8));
    if (grp == 0 && kin) {
      st8nt(a.pk + (s * (int64_t)K + n) * dk + 8 * col, div8(k8, gn8));
      st8(a.gam + s * dk + 8 * col, gn8);
    }
  }
  f8 acc = zero8(), acck = zero8();
  // pairs in chunks of G * UN, single-buffered: with eight elements per lane a second buffer
  // costs more occupancy than it hides latency, and so do larger chunks (at 16 lanes per pair,
  // two pairs per group leave room for five waves per SIMD on the delta rule, four pairs three)
  auto stream = [&](int ib, int ie, auto ld) {
    for (int i0 = ib; i0 < ie; i0 += G * UN) {
      f8 x[UN], y[UN];
      float wt[UN];
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int iu = i0 + u * G + grp;
        ld(iu < ie ? iu : ie - 1, x[u], y[u], wt[u]);  // clamped pair; its weight is masked at use
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const float wu = (i0 + u * G + grp < ie) ? wt[u] : 0.f;
        const float cq = group_sum<P>(dot8(x[u], qs)) * wu;
        acc = fma8(cq, y[u], acc);
        if (delta) {
          const float ck = group_sum<P>(dot8(x[u], ks)) * wu;
          acck = fma8(ck, y[u], acck);
        }
      }
    }
  };
  stream(0, rr, [&](int i, f8 &x, f8 &y, float &w) {
    const bool act = i < ra;
    const int64_t c = act ? wrap(off_a + i, a.act.cap) : wrap(off_f + (i - ra), a.frz.cap);
    const Arena &ar = act ? a.act : a.frz;
    x = ldh8nt(ar.U<_Float16>() + c * dk + 8 * colk);
    y = ldh8nt(ar.V<_Float16>() + c * dv + 8 * colv);
    w = ldnt(ar.s + c);
  });
  stream(rr, T, [&](int i, f8 &x, f8 &y, float &w) {
    const int64_t c = pad0 + i;
    x = ld8nt(a.pk + c * dk + 8 * colk);
    y = ld8nt(a.pw + c * dv + 8 * colv);
    w = ldnt(a.pc + c);
  });
  acc = cross_group_sum8<P>(acc);
  const f8 pq = DIAG ? acc : scale8(gamma, acc);
  if constexpr (RO) {
    if (grp == 0 && vin) st8(a.o + s * dv + 8 * col, pq);
    return;
  } else {
    f8 w8 = v8;
    if (delta) {
      acck = cross_group_sum8<P>(acck);
      w8 = scale8(be, sub8(v8, DIAG ? acck : scale8(al * gamma, acck)));
    }
    if constexpr (!DIAG) kq = group_sum<P>(dot8(k8, q8));
    const f8 o8 = add8(scale8(al, pq), scale8(kq, w8));
    const float gnew = al * gamma;
    if (grp == 0) {
      if (!DIAG && kin) st8nt(a.pk + (s * (int64_t)K + n) * dk + 8 * col, k8);
      if (vin) {
        st8nt(a.pw + (s * (int64_t)K + n) * dv + 8 * col, w8);
        st8(a.o + s * dv + 8 * col, o8);
      }
    }
    if (lane == 0) {
      a.pc[s * (int64_t)K + n] = 1.0f / gnew;
      Meta nm;
      nm.off_a = off_a;
      nm.off_f = off_f;
      nm.gamma = gnew;
      nm.packed = meta_pack(ra, rf, n + 1, flags);
      a.meta[s] = nm;
      const unsigned long long b = decode_bytes(dk, dv, K, rr, n, delta, KIND_FACTORED, 2, DIAG);
      __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// dense states, H = S^T stored [d_v][d_k]
// ---------------------------------------------------------------------------
constexpr int kMaxPad = 8;
#ifndef SS_DENSE_UN
#define SS_DENSE_UN 8  // row batch (in units of G rows) of the buffered dense kernel at d_k = 128
#endif
enum DenseMode : int { DM_DECODE = 0, DM_READOUT = 1, DM_FOLD = 2 };

// Stage segments of float4 data into LDS: the loads of a round (8 float4 per
// lane, clamped so they stay in bounds) are all issued before any is written.
struct Seg4 {
  float *dst;
  const float *src;
  int cnt;  // float4 count
};
template <int NSEG>
__device__ __forceinline__ void stage_lds(const Seg4 (&sg)[NSEG], int lane) {
  int tot = 0;
#pragma unroll
  for (int i = 0; i < NSEG; ++i) tot += sg[i].cnt;
  for (int e0 = 0; e0 < tot; e0 += 512) {
    float4 x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int e = e0 + q * 64 + lane;
      e = e < tot ? e : tot - 1;
      const float *p = sg[0].src;
#pragma unroll
      for (int i = 0, b = 0; i < NSEG; b += sg[i].cnt, ++i)
        if (e >= b && e < b + sg[i].cnt) p = sg[i].src + 4 * (e - b);
      x[q] = ld4(p);
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int e = e0 + q * 64 + lane;
#pragma unroll
      for (int i = 0, b = 0; i < NSEG; b += sg[i].cnt, ++i)
        if (e >= b && e < b + sg[i].cnt) st4(sg[i].dst + 4 * (e - b), x[q]);
    }
  }
}

// buffered dense region.  DM_DECODE / DM_READOUT: one wavefront per dense
// slot.  DM_FOLD: one wavefront per member of a compaction group; a dense
// member with a non-empty pad gets its pad folded into H.  Rows stream in
// batches of G * UN, double-buffered: the next batch is in flight while the
// current one is reduced.  LDS per wave: the pad's keys and w rows, the pad
// parts of p_q and p_k, and v.  The decode writes o, the slot record, c and a
// delta-rule w row; the new key and a scalar-rule w = v are copied into the
// pad by k_dense_append after it (a few small writes inside the row stream
// cost more than a pass of their own).
// DIAG (per-channel decay): the slot's decays gamma (d_k values) replace the scalar Gamma, so a
// dense state is S = diag(gamma) (H^T + sum_i k~_i w_i^T) with c_i = 1, rows are read with
// q~ = gamma' q and k~ = gamma' k (gamma' = gamma lambda), and a fold is
//   H_j <- gamma' (H_j + sum_i w_i,j k~_i) + w_j k  (element by element), gamma <- 1.
template <int P, int UN, int MODE, bool ANYDELTA, bool DIAG>
__global__ __launch_bounds__(256) void k_dense_buf(DenseArgs a) {
  constexpr int G = 64 / P, B = G * UN;
  constexpr bool DEC = MODE == DM_DECODE, RO = MODE == DM_READOUT, FO = MODE == DM_FOLD;
  extern __shared__ float smem[];
  const int wv = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 2);
  const int colk = kin ? col : (dk >> 2) - 1;  // clamped: loads stay in bounds
  float *W = smem + (size_t)wv * ((size_t)K * (dk + dv) + 3 * dv);  // pad w rows [K][d_v]
  float *PQ = W + (size_t)K * dv;                                      // pad part of p_q
  float *PK = PQ + dv;                                                 // pad part of p_k
  float *VS = PK + dv;                                                 // v
  float *KS = VS + dv;                                                 // pad keys [K][d_k]
  float *OS = PK;  // o, collected here once PK has been read (the row loop reads PK[j] before writing OS[j])
  float *WS = VS;  // the new pad w row, collected in place of v (v_j is read before w_j is written)
  uint32_t slot;
  if constexpr (FO) {
    const int mi = blockIdx.x * 4 + wv;
    if (mi >= a.n_members) return;
    const int sm = uniform(a.members[mi]);
    if (a.sel && a.sel[sm] == 0) return;  // compaction of listed states: this one is not listed
    const uint32_t mp = (uint32_t)uniform((int)a.meta[sm].packed);
    if (!(meta_flags(mp) & FLAG_DENSE)) return;
    slot = (uint32_t)uniform(a.meta[sm].off_a);
  } else {
    slot = blockIdx.x * 4u + (uint32_t)wv;
    if (slot >= min(a.counters[C_DENSE_COUNT], a.cap_d)) return;
  }
  // everything but the inputs is addressed by the slot: the record and the first two row
  // batches are issued together, then the pad (its fill comes from the record)
  const DenseSlot rec = a.dslot[slot];
  const float *H = a.dense + (int64_t)slot * dk * dv + 4 * colk;
  float *Hw = a.dense + (int64_t)slot * dk * dv + 4 * col;
  float4 hA[UN], hB[UN];
  auto load_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      hb[u] = ld4nt(H + (int64_t)(j < dv ? j : dv - 1) * dk);  // clamped row; q4, k4 are 0 off the key lanes
    }
  };
  if constexpr (!FO) {
    load_rows(hA, 0);
    if (B < dv) load_rows(hB, B);
  }
  const uint32_t packed = (uint32_t)uniform((int)rec.packed);
  const int n = meta_n(packed);
  if constexpr (FO) {
    if (n == 0) return;
    load_rows(hA, 0);
    if (B < dv) load_rows(hB, B);
  }
  const int64_t s = uniform(rec.s);
  const uint32_t flags = meta_flags(packed);
  const float gamma = uniformf(rec.gamma);
  const bool delta = ANYDELTA && DEC && (flags & FLAG_DELTA);
  const bool fold = FO || (DEC && n + 1 >= K);
  const float4 q4 = FO ? zero4() : sel4(kin, ld4nt(a.q + s * dk + 4 * colk));
  const float4 k4 = DEC ? sel4(kin, ld4nt(a.k + s * dk + 4 * colk)) : zero4();
  const float al = (DEC && !DIAG) ? uniformf(a.alpha[s]) : 1.f;
  float4 gn4 = one4();  // DIAG: the slot's decays after this step (readout and fold: as they are)
  if constexpr (DIAG) {
    const float4 g4 = ld4(a.dgam + (int64_t)slot * dk + 4 * colk);  // clamped lanes store nothing
    gn4 = DEC ? mul4(g4, ld4nt(a.alpha + s * dk + 4 * colk)) : g4;
  }
  const float4 qs = DIAG ? mul4(gn4, q4) : q4;
  const float4 ks = DIAG ? mul4(gn4, k4) : k4;
  const float be = delta ? uniformf(a.beta[s]) : 0.f;
  // the pad (keys, w rows) and v to LDS in one batch of loads
  const float *pks = a.pk + (int64_t)slot * K * dk;
  const float *pws = a.pw + (int64_t)slot * K * dv;
  float cq[kMaxPad], ck[kMaxPad], cf[kMaxPad];
#pragma unroll
  for (int i = 0; i < kMaxPad; ++i) {
    cf[i] = i < n ? uniformf(a.pc[(int64_t)slot * K + i]) : 0.f;
    cq[i] = ck[i] = 0.f;
  }
  {
    const Seg4 sg[3] = {{KS, pks, (n * dk) >> 2}, {W, pws, (n * dv) >> 2}, {VS, a.v + s * dv, DEC ? (dv >> 2) : 0}};
    stage_lds(sg, lane);
  }
  wave_sync();
  if constexpr (!FO) {
#pragma unroll
    for (int i = 0; i < kMaxPad; ++i) {
      if (i < n) {
        const float4 ki = *reinterpret_cast<const float4 *>(KS + i * dk + 4 * colk);
        cq[i] = uniformf(cf[i] * group_sum<P>(dot4(ki, qs)));
        if (delta) ck[i] = uniformf(cf[i] * group_sum<P>(dot4(ki, ks)));
      }
    }
  }
  wave_sync();
  if constexpr (!FO) {
    for (int j = lane; j < dv; j += 64) {
      float x = 0.f, y = 0.f;
#pragma unroll
      for (int i = 0; i < kMaxPad; ++i) {
        if (i < n) {
          const float wij = W[i * dv + j];
          x = fmaf(cq[i], wij, x);
          y = fmaf(ck[i], wij, y);
        }
      }
      PQ[j] = x;
      PK[j] = y;
    }
    wave_sync();
  }
  const float kq = DEC ? uniformf(group_sum<P>(dot4(k4, q4))) : 0.f;
  const float ag = al * gamma;       // DIAG: 1 (the decays are in gn4)
  const float sc = FO ? gamma : ag;  // a fold scales H and the pad by this (DIAG: by gn4)
  float *os = a.o + s * dv;
  float *pwn = a.pw + ((int64_t)slot * K + n) * dv;
  auto proc_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      const bool ok = j < dv;
      float w = 0.f;
      if constexpr (!FO) {
        const float pq = gamma * (group_sum<P>(dot4(hb[u], qs)) + (ok ? PQ[j] : 0.f));
        float oj = pq;
        if constexpr (DEC) {
          const float vj = ok ? VS[j] : 0.f;
          w = vj;
          if (delta) {
            const float pk = gamma * (group_sum<P>(dot4(hb[u], ks)) + (ok ? PK[j] : 0.f));
            w = be * (vj - al * pk);
          }
          oj = fmaf(al, pq, kq * w);
          if (delta && !fold && col == 0 && ok) WS[j] = w;
        }
        if (col == 0 && ok) OS[j] = oj;
      }
      // fold, first part: FO: H <- Gamma H;  DEC: H <- alpha Gamma H + w_j k  (DIAG: gn4 for the scalar)
      if (fold) {
        const float4 h = DIAG ? mul4(gn4, hb[u]) : scale4(sc, hb[u]);
        hb[u] = FO ? h : fma4(w, k4, h);
      }
    }
    if (fold) {
      // second part: H_j += sc c_i w_i,j k_i for every pad slot i, one key at a time
      for (int i = 0; i < n; ++i) {
        const float4 kr = *reinterpret_cast<const float4 *>(KS + i * dk + 4 * colk);
        const float4 ki = DIAG ? mul4(gn4, kr) : kr;
        const float si = DIAG ? cf[i] : sc * cf[i];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int j = j0 + u * G + grp;
          hb[u] = fma4(si * (j < dv ? W[i * dv + j] : 0.f), ki, hb[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * G + grp;
        if (j < dv && kin) st4nt(Hw + (int64_t)j * dk, hb[u]);  // streamed out: nothing reads it again this step
      }
    }
  };
  for (int j0 = 0; j0 < dv; j0 += 2 * B) {
    proc_rows(hA, j0);
    if (j0 + 2 * B < dv) load_rows(hA, j0 + 2 * B);
    if (j0 + B < dv) {
      proc_rows(hB, j0 + B);
      if (j0 + 3 * B < dv) load_rows(hB, j0 + 3 * B);
    }
  }
  // o and the new pad w row leave as whole float4 rows
  wave_sync();
  if constexpr (!FO) {
    for (int e = lane; e < (dv >> 2); e += 64) {
      st4nt(os + 4 * e, *reinterpret_cast<const float4 *>(OS + 4 * e));
      if (DEC && !fold && delta) st4nt(pwn + 4 * e, *reinterpret_cast<const float4 *>(WS + 4 * e));
    }
  }
  if constexpr (!RO) {
    if constexpr (DIAG) {  // the decays after the step, or 1 after a fold
      if (grp == 0 && kin) st4(a.dgam + (int64_t)slot * dk + 4 * col, fold ? one4() : gn4);
    }
    if (lane == 0) {
      if (DEC && !fold) a.pc[(int64_t)slot * K + n] = 1.0f / ag;
      DenseSlot nr = rec;
      nr.gamma = fold ? 1.0f : ag;
      nr.packed = meta_pack(0, 0, fold ? 0 : n + 1, flags);
      a.dslot[slot] = nr;
      if (DEC) {
        const unsigned long long b = decode_bytes(dk, dv, K, 0, n, delta, KIND_DENSE_BUFFERED, 4, DIAG);
        __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// The new pad entry of each dense slot that did not fold in the step just decoded: its key, and
// for the scalar rule its w = v, copied from the inputs in a pass of its own (delta-rule w rows
// depend on the state and are written by the decode).  The decode has already advanced the
// slot record, so the entry goes to pad slot n - 1; n = 0 means the step folded.
template <bool DIAG>
__global__ __launch_bounds__(256) void k_dense_append(DenseArgs a) {
  const int wv = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const uint32_t slot = blockIdx.x * 4u + (uint32_t)wv;
  if (slot >= min(a.counters[C_DENSE_COUNT], a.cap_d)) return;
  const DenseSlot rec = a.dslot[slot];
  const uint32_t packed = (uint32_t)uniform((int)rec.packed);
  const int n = meta_n(packed);
  if (n == 0) return;
  const int64_t s = uniform(rec.s);
  const int dk4 = a.dk >> 2, dv4 = (meta_flags(packed) & FLAG_DELTA) ? 0 : (a.dv >> 2);
  float *pkn = a.pk + ((int64_t)slot * a.K + n - 1) * a.dk;
  float *pwn = a.pw + ((int64_t)slot * a.K + n - 1) * a.dv;
  for (int e = lane; e < dk4 + dv4; e += 64) {
    // one 16-byte load and one 16-byte store per lane: source and destination are selected first
    const bool isk = e < dk4;
    const float *src = isk ? a.k + s * a.dk + 4 * e : a.v + s * a.dv + 4 * (e - dk4);
    float *dst = isk ? pkn + 4 * e : pwn + 4 * (e - dk4);
    float4 x = ld4nt(src);
    if constexpr (DIAG) {  // per-channel decay: the key is stored as k / gamma
      const float4 g = ld4(a.dgam + (int64_t)slot * a.dk + 4 * (isk ? e : dk4 - 1));
      x = isk ? div4(x, g) : x;
    }
    st4nt(dst, x);
  }
}

// plain dense recurrence (the dense baseline): every row read and written every
// step.  Same row streaming as the buffered kernel (double-buffered batches, v and o in LDS).
// DIAG: per-channel decay lambda (d_k values per state): H_j <- lambda H_j + w_j k, with
// w_j = beta (v_j - <H_j, lambda k>) for the delta rule, and o_j = <H_j, lambda q> + <k, q> w_j.
template <int P, int UN, bool RO, bool ANYDELTA, bool DIAG>
__global__ __launch_bounds__(256) void k_dense_plain(DenseArgs a) {
  constexpr int G = 64 / P, B = G * UN;
  extern __shared__ float smem[];
  const int wv = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const uint32_t slot = blockIdx.x * 4u + (uint32_t)wv;
  const uint32_t count = min(a.counters[C_DENSE_COUNT], a.cap_d);
  if (slot >= count) return;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv;
  const bool kin = col < (dk >> 2);
  const int colk = kin ? col : (dk >> 2) - 1;  // clamped: loads stay in bounds
  float *VS = smem + (size_t)wv * 2 * dv;  // v
  float *OS = VS + dv;                      // o, collected row by row
  const float *H = a.dense + (int64_t)slot * dk * dv + 4 * colk;
  float *Hw = a.dense + (int64_t)slot * dk * dv + 4 * col;
  float4 hA[UN], hB[UN];
  auto load_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      hb[u] = ld4nt(H + (int64_t)(j < dv ? j : dv - 1) * dk);  // clamped row; q4, k4 are 0 off the key lanes
    }
  };
  const DenseSlot rec = a.dslot[slot];
  load_rows(hA, 0);  // depends on the slot only: issued before the record arrives
  if (B < dv) load_rows(hB, B);
  const int64_t s = uniform(rec.s);
  const uint32_t flags = meta_flags((uint32_t)uniform((int)rec.packed));
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
  const float4 q4 = sel4(kin, ld4nt(a.q + s * dk + 4 * colk));
  const float4 k4 = RO ? zero4() : sel4(kin, ld4nt(a.k + s * dk + 4 * colk));
  const float al = (RO || DIAG) ? 1.f : uniformf(a.alpha[s]);
  const float be = delta ? uniformf(a.beta[s]) : 0.f;
  const float4 l4 = (DIAG && !RO) ? ld4nt(a.alpha + s * dk + 4 * colk) : one4();  // clamped lanes store nothing
  const float4 qs = (DIAG && !RO) ? mul4(l4, q4) : q4;
  const float4 ks = (DIAG && !RO) ? mul4(l4, k4) : k4;
  if constexpr (!RO) {
    const Seg4 sg[1] = {{VS, a.v + s * dv, dv >> 2}};
    stage_lds(sg, lane);
    wave_sync();
  }
  const float kq = RO ? 0.f : uniformf(group_sum<P>(dot4(k4, q4)));
  auto proc_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      const bool ok = j < dv;
      const float dq = group_sum<P>(dot4(hb[u], qs));
      float oj;
      if constexpr (RO) {
        oj = dq;
      } else {
        const float vj = ok ? VS[j] : 0.f;
        float w = vj;
        if (delta) {
          const float dkk = group_sum<P>(dot4(hb[u], ks));
          w = be * (vj - al * dkk);
        }
        oj = fmaf(al, dq, kq * w);
        if (ok && kin) st4nt(Hw + (int64_t)j * dk, fma4(w, k4, DIAG ? mul4(l4, hb[u]) : scale4(al, hb[u])));
      }
      if (col == 0 && ok) OS[j] = oj;
    }
  };
  for (int j0 = 0; j0 < dv; j0 += 2 * B) {
    proc_rows(hA, j0);
    if (j0 + 2 * B < dv) load_rows(hA, j0 + 2 * B);
    if (j0 + B < dv) {
      proc_rows(hB, j0 + B);
      if (j0 + 3 * B < dv) load_rows(hB, j0 + 3 * B);
    }
  }
  wave_sync();
  for (int e = lane; e < (dv >> 2); e += 64) st4nt(a.o + s * dv + 4 * e, *reinterpret_cast<const float4 *>(OS + 4 * e));
  if (!RO && lane == 0) {
    const unsigned long long b = decode_bytes(dk, dv, 0, 0, 0, delta, KIND_DENSE_PLAIN, 4, DIAG);
    __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool RO, bool AD, typename F, bool DG>
hipError_t decode_factored_p(const DecodeArgs &a, int P, hipStream_t st) {
  // a.N: upper bound of the list length
  const dim3 grid((unsigned)((a.N + kFactWaves - 1) / kFactWaves)), block(64 * kFactWaves);
  switch (P) {
    case 1: hipLaunchKernelGGL((k_decode_factored<1, 1, RO, AD, F, DG>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_factored<2, 1, RO, AD, F, DG>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_factored<4, 1, RO, AD, F, DG>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_factored<8, 2, RO, AD, F, DG>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_decode_factored<16, 2, RO, AD, F, DG>), grid, block, 0, st, a); break;
#ifndef SS_FACT_UN32
#define SS_FACT_UN32 2
#endif
    case 32: hipLaunchKernelGGL((k_decode_factored<32, SS_FACT_UN32, RO, AD, F, DG>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_decode_factored<64, 8, RO, AD, F, DG>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

#ifndef SS_FACT_H8_UN
#define SS_FACT_H8_UN 2
#endif
template <bool RO, bool AD, bool DG>
hipError_t decode_factored_h8_p(const DecodeArgs &a, int P, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  switch (P) {
    case 1: hipLaunchKernelGGL((k_decode_factored_h8<1, 1, RO, AD, DG>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_factored_h8<2, 1, RO, AD, DG>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_factored_h8<4, 2, RO, AD, DG>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_factored_h8<8, 2, RO, AD, DG>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_decode_factored_h8<16, SS_FACT_H8_UN, RO, AD, DG>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_decode_factored_h8<32, 4, RO, AD, DG>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool DG>
hipError_t decode_factored_h8_f(const DecodeArgs &a, bool readonly, bool any_delta, int P, hipStream_t st) {
  if (readonly) return decode_factored_h8_p<true, false, DG>(a, P, st);
  return any_delta ? decode_factored_h8_p<false, true, DG>(a, P, st) : decode_factored_h8_p<false, false, DG>(a, P, st);
}

template <typename F, bool DG>
hipError_t decode_factored_f(const DecodeArgs &a, bool readonly, bool any_delta, int P, hipStream_t st) {
  if (readonly) return decode_factored_p<true, false, F, DG>(a, P, st);
  return any_delta ? decode_factored_p<false, true, F, DG>(a, P, st) : decode_factored_p<false, false, F, DG>(a, P, st);
}

template <int P, int UN, bool AD, bool DG>
hipError_t dense_buf_mode(const DenseArgs &a, int mode, unsigned grid, hipStream_t st) {
  const size_t sh = sizeof(float) * 4 * ((size_t)a.K * (a.dk + a.dv) + 3 * (size_t)a.dv);
  const dim3 g(grid), b(256);
  if (mode == DM_DECODE) hipLaunchKernelGGL((k_dense_buf<P, UN, DM_DECODE, AD, DG>), g, b, sh, st, a);
  else if (mode == DM_READOUT) hipLaunchKernelGGL((k_dense_buf<P, UN, DM_READOUT, false, DG>), g, b, sh, st, a);
  else hipLaunchKernelGGL((k_dense_buf<P, UN, DM_FOLD, false, DG>), g, b, sh, st, a);
  return hipGetLastError();
}

template <bool AD, bool DG>
hipError_t dense_buf_pd(const DenseArgs &a, int mode, int P, unsigned grid, hipStream_t st) {
  switch (P) {
    case 1: return dense_buf_mode<1, 1, AD, DG>(a, mode, grid, st);
    case 2: return dense_buf_mode<2, 1, AD, DG>(a, mode, grid, st);
    case 4: return dense_buf_mode<4, 2, AD, DG>(a, mode, grid, st);
    case 8: return dense_buf_mode<8, 4, AD, DG>(a, mode, grid, st);
    case 16: return dense_buf_mode<16, 8, AD, DG>(a, mode, grid, st);
    case 32: return dense_buf_mode<32, SS_DENSE_UN, AD, DG>(a, mode, grid, st);
    case 64: return dense_buf_mode<64, 8, AD, DG>(a, mode, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool AD>
hipError_t dense_buf_p(const DenseArgs &a, int mode, int P, unsigned grid, hipStream_t st) {
  if (a.diag) return a.dgam ? dense_buf_pd<AD, true>(a, mode, P, grid, st) : hipErrorInvalidValue;
  return dense_buf_pd<AD, false>(a, mode, P, grid, st);
}

template <bool RO, bool AD, bool DG>
hipError_t dense_plain_pd(const DenseArgs &a, int P, unsigned grid, hipStream_t st) {
  const dim3 g(grid), b(256);
  const size_t sh = sizeof(float) * 4 * 2 * (size_t)a.dv;
  switch (P) {
    case 1: hipLaunchKernelGGL((k_dense_plain<1, 1, RO, AD, DG>), g, b, sh, st, a); break;
    case 2: hipLaunchKernelGGL((k_dense_plain<2, 1, RO, AD, DG>), g, b, sh, st, a); break;
    case 4: hipLaunchKernelGGL((k_dense_plain<4, 2, RO, AD, DG>), g, b, sh, st, a); break;
    case 8: hipLaunchKernelGGL((k_dense_plain<8, 4, RO, AD, DG>), g, b, sh, st, a); break;
    case 16: hipLaunchKernelGGL((k_dense_plain<16, 8, RO, AD, DG>), g, b, sh, st, a); break;
    case 32: hipLaunchKernelGGL((k_dense_plain<32, 8, RO, AD, DG>), g, b, sh, st, a); break;
    case 64: hipLaunchKernelGGL((k_dense_plain<64, 8, RO, AD, DG>), g, b, sh, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool RO, bool AD>
hipError_t dense_plain_p(const DenseArgs &a, int P, unsigned grid, hipStream_t st) {
  // a readout applies no decay: the per-channel variant is only needed for the step
  if (a.diag && !RO) return dense_plain_pd<RO, AD, true>(a, P, grid, st);
  return dense_plain_pd<RO, AD, false>(a, P, grid, st);
}

int pow2_at_least(int w) {
  int P = 1;
  while (P < w) P <<= 1;
  return P;
}

}  // namespace

int lanes_per_pair(int dk, int dv) { return pow2_at_least((dk > dv ? dk : dv) >> 2); }

hipError_t launch_decode_factored(const DecodeArgs &a, bool readonly, bool any_delta, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  const int P = lanes_per_pair(a.dk, a.dv);
  if (a.act.half && a.dk % 8 == 0 && a.dv % 8 == 0) {  // fp16 factors, eight elements per lane
    const int P8 = pow2_at_least((a.dk > a.dv ? a.dk : a.dv) >> 3);
    return a.gam ? decode_factored_h8_f<true>(a, readonly, any_delta, P8, st)
                 : decode_factored_h8_f<false>(a, readonly, any_delta, P8, st);
  }
  if (a.gam) {  // per-channel decay
    return a.act.half ? decode_factored_f<_Float16, true>(a, readonly, any_delta, P, st)
                      : decode_factored_f<float, true>(a, readonly, any_delta, P, st);
  }
  if (a.act.half) return decode_factored_f<_Float16, false>(a, readonly, any_delta, P, st);
  return decode_factored_f<float, false>(a, readonly, any_delta, P, st);
}

hipError_t launch_decode_dense(const DenseArgs &a, int64_t n_upper, bool readonly, bool any_delta, hipStream_t st) {
  if (n_upper <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_upper + 3) / 4);
  const int P = pow2_at_least(a.dk >> 2);
  if (a.pk) {
    if (a.K > kMaxPad) return hipErrorInvalidValue;
    const int mode = readonly ? DM_READOUT : DM_DECODE;
    hipError_t e = any_delta ? dense_buf_p<true>(a, mode, P, grid, st) : dense_buf_p<false>(a, mode, P, grid, st);
    if (e == hipSuccess && !readonly) {  // the pad entries of the step, in a pass of their own
      if (a.diag) hipLaunchKernelGGL(k_dense_append<true>, dim3(grid), dim3(256), 0, st, a);
      else hipLaunchKernelGGL(k_dense_append<false>, dim3(grid), dim3(256), 0, st, a);
      e = hipGetLastError();
    }
    return e;
  }
  if (readonly) return dense_plain_p<true, false>(a, P, grid, st);
  return any_delta ? dense_plain_p<false, true>(a, P, grid, st) : dense_plain_p<false, false>(a, P, grid, st);
}

hipError_t launch_dense_fold(const DenseArgs &a, hipStream_t st) {
  if (a.n_members <= 0 || !a.pk) return hipSuccess;
  if (a.K > kMaxPad) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((a.n_members + 3) / 4);
  return dense_buf_p<false>(a, DM_FOLD, pow2_at_least(a.dk >> 2), grid, st);
}

}  // namespace ss
