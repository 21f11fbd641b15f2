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
// record are written.
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
// its contribution vectors sit in LDS, the pad keys in registers.  The plain
// kernel (the dense baseline: the recurrence the dense Mamba-2 / GDN kernels
// run) reads and writes every row every step: H_j <- alpha H_j + w_j k.
#include "ss_internal.h"
#include "ss_wave.h"

namespace ss {

namespace {

// ---------------------------------------------------------------------------
// factored states
// ---------------------------------------------------------------------------
template <int P, int UN, bool RO, bool ANYDELTA>
__global__ __launch_bounds__(256) void k_decode_factored(DecodeArgs a) {
  constexpr int G = 64 / P;
  const int lane = threadIdx.x & 63;
  const uint32_t li = blockIdx.x * 4u + (uint32_t)uniform(threadIdx.x >> 6);
  if (li >= *a.fact_count) return;
  const int64_t s = uniform(a.fact_ids[li]);
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 2), vin = col < (dv >> 2);
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const uint32_t flags = meta_flags(packed);
  if (flags & FLAG_DENSE) return;  // the dense-region kernel serves this state
  const float4 q4 = kin ? ld4nt(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (!RO && kin) ? ld4nt(a.k + s * dk + 4 * col) : zero4();
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
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
  const int rr = ra + rf, T = rr + n;
  const int64_t pad0 = s * (int64_t)K - rr;  // pad slot of list index i is pad0 + i
  float4 acc = zero4(), acck = zero4();
  for (int i0 = 0; i0 < T; i0 += G * UN) {
    float4 x[UN], y[UN];
    float wt[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int i = i0 + u * G + grp;
      const float *xp, *yp, *wp;
      int64_t c;
      if (i < ra) {
        c = off_a + i;
        xp = a.act.u; yp = a.act.v; wp = a.act.s;
      } else if (i < rr) {
        c = off_f + (i - ra);
        xp = a.frz.u; yp = a.frz.v; wp = a.frz.s;
      } else {
        c = pad0 + i;
        xp = a.pk; yp = a.pw; wp = a.pc;
      }
      const bool ok = i < T;
      x[u] = (ok && kin) ? ld4nt(xp + c * dk + 4 * col) : zero4();
      y[u] = (ok && vin) ? ld4nt(yp + c * dv + 4 * col) : zero4();
      wt[u] = ok ? ldnt(wp + c) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const float cq = group_sum<P>(dot4(x[u], q4)) * wt[u];
      acc = fma4(cq, y[u], acc);
      if (delta) {
        const float ck = group_sum<P>(dot4(x[u], k4)) * wt[u];
        acck = fma4(ck, y[u], acck);
      }
    }
  }
  acc = cross_group_sum4<P>(acc);
  const float4 pq = scale4(gamma, acc);
  if constexpr (RO) {
    if (grp == 0 && vin) st4(a.o + s * dv + 4 * col, pq);
    return;
  } else {
    const float al = a.alpha[s];
    const float4 v4 = vin ? ld4nt(a.v + s * dv + 4 * col) : zero4();
    float4 w4 = v4;
    if (delta) {
      acck = cross_group_sum4<P>(acck);
      const float be = a.beta[s];
      w4 = scale4(be, sub4(v4, scale4(al * gamma, acck)));
    }
    const float kq = group_sum<P>(dot4(k4, q4));
    const float4 o4 = add4(scale4(al, pq), scale4(kq, w4));
    const float gnew = al * gamma;
    if (grp == 0) {
      if (kin) st4(a.pk + (s * (int64_t)K + n) * dk + 4 * col, k4);
      if (vin) {
        st4(a.pw + (s * (int64_t)K + n) * dv + 4 * col, w4);
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
      const unsigned long long b = decode_bytes(dk, dv, K, rr, n, delta, KIND_FACTORED);
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

// buffered dense region.  DM_DECODE / DM_READOUT: one wavefront per dense
// slot.  DM_FOLD: one wavefront per member of a compaction group; a dense
// member with a non-empty pad gets its pad folded into H.  Rows stream in
// batches of G * UN, double-buffered: the next batch is in flight while the
// current one is reduced.  LDS per wave: the pad's w rows, the pad parts of
// p_q and p_k, and v.
template <int P, int UN, int MODE, bool ANYDELTA>
__global__ __launch_bounds__(256) void k_dense_buf(DenseArgs a) {
  constexpr int G = 64 / P, B = G * UN;
  constexpr bool DEC = MODE == DM_DECODE, RO = MODE == DM_READOUT, FO = MODE == DM_FOLD;
  extern __shared__ float smem[];
  const int wv = uniform(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 2);
  float *W = smem + (size_t)wv * (K + 3) * dv;  // pad w rows [K][d_v]
  float *PQ = W + (size_t)K * dv;               // pad part of p_q
  float *PK = PQ + dv;                          // pad part of p_k
  float *VS = PK + dv;                          // v
  int64_t s;
  uint32_t slot;
  Meta m;
  uint32_t packed;
  if constexpr (FO) {
    const int mi = blockIdx.x * 4 + wv;
    if (mi >= a.n_members) return;
    s = uniform(a.members[mi]);
    m = a.meta[s];
    packed = (uint32_t)uniform((int)m.packed);
    if (!(meta_flags(packed) & FLAG_DENSE) || meta_n(packed) == 0) return;
    slot = (uint32_t)uniform(m.off_a);
  } else {
    slot = blockIdx.x * 4u + (uint32_t)wv;
    if (slot >= min(a.counters[C_DENSE_COUNT], a.cap_d)) return;
  }
  const float *H = a.dense + (int64_t)slot * dk * dv + 4 * col;
  float *Hw = a.dense + (int64_t)slot * dk * dv + 4 * col;
  float4 hA[UN], hB[UN];
  auto load_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      hb[u] = (j < dv && kin) ? ld4nt(H + (int64_t)j * dk) : zero4();
    }
  };
  load_rows(hA, 0);  // depends on the slot only: issued before the id lookup
  if constexpr (!FO) {
    s = uniform(a.dense_ids[slot]);
    m = a.meta[s];
    packed = (uint32_t)uniform((int)m.packed);
  }
  if (B < dv) load_rows(hB, B);
  const uint32_t flags = meta_flags(packed);
  const int n = meta_n(packed);
  const float gamma = uniformf(m.gamma);
  const bool delta = ANYDELTA && DEC && (flags & FLAG_DELTA);
  const bool fold = FO || (DEC && n + 1 >= K);
  const float4 q4 = (!FO && kin) ? ld4nt(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (DEC && kin) ? ld4nt(a.k + s * dk + 4 * col) : zero4();
  const float al = DEC ? uniformf(a.alpha[s]) : 1.f;
  const float be = delta ? uniformf(a.beta[s]) : 0.f;
  // the pad: w rows (and v) to LDS; each key is read once for its coefficients
  // (wave-uniform, kept in scalar registers) and re-read from cache by a fold
  const float *pks = a.pk + s * (int64_t)K * dk + 4 * col;
  const float *pws = a.pw + s * (int64_t)K * dv;
  float cq[kMaxPad], ck[kMaxPad], cf[kMaxPad];
#pragma unroll
  for (int i = 0; i < kMaxPad; ++i) {
    cf[i] = i < n ? uniformf(a.pc[s * (int64_t)K + i]) : 0.f;
    cq[i] = ck[i] = 0.f;
  }
  for (int e = lane; e < ((n * dv) >> 2); e += 64) st4(W + 4 * e, ld4(pws + 4 * e));
  if constexpr (DEC) {
    for (int e = lane; e < (dv >> 2); e += 64) st4(VS + 4 * e, ld4nt(a.v + s * dv + 4 * e));
  }
  if constexpr (!FO) {
#pragma unroll
    for (int i = 0; i < kMaxPad; ++i) {
      if (i < n) {
        const float4 ki = kin ? ld4(pks + (int64_t)i * dk) : zero4();
        cq[i] = uniformf(cf[i] * group_sum<P>(dot4(ki, q4)));
        if (delta) ck[i] = uniformf(cf[i] * group_sum<P>(dot4(ki, k4)));
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
  const float ag = al * gamma;
  const float sc = FO ? gamma : ag;  // a fold scales H and the pad by this
  float *os = a.o + s * dv;
  float *pwn = a.pw + (s * (int64_t)K + n) * dv;
  auto proc_rows = [&](float4 (&hb)[UN], int j0) {
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      const bool ok = j < dv;
      float w = 0.f;
      if constexpr (!FO) {
        const float pq = gamma * (group_sum<P>(dot4(hb[u], q4)) + (ok ? PQ[j] : 0.f));
        float oj = pq;
        if constexpr (DEC) {
          const float vj = ok ? VS[j] : 0.f;
          w = vj;
          if (delta) {
            const float pk = gamma * (group_sum<P>(dot4(hb[u], k4)) + (ok ? PK[j] : 0.f));
            w = be * (vj - al * pk);
          }
          oj = fmaf(al, pq, kq * w);
          if (!fold && col == 0 && ok) pwn[j] = w;
        }
        if (col == 0 && ok) os[j] = oj;
      }
      // fold, first part: FO: H <- Gamma H;  DEC: H <- alpha Gamma H + w_j k
      if (fold) hb[u] = FO ? scale4(sc, hb[u]) : fma4(w, k4, scale4(sc, hb[u]));
    }
    if (fold) {
      // second part: H_j += sc c_i w_i,j k_i for every pad slot i, one key at a time
      for (int i = 0; i < n; ++i) {
        const float4 ki = kin ? ld4(pks + (int64_t)i * dk) : zero4();
        const float si = sc * cf[i];
#pragma unroll
        for (int u = 0; u < UN; ++u) {
          const int j = j0 + u * G + grp;
          hb[u] = fma4(si * (j < dv ? W[i * dv + j] : 0.f), ki, hb[u]);
        }
      }
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * G + grp;
        if (j < dv && kin) st4(Hw + (int64_t)j * dk, hb[u]);
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
  if constexpr (!RO) {
    if (DEC && !fold && grp == 0 && kin) st4(a.pk + (s * (int64_t)K + n) * dk + 4 * col, k4);
    if (lane == 0) {
      if (DEC && !fold) a.pc[s * (int64_t)K + n] = 1.0f / ag;
      Meta nm = m;
      nm.gamma = fold ? 1.0f : ag;
      nm.packed = meta_pack(0, 0, fold ? 0 : n + 1, flags);
      a.meta[s] = nm;
      if (DEC) {
        const unsigned long long b = decode_bytes(dk, dv, K, 0, n, delta, KIND_DENSE_BUFFERED);
        __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

// plain dense recurrence (the dense baseline): every row read and written every step
template <int P, int UN, bool RO, bool ANYDELTA>
__global__ __launch_bounds__(256) void k_dense_plain(DenseArgs a) {
  constexpr int G = 64 / P;
  const int lane = threadIdx.x & 63;
  const uint32_t slot = blockIdx.x * 4u + (uint32_t)uniform(threadIdx.x >> 6);
  const uint32_t count = min(a.counters[C_DENSE_COUNT], a.cap_d);
  if (slot >= count) return;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv;
  const bool kin = col < (dk >> 2);
  const float *H = a.dense + (int64_t)slot * dk * dv + 4 * col;
  float *Hw = a.dense + (int64_t)slot * dk * dv + 4 * col;
  // first batch of rows: depends on the slot only, so it is issued before the id lookup
  float4 h[UN];
#pragma unroll
  for (int u = 0; u < UN; ++u) {
    const int j = u * G + grp;
    h[u] = (j < dv && kin) ? ld4nt(H + (int64_t)j * dk) : zero4();
  }
  const int64_t s = uniform(a.dense_ids[slot]);
  const uint32_t flags = meta_flags((uint32_t)uniform((int)a.meta[s].packed));
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
  const float4 q4 = kin ? ld4nt(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (!RO && kin) ? ld4nt(a.k + s * dk + 4 * col) : zero4();
  const float al = RO ? 1.f : a.alpha[s];
  const float be = delta ? a.beta[s] : 0.f;
  const float kq = RO ? 0.f : group_sum<P>(dot4(k4, q4));
  const float *vs = a.v + s * dv;
  float *os = a.o + s * dv;
  for (int j0 = 0; j0 < dv; j0 += G * UN) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * G + grp;
        h[u] = (j < dv && kin) ? ld4nt(H + (int64_t)j * dk) : zero4();
      }
    }
    float vj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      vj[u] = (!RO && j < dv) ? ldnt(vs + j) : 0.f;
    }
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      const float dq = group_sum<P>(dot4(h[u], q4));
      float oj;
      if constexpr (RO) {
        oj = dq;
      } else {
        float w = vj[u];
        if (delta) {
          const float dkk = group_sum<P>(dot4(h[u], k4));
          w = be * (vj[u] - al * dkk);
        }
        oj = fmaf(al, dq, kq * w);
        if (j < dv && kin) st4(Hw + (int64_t)j * dk, fma4(w, k4, scale4(al, h[u])));
      }
      if (col == 0 && j < dv) os[j] = oj;
    }
  }
  if (!RO && lane == 0) {
    const unsigned long long b = decode_bytes(dk, dv, 0, 0, 0, delta, KIND_DENSE_PLAIN);
    __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool RO, bool AD>
hipError_t decode_factored_p(const DecodeArgs &a, int P, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);  // a.N: upper bound of the list length
  switch (P) {
    case 1: hipLaunchKernelGGL((k_decode_factored<1, 1, RO, AD>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_factored<2, 1, RO, AD>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_factored<4, 1, RO, AD>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_factored<8, 2, RO, AD>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_decode_factored<16, 2, RO, AD>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_decode_factored<32, 4, RO, AD>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_decode_factored<64, 8, RO, AD>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int P, int UN, bool AD>
hipError_t dense_buf_mode(const DenseArgs &a, int mode, unsigned grid, hipStream_t st) {
  const size_t sh = sizeof(float) * 4 * (size_t)(a.K + 3) * a.dv;
  const dim3 g(grid), b(256);
  if (mode == DM_DECODE) hipLaunchKernelGGL((k_dense_buf<P, UN, DM_DECODE, AD>), g, b, sh, st, a);
  else if (mode == DM_READOUT) hipLaunchKernelGGL((k_dense_buf<P, UN, DM_READOUT, false>), g, b, sh, st, a);
  else hipLaunchKernelGGL((k_dense_buf<P, UN, DM_FOLD, false>), g, b, sh, st, a);
  return hipGetLastError();
}

template <bool AD>
hipError_t dense_buf_p(const DenseArgs &a, int mode, int P, unsigned grid, hipStream_t st) {
  switch (P) {
    case 1: return dense_buf_mode<1, 1, AD>(a, mode, grid, st);
    case 2: return dense_buf_mode<2, 1, AD>(a, mode, grid, st);
    case 4: return dense_buf_mode<4, 2, AD>(a, mode, grid, st);
    case 8: return dense_buf_mode<8, 4, AD>(a, mode, grid, st);
    case 16: return dense_buf_mode<16, 8, AD>(a, mode, grid, st);
    case 32: return dense_buf_mode<32, SS_DENSE_UN, AD>(a, mode, grid, st);
    case 64: return dense_buf_mode<64, 8, AD>(a, mode, grid, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool RO, bool AD>
hipError_t dense_plain_p(const DenseArgs &a, int P, unsigned grid, hipStream_t st) {
  const dim3 g(grid), b(256);
  switch (P) {
    case 1: hipLaunchKernelGGL((k_dense_plain<1, 1, RO, AD>), g, b, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_dense_plain<2, 1, RO, AD>), g, b, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_dense_plain<4, 2, RO, AD>), g, b, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_dense_plain<8, 4, RO, AD>), g, b, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_dense_plain<16, 8, RO, AD>), g, b, 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_dense_plain<32, 8, RO, AD>), g, b, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_dense_plain<64, 8, RO, AD>), g, b, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
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
  if (readonly) return decode_factored_p<true, false>(a, P, st);
  return any_delta ? decode_factored_p<false, true>(a, P, st) : decode_factored_p<false, false>(a, P, st);
}

hipError_t launch_decode_dense(const DenseArgs &a, int64_t n_upper, bool readonly, bool any_delta, hipStream_t st) {
  if (n_upper <= 0) return hipSuccess;
  const unsigned grid = (unsigned)((n_upper + 3) / 4);
  const int P = pow2_at_least(a.dk >> 2);
  if (a.pk) {
    if (a.K > kMaxPad) return hipErrorInvalidValue;
    const int mode = readonly ? DM_READOUT : DM_DECODE;
    return any_delta ? dense_buf_p<true>(a, mode, P, grid, st) : dense_buf_p<false>(a, mode, P, grid, st);
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
