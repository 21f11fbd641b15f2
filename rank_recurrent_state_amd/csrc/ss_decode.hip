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
// Dense states (SinkState 4.4 dense region; also the dense baseline) are
// stored transposed, H = S^T, row-major [d_v][d_k].  Row j of H is column j
// of S, and everything the step does to it depends on that row alone:
//   o_j = alpha <H_j, q> + <k, q> w_j,  w_j = v_j or beta (v_j - alpha <H_j, k>),
//   H_j <- alpha H_j + w_j k.
// So the dense kernel is a pure stream: one wavefront per state reads a
// batch of rows (P lanes per row, float4 per lane), reduces each row inside
// its lane group, and writes the rows back; nothing is held across rows and
// no workgroup barrier is needed.
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
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= a.N) return;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const bool kin = col < (dk >> 2), vin = col < (dv >> 2);
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const uint32_t flags = meta_flags(packed);
  if (flags & FLAG_DENSE) return;  // the dense-region kernel serves this state
  const float4 q4 = kin ? ld4(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (!RO && kin) ? ld4(a.k + s * dk + 4 * col) : zero4();
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
      x[u] = (ok && kin) ? ld4(xp + c * dk + 4 * col) : zero4();
      y[u] = (ok && vin) ? ld4(yp + c * dv + 4 * col) : zero4();
      wt[u] = ok ? wp[c] : 0.f;
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
    const float4 v4 = vin ? ld4(a.v + s * dv + 4 * col) : zero4();
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
      const unsigned long long b = decode_bytes(dk, dv, rr, n, delta, false);
      __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// ---------------------------------------------------------------------------
// dense states, H = S^T stored [d_v][d_k]
// ---------------------------------------------------------------------------
template <int P, int UN, bool RO, bool ANYDELTA>
__global__ __launch_bounds__(256) void k_decode_dense(DenseArgs a) {
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
    h[u] = (j < dv && kin) ? ld4(H + (int64_t)j * dk) : zero4();
  }
  const int64_t s = uniform(a.dense_ids[slot]);
  const uint32_t flags = meta_flags((uint32_t)uniform((int)a.meta[s].packed));
  const bool delta = ANYDELTA && !RO && (flags & FLAG_DELTA);
  const float4 q4 = kin ? ld4(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (!RO && kin) ? ld4(a.k + s * dk + 4 * col) : zero4();
  const float al = RO ? 1.f : a.alpha[s];
  const float be = delta ? a.beta[s] : 0.f;
  const float kq = RO ? 0.f : group_sum<P>(dot4(k4, q4));
  const float *vs = RO ? nullptr : a.v + s * dv;
  float *os = a.o + s * dv;
  for (int j0 = 0; j0 < dv; j0 += G * UN) {
    if (j0 > 0) {
#pragma unroll
      for (int u = 0; u < UN; ++u) {
        const int j = j0 + u * G + grp;
        h[u] = (j < dv && kin) ? ld4(H + (int64_t)j * dk) : zero4();
      }
    }
    float vj[UN];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      const int j = j0 + u * G + grp;
      vj[u] = (!RO && j < dv) ? vs[j] : 0.f;
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
    const unsigned long long b = decode_bytes(dk, dv, 0, 0, delta, true);
    __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <bool RO, bool AD>
hipError_t decode_factored_p(const DecodeArgs &a, int P, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
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

template <bool RO, bool AD>
hipError_t decode_dense_p(const DenseArgs &a, int P, unsigned grid, hipStream_t st) {
  const dim3 g(grid), b(256);
  switch (P) {
    case 1: hipLaunchKernelGGL((k_decode_dense<1, 1, RO, AD>), g, b, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_dense<2, 1, RO, AD>), g, b, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_dense<4, 2, RO, AD>), g, b, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_dense<8, 4, RO, AD>), g, b, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_decode_dense<16, 8, RO, AD>), g, b, 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_decode_dense<32, 8, RO, AD>), g, b, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_decode_dense<64, 8, RO, AD>), g, b, 0, st, a); break;
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
  if (readonly) return decode_dense_p<true, false>(a, P, grid, st);
  return any_delta ? decode_dense_p<false, true>(a, P, grid, st) : decode_dense_p<false, false>(a, P, grid, st);
}

}  // namespace ss
