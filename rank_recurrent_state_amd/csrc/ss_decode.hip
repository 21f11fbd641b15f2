// ss_decode.hip -- decode step and read-only readout.
//
// Factored states (SinkState 4.2 "(i) Buffering", 4.4 "Kernel fusion"): one
// 64-lane wavefront per state.  The factors are streamed once: every
// component (active and frozen region) and every filled pad slot is a pair
// (x in R^{d_k}, y in R^{d_v}) with a weight; the wave computes
// coef = weight * <x, q> and accumulates coef * y.  Lanes are split into
// 64/P groups of P lanes (P = next power of two >= max(d_k, d_v)/4); a group
// reads one pair per step as float4 lanes, reduces <x, q> with DPP inside the
// group and keeps a float4 slice of the d_v-vector accumulator.  The decay is
// applied through Gamma (accumulated since the last compaction), so the
// factors are never rewritten; only the new pad slot, o and the 16-byte
// record are written.
//
//   p_q = S_{t-1}^T q,  p_k = S_{t-1}^T k  (delta rule only)
//   w   = v (scalar rule)  or  beta (v - alpha p_k)  (Gated DeltaNet, SEED eq. (2))
//   o   = alpha p_q + <k, q> w            (= S_t^T q, read after the update)
//   pad slot n <- (k, w, 1 / (alpha Gamma)),  Gamma <- alpha Gamma
//
// Dense states (SinkState 4.4 dense region; also the dense baseline): one
// 256-thread workgroup per state holds S in registers, so S is read once and
// written once: S <- alpha S + k w^T, o = alpha S_{t-1}^T q + <k, q> w.
#include "ss_internal.h"
#include "ss_wave.h"

namespace ss {

namespace {

template <int P, bool DELTA>
__device__ __forceinline__ void stream_pairs(const float *__restrict__ X, const float *__restrict__ Y,
                                             const float *__restrict__ Wt, int cnt, int dk, int dv, int grp,
                                             int col, bool kin, bool vin, float4 q4, float4 k4, float4 &acc,
                                             float4 &acck) {
  constexpr int G = 64 / P;
  constexpr int UN = 2;
  for (int i0 = 0; i0 < cnt; i0 += G * UN) {
    float4 x[UN], y[UN];
    float wt[UN];
#pragma unroll
    for (int j = 0; j < UN; ++j) {
      const int i = i0 + j * G + grp;
      const bool ok = i < cnt;
      x[j] = (ok && kin) ? ld4(X + (int64_t)i * dk + 4 * col) : zero4();
      y[j] = (ok && vin) ? ld4(Y + (int64_t)i * dv + 4 * col) : zero4();
      wt[j] = ok ? Wt[i] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < UN; ++j) {
      const float cq = group_sum<P>(dot4(x[j], q4)) * wt[j];
      acc = fma4(cq, y[j], acc);
      if constexpr (DELTA) {
        const float ck = group_sum<P>(dot4(x[j], k4)) * wt[j];
        acck = fma4(ck, y[j], acck);
      }
    }
  }
}

template <int P, bool RO, bool ANYDELTA>
__global__ __launch_bounds__(256) void k_decode_factored(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= a.N) return;
  const int grp = lane / P, col = lane % P;
  const int dk = a.dk, dv = a.dv, K = a.K;
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const uint32_t flags = meta_flags(packed);
  if (flags & FLAG_DENSE) return;
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
  const bool kin = col < (dk >> 2), vin = col < (dv >> 2);
  const float4 q4 = kin ? ld4(a.q + s * dk + 4 * col) : zero4();
  const float4 k4 = (!RO && kin) ? ld4(a.k + s * dk + 4 * col) : zero4();
  float4 acc = zero4(), acck = zero4();
  const float *pk = a.pk + s * (int64_t)K * dk;
  const float *pw = a.pw + s * (int64_t)K * dv;
  const float *pc = a.pc + s * (int64_t)K;
  if (delta) {
    stream_pairs<P, true>(a.act.u + (int64_t)off_a * dk, a.act.v + (int64_t)off_a * dv, a.act.s + off_a, ra, dk, dv,
                          grp, col, kin, vin, q4, k4, acc, acck);
    stream_pairs<P, true>(a.frz.u + (int64_t)off_f * dk, a.frz.v + (int64_t)off_f * dv, a.frz.s + off_f, rf, dk, dv,
                          grp, col, kin, vin, q4, k4, acc, acck);
    stream_pairs<P, true>(pk, pw, pc, n, dk, dv, grp, col, kin, vin, q4, k4, acc, acck);
  } else {
    stream_pairs<P, false>(a.act.u + (int64_t)off_a * dk, a.act.v + (int64_t)off_a * dv, a.act.s + off_a, ra, dk, dv,
                           grp, col, kin, vin, q4, k4, acc, acck);
    stream_pairs<P, false>(a.frz.u + (int64_t)off_f * dk, a.frz.v + (int64_t)off_f * dv, a.frz.s + off_f, rf, dk,
                           dv, grp, col, kin, vin, q4, k4, acc, acck);
    stream_pairs<P, false>(pk, pw, pc, n, dk, dv, grp, col, kin, vin, q4, k4, acc, acck);
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
      const unsigned long long b = decode_bytes(dk, dv, ra + rf, n, delta, false);
      __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Dense state: 256 threads; thread t owns column slice c = t % C4 (float4) of
// rows g, g + RG, ... with g = t / C4, RG = 256 / C4.
template <bool RO, int NR>
__global__ __launch_bounds__(256) void k_decode_dense(DenseArgs a) {
  __shared__ float4 part_q[256];
  __shared__ float4 part_k[256];
  __shared__ float4 tot_q[64];
  __shared__ float4 tot_k[64];
  __shared__ float sq[256];
  __shared__ float sk[256];
  __shared__ float skq;
  const int t = threadIdx.x;
  const int dk = a.dk, dv = a.dv;
  const int C4 = dv >> 2, RG = 256 / C4;
  const int c = t % C4, g = t / C4;
  const bool act = t < RG * C4;
  const uint32_t count = min(a.counters[C_DENSE_COUNT], a.cap_d);
  for (uint32_t slot = blockIdx.x; slot < count; slot += gridDim.x) {
    const int64_t s = a.dense_ids[slot];
    const uint32_t flags = meta_flags(a.meta[s].packed);
    const bool delta = flags & FLAG_DELTA;
    float *S = a.dense + (int64_t)slot * dk * dv;
    __syncthreads();  // LDS of the previous state is no longer read
    if (t < dk) {
      sq[t] = a.q[s * dk + t];
      if (!RO) sk[t] = a.k[s * dk + t];
    }
    __syncthreads();
    float4 reg[NR];
    float4 pq = zero4(), pk = zero4();
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int row = g + j * RG;
      if (act && row < dk) {
        reg[j] = ld4(S + (int64_t)row * dv + 4 * c);
        pq = fma4(sq[row], reg[j], pq);
        if (!RO && delta) pk = fma4(sk[row], reg[j], pk);
      } else {
        reg[j] = zero4();
      }
    }
    if (act) {
      part_q[t] = pq;
      part_k[t] = pk;
    }
    if (!RO && t < 64) {  // <k, q> on wave 0
      float x = 0.f;
      for (int i = t; i < dk; i += 64) x += sq[i] * sk[i];
      x = wave_sum(x);
      if (t == 0) skq = x;
    }
    __syncthreads();
    if (t < C4) {
      float4 aq = zero4(), ak = zero4();
      for (int gg = 0; gg < RG; ++gg) {
        aq = add4(aq, part_q[gg * C4 + t]);
        if (delta) ak = add4(ak, part_k[gg * C4 + t]);
      }
      tot_q[t] = aq;
      tot_k[t] = ak;
    }
    __syncthreads();
    if constexpr (RO) {
      if (act && g == 0) st4(a.o + s * dv + 4 * c, tot_q[c]);
    } else {
      if (act) {
        const float al = a.alpha[s];
        const float4 v4 = ld4(a.v + s * dv + 4 * c);
        float4 w4 = v4;
        if (delta) w4 = scale4(a.beta[s], sub4(v4, scale4(al, tot_k[c])));
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          const int row = g + j * RG;
          if (row < dk) st4(S + (int64_t)row * dv + 4 * c, fma4(sk[row], w4, scale4(al, reg[j])));
        }
        if (g == 0) st4(a.o + s * dv + 4 * c, add4(scale4(al, tot_q[c]), scale4(skq, w4)));
      }
      if (t == 0) {
        const unsigned long long b = decode_bytes(dk, dv, 0, 0, delta, true);
        __hip_atomic_fetch_add(&a.acct[s & (kAcctSlots - 1)], b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
}

template <bool RO, bool AD>
hipError_t decode_factored_p(const DecodeArgs &a, int P, hipStream_t st) {
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  switch (P) {
    case 1: hipLaunchKernelGGL((k_decode_factored<1, RO, AD>), grid, block, 0, st, a); break;
    case 2: hipLaunchKernelGGL((k_decode_factored<2, RO, AD>), grid, block, 0, st, a); break;
    case 4: hipLaunchKernelGGL((k_decode_factored<4, RO, AD>), grid, block, 0, st, a); break;
    case 8: hipLaunchKernelGGL((k_decode_factored<8, RO, AD>), grid, block, 0, st, a); break;
    case 16: hipLaunchKernelGGL((k_decode_factored<16, RO, AD>), grid, block, 0, st, a); break;
    case 32: hipLaunchKernelGGL((k_decode_factored<32, RO, AD>), grid, block, 0, st, a); break;
    case 64: hipLaunchKernelGGL((k_decode_factored<64, RO, AD>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool RO>
hipError_t decode_dense_nr(const DenseArgs &a, int nr, unsigned grid, hipStream_t st) {
  const dim3 g(grid), b(256);
  if (nr <= 1) hipLaunchKernelGGL((k_decode_dense<RO, 1>), g, b, 0, st, a);
  else if (nr <= 2) hipLaunchKernelGGL((k_decode_dense<RO, 2>), g, b, 0, st, a);
  else if (nr <= 4) hipLaunchKernelGGL((k_decode_dense<RO, 4>), g, b, 0, st, a);
  else if (nr <= 8) hipLaunchKernelGGL((k_decode_dense<RO, 8>), g, b, 0, st, a);
  else if (nr <= 12) hipLaunchKernelGGL((k_decode_dense<RO, 12>), g, b, 0, st, a);
  else if (nr <= 16) hipLaunchKernelGGL((k_decode_dense<RO, 16>), g, b, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

int lanes_per_pair(int dk, int dv) {
  const int w = (dk > dv ? dk : dv) >> 2;
  int P = 1;
  while (P < w) P <<= 1;
  return P;
}

int dense_rows_per_thread(int dk, int dv) {
  const int C4 = dv >> 2;
  const int RG = 256 / C4;
  return (dk + RG - 1) / RG;
}

hipError_t launch_decode_factored(const DecodeArgs &a, bool readonly, bool any_delta, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  const int P = lanes_per_pair(a.dk, a.dv);
  if (readonly) return any_delta ? decode_factored_p<true, true>(a, P, st) : decode_factored_p<true, false>(a, P, st);
  return any_delta ? decode_factored_p<false, true>(a, P, st) : decode_factored_p<false, false>(a, P, st);
}

hipError_t launch_decode_dense(const DenseArgs &a, int64_t grid_upper, bool readonly, hipStream_t st) {
  if (grid_upper <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(grid_upper < 4096 ? grid_upper : 4096);
  const int nr = dense_rows_per_thread(a.dk, a.dv);
  return readonly ? decode_dense_nr<true>(a, nr, grid, st) : decode_dense_nr<false>(a, nr, grid, st);
}

}  // namespace ss
