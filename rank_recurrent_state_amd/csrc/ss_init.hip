// ss_init.hip -- randomized block SVD initialization of dense states after
// prefill (SinkState 4.1; 4.2 "Randomized SVD initialization after prefill",
// Figure 6(a); the randomized range finder with subspace iteration of Halko,
// Martinsson and Tropp, 2011).
//
// The pages write the state as H = S^T (d_v x d_k, y = H q); the library
// holds S (d_k x d_v, o = S^T q).  For block k, from the caller's Gaussian
// Omega_k (d_k x b):
//   repeat `iters` times:  Y = S^T Omega,  Q = orth(Y),  Omega = S Q
//   block SVD:  Omega = X diag(sigma) W^T,  u = X,  v = Q W
// The first block's largest sigma is sigma_0.  Components with
// sigma >= eps sigma_0 and sigma > 0 are kept; if one is below, no further
// block is taken; otherwise the block is subtracted from the residual
// (S <- S - X diag(sigma) (Q W)^T) and the next block starts from it.
//
// One 256-thread workgroup per state.  The residual lives in LDS when it fits
// (rows padded by one float, so that both row and column walks are free of
// bank conflicts), else in a caller-given workspace.  The products S^T Omega
// and S Q and the subtraction use all threads (a thread owns one row of the
// product and four of its block columns), with Omega and
// Q in LDS; orth is the CGS2 thin QR and the block SVD is the thin QR of
// Omega followed by one-sided Jacobi on its R, both on wavefront 0.
#include <mutex>
#include <unordered_map>

#include "ss_internal.h"
#include "ss_linalg.h"
#include "ss_wave.h"

namespace ss {

namespace {

constexpr int kDMax = 256;

template <int NSK, int NSV, bool LDSS>
__global__ __launch_bounds__(256) void k_rsvd(RsvdArgs a) {
  extern __shared__ float smem[];  // the residual, [d_k][d_v + 1], when LDSS
  __shared__ float Om[kMaxM][kDMax];  // Omega, then X diag(sigma) for the subtraction (column c at Om[c])
  __shared__ float Qv[kMaxM][kDMax];  // Y, then Q, then Q W
  __shared__ float Rq[256], Cm[256], Vh[256];
  __shared__ float sg[kMaxM];
  __shared__ int perm[kMaxM];
  __shared__ int ctl[2];  // [0]: components kept so far, [1]: stop
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t s = blockIdx.x;
  const int dk = a.dk, dv = a.dv, b = a.b;
  const float *S = a.S + s * dk * dv;
  const int ld = LDSS ? dv + 1 : dv;                // row stride of the residual
  float *Wr = LDSS ? smem : a.work + s * dk * dv;   // the residual
  for (int e = tid; e < dk * dv; e += 256) {
    const int i = e / dv, j = e - i * dv;
    Wr[i * ld + j] = S[e];
  }
  if (tid == 0) {
    ctl[0] = 0;
    ctl[1] = 0;
  }
  const float eps = a.eps[s];
  float sigma0 = 0.f;
  __syncthreads();
  for (int blk = 0; blk < a.nb; ++blk) {
    if (ctl[1] || ctl[0] >= a.max_rank) break;  // uniform: written before the last barrier
    const float *om = a.omega + ((s * a.nb + blk) * (int64_t)dk) * b;
    for (int e = tid; e < dk * b; e += 256) {
      const int i = e / b, c = e - i * b;
      Om[c][i] = om[e];
    }
    __syncthreads();
    for (int it = 0; it < a.iters; ++it) {
      // Y = S^T Omega: a thread owns row j of Y and a group of 4 of its columns
      for (int o = tid; o < dv * ((b + 3) >> 2); o += 256) {
        const int j = o % dv, c0 = 4 * (o / dv);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < dk; ++i) {
          const float w = Wr[i * ld + j];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c0 + u < b) acc[u] = fmaf(w, Om[c0 + u][i], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + u < b) Qv[c0 + u][j] = acc[u];
      }
      __syncthreads();
      if (wv == 0) {  // Q = orth(Y)
        float y[kMaxM][NSV];
#pragma unroll
        for (int c = 0; c < kMaxM; ++c)
#pragma unroll
          for (int t = 0; t < NSV; ++t) {
            const int j = lane + 64 * t;
            y[c][t] = (c < b && j < dv) ? Qv[c][j] : 0.f;
          }
        cgs2_one<NSV>(y, b, lane, Rq);
#pragma unroll
        for (int c = 0; c < kMaxM; ++c)
#pragma unroll
          for (int t = 0; t < NSV; ++t) {
            const int j = lane + 64 * t;
            if (c < b && j < dv) Qv[c][j] = y[c][t];
          }
      }
      __syncthreads();
      // Omega = S Q: a thread owns row i of Omega and a group of 4 of its columns
      for (int o = tid; o < dk * ((b + 3) >> 2); o += 256) {
        const int i = o % dk, c0 = 4 * (o / dk);
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
        const float *row = Wr + i * ld;
        for (int j = 0; j < dv; ++j) {
          const float w = row[j];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (c0 + u < b) acc[u] = fmaf(w, Qv[c0 + u][j], acc[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (c0 + u < b) Om[c0 + u][i] = acc[u];
      }
      __syncthreads();
    }
    // block SVD of Omega (d_k x b) and the kept components, on wavefront 0
    if (wv == 0) {
      float x[kMaxM][NSK];
#pragma unroll
      for (int c = 0; c < kMaxM; ++c)
#pragma unroll
        for (int t = 0; t < NSK; ++t) {
          const int i = lane + 64 * t;
          x[c][t] = (c < b && i < dk) ? Om[c][i] : 0.f;
        }
      cgs2_one<NSK>(x, b, lane, Rq);  // Omega = Q2 R2
      wave_sync();
      for (int e = lane; e < 256; e += 64) {
        Cm[e] = Rq[e];
        Vh[e] = (e & 15) == (e >> 4) ? 1.f : 0.f;
      }
      wave_sync();
      jacobi16(Cm, Vh, b, lane);  // R2 J = Uh diag(sigma)
      if (lane < kMaxM) {
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) q = fmaf(Cm[lane * 16 + i], Cm[lane * 16 + i], q);
        sg[lane] = lane < b ? sqrtf(q) : -1.f;
      }
      wave_sync();
      float mine = 0.f;
      int rank = 0;
      if (lane < b) {  // descending, ties by index
        mine = sg[lane];
        for (int i = 0; i < b; ++i) rank += (sg[i] > mine) || (sg[i] == mine && i < lane);
      }
      wave_sync();
      if (lane < b) perm[rank] = lane;
      wave_sync();
      if (blk == 0) sigma0 = sg[perm[0]];
      const int R0 = ctl[0];
      int kept = 0;
      for (int c = 0; c < b && R0 + kept < a.max_rank; ++c) {
        const float sc = sg[perm[c]];
        if (!(sc >= eps * sigma0 && sc > 0.f)) break;
        ++kept;
      }
      // u = Q2 Uh (column perm[c] of R2 J, normalized), v = Q W; written in sorted order
      float vq[kMaxM][NSV];
#pragma unroll
      for (int c = 0; c < kMaxM; ++c)
#pragma unroll
        for (int t = 0; t < NSV; ++t) vq[c][t] = 0.f;
#pragma unroll
      for (int c = 0; c < kMaxM; ++c) {
        if (c < b) {
          const int pc = perm[c];
#pragma unroll
          for (int tt = 0; tt < kMaxM; ++tt) {
            const float wj = tt < b ? Vh[pc * 16 + tt] : 0.f;
#pragma unroll
            for (int t = 0; t < NSV; ++t) {
              const int j = lane + 64 * t;
              vq[c][t] = fmaf(wj, (tt < b && j < dv) ? Qv[tt][j] : 0.f, vq[c][t]);
            }
          }
        }
      }
      float xu[kMaxM][NSK];
#pragma unroll
      for (int c = 0; c < kMaxM; ++c) {
#pragma unroll
        for (int t = 0; t < NSK; ++t) xu[c][t] = 0.f;
        if (c < b) {
          const int pc = perm[c];
          const float sc = sg[pc];
          const float inv = sc > 0.f ? 1.0f / sc : 0.f;
#pragma unroll
          for (int tt = 0; tt < kMaxM; ++tt) {
            const float cu = tt < b ? Cm[pc * 16 + tt] * inv : 0.f;
#pragma unroll
            for (int t = 0; t < NSK; ++t) xu[c][t] = fmaf(cu, x[tt][t], xu[c][t]);
          }
        }
      }
      wave_sync();
      // outputs, and X diag(sigma) and Q W to LDS for the subtraction
#pragma unroll
      for (int c = 0; c < kMaxM; ++c) {
        if (c < b) {
          const float sc = sg[perm[c]];
          float *uo = a.u + (s * a.max_rank + R0 + c) * (int64_t)dk;
          float *vo = a.v + (s * a.max_rank + R0 + c) * (int64_t)dv;
#pragma unroll
          for (int t = 0; t < NSK; ++t) {
            const int i = lane + 64 * t;
            if (i < dk) {
              if (c < kept) uo[i] = xu[c][t];
              Om[c][i] = sc * xu[c][t];
            }
          }
#pragma unroll
          for (int t = 0; t < NSV; ++t) {
            const int j = lane + 64 * t;
            if (j < dv) {
              if (c < kept) vo[j] = vq[c][t];
              Qv[c][j] = vq[c][t];
            }
          }
          if (lane == 0 && c < kept) a.sigma[s * a.max_rank + R0 + c] = sc;
        }
      }
      if (lane == 0) {
        ctl[0] = R0 + kept;
        ctl[1] = kept < b ? 1 : 0;
      }
    }
    __syncthreads();
    if (ctl[1] || ctl[0] >= a.max_rank || blk + 1 >= a.nb) break;
    // the block leaves the residual: S <- S - X diag(sigma) (Q W)^T
    for (int e = tid; e < dk * dv; e += 256) {
      const int i = e / dv, j = e - i * dv;
      float w = Wr[i * ld + j];
#pragma unroll
      for (int c = 0; c < kMaxM; ++c)
        if (c < b) w = fmaf(-Om[c][i], Qv[c][j], w);
      Wr[i * ld + j] = w;
    }
    __syncthreads();
  }
  if (tid == 0) a.rank[s] = ctl[0];
}

}  // namespace

// the residual in LDS when it fits beside the kernel's 33 KB of static LDS
bool rsvd_residual_in_lds(int dk, int dv) { return sizeof(float) * (size_t)dk * (dv + 1) <= 120 * 1024; }

hipError_t launch_rsvd_init(const RsvdArgs &a, hipStream_t st) {
  if (a.n <= 0) return hipSuccess;
  const int nk = a.dk <= 64 ? 1 : a.dk <= 128 ? 2 : 4, nv = a.dv <= 64 ? 1 : a.dv <= 128 ? 2 : 4;
  const dim3 g((unsigned)a.n), b(256);
  const size_t sh = sizeof(float) * (size_t)a.dk * (a.dv + 1);
  const bool lds = rsvd_residual_in_lds(a.dk, a.dv);
#define SS_RSVD(K, V)                                                                        \
  if (nk == K && nv == V) {                                                                  \
    if (lds) hipLaunchKernelGGL((k_rsvd<K, V, true>), g, b, sh, st, a);                      \
    else hipLaunchKernelGGL((k_rsvd<K, V, false>), g, b, 0, st, a);                          \
    return hipGetLastError();                                                                \
  }
  SS_RSVD(1, 1) SS_RSVD(1, 2) SS_RSVD(1, 4) SS_RSVD(2, 1) SS_RSVD(2, 2) SS_RSVD(2, 4) SS_RSVD(4, 1) SS_RSVD(4, 2)
  SS_RSVD(4, 4)
#undef SS_RSVD
  return hipErrorInvalidValue;
}

// Fixed workspace of the allocation-free initialization entry point: the residuals of a call
// whose states do not fit the kernel's LDS live here instead of in a caller's buffer.  The array
// is a file-scope device variable, so each GPU the library runs on holds its own copy for the
// life of the process.  In host code its name stands for no device address: the address is
// asked of the runtime once per device (with that device current) and kept.
namespace {
__device__ __align__(256) float scratch[kRsvdScratchFloats];
std::mutex g_scratch_mu;
std::unordered_map<int, float *> g_scratch_ptr;  // device -> address of its copy of `scratch`
}  // namespace

hipError_t rsvd_scratch(float **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = g_scratch_ptr.emplace(dev, static_cast<float *>(ptr)).first;
  }
  *out = it->second;
  return hipSuccess;
}

}  // namespace ss
