// ss_consolidate.hip -- consolidation of the frozen part, on the GPU.
//
// SinkState 4.3 "Asynchronous CPU Consolidation", Figure 7(a): the frozen
// components of a state are replaced by the exact SVD of their sum, and the
// singular values below eps * sigma_0 are dropped, sigma_0 being the state's
// largest stored singular value (the first entry of the active list or of
// the frozen list, both descending).  The active part, the pad and Gamma
// stay as they are; Gamma scales every component alike, so the work is done
// on the stored values.
//
// One 256-thread workgroup per state; the frozen part is staged in LDS:
//   1. B = U_F diag(sigma_F) (d_k x f) and V_F (d_v x f) from the frozen ring.
//   2. Thin QR V_F = Q R by CGS2 over the workgroup: one wavefront per dot
//      product, one thread per row for the updates.  A column whose residual
//      is at most 1e-5 of its own norm is dependent: it is zeroed, and so is
//      its row of R, so it cannot create a component.
//   3. B <- B R^T (one thread per row, in place): the frozen part is B Q^T
//      with Q orthonormal.
//   4. One-sided (Hestenes) Jacobi on the columns of B: 8 lanes per column
//      pair, up to 32 pairs per round in round-robin (circle) order, one
//      barrier per round; the rotations are accumulated in Y (f x f).  At
//      convergence B = X diag(s), and the frozen part is X diag(s) (Q Y)^T.
//   5. Sort s; keep s >= eps sigma_0 (and s > 0); write u = B_j / s_j,
//      v = Q Y_j and s_j over the state's frozen slots.  The result never has
//      more components than the old frozen part, and every global read is done
//      in step 1, so the write is in place: the group's ring segment keeps its
//      size until the group's next compaction re-packs it.
#include "ss_internal.h"
#include "ss_linalg.h"
#include "ss_wave.h"

namespace ss {

namespace {

constexpr int kCT = 256;         // threads per workgroup
constexpr int kConsSweeps = 32;  // Jacobi sweep limit

__global__ __launch_bounds__(256) void k_consolidate(ConsolidateArgs a) {
  extern __shared__ float sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = uniform(a.members[blockIdx.x]);
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  if (meta_flags(packed) & FLAG_DENSE) return;
  const int ra = meta_ra(packed), rf = meta_rf(packed), n = meta_n(packed);
  if (rf == 0 || rf > a.fmax) return;  // the host sizes fmax to the pool's largest frozen part
  const int dk = a.dk, dv = a.dv, F2 = (a.fmax + 1) & ~1;
  float *B = sm;                                // [F2][dk]: column j at B + j dk
  float *Q = B + (size_t)F2 * dk;               // [fmax][dv]
  float *Y = Q + (size_t)a.fmax * dv;           // [F2][F2]: R(i, j) at Y[j F2 + i], then the rotations
  float *sg = Y + (size_t)F2 * F2;              // [F2]: frozen sigma, later the column norms
  float *dt = sg + F2;                          // [F2]: dot products
  int *perm = reinterpret_cast<int *>(dt + F2);  // [F2]
  float *ctl = reinterpret_cast<float *>(perm + F2);  // [2]
  int *flag = reinterpret_cast<int *>(ctl + 2);       // [2]: rotation seen, per sweep parity
  const int64_t capF = a.frz.cap;
  const int off_f = uniform(m.off_f);

  // ---- 1. stage the frozen part --------------------------------------------------------------
  for (int j = tid; j < rf; j += kCT) sg[j] = a.frz.s[wrap(off_f + j, capF)];
  for (int e = tid; e < F2 * F2; e += kCT) Y[e] = 0.f;
  if (rf & 1)
    for (int e = tid; e < dk; e += kCT) B[(size_t)rf * dk + e] = 0.f;
  if (tid < 2) flag[tid] = 0;
  __syncthreads();
  float s0 = sg[0];
  if (ra > 0) s0 = fmaxf(s0, a.act.s[m.off_a]);
  const float thr = a.eps[s] * s0;
  {
    const int dk4 = dk >> 2, tot4 = dk4 + (dv >> 2);
    for (int e = tid; e < rf * tot4; e += kCT) {
      const int j = e / tot4, c = e - j * tot4;
      const int64_t pos = wrap(off_f + j, capF);
      if (c < dk4) st4(B + (size_t)j * dk + 4 * c, scale4(sg[j], ld4(a.frz.u + pos * dk + 4 * c)));
      else st4(Q + (size_t)j * dv + 4 * (c - dk4), ld4(a.frz.v + pos * dv + 4 * (c - dk4)));
    }
  }
  __syncthreads();

  // ---- 2. CGS2 thin QR of V_F ----------------------------------------------------------------
  for (int j = 0; j < rf; ++j) {
    float *qj = Q + (size_t)j * dv;
    for (int pass = 0; pass < 2; ++pass) {
      const int hi = pass == 0 ? j + 1 : j;  // the first pass also takes |q_j|^2 (i = j)
      for (int i = w; i < hi; i += 4) {
        const float *qi = Q + (size_t)i * dv;
        float x = 0.f;
        for (int e = lane; e < dv; e += 64) x = fmaf(qi[e], qj[e], x);
        x = wave_sum_u(x);
        if (lane == 0) dt[i] = x;
      }
      __syncthreads();
      if (tid < dv) {
        float x = qj[tid];
        for (int i = 0; i < j; ++i) x = fmaf(-dt[i], Q[(size_t)i * dv + tid], x);
        qj[tid] = x;
      }
      if (tid < j) Y[(size_t)j * F2 + tid] += dt[tid];
      __syncthreads();
    }
    if (w == 0) {
      float x = 0.f;
      for (int e = lane; e < dv; e += 64) x = fmaf(qj[e], qj[e], x);
      x = wave_sum_u(x);
      if (lane == 0) ctl[0] = x;
    }
    __syncthreads();
    const float n0 = dt[j], nu = ctl[0];
    const bool keep = nu > 0.f && nu > kTau2 * n0;
    const float su = sqrtf(nu), iu = keep ? 1.0f / su : 0.f;
    if (tid < dv) qj[tid] *= iu;
    if (tid == 0) Y[(size_t)j * F2 + j] = keep ? su : 0.f;
    __syncthreads();
  }

  // ---- 3. B <- B R^T, then Y <- I ------------------------------------------------------------
  if (tid < dk) {
    for (int jp = 0; jp < rf; ++jp) {
      float acc = 0.f;
      for (int i = jp; i < rf; ++i) acc = fmaf(B[(size_t)i * dk + tid], Y[(size_t)i * F2 + jp], acc);
      B[(size_t)jp * dk + tid] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < F2 * F2; e += kCT) {
    const int c = e / F2;
    Y[e] = (e - c * F2) == c ? 1.f : 0.f;
  }
  __syncthreads();

  // ---- 4. one-sided Jacobi on B's columns ----------------------------------------------------
  const int M = (rf + 1) & ~1;  // an odd count is paired with B's zero column rf
  int sweeps = 0;
  if (M >= 2) {
    const int np = M >> 1, rounds = M - 1, grp = tid >> 3, sub = tid & 7;
    for (int sw = 0; sw < kConsSweeps; ++sw) {
      ++sweeps;
      int *fl = flag + (sw & 1);
      for (int k = 0; k < rounds; ++k) {
        for (int p = grp; p < np; p += kCT / 8) {
          const int ci = p == 0 ? k : (k + p) % (M - 1);
          const int cj = p == 0 ? M - 1 : (k - p + (M - 1)) % (M - 1);
          float *x = B + (size_t)ci * dk, *y = B + (size_t)cj * dk;
          float aa = 0.f, bb = 0.f, gg = 0.f;
          for (int e = sub; e < dk; e += 8) {
            const float xe = x[e], ye = y[e];
            aa = fmaf(xe, xe, aa);
            bb = fmaf(ye, ye, bb);
            gg = fmaf(xe, ye, gg);
          }
          aa = group_sum<8>(aa);
          bb = group_sum<8>(bb);
          gg = group_sum<8>(gg);
          const bool rot = gg != 0.f && fabsf(gg) > kTolJ * __builtin_amdgcn_sqrtf(aa * bb);
          if (rot) {
            // zeta = (|y|^2 - |x|^2) / (2 x.y); t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)) zeroes x'.y'
            const float zeta = (bb - aa) * (0.5f * __builtin_amdgcn_rcpf(gg));
            const float az = fabsf(zeta);
            const float t = az > 1e10f ? 0.5f * __builtin_amdgcn_rcpf(zeta)
                                       : copysignf(__builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(fmaf(zeta, zeta, 1.f))), zeta);
            const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), sn = c * t;
            for (int e = sub; e < dk; e += 8) {
              const float xe = x[e], ye = y[e];
              x[e] = c * xe - sn * ye;
              y[e] = sn * xe + c * ye;
            }
            float *yx = Y + (size_t)ci * F2, *yy = Y + (size_t)cj * F2;
            for (int e = sub; e < rf; e += 8) {
              const float xe = yx[e], ye = yy[e];
              yx[e] = c * xe - sn * ye;
              yy[e] = sn * xe + c * ye;
            }
            if (sub == 0) *fl = 1;
          }
        }
        __syncthreads();
      }
      const int any = *fl;
      __syncthreads();  // every thread has read this sweep's flag before it is cleared for sweep sw + 2
      if (tid == 0) *fl = 0;
      if (!any) break;
    }
  }

  // ---- 5. norms, order, truncation, in-place write -------------------------------------------
  for (int j = w; j < rf; j += 4) {
    const float *bj = B + (size_t)j * dk;
    float x = 0.f;
    for (int e = lane; e < dk; e += 64) x = fmaf(bj[e], bj[e], x);
    x = wave_sum_u(x);
    if (lane == 0) sg[j] = sqrtf(x);
  }
  __syncthreads();
  if (tid < rf) {
    const float v = sg[tid];
    int rk = 0;
    for (int i = 0; i < rf; ++i) {
      const float u = sg[i];
      rk += (u > v || (u == v && i < tid)) ? 1 : 0;
    }
    perm[rk] = tid;
  }
  int kept = 0;
  for (int i = 0; i < rf; ++i) kept += (sg[i] > 0.f && sg[i] >= thr) ? 1 : 0;
  __syncthreads();
  for (int e = tid; e < kept * dk; e += kCT) {
    const int k = e / dk, i = e - k * dk, j = perm[k];
    a.frz.u[wrap(off_f + k, capF) * dk + i] = B[(size_t)j * dk + i] * (1.0f / sg[j]);
  }
  for (int e = tid; e < kept * dv; e += kCT) {
    const int k = e / dv, i = e - k * dv, j = perm[k];
    const float *yj = Y + (size_t)j * F2;
    float acc = 0.f;
    for (int c = 0; c < rf; ++c) acc = fmaf(Q[(size_t)c * dv + i], yj[c], acc);
    a.frz.v[wrap(off_f + k, capF) * dv + i] = acc;
  }
  if (tid < kept) a.frz.s[wrap(off_f + tid, capF)] = sg[perm[tid]];
  if (tid == 0) {
    a.meta[s].packed = meta_pack(ra, kept, n, meta_flags(packed));
    const unsigned long long f = (unsigned long long)rf * rf;
    const unsigned long long flops = 4ull * dv * f + (unsigned long long)dk * f +
                                     (unsigned long long)sweeps * (rf * (rf - 1) / 2) * (12ull * dk + 6ull * rf) +
                                     2ull * dv * rf * kept;
    const int slot = blockIdx.x % kAcctSlots;
    atomicAdd(a.acct_flops + slot, flops);
    atomicAdd(a.acct_states + slot, 1ull);
    atomicAdd(a.acct_removed + slot, (unsigned long long)(rf - kept));
  }
}

}  // namespace

size_t consolidate_lds_bytes(int dk, int dv, int fmax) {
  const size_t F2 = (size_t)((fmax + 1) & ~1);
  return sizeof(float) * (F2 * dk + (size_t)fmax * dv + F2 * F2 + 3 * F2 + 4);
}

hipError_t launch_consolidate(const ConsolidateArgs &a, hipStream_t st) {
  if (a.n_members <= 0 || a.fmax <= 0) return hipSuccess;
  const size_t sh = consolidate_lds_bytes(a.dk, a.dv, a.fmax);
  if (sh > kConsolidateLdsMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_consolidate, dim3((unsigned)a.n_members), dim3(kCT), sh, st, a);
  return hipGetLastError();
}

}  // namespace ss
