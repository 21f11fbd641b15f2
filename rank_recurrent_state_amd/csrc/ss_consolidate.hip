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
// One 256-thread workgroup per state; the frozen part goes through one LDS
// panel A (f columns) and the small matrix Y (f x f):
//   1. V_F (d_v x f) from the frozen ring into A.
//   2. Thin QR V_F = Q R by CGS2 over the workgroup: one wavefront per dot
//      product, one thread per row for the updates; R goes to Y.  A column
//      whose residual is at most 1e-5 of its own norm is dependent: it is
//      zeroed, and so is its row of R, so it cannot create a component.
//      Q is parked in the state's own frozen v slots (their old contents are
//      consumed), which frees A.
//   3. B = U_F diag(sigma_F) R^T into A (one thread per row): the frozen
//      part is B Q^T with Q orthonormal.
//   4. One-sided (Hestenes) Jacobi on the columns of B: 8 lanes per column
//      pair, up to 32 pairs per round in round-robin (circle) order, one
//      barrier per round; the rotations are accumulated in Y (f x f).  The
//      columns' squared norms are taken at the start of each sweep and then
//      carried (a - t g, b + t g after a rotation by t = tan theta), so a pair
//      computes only its inner product.  At convergence B = X diag(s), and the
//      frozen part is X diag(s) (Q Y)^T.
//   5. Sort s; keep s >= eps sigma_0 (and s > 0); write u = B_j / s_j and
//      s_j over the state's frozen slots, bring Q back into A, and write
//      v = Q Y_j.  The result never has more components than the old frozen
//      part, so the write is in place: the group's ring segment keeps its size
//      until the group's next compaction re-packs it.
// Column strides in LDS are odd multiples of 8 floats, so the 8 lanes of a
// Jacobi pair and the 8 pairs of a wavefront (consecutive columns) fall in
// distinct banks.
#include <type_traits>

#include "ss_internal.h"
#include "ss_linalg.h"
#include "ss_wave.h"

namespace ss {

namespace {

constexpr int kCT = 256;         // threads per workgroup
constexpr int kConsSweeps = 32;  // Jacobi sweep limit

// smallest stride >= d that is an odd multiple of 8 floats
__host__ __device__ inline int bank_stride(int d) { return ((d + 7) / 8 | 1) * 8; }

// KE: elements per lane of a Jacobi column pair (8 lanes per pair), KE * 8 >= max(d_k, f)
template <int KE, typename F>
__global__ __launch_bounds__(256) void k_consolidate(ConsolidateArgs a) {
  extern __shared__ float sm[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int s = uniform(a.members[blockIdx.x]);
  const Meta m = a.snap ? a.snap[blockIdx.x] : a.meta[s];
  const bool staged = a.st_u != nullptr;  // asynchronous form: results to staging, rings and records untouched
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  if (meta_flags(packed) & FLAG_DENSE) return;
  const int ra = meta_ra(packed), rf = meta_rf(packed), n = meta_n(packed);
  if (rf == 0 || rf > a.fmax) return;  // the host sizes fmax to the pool's largest frozen part
  const int dk = a.dk, dv = a.dv, F2 = (a.fmax + 1) & ~1;
  const int bs = bank_stride(dk), ys = bank_stride(F2);
  float *A = sm;                                      // [F2][max(bs, dv)]: Q (stride dv), then B (stride bs)
  float *Y = A + (size_t)F2 * (bs > dv ? bs : dv);    // [F2][ys]: R(i, j) at Y[j ys + i], then the rotations
  float *sg = Y + (size_t)F2 * ys;                    // [F2]: frozen sigma, later the column norms
  float *dt = sg + F2;                                // [F2]: dot products
  int *perm = reinterpret_cast<int *>(dt + F2);       // [F2]
  float *ctl = reinterpret_cast<float *>(perm + F2);  // [2]
  int *flag = reinterpret_cast<int *>(ctl + 2);       // [2]: rotation seen, per sweep parity
  // where Q is parked: fp32 factors park it in the frozen v slots; fp16 factors would round it, so
  // they park it in LDS after the other arrays ([F2][d_v]); the asynchronous form must not write
  // the rings and parks it in its own staging rows (fp32), keeping the LDS of the in-place form
  constexpr bool kHalf = !std::is_same<F, float>::value;
  const size_t sbase = (size_t)blockIdx.x * a.fmax;  // staging rows of this member
  float *QL = sm + ((reinterpret_cast<float *>(flag + 2) - sm + 3) & ~(ptrdiff_t)3);  // float4-aligned
  const int64_t capF = a.frz.cap;
  const int off_f = uniform(m.off_f);
  const int dk4 = dk >> 2, dv4 = dv >> 2;
  auto qpark = [&](int j) -> float * {
    if (staged) return a.st_v + (sbase + j) * dv;
    return kHalf ? QL + (size_t)j * dv : reinterpret_cast<float *>(a.frz.V<F>()) + wrap(off_f + j, capF) * dv;
  };

  // ---- 1. stage V_F --------------------------------------------------------------------------
  for (int j = tid; j < rf; j += kCT) sg[j] = a.frz.s[wrap(off_f + j, capF)];
  for (int e = tid; e < F2 * ys; e += kCT) Y[e] = 0.f;
  if (tid < 2) flag[tid] = 0;
  for (int e = tid; e < rf * dv4; e += kCT) {
    const int j = e / dv4, c = e - j * dv4;
    st4(A + (size_t)j * dv + 4 * c, ldf4(a.frz.V<F>() + wrap(off_f + j, capF) * dv + 4 * c));
  }
  __syncthreads();
  float s0 = sg[0];
  if (ra > 0) s0 = fmaxf(s0, a.act.s[m.off_a]);
  const float thr = a.eps[s] * s0;

  // ---- 2. CGS2 thin QR of V_F ----------------------------------------------------------------
  for (int j = 0; j < rf; ++j) {
    float *qj = A + (size_t)j * dv;
    for (int pass = 0; pass < 2; ++pass) {
      const int hi = pass == 0 ? j + 1 : j;  // the first pass also takes |q_j|^2 (i = j)
      for (int i = w; i < hi; i += 4) {
        const float *qi = A + (size_t)i * dv;
        float x = 0.f;
        for (int e = lane; e < dv; e += 64) x = fmaf(qi[e], qj[e], x);
        x = wave_sum_u(x);
        if (lane == 0) dt[i] = x;
      }
      __syncthreads();
      if (tid < dv) {
        float x = qj[tid];
#pragma unroll 8
        for (int i = 0; i < j; ++i) x = fmaf(-dt[i], A[(size_t)i * dv + tid], x);
        qj[tid] = x;
      }
      if (tid < j) Y[(size_t)j * ys + tid] += dt[tid];
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
    if (tid == 0) Y[(size_t)j * ys + j] = keep ? su : 0.f;
    __syncthreads();
  }
  // park Q (V_F has been consumed)
  for (int e = tid; e < rf * dv4; e += kCT) {
    const int j = e / dv4, c = e - j * dv4;
    st4(qpark(j) + 4 * c, ld4(A + (size_t)j * dv + 4 * c));
  }
  __syncthreads();

  // ---- 3. B = U_F diag(sigma_F) R^T into A, then Y <- I --------------------------------------
  for (int e = tid; e < rf * dk4; e += kCT) {
    const int j = e / dk4, c = e - j * dk4;
    st4(A + (size_t)j * bs + 4 * c, scale4(sg[j], ldf4(a.frz.U<F>() + wrap(off_f + j, capF) * dk + 4 * c)));
  }
  if (rf & 1)  // an odd count is paired with a zero column in the Jacobi
    for (int e = tid; e < dk; e += kCT) A[(size_t)rf * bs + e] = 0.f;
  __syncthreads();
  if (tid < dk) {
    for (int jp = 0; jp < rf; ++jp) {  // column jp reads columns >= jp only: in place, row-private
      float acc = 0.f;
#pragma unroll 8
      for (int i = jp; i < rf; ++i) acc = fmaf(A[(size_t)i * bs + tid], Y[(size_t)i * ys + jp], acc);
      A[(size_t)jp * bs + tid] = acc;
    }
  }
  __syncthreads();
  for (int e = tid; e < F2 * ys; e += kCT) {
    const int c = e / ys;
    Y[e] = (e - c * ys) == c ? 1.f : 0.f;
  }
  __syncthreads();

  // ---- 4. one-sided Jacobi on B's columns ----------------------------------------------------
  const int M = (rf + 1) & ~1;
  int sweeps = 0;
  if (M >= 2) {
    const int np = M >> 1, rounds = M - 1, grp = tid >> 3, sub = tid & 7;
    float *nrm = dt;  // the carried squared column norms (dt is free after the QR)
    const float tol2 = kTolJ * kTolJ;
    for (int sw = 0; sw < kConsSweeps; ++sw) {
      ++sweeps;
      int *fl = flag + (sw & 1);
      for (int j = w; j < M; j += 4) {
        const float *bj = A + (size_t)j * bs;
        float x = 0.f;
        for (int e = lane; e < dk; e += 64) x = fmaf(bj[e], bj[e], x);
        x = wave_sum_u(x);
        if (lane == 0) nrm[j] = x;
      }
      __syncthreads();
      for (int k = 0; k < rounds; ++k) {
        for (int p = grp; p < np; p += kCT / 8) {
          const int ci = p == 0 ? k : (k + p) % (M - 1);
          const int cj = p == 0 ? M - 1 : (k - p + (M - 1)) % (M - 1);
          float *x = A + (size_t)ci * bs, *y = A + (size_t)cj * bs;
          float xr[KE], yr[KE];
#pragma unroll
          for (int t = 0; t < KE; ++t) {  // all loads in flight at once (clamped index, then select)
            const int e = sub + 8 * t, ec = e < dk ? e : 0;
            xr[t] = self(e < dk, x[ec]);
            yr[t] = self(e < dk, y[ec]);
          }
          float gg = 0.f;
#pragma unroll
          for (int t = 0; t < KE; ++t) gg = fmaf(xr[t], yr[t], gg);
          gg = group_sum<8>(gg);
          const float aa = nrm[ci], bb = nrm[cj];
          // |a b|: a carried norm may round below zero; then g = 0 must still not rotate
          const bool rot = gg * gg > tol2 * fabsf(aa * bb);
          if (rot) {
            // t = tan of the rotation angle that zeroes x'.y', the root of smaller magnitude, in
            // Rutishauser's form: t = sign(d) 2 g / (|d| + sqrt(d^2 + 4 g^2)), d = b - a
            const float d = bb - aa, g2 = gg + gg;
            const float t = (d < 0.f ? -g2 : g2) * __builtin_amdgcn_rcpf(fabsf(d) + __builtin_amdgcn_sqrtf(fmaf(d, d, g2 * g2)));
            const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), sn = c * t;
            float *yx = Y + (size_t)ci * ys, *yy = Y + (size_t)cj * ys;
            float ux[KE], uy[KE];
#pragma unroll
            for (int q = 0; q < KE; ++q) {
              const int e = sub + 8 * q, ec = e < rf ? e : 0;
              ux[q] = yx[ec];
              uy[q] = yy[ec];
            }
#pragma unroll
            for (int q = 0; q < KE; ++q) {
              const int e = sub + 8 * q;
              if (e < dk) {
                x[e] = c * xr[q] - sn * yr[q];
                y[e] = sn * xr[q] + c * yr[q];
              }
              if (e < rf) {
                yx[e] = c * ux[q] - sn * uy[q];
                yy[e] = sn * ux[q] + c * uy[q];
              }
            }
            if (sub == 0) {
              nrm[ci] = fmaf(-t, gg, aa);
              nrm[cj] = fmaf(t, gg, bb);
              *fl = 1;
            }
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
    const float *bj = A + (size_t)j * bs;
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
    const float x = A[(size_t)j * bs + i] * (1.0f / sg[j]);
    if (staged) a.st_u[(sbase + k) * dk + i] = x;
    else stf(a.frz.U<F>() + wrap(off_f + k, capF) * dk + i, x);
  }
  if (tid < kept) {
    if (staged) a.st_s[sbase + tid] = sg[perm[tid]];
    else a.frz.s[wrap(off_f + tid, capF)] = sg[perm[tid]];
  }
  __syncthreads();  // B is consumed: bring Q back into A
  for (int e = tid; e < rf * dv4; e += kCT) {
    const int j = e / dv4, c = e - j * dv4;
    st4(A + (size_t)j * dv + 4 * c, ld4(qpark(j) + 4 * c));
  }
  __syncthreads();
  for (int e = tid; e < kept * dv; e += kCT) {
    const int k = e / dv, i = e - k * dv, j = perm[k];
    const float *yj = Y + (size_t)j * ys;
    float acc = 0.f;
#pragma unroll 8
    for (int c = 0; c < rf; ++c) acc = fmaf(A[(size_t)c * dv + i], yj[c], acc);
    if (staged) a.st_v[(sbase + k) * dv + i] = acc;
    else stf(a.frz.V<F>() + wrap(off_f + k, capF) * dv + i, acc);
  }
  if (tid == 0) {
    if (staged) a.st_cnt[blockIdx.x] = kept;
    else a.meta[s].packed = meta_pack(ra, kept, n, meta_flags(packed));
    const unsigned long long f = (unsigned long long)rf * rf;
    const unsigned long long flops = 4ull * dv * f + (unsigned long long)dk * f +
                                     (unsigned long long)sweeps * (rf * (rf - 1) / 2) * (12ull * dk + 6ull * rf) +
                                     2ull * dv * rf * kept;
    const int slot = blockIdx.x % kAcctSlots;
    atomicAdd(a.acct_flops + slot, flops);
    atomicAdd(a.acct_states + slot, 1ull);
    if (!staged) atomicAdd(a.acct_removed + slot, (unsigned long long)(rf - kept));
  }
}

template <typename F>
hipError_t consolidate_f(const ConsolidateArgs &a, int need, size_t sh, hipStream_t st) {
  const dim3 g((unsigned)a.n_members), b(kCT);
  if (need <= 16) hipLaunchKernelGGL((k_consolidate<2, F>), g, b, sh, st, a);
  else if (need <= 32) hipLaunchKernelGGL((k_consolidate<4, F>), g, b, sh, st, a);
  else if (need <= 64) hipLaunchKernelGGL((k_consolidate<8, F>), g, b, sh, st, a);
  else if (need <= 128) hipLaunchKernelGGL((k_consolidate<16, F>), g, b, sh, st, a);
  else hipLaunchKernelGGL((k_consolidate<32, F>), g, b, sh, st, a);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_cons_snapshot(const Meta *meta, const int32_t *members, int32_t n,
                                                       Meta *snap) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) snap[i] = meta[members[i]];
}

// one wavefront per member: the staged frozen part replaces the stored one in place (it never has
// more components), where the record still matches the snapshot the result was computed from
template <typename F>
__global__ __launch_bounds__(256) void k_cons_install(InstallArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (i >= a.n_members) return;
  const int s = uniform(a.members[i]);
  const Meta m = a.meta[s], sm = a.snap[i];
  const uint32_t pk = (uint32_t)uniform((int)m.packed), spk = (uint32_t)uniform((int)sm.packed);
  const int rf0 = meta_rf(spk);
  if (rf0 == 0 || rf0 > a.fmax) return;  // the kernel skipped this state
  if ((meta_flags(pk) & FLAG_DENSE) || meta_ra(pk) != meta_ra(spk) || meta_rf(pk) != meta_rf(spk)) return;
  const int kept = uniform(a.st_cnt[i]);
  const int64_t capF = a.frz.cap, off_f = uniform(m.off_f);
  const size_t sbase = (size_t)i * a.fmax;
  const int dk = a.dk, dv = a.dv;
  for (int k = 0; k < kept; ++k) {
    const int64_t c = wrap(off_f + k, capF);
    for (int e = lane; e < dk; e += 64) stf(a.frz.U<F>() + c * dk + e, a.st_u[(sbase + k) * dk + e]);
    for (int e = lane; e < dv; e += 64) stf(a.frz.V<F>() + c * dv + e, a.st_v[(sbase + k) * dv + e]);
    if (lane == 0) a.frz.s[c] = a.st_s[sbase + k];
  }
  if (lane == 0) {
    a.meta[s].packed = meta_pack(meta_ra(pk), kept, meta_n(pk), meta_flags(pk));
    atomicAdd(a.acct_removed + (s & (kAcctSlots - 1)), (unsigned long long)(rf0 - kept));
    atomicAdd(a.installed, 1u);
  }
}

// Host-core form, download side: one wavefront per member copies the frozen part the snapshot
// record names (u, v, sigma, as fp32) into the member's staging rows, and the state's sigma_0
// (the larger of its first active and first frozen value); cnt is the frozen count, or 0 for a
// state the consolidation leaves alone (dense, no frozen part, or more than fmax components).
template <typename F>
__global__ __launch_bounds__(256) void k_cons_gather(GatherArgs a) {
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (i >= a.n_members) return;
  const Meta m = a.snap[i];
  const uint32_t pk = (uint32_t)uniform((int)m.packed);
  const int ra = meta_ra(pk), rf = meta_rf(pk);
  const bool ok = !(meta_flags(pk) & FLAG_DENSE) && rf > 0 && rf <= a.fmax;
  if (lane == 0) a.st_cnt[i] = ok ? rf : 0;
  if (!ok) return;
  const int64_t capF = a.frz.cap, off_f = uniform(m.off_f);
  const size_t sbase = (size_t)i * a.fmax;
  const int dk = a.dk, dv = a.dv;
  for (int k = 0; k < rf; ++k) {
    const int64_t c = wrap(off_f + k, capF);
    for (int e = lane; e < dk; e += 64) a.st_u[(sbase + k) * dk + e] = ldf(a.frz.U<F>() + c * dk + e);
    for (int e = lane; e < dv; e += 64) a.st_v[(sbase + k) * dv + e] = ldf(a.frz.V<F>() + c * dv + e);
    if (lane == 0) a.st_s[sbase + k] = a.frz.s[c];
  }
  if (lane == 0) {
    const float s_act = ra > 0 ? a.act.s[wrap((int64_t)m.off_a, a.act.cap)] : 0.f;
    const float s_frz = a.frz.s[wrap(off_f, capF)];
    a.st_s0[i] = s_act > s_frz ? s_act : s_frz;
  }
}

}  // namespace

hipError_t launch_cons_gather(const GatherArgs &a, hipStream_t st) {
  if (a.n_members <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_members + 3) / 4)), block(256);
  if (a.frz.half) hipLaunchKernelGGL(k_cons_gather<_Float16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_cons_gather<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_cons_snapshot(const Meta *meta, const int32_t *members, int32_t n, Meta *snap, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cons_snapshot, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, meta, members, n, snap);
  return hipGetLastError();
}

hipError_t launch_cons_install(const InstallArgs &a, hipStream_t st) {
  if (a.n_members <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_members + 3) / 4)), block(256);
  if (a.frz.half) hipLaunchKernelGGL(k_cons_install<_Float16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_cons_install<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

size_t consolidate_lds_bytes(int dk, int dv, int fmax, bool q_in_lds) {
  const int F2 = (fmax + 1) & ~1, bs = bank_stride(dk);
  return sizeof(float) * ((size_t)F2 * (bs > dv ? bs : dv) + (size_t)F2 * bank_stride(F2) + 3 * (size_t)F2 + 4 +
                          (q_in_lds ? (size_t)F2 * dv + 4 : 0));
}

hipError_t launch_consolidate(const ConsolidateArgs &a, hipStream_t st) {
  if (a.n_members <= 0 || a.fmax <= 0) return hipSuccess;
  const size_t sh = consolidate_lds_bytes(a.dk, a.dv, a.fmax, a.frz.half != 0 && a.st_u == nullptr);
  if (sh > kConsolidateLdsMax) return hipErrorInvalidValue;
  const int need = a.dk > a.fmax ? a.dk : a.fmax;  // elements of a column pair: 8 lanes x KE
  if (need > 256) return hipErrorInvalidValue;
  return a.frz.half ? consolidate_f<_Float16>(a, need, sh, st) : consolidate_f<float>(a, need, sh, st);
}

}  // namespace ss
