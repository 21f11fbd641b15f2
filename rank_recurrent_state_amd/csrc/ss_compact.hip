// ss_compact.hip -- Brand compaction, dense materialization, pool scatter.
//
// Compaction (SinkState 3.2 Design 1 and 4.2 "(ii) Top-subspace SVD"): one
// 64-lane wavefront per state of the group, four states per workgroup.
//   1. U_C = [U_active | pad keys] (d_k x m), V_C = [V_active | pad w]
//      (d_v x m), weights Gamma * (sigma_active, c); m = r_a + n <= 16.
//      The d_k side of every column lives on lanes 0-31, the d_v side on
//      lanes 32-63, four consecutive elements per lane and float4 block.
//   2. Thin QR of both sides by classical Gram-Schmidt, a second projection
//      pass only for a column whose first pass kept less than a tenth of its
//      squared norm; a column whose residual is at most 1e-5 of its own norm
//      is taken as dependent and zeroed (its R row is then zero too, so it
//      cannot create a spurious component).
//   3. Core C = R_L diag(w) R_R^T (m x m) in LDS.
//   4. One-sided (Hestenes) Jacobi SVD of C on its columns only: 8 lanes per
//      column pair, pairs in round-robin (circle) order so that m/2 disjoint
//      pairs rotate at once; sweeps until no pair is off-orthogonal by more
//      than 1e-6.  The right singular vectors follow from C afterwards.
//   5. Sort the local singular values; merge them with the frozen ones
//      (scaled by Gamma; with per-channel decay by |gamma u_f|, and sorted
//      again) in descending order, local first on ties; drop
//      sigma < eps * sigma_max and sigma = 0 (SinkState 4.1, 4.2 example).
//   6. U' = Q_L U_hat, V' = Q_R V_hat for the kept local components; kept
//      frozen components are copied.  The first r of the merged list go to
//      the group's other active segment, the rest to its other frozen segment.
//   7. With promotion on, a state left with more than L components is queued
//      for the dense region (SinkState 4.4).
// No global-memory intermediates: QR factors live in registers, the small
// matrices in LDS (SinkState 4.4: fused chains of factor algebra).
#include <hipcub/hipcub.hpp>

#include <type_traits>

#include "ss_internal.h"
#include "ss_linalg.h"
#include "ss_wave.h"

namespace ss {

namespace {

constexpr int kMaxFrozen = 256;  // frozen components per state (max_frozen <= 255)
// LDS per wavefront, in floats
constexpr int kOffRl = 0, kOffRr = 256, kOffCm = 512, kOffVh = 768, kOffScw = 1024, kOffSgs = 1040, kOffSraw = 1056,
              kOffPerm = 1072, kOffPosL = 1088, kOffFs = 1104, kOffPosF = kOffFs + kMaxFrozen,
              kLdsPerWave = kOffPosF + kMaxFrozen;
// per-channel decay adds, per wavefront: the frozen sigma before sorting, the sorted order, the norms
constexpr int kOffFraw = kLdsPerWave, kOffForig = kOffFraw + kMaxFrozen, kOffFnorm = kOffForig + kMaxFrozen,
              kLdsPerWaveDiag = kOffFnorm + kMaxFrozen;

// A member's slots in its group's new ring segments: upper bounds of its new active and frozen
// counts that the stored record already fixes, so that every member's place in the segment is a
// prefix sum taken before the compaction runs (no allocation inside it).  A merge keeps at most
// ra + rf + n components and at most r + fcap, the first r of them active; a state moved unchanged
// keeps ra and rf.  With the ring's invariant (frozen components only behind a full active part)
// neither bound exceeds the old slot plus the pad size K, which bounds the ring usage on the host.
__device__ __forceinline__ void slot_sizes(int ra, int rf, int n, int r, int fcap, int &sa, int &sf) {
  int t = ra + rf + n;
  if (t > r + fcap) t = r + fcap;
  const int ta = t < r ? t : r;
  sa = ta > ra ? ta : ra;
  sf = t - ta > rf ? t - ta : rf;
}

// copy one fp32 component (u, v) into factor storage of type F, with float4 lanes
template <typename F>
__device__ __forceinline__ void copy_comp(const float *su, const float *sv, F *du, F *dv_, int dk, int dv, int lane) {
  const int dk4 = dk >> 2, tot = dk4 + (dv >> 2);
  for (int e = lane; e < tot; e += 64) {
    if (e < dk4) stf4(du + 4 * e, ld4(su + 4 * e));
    else stf4(dv_ + 4 * (e - dk4), ld4(sv + 4 * (e - dk4)));
  }
}

// streaming store into factor storage: the copied components are read again only by the next
// decode step, after the rest of the compaction has gone through the caches
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stf4nt(float *p, float4 v) {
  const f32x4_t x = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(x, reinterpret_cast<f32x4_t *>(p));
}
__device__ __forceinline__ void stf4nt(_Float16 *p, float4 v) {
  half4_t h;
  h.x = (_Float16)v.x;
  h.y = (_Float16)v.y;
  h.z = (_Float16)v.z;
  h.w = (_Float16)v.w;
  __builtin_nontemporal_store(h, reinterpret_cast<half4_t *>(p));
}

__device__ __forceinline__ void stfnt(float *p, float v) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void stfnt(_Float16 *p, float v) { __builtin_nontemporal_store((_Float16)v, p); }
__device__ __forceinline__ float ldfnt(const float *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ float ldfnt(const _Float16 *p) { return (float)__builtin_nontemporal_load(p); }

// Copy `cnt` components (u, v) starting at ring position c0 of arena `src`
// to the positions dst_of(f) (a component for which it returns false is dropped).
// A component is d_k / 4 + d_v / 4 float4 chunks (u's, then v's); lane l moves chunks l, l + 64, ...
// of every component, so its offsets inside a component are fixed and only the component's slots
// (wave-uniform) change from one to the next.  UNC components per round keep their loads in flight
// together; the source is read once and the destination written once, both with the nontemporal
// hint.  dst_of is called with a wave-uniform f by every lane.
template <typename F, typename DstOf>
__device__ __forceinline__ void copy_comps(const Arena &src, int64_t c0, int cnt, int dk, int dv, int lane,
                                           DstOf dst_of) {
  constexpr int UNC = 4;
  const int dk4 = dk >> 2, tot4 = dk4 + (dv >> 2);
  for (int cb = 0; cb < tot4; cb += 64) {
    const int c = cb + lane;
    const bool on = c < tot4;
    const bool isu = c < dk4;
    const int off = !on ? 0 : (isu ? 4 * c : 4 * (c - dk4));  // element offset inside u or v (0 when off)
    const F *sbase = (isu ? src.U<F>() : src.V<F>()) + off;     // this lane's side, taken once
    const uint32_t sd = isu ? (uint32_t)dk : (uint32_t)dv;
    for (int f0 = 0; f0 < cnt; f0 += UNC) {
      float4 x[UNC];
#pragma unroll
      for (int q = 0; q < UNC; ++q) {
        const int f = f0 + q < cnt ? f0 + q : cnt - 1;  // clamped (cnt >= 1 inside the loop)
        const int64_t cs = wrap(c0 + f, src.cap);
        x[q] = ldf4nt(sbase + cs * (int64_t)sd);
      }
#pragma unroll
      for (int q = 0; q < UNC; ++q) {
        if (f0 + q < cnt) {
          F *du, *dvp;
          if (dst_of(f0 + q, du, dvp) && on) stf4nt(isu ? du + off : dvp + off, x[q]);  // one 16-byte store
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Brand compaction with the two sides of a state split across the halves of its wavefront (one
// wavefront per state, four per workgroup).  Lanes [0, 32) hold the d_k side of every column
// ([U_a | K]), lanes [32, 64) the d_v side ([V_a | W]); a lane keeps NB float4 blocks of each
// column (element 128 b + 4 l + c of its side's vector in lane l of the half, block b, component
// c).  Both sides' Gram-Schmidt then runs as one instruction stream, and each pair of dot products
// (one per side) is one sum over 32 lanes.
//
// DIAG (per-channel decay): the state is diag(gamma) times its stored parts, gamma holding the
// decays accumulated per key channel since the last compaction.  The active columns and the pad
// keys enter the QR scaled by gamma; each frozen u_f is scaled by gamma and given unit norm again
// (sigma_f takes the norm), and the frozen list is sorted again by the new sigma (stored order on
// ties) before the merge; gamma is reset to 1.
// ---------------------------------------------------------------------------------------------
template <int NB>
__device__ __forceinline__ float dotb(const float4 (&x)[NB], const float4 (&y)[NB]) {
  float acc = dot4(x[0], y[0]);
#pragma unroll
  for (int b = 1; b < NB; ++b) acc += dot4(x[b], y[b]);
  return acc;
}

template <int NB, typename F, bool DIAG>
__global__ __launch_bounds__(256) void k_compact_h(CompactArgs a) {
  __shared__ __align__(16) float lds[4][DIAG ? kLdsPerWaveDiag : kLdsPerWave];
  const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int side = lane >> 5, r = lane & 31;
  const int mi = blockIdx.x * 4 + w;
  float *Rl = lds[w] + kOffRl;
  float *Rr = lds[w] + kOffRr;
  float *Cm = lds[w] + kOffCm;
  float *Vh = lds[w] + kOffVh;
  float *scw = lds[w] + kOffScw;
  float *sgs = lds[w] + kOffSgs;
  float *sraw = lds[w] + kOffSraw;
  int *perm = reinterpret_cast<int *>(lds[w] + kOffPerm);
  int *posL = reinterpret_cast<int *>(lds[w] + kOffPosL);
  float *fsl = lds[w] + kOffFs;
  int *posF = reinterpret_cast<int *>(lds[w] + kOffPosF);
  const int dk = a.dk, dv = a.dv, K = a.K, rr_ = a.r;
  const int dme = side ? dv : dk;  // length of this lane's side of a column
  const int64_t capA = a.act.cap, capF = a.frz.cap;

  // ---- phase A: what this wave's state becomes -------------------------------------------
  bool live = mi < a.n_members;  // a member of the group held in factored form
  int s = 0, ra = 0, rf = 0, n = 0, off_a = 0, off_f = 0;
  uint32_t flags = 0;
  float gamma = 1.0f;
  if (live) {
    s = uniform(a.members[mi]);
    const Meta m = a.meta[s];
    const uint32_t packed = (uint32_t)uniform((int)m.packed);
    flags = meta_flags(packed);
    if (flags & FLAG_DENSE) {
      live = false;
    } else {
      ra = meta_ra(packed);
      rf = meta_rf(packed);
      n = meta_n(packed);
      off_a = uniform(m.off_a);
      off_f = uniform(m.off_f);
      gamma = uniformf(m.gamma);
    }
  }
  // an unselected member (compaction of listed states) keeps its pad and Gamma and only moves
  const bool keep = live && a.sel != nullptr && a.sel[s] == 0;
  const bool work = live && n > 0 && !keep;  // a Brand update; otherwise the components move unchanged
  const int mcol = ra + n;
  int kl = 0, kf = 0, total = 0, ra2 = ra, rf2 = rf, sweeps = 0;
  int proj = 0;  // column projections made by the Gram-Schmidt passes
  bool jlimit = false;
  float4 x[kMaxM][NB];
  // DIAG: the state's decays on this lane's rows of the d_k side, 1 on the d_v side and past d_k
  float4 g4[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) g4[b] = make_float4(1.f, 1.f, 1.f, 1.f);
  if (DIAG && work && side == 0) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int e = 128 * b + 4 * r;
      if (e < dk) g4[b] = ld4(a.gam + (int64_t)s * dk + e);
    }
  }
  if (work) {
    if constexpr (DIAG) {
      // the frozen singular values become sigma_f |gamma u_f| and their order is taken again
      // (descending, stored order on ties); the norms on the d_k half, four components in flight
      float *fraw = lds[w] + kOffFraw, *fnrm = lds[w] + kOffFnorm;
      int *forig = reinterpret_cast<int *>(lds[w] + kOffForig);
      for (int f0 = 0; f0 < rf; f0 += 4) {
        float4 y[4][NB];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int f = f0 + c < rf ? f0 + c : rf - 1;  // clamped (rf >= 1 inside the loop)
          const F *fu = a.frz.U<F>() + wrap(off_f + f, capF) * dk;
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const int e = 128 * b + 4 * r;
            y[c][b] = zero4();
            if (side == 0 && e < dk) {
              const float4 t = ldf4nt(fu + e);
              y[c][b] = make_float4(t.x * g4[b].x, t.y * g4[b].y, t.z * g4[b].z, t.w * g4[b].w);
            }
          }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float nn = group_sum<32>(dotb<NB>(y[c], y[c]));  // lanes of the d_k half
          if (lane == 0 && f0 + c < rf) fnrm[f0 + c] = sqrtf(nn);
        }
      }
      wave_sync();
      for (int f = lane; f < rf; f += 64) fraw[f] = a.frz.s[wrap(off_f + f, capF)] * fnrm[f];
      wave_sync();
      for (int f = lane; f < rf; f += 64) {
        const float xv = fraw[f];
        int rk = 0;
        for (int g = 0; g < rf; ++g) {
          const float yv = fraw[g];
          rk += (yv > xv) || (yv == xv && g < f);
        }
        fsl[rk] = xv;
        forig[rk] = f;
      }
      wave_sync();
    } else {
      // frozen singular values (scaled by Gamma) to LDS: the merge searches them there
      for (int f = lane; f < rf; f += 64) fsl[f] = a.frz.s[wrap(off_f + f, capF)] * gamma;
    }
    // columns: [U_a | K] on the d_k lanes, [V_a | W] on the d_v lanes; this lane's side's arena and
    // pad bases and row length are taken once, so a column costs one multiply-add per address
    {
      const F *act_b = side ? a.act.V<F>() : a.act.U<F>();
      const float *pad_b = (side ? a.pw : a.pk) + (int64_t)s * K * dme;
#pragma unroll
      for (int jj = 0; jj < kMaxM; ++jj) {
        const bool valid = jj < mcol;
        const int j = valid ? jj : mcol - 1;  // clamped: the loads stay in bounds (mcol >= 1 here)
        const bool isact = j < ra;
        const int64_t ca = wrap(off_a + (isact ? j : 0), capA);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = 128 * b + 4 * r;
          const bool ok = valid && e < dme;
          const int eo = e < dme ? e : 0;
          float4 v;
          if (isact) {  // wave-uniform branch
            v = ldf4nt(act_b + ca * dme + eo);
          } else {
            v = ld4nt(pad_b + (j - ra) * dme + eo);
          }
          if constexpr (DIAG) v = make_float4(v.x * g4[b].x, v.y * g4[b].y, v.z * g4[b].z, v.w * g4[b].w);
          x[jj][b] = sel4(ok, v);  // DIAG: active columns and pad keys carry the decays
        }
      }
    }
    if (lane < kMaxM) {
      float wgt = 0.f;
      if (lane < ra) wgt = a.act.s[wrap(off_a + lane, capA)] * gamma;
      else if (lane < mcol) wgt = a.pc[(int64_t)s * K + (lane - ra)] * gamma;
      scw[lane] = wgt;
    }
    // Gram-Schmidt of both sides at once with selective reorthogonalization (the test of Daniel,
    // Gragg, Kaufman and Stewart, 1976, with a lower threshold): one classical pass leaves along the
    // earlier columns a rounding residue of a few unit roundoffs times the column's input norm, so
    // relative to what remains it is that residue times sqrt(n0 / nu).  A second pass runs only when
    // the first one kept less than kReorth2 of the squared norm, i.e. when that factor exceeds
    // sqrt(10) (for both sides at once, so the wave stays uniform); above it one pass is orthogonal
    // to a few unit roundoffs already.  R goes to LDS row-major, R[i * 16 + jj] = R(i, jj).  A
    // column whose residual is at most 1e-5 of its input norm is dependent: it and its R row are
    // zeroed.
    float *Rs = side ? Rr : Rl;
#pragma unroll
    for (int jj = 0; jj < kMaxM; ++jj) {
      if (jj < mcol) {
        const float n0 = group_sum<32>(dotb<NB>(x[jj], x[jj]));
        float nu = n0;
        if (jj > 0) {
          float du[kMaxM];  // R(i, jj), i < jj: the same value in every lane of the side
#pragma unroll
          for (int i = 0; i < jj; ++i) du[i] = group_sum<32>(dotb<NB>(x[i], x[jj]));
#pragma unroll
          for (int i = 0; i < jj; ++i) {
#pragma unroll
            for (int b = 0; b < NB; ++b) x[jj][b] = fma4(-du[i], x[i][b], x[jj][b]);
          }
          nu = group_sum<32>(dotb<NB>(x[jj], x[jj]));
          proj += jj;
          if (__builtin_amdgcn_ballot_w64(nu < kReorth2 * n0) != 0ull) {  // the second pass (wave-uniform)
#pragma unroll
            for (int i = 0; i < jj; ++i) {
              const float e = group_sum<32>(dotb<NB>(x[i], x[jj]));
#pragma unroll
              for (int b = 0; b < NB; ++b) x[jj][b] = fma4(-e, x[i][b], x[jj][b]);
              du[i] += e;
            }
            nu = group_sum<32>(dotb<NB>(x[jj], x[jj]));
            proj += jj;
          }
          if (r == 0) {  // one lane per side writes the column's entries above the diagonal
#pragma unroll
            for (int i = 0; i < jj; ++i) Rs[i * 16 + jj] = du[i];
          }
        }
        const bool kk = nu > 0.f && nu > kTau2 * n0;
        const float su = sqrtf(nu);
        const float iv = kk ? 1.0f / su : 0.f;
#pragma unroll
        for (int b = 0; b < NB; ++b) x[jj][b] = scale4(iv, x[jj][b]);
        if (r < kMaxM && r >= jj) Rs[r * 16 + jj] = r == jj ? (kk ? su : 0.f) : 0.f;
      } else {
#pragma unroll
        for (int b = 0; b < NB; ++b) x[jj][b] = zero4();
        if (r < kMaxM) Rs[r * 16 + jj] = 0.f;
      }
    }
    wave_sync();
    // core C = R_L diag(w) R_R^T: lane l forms C(i, j) for i = l mod 16 and the four j = l / 16 + 4 q
    // from row i of R_L and rows j of R_R (both upper triangular, so the sum over t runs over
    // t >= max(i, j); the zero terms below it leave the sum unchanged).  C goes to Vh column-major
    // (kept: the rotations are recovered from it below) and, in jacobi16c's layout, over R_L and R_R
    // once every lane has read them.
    float *Bj = Rl;  // Rl and Rr: 512 floats
    {
      const int i = lane & 15, j0 = lane >> 4;
      float cv[4];
      float rl[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a4 = *reinterpret_cast<const float4 *>(Rl + i * 16 + 4 * q);
        const float4 w4 = *reinterpret_cast<const float4 *>(scw + 4 * q);
        rl[4 * q] = a4.x * w4.x;
        rl[4 * q + 1] = a4.y * w4.y;
        rl[4 * q + 2] = a4.z * w4.z;
        rl[4 * q + 3] = a4.w * w4.w;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 4 * q;
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float4 b4 = *reinterpret_cast<const float4 *>(Rr + j * 16 + 4 * h);
          acc = fmaf(rl[4 * h], b4.x, acc);
          acc = fmaf(rl[4 * h + 1], b4.y, acc);
          acc = fmaf(rl[4 * h + 2], b4.z, acc);
          acc = fmaf(rl[4 * h + 3], b4.w, acc);
        }
        cv[q] = acc;
      }
      wave_sync();
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 4 * q;
        Vh[j * 16 + i] = cv[q];
        Bj[j * 32 + 4 * (i >> 1) + (i & 1)] = cv[q];
      }
    }
    wave_sync();
    sweeps = jacobi16c(Bj, mcol, lane, &jlimit);
    // the singular values s_j = |b_j| and the left singular vectors u_j = b_j / s_j of C, to Cm
    // column-major: lane l takes rows 4 (l & 3) to 4 (l & 3) + 3 of column l / 4 (a column with
    // s_j = 0 stays zero); 1 / s_j goes to sinv (over R_R, once every lane has read B)
    float *sinv = Rr;
    {
      const int col = lane >> 2;
      const float4 *q = reinterpret_cast<const float4 *>(Bj) + 8 * col + 2 * (lane & 3);
      const float4 u0 = q[0], u1 = q[1];
      const float sj = __builtin_amdgcn_sqrtf(
          group_sum<4>(fmaf(u0.x, u0.x, fmaf(u0.y, u0.y, fmaf(u1.x, u1.x, u1.y * u1.y)))));
      const float is = sj > 0.f ? __builtin_amdgcn_rcpf(sj) : 0.f;
      *reinterpret_cast<float4 *>(Cm + 16 * col + 4 * (lane & 3)) =
          make_float4(u0.x * is, u0.y * is, u1.x * is, u1.y * is);
      wave_sync();
      if ((lane & 3) == 0) {
        sraw[col] = col < mcol ? sj : -1.f;
        sinv[col] = is;
      }
    }
    wave_sync();
    // right singular vectors of C: V(:, j) = C^T b_j / s_j^2 = C^T u_j / s_j (see jacobi16c), lane l
    // forming rows l mod 16 of the four columns l / 16 + 4 q; C is read whole before V overwrites it
    {
      const int row = lane & 15, j0 = lane >> 4;
      float c0[16];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 a4 = *reinterpret_cast<const float4 *>(Vh + row * 16 + 4 * q);
        c0[4 * q] = a4.x;
        c0[4 * q + 1] = a4.y;
        c0[4 * q + 2] = a4.z;
        c0[4 * q + 3] = a4.w;
      }
      float vq[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = j0 + 4 * q;
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float4 b4 = *reinterpret_cast<const float4 *>(Cm + j * 16 + 4 * h);
          acc = fmaf(c0[4 * h], b4.x, acc);
          acc = fmaf(c0[4 * h + 1], b4.y, acc);
          acc = fmaf(c0[4 * h + 2], b4.z, acc);
          acc = fmaf(c0[4 * h + 3], b4.w, acc);
        }
        vq[q] = acc * sinv[j];
      }
      wave_sync();
#pragma unroll
      for (int q = 0; q < 4; ++q) Vh[(j0 + 4 * q) * 16 + row] = vq[q];
    }
    wave_sync();
    if (lane < mcol) {
      const float my = sraw[lane];
      int rank = 0;
      for (int i = 0; i < mcol; ++i) {
        const float o = sraw[i];
        rank += (o > my) || (o == my && i < lane);
      }
      perm[rank] = lane;
      sgs[rank] = my;
    }
    wave_sync();

    // merge with the frozen part and truncate: both lists are descending; on ties the local
    // component comes first; drop sigma < eps * sigma_max and sigma = 0
    const float smax = fmaxf(sgs[0], rf > 0 ? fsl[0] : 0.f);
    const float thr = a.eps[s] * smax;
    kl = __builtin_popcountll(__builtin_amdgcn_ballot_w64(lane < mcol && sgs[lane] >= thr && sgs[lane] > 0.f));
    for (int f0 = 0; f0 < rf; f0 += 64) {
      const int f = f0 + lane;
      kf += __builtin_popcountll(__builtin_amdgcn_ballot_w64(f < rf && fsl[f] >= thr && fsl[f] > 0.f));
    }
    total = kl + kf;
    const int cap_total = rr_ + a.fcap;
    if (total > cap_total) {
      if (lane == 0)
        __hip_atomic_fetch_add(&a.counters[C_CAP_TRUNC], (uint32_t)(total - cap_total), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
      total = cap_total;
    }
    ra2 = total < rr_ ? total : rr_;
    rf2 = total - ra2;
    if (lane < kl) {  // local i goes after the frozen ones strictly greater than it
      const float xv = sgs[lane];
      int lo = 0, hi = kf;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (fsl[mid] > xv) lo = mid + 1;
        else hi = mid;
      }
      posL[lane] = lane + lo;
    }
    for (int f = lane; f < kf; f += 64) {  // frozen f goes after the local ones >= it
      const float xv = fsl[f];
      int c = 0;
      for (int i = 0; i < kl; ++i) c += sgs[i] >= xv ? 1 : 0;
      posF[f] = f + c;
    }
    wave_sync();
  }

  // ---- placement: the member's slots in the group's new segments ---------------------------
  if (!live) return;
  {
    int sa, sf;
    slot_sizes(ra, rf, n, rr_, a.fcap, sa, sf);
    if (ra2 > sa || rf2 > sf) {  // cannot happen (the slots bound the counts); never overwrite a neighbour
      if (lane == 0) *a.hflag = 1u;
      return;
    }
  }
  const unsigned long long rel = a.slot_in[mi] + a.slot_blk[mi / kSlotBlock];
  const unsigned long long va = a.ring_a->begin + (rel & 0xffffffffull), vf = a.ring_f->begin + (rel >> 32);
  // the ring is full (the ring set-up has raised the pool's flag): the state keeps its old form
  if (va + ra2 > a.ring_a->limit || vf + rf2 > a.ring_f->limit) return;
  const int64_t dst_a = (int64_t)(va % (unsigned long long)capA), dst_f = (int64_t)(vf % (unsigned long long)capF);

  // ---- phase B: write the new components and the record ------------------------------------
  if (!work) {  // nothing buffered (or not selected): the components move unchanged
    copy_comps<F>(a.act, off_a, ra, dk, dv, lane, [&](int f, F *&du, F *&dvp) {
      const int64_t c = wrap(dst_a + f, capA);
      du = a.act.U<F>() + c * dk;
      dvp = a.act.V<F>() + c * dv;
      return true;
    });
    copy_comps<F>(a.frz, off_f, rf, dk, dv, lane, [&](int f, F *&du, F *&dvp) {
      const int64_t c = wrap(dst_f + f, capF);
      du = a.frz.U<F>() + c * dk;
      dvp = a.frz.V<F>() + c * dv;
      return true;
    });
    // an empty pad means Gamma = 1 (no step since the last compaction) and sigma takes it in;
    // an unselected member keeps Gamma with its pad
    const float gs = keep ? 1.0f : gamma;
    for (int f = lane; f < ra; f += 64) a.act.s[wrap(dst_a + f, capA)] = a.act.s[wrap(off_a + f, capA)] * gs;
    for (int f = lane; f < rf; f += 64) a.frz.s[wrap(dst_f + f, capF)] = a.frz.s[wrap(off_f + f, capF)] * gs;
    if (lane == 0) {
      Meta nm;
      nm.off_a = (int32_t)dst_a;
      nm.off_f = (int32_t)dst_f;
      nm.gamma = keep ? gamma : 1.0f;
      nm.packed = meta_pack(ra, rf, keep ? n : 0, flags);
      a.meta[s] = nm;
    }
    return;
  }
  // merged position pos -> slot of the new active (pos < r) or frozen component
  auto slot_u = [&](int pos) -> F * {
    return pos < rr_ ? a.act.U<F>() + wrap(dst_a + pos, capA) * dk : a.frz.U<F>() + wrap(dst_f + pos - rr_, capF) * dk;
  };
  auto slot_v = [&](int pos) -> F * {
    return pos < rr_ ? a.act.V<F>() + wrap(dst_a + pos, capA) * dv : a.frz.V<F>() + wrap(dst_f + pos - rr_, capF) * dv;
  };
  auto slot_s = [&](int pos) -> float * {
    return pos < rr_ ? a.act.s + wrap(dst_a + pos, capA) : a.frz.s + wrap(dst_f + pos - rr_, capF);
  };
  // kept local components: U' = Q_L U_hat (d_k lanes), V' = Q_R V_hat (d_v lanes)
  for (int i = 0; i < kl; ++i) {
    const int pos = uniform(posL[i]);  // i is wave-uniform
    if (pos >= total) continue;
    const int j = uniform(perm[i]);
    const float *cf = (side ? Vh : Cm) + j * 16;  // u_j or v_j of C
    float4 o[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) o[b] = zero4();
#pragma unroll
    for (int tt = 0; tt < kMaxM; ++tt) {
      const float c = cf[tt];
#pragma unroll
      for (int b = 0; b < NB; ++b) o[b] = fma4(c, x[tt][b], o[b]);
    }
    F *dst = side ? slot_v(pos) : slot_u(pos);
#pragma unroll
    for (int b = 0; b < NB; ++b) {  // rounded to the storage type here (fp16 factors: at every compaction)
      const int e = 128 * b + 4 * r;
      if (e < dme) stf4nt(dst + e, o[b]);
    }
  }
  if (lane < kl && posL[lane] < total) *slot_s(posL[lane]) = sgs[lane];
  if constexpr (DIAG) {
    // kept frozen components in sorted order: u <- gamma u / |gamma u|, v copied; gamma <- 1
    const float *fnrm = lds[w] + kOffFnorm;
    const int *forig = reinterpret_cast<const int *>(lds[w] + kOffForig);
    constexpr int FC = 4;  // components in flight: all loads of a batch are issued before its stores
    for (int f0 = 0; f0 < kf; f0 += FC) {
      float4 y[FC][NB];
#pragma unroll
      for (int c = 0; c < FC; ++c) {
        const int f = f0 + c < kf ? f0 + c : kf - 1;  // clamped (kf >= 1 inside the loop)
        const int64_t cs = wrap(off_f + uniform(forig[f]), capF);  // f is wave-uniform
        const F *src = side ? a.frz.V<F>() + cs * dv : a.frz.U<F>() + cs * dk;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = 128 * b + 4 * r;
          y[c][b] = ldf4nt(src + (e < dme ? e : 0));
        }
      }
#pragma unroll
      for (int c = 0; c < FC; ++c) {
        const int f = f0 + c;
        if (f >= kf) break;
        const int pos = uniform(posF[f]);  // f is wave-uniform
        if (pos >= total) continue;
        const float inv = side ? 1.f : __builtin_amdgcn_rcpf(uniformf(fnrm[uniform(forig[f])]));
        F *dst = side ? slot_v(pos) : slot_u(pos);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int e = 128 * b + 4 * r;
          const float4 t = y[c][b];
          if (e < dme)
            stf4nt(dst + e, make_float4(t.x * g4[b].x * inv, t.y * g4[b].y * inv, t.z * g4[b].z * inv,
                                        t.w * g4[b].w * inv));
        }
      }
    }
    if (side == 0) {
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        const int e = 128 * b + 4 * r;
        if (e < dk) st4(a.gam + (int64_t)s * dk + e, make_float4(1.f, 1.f, 1.f, 1.f));
      }
    }
  } else {
    // kept frozen components: copied, sigma scaled by Gamma
    copy_comps<F>(a.frz, off_f, kf, dk, dv, lane, [&](int f, F *&du, F *&dvp) {
      const int pos = uniform(posF[f]);  // f is wave-uniform
      if (pos >= total) return false;
      du = slot_u(pos);
      dvp = slot_v(pos);
      return true;
    });
  }
  for (int f = lane; f < kf; f += 64) {
    const int pos = posF[f];
    if (pos < total) *slot_s(pos) = fsl[f];
  }
  if (lane == 0) {
    Meta nm;
    nm.off_a = (int32_t)dst_a;
    nm.off_f = (int32_t)dst_f;
    nm.gamma = 1.0f;
    nm.packed = meta_pack(ra2, rf2, 0, flags);
    a.meta[s] = nm;
    if (a.promote && total > a.L) {
      const uint32_t idx =
          __hip_atomic_fetch_add(&a.counters[C_PROMOTE_COUNT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.promote_list[idx] = s;
    }
    if (jlimit) __hip_atomic_fetch_add(&a.counters[C_JACOBI_LIMIT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long D = (unsigned long long)(dk + dv), mm = (unsigned long long)mcol;
    const unsigned long long flops = 4ull * D * (unsigned long long)proj + 4ull * mm * mm * mm +
                                     6ull * mm * mm * (mm - 1) * (unsigned long long)sweeps +
                                     2ull * D * mm * (unsigned long long)kl;
    __hip_atomic_fetch_add(&a.acct_flops[s & (kAcctSlots - 1)], flops, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_add(&a.acct_states[s & (kAcctSlots - 1)], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Materialize dense states into new slots of the dense region, stored as
// H = S^T row-major [d_v][d_k]: H[j][i] = sum_c sigma_c v_c[j] u_c[i].  Three launches:
//   k_mat_reserve  one thread: the states of the list take consecutive slots from the
//                  dense count (base + list index);
//   k_mat_rows     one workgroup per (state, block of RPB rows), so a few promotions still
//                  spread over many CUs: thread t owns float4 column t % (d_k/4) of rows
//                  t / (d_k/4) + RG * jj (jj < kMatRows); components are staged through
//                  LDS in chunks of kMatCH (u whole, v only the block's rows);
//   k_mat_finish   one thread per state: the dense record, the slot record, the slot's
//                  per-channel decays (set to 1), counters.
// The state's record is rewritten only by the last launch, after every row block has read
// where its components are.
constexpr int kMatCH = 16;
constexpr int kMatRows = 2;

__device__ __forceinline__ uint32_t mat_count(const MaterializeArgs &a) {
  return a.count ? *a.count : (uint32_t)a.fixed_count;
}

__global__ void k_mat_reserve(MaterializeArgs a) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const uint32_t base = a.counters[C_DENSE_COUNT];
  a.counters[C_MAT_BASE] = base;
  a.counters[C_DENSE_COUNT] = base + mat_count(a);  // may pass cap_d: readers clamp, k_mat_finish reports it
}

template <typename F>
__global__ __launch_bounds__(256) void k_mat_rows(MaterializeArgs a, int RB) {
  extern __shared__ float smem[];
  const int t = threadIdx.x;
  const int dk = a.dk, dv = a.dv;
  const int C4 = dk >> 2, RG = 256 / C4, RPB = RG * kMatRows;
  const int c = t % C4, g = t / C4;
  const bool act = t < RG * C4;
  float *su = smem;                  // [CH][dk]
  float *sv = smem + kMatCH * dk;    // [CH][RPB]
  float *ss = sv + kMatCH * RPB;     // [CH]
  const uint32_t cnt = mat_count(a);
  const uint32_t base = a.counters[C_MAT_BASE];
  for (int64_t idx = blockIdx.x; idx < (int64_t)cnt * RB; idx += gridDim.x) {  // uniform over the block
    const int li = (int)(idx / RB), rb = (int)(idx - (int64_t)li * RB);
    const int64_t slot = (int64_t)base + li;
    if (slot >= a.cap_d) continue;  // k_mat_finish reports it
    const int s = a.list[li];
    const Meta m = a.meta[s];
    int n1, n2;
    int64_t o0 = 0;
    float scale = 1.0f;
    if (a.csr_off) {
      o0 = a.csr_off[s];
      n1 = (int)(a.csr_off[s + 1] - o0);
      n2 = 0;
    } else {
      n1 = (int)meta_ra(m.packed);
      n2 = (int)meta_rf(m.packed);
      scale = m.gamma;
    }
    // element i of u (or v) of component comp: the CSR row (initial states) or the ring slot
    auto comp_u = [&](int comp, int i) -> float {
      if (a.csr_off) return a.csr_u[(o0 + comp) * dk + i];
      return ldf(comp < n1 ? a.act.U<F>() + wrap(m.off_a + comp, a.act.cap) * dk + i
                           : a.frz.U<F>() + wrap(m.off_f + comp - n1, a.frz.cap) * dk + i);
    };
    auto comp_v = [&](int comp, int j) -> float {
      if (a.csr_off) return a.csr_v[(o0 + comp) * dv + j];
      return ldf(comp < n1 ? a.act.V<F>() + wrap(m.off_a + comp, a.act.cap) * dv + j
                           : a.frz.V<F>() + wrap(m.off_f + comp - n1, a.frz.cap) * dv + j);
    };
    auto comp_s = [&](int comp) -> float {
      if (a.csr_off) return a.csr_s[o0 + comp];
      return comp < n1 ? a.act.s[wrap(m.off_a + comp, a.act.cap)] : a.frz.s[wrap(m.off_f + comp - n1, a.frz.cap)];
    };
    const int total = n1 + n2;
    const int j0 = rb * RPB, j1 = j0 + RPB < dv ? j0 + RPB : dv;
    float *H = a.dense + slot * dk * dv;
    const int64_t di = a.dsrc_idx ? a.dsrc_idx[s] : -1;
    if (di >= 0) {  // given dense: rows j0..j1 of H = S^T
      const float *S = a.dsrc + di * dk * dv;
      if (act)
        for (int j = j0 + g; j < j1; j += RG) {
          const float *col = S + (int64_t)(4 * c) * dv + j;
          st4(H + (int64_t)j * dk + 4 * c, make_float4(col[0], col[dv], col[2 * dv], col[3 * dv]));
        }
      continue;
    }
    float4 acc[kMatRows];
#pragma unroll
    for (int jj = 0; jj < kMatRows; ++jj) acc[jj] = zero4();
    for (int c0 = 0; c0 < total; c0 += kMatCH) {
      __syncthreads();
      for (int e = t; e < kMatCH * dk; e += 256) {
        const int cc = e / dk, i = e - cc * dk, comp = c0 + cc;
        su[e] = comp < total ? comp_u(comp, i) : 0.f;
      }
      for (int e = t; e < kMatCH * RPB; e += 256) {
        const int cc = e / RPB, jr = e - cc * RPB, comp = c0 + cc, j = j0 + jr;
        sv[e] = (comp < total && j < j1) ? comp_v(comp, j) : 0.f;
      }
      if (t < kMatCH) {
        const int comp = c0 + t;
        ss[t] = comp < total ? scale * comp_s(comp) : 0.f;
      }
      __syncthreads();
      if (act) {
        const int lim = (total - c0) < kMatCH ? (total - c0) : kMatCH;
        for (int cc = 0; cc < lim; ++cc) {
          const float4 u4 = *reinterpret_cast<const float4 *>(su + cc * dk + 4 * c);
          const float sc = ss[cc];
#pragma unroll
          for (int jj = 0; jj < kMatRows; ++jj) acc[jj] = fma4(sc * sv[cc * RPB + g + RG * jj], u4, acc[jj]);
        }
      }
    }
    if (act) {
#pragma unroll
      for (int jj = 0; jj < kMatRows; ++jj) {
        const int j = j0 + g + RG * jj;
        if (j < j1) st4(H + (int64_t)j * dk + 4 * c, acc[jj]);
      }
    }
  }
}

__global__ __launch_bounds__(256) void k_mat_finish(MaterializeArgs a) {
  const uint32_t li = blockIdx.x * 256u + threadIdx.x;
  if (li >= mat_count(a)) return;
  const int64_t slot = (int64_t)a.counters[C_MAT_BASE] + li;
  const int s = a.list[li];
  if (slot >= a.cap_d) {
    __hip_atomic_fetch_add(&a.counters[C_ERR_DENSE_CAP], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *a.hflag = 1u;
    return;
  }
  const uint32_t flags = meta_flags(a.meta[s].packed) & FLAG_DELTA;
  Meta nm;
  nm.off_a = (int32_t)slot;
  nm.off_f = 0;
  nm.gamma = 1.0f;
  nm.packed = meta_pack(0, 0, 0, flags | FLAG_DENSE);
  a.meta[s] = nm;
  DenseSlot ds;
  ds.s = s;
  ds.packed = meta_pack(0, 0, 0, flags | FLAG_DENSE);  // empty pad
  ds.gamma = 1.0f;
  ds.spare = 0u;
  a.dslot[slot] = ds;
  if (a.dgam)  // per-channel decay: the new slot starts with no decay accumulated
    for (int e = 0; e < a.dk; ++e) a.dgam[slot * a.dk + e] = 1.f;
  if (!a.csr_off) __hip_atomic_fetch_add(&a.counters[C_PROMOTIONS], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Pool creation: place the CSR components of every state into its slice of
// the group's first segments, or queue it for the dense region.
template <typename F>
__global__ __launch_bounds__(256) void k_scatter(ScatterArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= a.N) return;
  const int64_t o0 = a.csr_off[s], o1 = a.csr_off[s + 1];
  const int R = (int)(o1 - o0);
  const uint32_t flags = a.rule[s] ? FLAG_DELTA : 0u;
  if (a.force_dense || R > a.L || (a.dense_mask && a.dense_mask[s])) {
    if (lane == 0) {
      const uint32_t idx =
          __hip_atomic_fetch_add(&a.counters[C_PROMOTE_COUNT], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.dense_list[idx] = (int32_t)s;
      Meta nm;
      nm.off_a = -1;
      nm.off_f = -1;
      nm.gamma = 1.0f;
      nm.packed = meta_pack(0, 0, 0, flags);
      a.meta[s] = nm;
    }
    return;
  }
  const int64_t dst_a = a.dst_a[s], dst_f = a.dst_f[s];
  const int ra = R < a.r ? R : a.r, rf = R - ra;
  const int dk = a.dk, dv = a.dv;
  for (int c = 0; c < R; ++c) {
    const float *su = a.csr_u + (o0 + c) * dk, *sv = a.csr_v + (o0 + c) * dv;
    const bool isa = c < ra;
    F *du = isa ? a.act.U<F>() + (dst_a + c) * dk : a.frz.U<F>() + (dst_f + c - ra) * dk;
    F *dvv = isa ? a.act.V<F>() + (dst_a + c) * dv : a.frz.V<F>() + (dst_f + c - ra) * dv;
    copy_comp<F>(su, sv, du, dvv, dk, dv, lane);
    if (lane == 0) (isa ? a.act.s[dst_a + c] : a.frz.s[dst_f + c - ra]) = a.csr_s[o0 + c];
  }
  if (lane == 0) {
    Meta nm;
    nm.off_a = (int32_t)dst_a;
    nm.off_f = (int32_t)dst_f;
    nm.gamma = 1.0f;
    nm.packed = meta_pack(ra, rf, 0, flags);
    a.meta[s] = nm;
  }
}

__global__ __launch_bounds__(256) void k_prune_factored(const int32_t *src, const uint32_t *src_count, int32_t *dst,
                                                        uint32_t *dst_count, const Meta *meta) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  const int lane = threadIdx.x & 63;
  int32_t s = -1;
  bool keep = false;
  if (i < *src_count) {
    s = src[i];
    keep = !(meta_flags(meta[s].packed) & FLAG_DENSE);
  }
  const unsigned long long mask = __builtin_amdgcn_ballot_w64(keep);
  if (mask == 0ull) return;
  uint32_t base = 0;
  if (lane == 0)
    base = __hip_atomic_fetch_add(dst_count, (uint32_t)__builtin_popcountll(mask), __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
  base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
  if (keep) dst[base + __builtin_popcountll(mask & ((1ull << lane) - 1ull))] = s;
}

// A group's ring slots, first pass: per member its slot sizes packed as (active | frozen << 32),
// scanned (exclusive) within blocks of kSlotBlock members; each block's total goes to blk.
__global__ __launch_bounds__(kSlotBlock) void k_slot_scan(const int32_t *members, int n_members, const Meta *meta,
                                                          int r, int fcap, unsigned long long *in_blk,
                                                          unsigned long long *blk) {
  using Scan = hipcub::BlockScan<unsigned long long, kSlotBlock>;
  __shared__ typename Scan::TempStorage tmp;
  const int mi = blockIdx.x * kSlotBlock + threadIdx.x;
  unsigned long long v = 0;
  if (mi < n_members) {
    const uint32_t packed = meta[members[mi]].packed;
    if (!(meta_flags(packed) & FLAG_DENSE)) {
      int sa, sf;
      slot_sizes((int)meta_ra(packed), (int)meta_rf(packed), (int)meta_n(packed), r, fcap, sa, sf);
      v = (unsigned long long)sa | ((unsigned long long)sf << 32);
    }
  }
  unsigned long long ex, tot;
  Scan(tmp).ExclusiveSum(v, ex, tot);
  if (mi < n_members) in_blk[mi] = ex;
  if (threadIdx.x == 0) blk[blockIdx.x] = tot;
}

// Ring set-up of a compaction, after k_slot_scan: the block totals become block offsets, each
// ring's new segment is [begin, begin + its slots) from the old head, and the limit is the oldest
// live segment's start plus the capacity (seg_x[2 g] / seg_x[2 g + 1]: virtual start / end of
// group g's segment, start == end: none).  A segment past its limit raises the pool's flag.
// A group of at most kSlotBlock members (small != 0) is scanned here whole, without k_slot_scan.
__global__ __launch_bounds__(kSlotBlock) void k_ring_begin(Ring *ra, Ring *rf, const unsigned long long *seg_a,
                                                           const unsigned long long *seg_f, int n_groups,
                                                           int64_t cap_a, int64_t cap_f, uint32_t *counters,
                                                           unsigned long long *blk, int n_blk, uint32_t *hflag,
                                                           int small, const int32_t *members, int n_members,
                                                           const Meta *meta, int r, int fcap,
                                                           unsigned long long *in_blk) {
  using Scan = hipcub::BlockScan<unsigned long long, kSlotBlock>;
  __shared__ typename Scan::TempStorage tmp;
  unsigned long long carry = 0;
  if (small) {
    const int mi = (int)threadIdx.x;
    unsigned long long v = 0;
    if (mi < n_members) {
      const uint32_t packed = meta[members[mi]].packed;
      if (!(meta_flags(packed) & FLAG_DENSE)) {
        int sa, sf;
        slot_sizes((int)meta_ra(packed), (int)meta_rf(packed), (int)meta_n(packed), r, fcap, sa, sf);
        v = (unsigned long long)sa | ((unsigned long long)sf << 32);
      }
    }
    unsigned long long ex;
    Scan(tmp).ExclusiveSum(v, ex, carry);
    if (mi < n_members) in_blk[mi] = ex;
    if (threadIdx.x == 0) blk[0] = 0ull;
  } else {
    for (int b0 = 0; b0 < n_blk; b0 += kSlotBlock) {
      const int b = b0 + (int)threadIdx.x;
      const unsigned long long v = b < n_blk ? blk[b] : 0ull;
      unsigned long long ex, tot;
      Scan(tmp).ExclusiveSum(v, ex, tot);
      __syncthreads();  // tmp is used again
      if (b < n_blk) blk[b] = carry + ex;
      carry += tot;
    }
  }
  if (threadIdx.x != 0) return;
  counters[C_PROMOTE_COUNT] = 0u;  // the compaction's promotion list starts empty
  counters[C_FACT1] = 0u;          // scratch length for a pruning of the factored-state list
  unsigned long long ta = ra->head, tf = rf->head;
  for (int g = 0; g < n_groups; ++g) {
    if (seg_a[2 * g + 1] > seg_a[2 * g] && seg_a[2 * g] < ta) ta = seg_a[2 * g];
    if (seg_f[2 * g + 1] > seg_f[2 * g] && seg_f[2 * g] < tf) tf = seg_f[2 * g];
  }
  ra->limit = ta + (unsigned long long)cap_a;
  rf->limit = tf + (unsigned long long)cap_f;
  ra->begin = ra->head;
  rf->begin = rf->head;
  ra->head = ra->begin + (carry & 0xffffffffull);
  rf->head = rf->begin + (carry >> 32);
  if (ra->head > ra->limit || rf->head > rf->limit) {  // the members whose slots pass it keep their old form
    ra->overflow += 1ull;
    *hflag = 1u;
  }
}

__global__ void k_ring_end(Ring *ra, Ring *rf, unsigned long long *seg_a, unsigned long long *seg_f, int g) {
  if (threadIdx.x != 0) return;
  seg_a[2 * g] = ra->begin;
  seg_a[2 * g + 1] = ra->head;
  seg_f[2 * g] = rf->begin;
  seg_f[2 * g + 1] = rf->head;
}

// one wavefront per state: copy its live components to the new rings
template <typename F>
__global__ __launch_bounds__(256) void k_repack(RepackArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t s = (int64_t)blockIdx.x * 4 + uniform(threadIdx.x >> 6);
  if (s >= a.N) return;
  const int64_t na = a.new_a[s], nf = a.new_f[s];
  if (na < 0) return;
  const Meta m = a.meta[s];
  const uint32_t packed = (uint32_t)uniform((int)m.packed);
  const int ra = meta_ra(packed), rf = meta_rf(packed);
  const int dk = a.dk, dv = a.dv;
  copy_comps<F>(a.src_a, m.off_a, ra, dk, dv, lane, [&](int f, F *&du, F *&dvp) {
    du = a.dst_a.U<F>() + wrap(na + f, a.dst_a.cap) * dk;
    dvp = a.dst_a.V<F>() + wrap(na + f, a.dst_a.cap) * dv;
    return true;
  });
  copy_comps<F>(a.src_f, m.off_f, rf, dk, dv, lane, [&](int f, F *&du, F *&dvp) {
    du = a.dst_f.U<F>() + wrap(nf + f, a.dst_f.cap) * dk;
    dvp = a.dst_f.V<F>() + wrap(nf + f, a.dst_f.cap) * dv;
    return true;
  });
  for (int f = lane; f < ra; f += 64) a.dst_a.s[wrap(na + f, a.dst_a.cap)] = a.src_a.s[wrap(m.off_a + f, a.src_a.cap)];
  for (int f = lane; f < rf; f += 64) a.dst_f.s[wrap(nf + f, a.dst_f.cap)] = a.src_f.s[wrap(m.off_f + f, a.src_f.cap)];
  if (lane == 0) {
    Meta nm = m;
    nm.off_a = (int32_t)na;
    nm.off_f = (int32_t)nf;
    a.meta[s] = nm;
  }
}

// layout index li -> (ord slot, member) -> state; its component counts (0 for dense states)
__global__ __launch_bounds__(256) void k_layout_counts(LayoutArgs a) {
  const int64_t li = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (li >= a.N) return;
  int lo = 0, hi = a.G - 1;  // the ord slot k with lstart[k] <= li < lstart[k + 1]
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.lstart[mid] <= li) lo = mid;
    else hi = mid - 1;
  }
  const int g = a.ord[lo];
  const int32_t s = a.members[a.gstart[g] + (li - a.lstart[lo])];
  const uint32_t pk = a.meta[s].packed;
  const bool dense = meta_flags(pk) & FLAG_DENSE;
  a.cnt_a[li] = dense ? 0 : (int64_t)meta_ra(pk);
  a.cnt_f[li] = dense ? 0 : (int64_t)meta_rf(pk);
}

__global__ __launch_bounds__(256) void k_layout_scatter(LayoutArgs a) {
  const int64_t li = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (li >= a.N) return;
  int lo = 0, hi = a.G - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.lstart[mid] <= li) lo = mid;
    else hi = mid - 1;
  }
  const int g = a.ord[lo];
  const int32_t s = a.members[a.gstart[g] + (li - a.lstart[lo])];
  const bool dense = meta_flags(a.meta[s].packed) & FLAG_DENSE;
  a.new_a[s] = dense ? -1 : a.off_a[li];
  a.new_f[s] = dense ? -1 : a.off_f[li];
}

// group segments and ring heads from the scans (one thread per ord slot)
__global__ void k_layout_segs(LayoutArgs a) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = a.N;
  const unsigned long long tot_a = n ? (unsigned long long)(a.off_a[n - 1] + a.cnt_a[n - 1]) : 0ull;
  const unsigned long long tot_f = n ? (unsigned long long)(a.off_f[n - 1] + a.cnt_f[n - 1]) : 0ull;
  if (k < a.G) {
    const int g = a.ord[k];
    const int64_t b0 = a.lstart[k], b1 = a.lstart[k + 1];
    const unsigned long long sa = b0 < n ? (unsigned long long)a.off_a[b0] : tot_a;
    const unsigned long long sf = b0 < n ? (unsigned long long)a.off_f[b0] : tot_f;
    const unsigned long long ea = b1 > b0 ? (unsigned long long)(a.off_a[b1 - 1] + a.cnt_a[b1 - 1]) : sa;
    const unsigned long long ef = b1 > b0 ? (unsigned long long)(a.off_f[b1 - 1] + a.cnt_f[b1 - 1]) : sf;
    a.seg[2 * g] = sa;
    a.seg[2 * g + 1] = ea;
    a.seg[2 * a.G + 2 * g] = sf;
    a.seg[2 * a.G + 2 * g + 1] = ef;
  }
  if (k == 0) {
    a.ring[0].head = a.ring[0].begin = tot_a;
    a.ring[1].head = a.ring[1].begin = tot_f;
    a.ring[0].overflow = a.ring[1].overflow = 0ull;
  }
}

// list[i] = tmp[i] for i < *tmp_count; the length goes to *count and to a host-visible word
__global__ __launch_bounds__(256) void k_copy_list(const int32_t *tmp, const uint32_t *tmp_count, int32_t *list,
                                                   uint32_t *count, uint32_t *host) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  const uint32_t c = *tmp_count;
  if (i < c) list[i] = tmp[i];
  if (i == 0) {
    *count = c;
    *host = c;
  }
}

__global__ void k_zero_u32(uint32_t *p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

__global__ void k_fill_f32(float *p, int64_t n, float x) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = x;
}

template <int NB, typename F, bool DG>
hipError_t compact_h(const CompactArgs &a, hipStream_t st) {
  const dim3 grid((unsigned)((a.n_members + 3) / 4)), block(256);
  hipLaunchKernelGGL((k_compact_h<NB, F, DG>), grid, block, 0, st, a);
  return hipGetLastError();
}


}  // namespace

hipError_t launch_compact(const CompactArgs &a, hipStream_t st) {
  if (a.n_members <= 0) return hipSuccess;
  const int d = a.dk > a.dv ? a.dk : a.dv;
  if (d > 256) return hipErrorInvalidValue;
  // the two sides of a state on the two halves of its wavefront; a.gam: per-channel decay
  if (a.gam) {
    if (d <= 128) return a.act.half ? compact_h<1, _Float16, true>(a, st) : compact_h<1, float, true>(a, st);
    return a.act.half ? compact_h<2, _Float16, true>(a, st) : compact_h<2, float, true>(a, st);
  }
  if (d <= 128) return a.act.half ? compact_h<1, _Float16, false>(a, st) : compact_h<1, float, false>(a, st);
  return a.act.half ? compact_h<2, _Float16, false>(a, st) : compact_h<2, float, false>(a, st);
}

hipError_t launch_materialize(const MaterializeArgs &a, int64_t grid_upper, hipStream_t st) {
  if (grid_upper <= 0) return hipSuccess;
  const int C4 = a.dk >> 2, RPB = (256 / C4) * kMatRows, RB = (a.dv + RPB - 1) / RPB;
  const int64_t want = grid_upper * RB;
  const unsigned grid = (unsigned)(want < 4096 ? want : 4096);
  const size_t sh = sizeof(float) * ((size_t)kMatCH * (a.dk + RPB) + kMatCH);
  hipLaunchKernelGGL(k_mat_reserve, dim3(1), dim3(64), 0, st, a);
  if (a.act.half) hipLaunchKernelGGL(k_mat_rows<_Float16>, dim3(grid), dim3(256), sh, st, a, RB);
  else hipLaunchKernelGGL(k_mat_rows<float>, dim3(grid), dim3(256), sh, st, a, RB);
  hipLaunchKernelGGL(k_mat_finish, dim3((unsigned)((grid_upper + 255) / 256)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_scatter(const ScatterArgs &a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  if (a.act.half) hipLaunchKernelGGL(k_scatter<_Float16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_scatter<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prune_factored(int32_t *list, uint32_t *count, int32_t *tmp, uint32_t *tmp_count, int64_t n_upper,
                                 const Meta *meta, uint32_t *host_count, hipStream_t st) {
  if (n_upper <= 0) return hipSuccess;
  const dim3 grid((unsigned)((n_upper + 255) / 256)), block(256);
  hipLaunchKernelGGL(k_prune_factored, grid, block, 0, st, list, count, tmp, tmp_count, meta);
  hipLaunchKernelGGL(k_copy_list, grid, block, 0, st, tmp, tmp_count, list, count, host_count);
  return hipGetLastError();
}

hipError_t launch_ring_begin(const RingBeginArgs &b, hipStream_t st) {
  const int n_blk = (b.n_members + kSlotBlock - 1) / kSlotBlock;
  const int small = n_blk <= 1 ? 1 : 0;  // one block: scanned by k_ring_begin itself
  if (!small)
    hipLaunchKernelGGL(k_slot_scan, dim3((unsigned)n_blk), dim3(kSlotBlock), 0, st, b.members, b.n_members, b.meta, b.r,
                       b.fcap, b.slot_in, b.slot_blk);
  hipLaunchKernelGGL(k_ring_begin, dim3(1), dim3(kSlotBlock), 0, st, b.ring_a, b.ring_f, b.seg_a, b.seg_f, b.n_groups,
                     b.cap_a, b.cap_f, b.counters, b.slot_blk, n_blk, b.hflag, small, b.members, b.n_members, b.meta,
                     b.r, b.fcap, b.slot_in);
  return hipGetLastError();
}

hipError_t launch_ring_end(Ring *ra, Ring *rf, unsigned long long *seg_a, unsigned long long *seg_f, int g,
                           hipStream_t st) {
  hipLaunchKernelGGL(k_ring_end, dim3(1), dim3(64), 0, st, ra, rf, seg_a, seg_f, g);
  return hipGetLastError();
}

size_t layout_scan_bytes(int64_t N) {
  size_t bytes = 0;
  if (hipcub::DeviceScan::ExclusiveSum(nullptr, bytes, (const int64_t *)nullptr, (int64_t *)nullptr, (int)N) !=
      hipSuccess)
    return 0;
  return bytes;
}

hipError_t launch_ring_layout(const LayoutArgs &a, hipStream_t st) {
  if (a.N <= 0 || a.G <= 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((a.N + 255) / 256)), block(256);
  hipLaunchKernelGGL(k_layout_counts, grid, block, 0, st, a);
  hipError_t e = hipGetLastError();
  size_t bytes = a.scan_bytes;
  if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(a.scan_tmp, bytes, a.cnt_a, a.off_a, (int)a.N, st);
  bytes = a.scan_bytes;
  if (e == hipSuccess) e = hipcub::DeviceScan::ExclusiveSum(a.scan_tmp, bytes, a.cnt_f, a.off_f, (int)a.N, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_layout_scatter, grid, block, 0, st, a);
  hipLaunchKernelGGL(k_layout_segs, dim3((unsigned)((a.G + 63) / 64)), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_repack(const RepackArgs &a, hipStream_t st) {
  if (a.N <= 0) return hipSuccess;
  const dim3 grid((unsigned)((a.N + 3) / 4)), block(256);
  if (a.src_a.half) hipLaunchKernelGGL(k_repack<_Float16>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(k_repack<float>, grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float *p, int64_t n, float x, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n, x);
  return hipGetLastError();
}

hipError_t launch_zero_u32(uint32_t *p, int n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

}  // namespace ss
