// ss_linalg.h -- wavefront-level small dense linear algebra for the compaction
// and the initialization kernels: thin QR by classical Gram-Schmidt with one
// re-orthogonalization pass (CGS2) on register-resident columns (the
// initialization; the compaction's selective Gram-Schmidt uses the thresholds
// below), and one-sided (Hestenes) Jacobi SVDs of a 16 x 16 matrix in LDS, with
// the rotations accumulated (jacobi16) or the columns only (jacobi16c).
#pragma once
#include "ss_internal.h"
#include "ss_wave.h"

namespace ss {

constexpr float kTau2 = 1e-10f;  // (1e-5)^2: CGS2 dependent-column test on squared norms
constexpr float kReorth2 = 0.1f;  // selective Gram-Schmidt: second pass below this share of the squared norm
constexpr float kTolJ = 1e-6f;   // Jacobi: rotate while |a_i.a_j| > tol |a_i| |a_j|
constexpr int kMaxSweeps = 16;

// Single-sided CGS2: in-place thin QR of the register-resident columns u[0..m) (element e of a
// column in lane e % 64, register e / 64).  R goes to LDS column-major 16 x 16:
// R[j * 16 + i] = R(i, j).  A column whose residual is at most 1e-5 of its input norm is
// dependent: it and its R row are zeroed.
template <int NS>
__device__ __forceinline__ void cgs2_one(float (&u)[kMaxM][NS], int m, int lane, float *Ru) {
#pragma unroll
  for (int j = 0; j < kMaxM; ++j) {
    if (j < m) {
      float n0 = 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t) n0 = fmaf(u[j][t], u[j][t], n0);
      n0 = wave_sum_u(n0);
      float ru[kMaxM];
#pragma unroll
      for (int i = 0; i < kMaxM; ++i) ru[i] = 0.f;
#pragma unroll
      for (int pass = 0; pass < 2; ++pass) {
        float du[kMaxM];
#pragma unroll
        for (int i = 0; i < j; ++i) {
          float x = 0.f;
#pragma unroll
          for (int t = 0; t < NS; ++t) x = fmaf(u[i][t], u[j][t], x);
          du[i] = wave_sum_u(x);
        }
#pragma unroll
        for (int i = 0; i < j; ++i) {
          ru[i] += du[i];
#pragma unroll
          for (int t = 0; t < NS; ++t) u[j][t] = fmaf(-du[i], u[i][t], u[j][t]);
        }
      }
      float nu = 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t) nu = fmaf(u[j][t], u[j][t], nu);
      nu = wave_sum_u(nu);
      const bool ku = nu > 0.f && nu > kTau2 * n0;
      const float su = sqrtf(nu);
      const float iu = ku ? 1.0f / su : 0.f;
#pragma unroll
      for (int t = 0; t < NS; ++t) u[j][t] *= iu;
      if (lane < kMaxM) {
        float xu = 0.f;
#pragma unroll
        for (int i = 0; i < kMaxM; ++i)
          if (i == lane && i < j) xu = ru[i];
        if (lane == j) xu = ku ? su : 0.f;
        Ru[j * 16 + lane] = xu;
      }
    } else {
#pragma unroll
      for (int t = 0; t < NS; ++t) u[j][t] = 0.f;
      if (lane < kMaxM) Ru[j * 16 + lane] = 0.f;
    }
  }
}

// One-sided Jacobi on the 16 x 16 column-major C (columns >= m are zero),
// accumulating the rotations into Vh.  Returns the number of sweeps run.
// Pairs follow the round-robin (circle) order on M = m rounded up to even:
// in round k, pair 0 is (k, M-1) and pair p > 0 is ((k+p) mod (M-1),
// (k-p) mod (M-1)); both indices advance by one (mod M-1) from a round to
// the next, so they are carried in registers instead of recomputed.  The
// rotation zeroes the pair's inner product: zeta = (|y|^2 - |x|^2) / (2 x.y),
// t = sign(zeta) / (|zeta| + sqrt(1 + zeta^2)), c = 1 / sqrt(1 + t^2), s = c t,
// with the hardware reciprocal and reciprocal square root (about 1 ulp).
// *limit (when given) is set if the last allowed sweep still rotated.
__device__ inline int jacobi16(float *Cm, float *Vh, int m, int lane, bool *limit = nullptr) {
  if (limit) *limit = false;
  const int M = (m + 1) & ~1;
  if (M < 2) return 0;
  const int np = M >> 1, rounds = M - 1;
  const int p = lane >> 3, sub = lane & 7;
  const bool act = p < np;
  int sweep = 0;
  while (sweep < kMaxSweeps) {
    ++sweep;
    bool any = false;
    int ci = p == 0 ? 0 : p % (M - 1);
    int cj = p == 0 ? M - 1 : (M - 1 - p) % (M - 1);
    for (int k = 0; k < rounds; ++k) {
      float x0 = 0.f, x1 = 0.f, y0 = 0.f, y1 = 0.f;
      if (act) {
        x0 = Cm[ci * 16 + sub];
        x1 = Cm[ci * 16 + sub + 8];
        y0 = Cm[cj * 16 + sub];
        y1 = Cm[cj * 16 + sub + 8];
      }
      float aa = fmaf(x0, x0, x1 * x1), bb = fmaf(y0, y0, y1 * y1), gg = fmaf(x0, y0, x1 * y1);
      aa = group_sum<8>(aa);
      bb = group_sum<8>(bb);
      gg = group_sum<8>(gg);
      const bool rot = act && gg != 0.f && fabsf(gg) > kTolJ * __builtin_amdgcn_sqrtf(aa * bb);
      if (rot) {
        const float zeta = (bb - aa) * (0.5f * __builtin_amdgcn_rcpf(gg));
        const float az = fabsf(zeta);
        const float t = az > 1e10f ? 0.5f * __builtin_amdgcn_rcpf(zeta)
                                   : copysignf(__builtin_amdgcn_rcpf(az + __builtin_amdgcn_sqrtf(fmaf(zeta, zeta, 1.f))), zeta);
        const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), sn = c * t;
        Cm[ci * 16 + sub] = c * x0 - sn * y0;
        Cm[ci * 16 + sub + 8] = c * x1 - sn * y1;
        Cm[cj * 16 + sub] = sn * x0 + c * y0;
        Cm[cj * 16 + sub + 8] = sn * x1 + c * y1;
        const float vx0 = Vh[ci * 16 + sub], vx1 = Vh[ci * 16 + sub + 8];
        const float vy0 = Vh[cj * 16 + sub], vy1 = Vh[cj * 16 + sub + 8];
        Vh[ci * 16 + sub] = c * vx0 - sn * vy0;
        Vh[ci * 16 + sub + 8] = c * vx1 - sn * vy1;
        Vh[cj * 16 + sub] = sn * vx0 + c * vy0;
        Vh[cj * 16 + sub + 8] = sn * vx1 + c * vy1;
      }
      any = any || (__builtin_amdgcn_ballot_w64(rot) != 0ull);
      wave_sync();
      ci = (ci + 1 == M - 1) ? 0 : ci + 1;
      if (p != 0) cj = (cj + 1 == M - 1) ? 0 : cj + 1;
    }
    if (!any) break;
    if (limit && sweep == kMaxSweeps) *limit = true;
  }
  return sweep;
}

// (a << 7) + b in one instruction (the compiler emits a shift and an add for it)
__device__ __forceinline__ uint32_t lshl7_add(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_lshl_add_u32 %0, %1, 7, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// One-sided Jacobi on the columns of a 16 x 16 matrix B (columns >= m zero) with the same pairs,
// order, stopping rule and rotation as jacobi16, but without accumulating the rotations: only B
// turns (B = C J), and the caller recovers J from C.  At convergence B^T B = diag(s^2) and
// C^T C = J diag(s^2) J^T, so C^T B = J diag(s^2): column j of J is C^T b_j / s_j^2 for s_j > 0
// (the columns with s_j = 0 carry no component).
//
// Each round computes only the pair's inner product g; the squared norms a, b of the pair's columns
// are carried and, after a rotation by t = tan(theta), updated to a - t g and b + t g (the rotation
// zeroes g).  They are recomputed from the columns at the start of every sweep, so the rounding of
// the updates never accumulates past one sweep.  Layout of Bj (512 floats of LDS): column j is 8
// chunks of 4 floats, chunk c = {B(2c, j), B(2c + 1, j), |b_j|^2, unused}.  The lane holding rows
// 2c, 2c + 1 of a pair's column reads them and the column's norm with one 16-byte access, and every
// lane keeps its chunk's copy of the norm current, so no lane waits on another for a norm.
//
// t is the root of smaller magnitude of t^2 + 2 zeta t - 1 = 0 with zeta = (b - a) / (2 g), written
// without zeta: t = sign(d) 2 g / (|d| + sqrt(d^2 + 4 g^2)), d = b - a (Rutishauser's form; no
// division by g and no large-zeta branch); c = 1 / sqrt(1 + t^2), s = c t.  The round-robin
// schedule is the same every sweep and is packed once: 4 bits per round of this lane's pair's
// column indices.
__device__ inline int jacobi16c(float *Bj, int m, int lane, bool *limit = nullptr) {
  if (limit) *limit = false;
  const int M = (m + 1) & ~1;
  if (M < 2) return 0;
  const int np = M >> 1, rounds = M - 1;
  const int p = lane >> 3, sub = lane & 7;
  const bool act = p < np;
  const float tol2 = kTolJ * kTolJ;
  // rounds 0-7 in lo, 8-14 in hi; inactive pairs read column 0 and never rotate
  uint32_t ilo = 0, ihi = 0, jlo = 0, jhi = 0;
  {
    int ci = p == 0 ? 0 : p % (M - 1);
    int cj = p == 0 ? M - 1 : (M - 1 - p) % (M - 1);
    for (int k = 0; k < rounds; ++k) {
      const uint32_t ii = act ? (uint32_t)ci : 0u, jj = act ? (uint32_t)cj : 0u;
      if (k < 8) {
        ilo |= ii << (4 * k);
        jlo |= jj << (4 * k);
      } else {
        ihi |= ii << (4 * (k - 8));
        jhi |= jj << (4 * (k - 8));
      }
      ci = (ci + 1 == M - 1) ? 0 : ci + 1;
      if (p != 0) cj = (cj + 1 == M - 1) ? 0 : cj + 1;
    }
  }
  // LDS byte address of this lane's chunk of column 0; column i's is 128 i past it
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) v4f lds_v4f;
  const uint32_t base = (uint32_t)(size_t)(lds_v4f *)(reinterpret_cast<v4f *>(Bj) + sub);
  int sweep = 0;
  bool any = false;
  auto round = [&](uint32_t iw, uint32_t jw, int sh) {
    lds_v4f *px = (lds_v4f *)(size_t)lshl7_add(__builtin_amdgcn_ubfe(iw, sh, 4), base);
    lds_v4f *py = (lds_v4f *)(size_t)lshl7_add(__builtin_amdgcn_ubfe(jw, sh, 4), base);
    const v4f x = *px, y = *py;
    const float gg = group_sum<8>(fmaf(x.x, y.x, x.y * y.y));
    // |a b|: a carried norm may round below zero; then g = 0 must still not rotate
    const bool rot = act && gg * gg > tol2 * fabsf(x.z * y.z);
    if (rot) {
      const float d = y.z - x.z, g2 = gg + gg;
      const float t = (d < 0.f ? -g2 : g2) * __builtin_amdgcn_rcpf(fabsf(d) + __builtin_amdgcn_sqrtf(fmaf(d, d, g2 * g2)));
      const float c = __builtin_amdgcn_rsqf(fmaf(t, t, 1.f)), sn = c * t;
      *px = v4f{c * x.x - sn * y.x, c * x.y - sn * y.y, fmaf(-t, gg, x.z), 0.f};
      *py = v4f{sn * x.x + c * y.x, sn * x.y + c * y.y, fmaf(t, gg, y.z), 0.f};
    }
    any = any || (__builtin_amdgcn_ballot_w64(rot) != 0ull);
    wave_sync();
  };
  while (sweep < kMaxSweeps) {
    ++sweep;
    {  // norms: lane l sums chunks 2 (l & 3) and 2 (l & 3) + 1 of column l / 4, four lanes per column
      float4 *q = reinterpret_cast<float4 *>(Bj) + 8 * (lane >> 2) + 2 * (lane & 3);
      const float4 u0 = q[0], u1 = q[1];
      const float xx = group_sum<4>(fmaf(u0.x, u0.x, fmaf(u0.y, u0.y, fmaf(u1.x, u1.x, u1.y * u1.y))));
      reinterpret_cast<float *>(q)[2] = xx;
      reinterpret_cast<float *>(q)[6] = xx;
    }
    wave_sync();
    any = false;
    const int r0 = rounds < 8 ? rounds : 8;
    for (int k = 0; k < r0; ++k) round(ilo, jlo, 4 * k);
    for (int k = 8; k < rounds; ++k) round(ihi, jhi, 4 * (k - 8));
    if (!any) break;
    if (limit && sweep == kMaxSweeps) *limit = true;
  }
  return sweep;
}

}  // namespace ss
