// ss_wave.h -- wavefront (64-lane) reductions for gfx950.
//
// Sums over aligned groups of P lanes use DPP inside a row of 16 lanes
// (quad permutes, half-row and row mirrors: each step folds two aligned
// halves of a 2^j block, so every lane of the block ends with the block sum),
// ds_swizzle for the 16-lane stride inside a half-wave and ds_bpermute for
// the 32-lane stride.
#pragma once
#include <hip/hip_runtime.h>

namespace ss {

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// lane i reads lane i ^ MASK inside each 32-lane half (MASK < 32)
template <int MASK>
__device__ __forceinline__ float swz_xor(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), (MASK << 10) | 0x1F));
}

__device__ __forceinline__ float xor32(float x) {
  const int lane = __lane_id();
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, x)));
}

// sum over each aligned block of P lanes (P a power of two, 1..64)
template <int P>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (P >= 2) x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
  if constexpr (P >= 4) x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
  if constexpr (P >= 8) x += dpp<0x141>(x);   // row_half_mirror
  if constexpr (P >= 16) x += dpp<0x140>(x);  // row_mirror
  if constexpr (P >= 32) x += swz_xor<16>(x);
  if constexpr (P >= 64) x += xor32(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return group_sum<64>(x); }

template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_rows(float x) {
  return __builtin_bit_cast(float,
                            __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, ROWMASK, 0xF, false));
}

// sum over the 64 lanes as a wave-uniform value: row sums by DPP, then row 0 -> 1 and
// row 2 -> 3 (row_bcast:15), rows 0-1 -> 2-3 (row_bcast:31); lane 63 holds the total and is
// read into a scalar register, so no LDS permute is involved
__device__ __forceinline__ float wave_sum_u(float x) {
  x += dpp<0xB1>(x);
  x += dpp<0x4E>(x);
  x += dpp<0x141>(x);
  x += dpp<0x140>(x);
  x += dpp_rows<0x142, 0xA>(x);
  x += dpp_rows<0x143, 0xC>(x);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}

// lane i reads lane i ^ S (S a power of two < 64)
template <int S>
__device__ __forceinline__ float lane_xor(float x) {
  if constexpr (S >= 32) return xor32(x);
  else return swz_xor<S>(x);
}

// sum over lanes that differ only in bits >= log2(P): lanes with the same
// position inside their P-block end with the same total
template <int P>
__device__ __forceinline__ float cross_group_sum(float x) {
  if constexpr (P <= 1) x += lane_xor<1>(x);
  if constexpr (P <= 2) x += lane_xor<2>(x);
  if constexpr (P <= 4) x += lane_xor<4>(x);
  if constexpr (P <= 8) x += lane_xor<8>(x);
  if constexpr (P <= 16) x += lane_xor<16>(x);
  if constexpr (P <= 32) x += lane_xor<32>(x);
  return x;
}

__device__ __forceinline__ float4 add4(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
__device__ __forceinline__ float4 sub4(float4 a, float4 b) { return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w); }
__device__ __forceinline__ float4 scale4(float s, float4 a) { return make_float4(s * a.x, s * a.y, s * a.z, s * a.w); }
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 zero4() { return make_float4(0.f, 0.f, 0.f, 0.f); }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
  return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}

template <int P>
__device__ __forceinline__ float4 cross_group_sum4(float4 a) {
  return make_float4(cross_group_sum<P>(a.x), cross_group_sum<P>(a.y), cross_group_sum<P>(a.z),
                     cross_group_sum<P>(a.w));
}

__device__ __forceinline__ float4 ld4(const float *p) { return *reinterpret_cast<const float4 *>(p); }
// streaming (read-once) loads: the nontemporal hint keeps them from displacing reused lines
__device__ __forceinline__ float4 ld4nt(const float *p) {
  return make_float4(__builtin_nontemporal_load(p), __builtin_nontemporal_load(p + 1), __builtin_nontemporal_load(p + 2),
                     __builtin_nontemporal_load(p + 3));
}
__device__ __forceinline__ float ldnt(const float *p) { return __builtin_nontemporal_load(p); }

// Guarded loads are written as an unconditional load from an address that is
// always valid (the caller clamps it), followed by a select: a load placed
// inside a branch is followed by a wait for its data, which would serialize
// the loads of a batch.
__device__ __forceinline__ float4 sel4(bool ok, float4 v) {
  return make_float4(ok ? v.x : 0.f, ok ? v.y : 0.f, ok ? v.z : 0.f, ok ? v.w : 0.f);
}
__device__ __forceinline__ float self(bool ok, float v) { return ok ? v : 0.f; }
__device__ __forceinline__ void st4(float *p, float4 v) { *reinterpret_cast<float4 *>(p) = v; }
// streaming (write-once, read much later) stores
__device__ __forceinline__ void st4nt(float *p, float4 v) {
  __builtin_nontemporal_store(v.x, p);
  __builtin_nontemporal_store(v.y, p + 1);
  __builtin_nontemporal_store(v.z, p + 2);
  __builtin_nontemporal_store(v.w, p + 3);
}

// Factor storage element types: float, or _Float16 (four elements = 8 bytes per lane).
// Conversions to fp16 round to nearest, ties to even (the hardware's default mode).
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 ldf4(const float *p) { return ld4(p); }
__device__ __forceinline__ float4 ldf4(const _Float16 *p) {
  const half4_t h = *reinterpret_cast<const half4_t *>(p);
  return make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
}
__device__ __forceinline__ float4 ldf4nt(const float *p) { return ld4nt(p); }
__device__ __forceinline__ float4 ldf4nt(const _Float16 *p) {
  const half4_t h = __builtin_nontemporal_load(reinterpret_cast<const half4_t *>(p));
  return make_float4((float)h.x, (float)h.y, (float)h.z, (float)h.w);
}
__device__ __forceinline__ void stf4(float *p, float4 v) { st4(p, v); }
__device__ __forceinline__ void stf4(_Float16 *p, float4 v) {
  half4_t h;
  h.x = (_Float16)v.x;
  h.y = (_Float16)v.y;
  h.z = (_Float16)v.z;
  h.w = (_Float16)v.w;
  *reinterpret_cast<half4_t *>(p) = h;
}
__device__ __forceinline__ float ldf(const float *p) { return *p; }
__device__ __forceinline__ float ldf(const _Float16 *p) { return (float)*p; }
__device__ __forceinline__ void stf(float *p, float v) { *p = v; }
__device__ __forceinline__ void stf(_Float16 *p, float v) { *p = (_Float16)v; }

// make this lane's LDS writes visible to the other lanes of the wavefront
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniformf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

}  // namespace ss
