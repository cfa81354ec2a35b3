// kda_device.h -- device-side helpers shared by the libkda kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// bfloat16 stored as raw 16-bit patterns in memory.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16, round to nearest even (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// Element type traits for the io dtype.
template <typename T>
struct io;

template <>
struct io<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};

template <>
struct io<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
  __device__ __forceinline__ static void store(bf16_t* p, float x) { p->bits = f32_to_bf16(x); }
};

// Load 4 consecutive io elements as floats.
__device__ __forceinline__ f32x4 load4(const float* p) {
  return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  f32x4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xFFFF0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xFFFF0000u);
  return r;
}

// Raw storage of 4 consecutive io elements (loaded now, widened later).
template <typename T>
struct raw4;
template <>
struct raw4<float> {
  typedef f32x4 type;
};
template <>
struct raw4<bf16_t> {
  typedef uint2 type;
};
__device__ __forceinline__ f32x4 load4raw(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
__device__ __forceinline__ uint2 load4raw(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ f32x4 cvt4(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 cvt4(uint2 u) {
  f32x4 r;
  r[0] = __uint_as_float(u.x << 16);
  r[1] = __uint_as_float(u.x & 0xFFFF0000u);
  r[2] = __uint_as_float(u.y << 16);
  r[3] = __uint_as_float(u.y & 0xFFFF0000u);
  return r;
}

// Store 4 consecutive io elements.
__device__ __forceinline__ void store4(float* p, f32x4 x) { *reinterpret_cast<f32x4*>(p) = x; }
__device__ __forceinline__ void store4(bf16_t* p, f32x4 x) {
  uint2 u;
  u.x = f32x2_to_bf16x2(x[0], x[1]);
  u.y = f32x2_to_bf16x2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = u;
}

// -softplus(z) = -log(1 + e^z) without overflow: -(max(z, 0) + log1p(e^{-|z|})),
// with log1p(t) taken as t (1 - t/2) below t = 2^-10 (error below t^3 / 3)
__device__ __forceinline__ float neg_softplus(float z) {
  const float t = __expf(-fabsf(z));
  const float l = t < 0x1p-10f ? t * (1.f - 0.5f * t) : __logf(1.f + t);
  return -(fmaxf(z, 0.f) + l);
}

// One DPP move (bound_ctrl: lanes without a source read 0).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N consecutive lanes (N = 4, 8, 16 or 32) with
// DPP moves inside each row of 16 lanes and one swizzle across the two rows
// of a 32-lane half; every lane of a group receives the group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 4 || N == 8 || N == 16 || N == 32, "group of 4 to 32 lanes");
  x += dpp_mov<0xB1>(x);                        // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);                        // quad_perm [2,3,0,1]: quad sums
  if constexpr (N >= 8) x += dpp_mov<0x141>(x);  // row_half_mirror: sums over 8 lanes
  if constexpr (N >= 16) x += dpp_mov<0x140>(x); // row_mirror: sums over 16 lanes
  if constexpr (N == 32)  // xor 16 within each 32-lane half (and_mask 0x1F, xor_mask 0x10)
    x += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x401F));
  return x;
}

// Cross-lane xor shuffle within a 64-wide wavefront.
__device__ __forceinline__ float shfl_xor(float x, int m) { return __shfl_xor(x, m, 64); }

}  // namespace kda
