// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// ---- 16-bit float <-> float32 (bit exact, no library dependency) -----------
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
  _Float16 v = __builtin_bit_cast(_Float16, (uint16_t)h);
  return (float)v;
}

// float32 -> bf16 bits, round to nearest even (finite inputs; NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (u >> 16) | 0x40u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // v_cvt_f16_f32: round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Output element store helper: OUT_BF16 selects bf16, otherwise f16.
template <bool OUT_BF16>
__device__ __forceinline__ uint32_t f32_to_out_bits(float f) {
  if constexpr (OUT_BF16) return f32_to_bf16_bits(f);
  else return f32_to_f16_bits(f);
}

template <bool OUT_BF16>
__device__ __forceinline__ float out_bits_to_f32(uint32_t h) {
  if constexpr (OUT_BF16) return bf16_bits_to_f32(h);
  else return f16_bits_to_f32(h);
}

// Four consecutive 16-bit bias values b[n .. n+3] as float32, zero past n_end.
// vec: b + n is 8-byte aligned and n + 3 < n_end, one 8-byte load.
__device__ __forceinline__ f32x4 load_bias4(const void* b, int64_t n, int64_t n_end, bool bf16, bool vec) {
  const uint16_t* h = static_cast<const uint16_t*>(b);
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  if (vec) {
    const uint2 w = *reinterpret_cast<const uint2*>(h + n);
    const uint32_t u[4] = {w.x & 0xFFFFu, w.x >> 16, w.y & 0xFFFFu, w.y >> 16};
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = bf16 ? bf16_bits_to_f32(u[r]) : f16_bits_to_f32(u[r]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < n_end) v[r] = bf16 ? bf16_bits_to_f32(h[n + r]) : f16_bits_to_f32(h[n + r]);
  }
  return v;
}

// ---- wave reductions ----------------------------------------------------------
// Maximum of absolute values (floats >= +0, not NaN, whose bit patterns order
// as unsigned integers) over aligned groups of `width` adjacent lanes (a power
// of two, at most kWave), every lane of a group receiving it. Within a 16-lane
// row each step is one DPP-modified integer max: quad_perm [1,0,3,2] and
// [2,3,0,1] read lane ^ 1 and lane ^ 2; row_half_mirror reads lane 7 - i of
// each 8-lane half row and row_mirror lane 15 - i of each row, which lie in the
// partner group once the smaller groups hold their maxima. Wider steps permute
// through LDS.
template <int CTRL>
__device__ __forceinline__ uint32_t umax_dpp(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, true);
  return v > o ? v : o;
}

__device__ __forceinline__ float wave_max_xor(float v, int width) {
  uint32_t u = __float_as_uint(v);
  if (width >= 2) u = umax_dpp<0xB1>(u);
  if (width >= 4) u = umax_dpp<0x4E>(u);
  if (width >= 8) u = umax_dpp<0x141>(u);
  if (width >= 16) u = umax_dpp<0x140>(u);
  for (int off = 16; off < width; off <<= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)u, off, kWave);
    u = u > o ? u : o;
  }
  return __uint_as_float(u);
}

// Round a positive float32 up to a power of two (bitwise; powers of two unchanged).
__device__ __forceinline__ float ue8m0_ceil(float s) {
  uint32_t u = __float_as_uint(s);
  if (u & 0x007FFFFFu) u = (u & 0x7F800000u) + 0x00800000u;
  return __uint_as_float(u);
}

}  // namespace q8
