// 8-bit activation quantization kernels for gfx950.
//
// "Implementation: Sgl project Sglang GEMM Interface", Description >
// Quantization Routines: per-token-group 8-bit quantization (FP8 e4m3fn or
// INT8) with epsilon, clipping range and optional UE8M0 scales; per-token
// (one group per row) and per-tensor (static or dynamic) variants.
//
// Per group, in float32 with round-to-nearest-even:
//   a = max|x|, s = max(a, eps) / qmax, UE8M0: s -> next power of two,
//   y = clamp(x / s, qmin, qmax), code = e4m3fn(y) (hardware RNE convert) or
//   rint(y) for INT8.
// x / s is the correctly rounded IEEE quotient: an exact multiply by 1/s for
// power-of-two scales, a reciprocal with two FMA residual corrections
// otherwise (see Divider).
//
// Kernels
//   quant_group_wave   groups of 8..512 elements (power of two): each lane
//                      loads 8 consecutive elements (16 B for bf16/f16), the
//                      group's lanes are adjacent in one wave and reduce their
//                      absolute maximum with xor shuffles. HBM-bound.
//   quant_group_rowwave groups of up to 2048 elements that are a multiple of
//                      8 (other than the powers of two above): one wave per
//                      group held in registers, xor-shuffle reduction, codes.
//   quant_group_regs   longer groups of up to 8192 elements (per-token rows):
//                      one workgroup per group held in registers, block
//                      reduction, codes. Both issue every load before the
//                      first use.
//   quant_group_block  any other group size (odd sizes, unaligned strides,
//                      longer rows): one workgroup per group, block reduction,
//                      then a second pass that re-reads the group (L2 hit).
//   quant_fused_wave,  fused SiLU-and-mul (y = silu(gate) * up) and/or masked
//   quant_fused_block  rows: groups of 16..512 (power of two) per lane group,
//                      any other group size one workgroup per group.
//   amax_partials +    per-tensor dynamic: per-workgroup maxima into the
//   quant_tensor       workspace, then every workgroup reduces them (the max
//                      is order independent, so the result is deterministic)
//                      and quantizes a grid-stride slice. Static mode reads
//                      the given scale instead.
#include "q8_internal.h"
#include "q8_device.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;
constexpr int kTensorPartials = 512;
// Groups that are multiples of 8 but not taken by the power-of-two kernel: up
// to kRowWaveMaxGroup elements get one wave each, up to kThreads * 8 * 4 one
// workgroup each. On bf16 [8192, 2048] one wave per row ran 1.6x faster than
// one workgroup per row, on bf16 [8192, 4096] and [4096, 7168] 10-13 % slower.
constexpr int64_t kRowWaveMaxGroup = 2048;

// ---- element loads -----------------------------------------------------------
// Eight consecutive elements as loaded (one 16-byte load for bf16/f16, two for
// float32), converted to float32 on use: a 16-bit vector waiting in registers
// takes 4 of them rather than 8.
template <int XT>
struct Vec8 {
  uint4 w[XT == Q8_F32 ? 2 : 1];
  __device__ __forceinline__ void load(const void* base, int64_t idx) {
    if constexpr (XT == Q8_F32) {
      const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + idx);
      w[0] = p[0];
      w[1] = p[1];
    } else {
      w[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + idx);
    }
  }
  __device__ __forceinline__ void get(float (&f)[8]) const {
    if constexpr (XT == Q8_F32) {
      const uint32_t u[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = __uint_as_float(u[i]);
    } else {
      const uint32_t u[4] = {w[0].x, w[0].y, w[0].z, w[0].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (XT == Q8_BF16) {
          f[2 * i] = __uint_as_float(u[i] << 16);
          f[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
        } else {
          f[2 * i] = f16_bits_to_f32(u[i] & 0xFFFFu);
          f[2 * i + 1] = f16_bits_to_f32(u[i] >> 16);
        }
      }
    }
  }
};

template <int XT>
__device__ __forceinline__ void load8(const void* base, int64_t idx, float (&f)[8]) {
  Vec8<XT> v;
  v.load(base, idx);
  v.get(f);
}

template <int XT>
__device__ __forceinline__ float load1(const void* base, int64_t idx) {
  if constexpr (XT == Q8_F32) return static_cast<const float*>(base)[idx];
  else if constexpr (XT == Q8_BF16) return bf16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
  else return f16_bits_to_f32(static_cast<const uint16_t*>(base)[idx]);
}

// ---- scale and codes -----------------------------------------------------------
template <bool UE>
__device__ __forceinline__ float group_scale(float amax, float eps, float qmax) {
  float s = fmaxf(amax, eps) / qmax;
  return UE ? ue8m0_ceil(s) : s;
}

// y = clamp(x / s), with x / s the correctly rounded IEEE quotient.
// * UE8M0: s is a power of two and x * (1/s) is that same value whenever 1/s
//   is a normal float.
// * Otherwise: y0 = x * r with r = RN(1/s), then two residual corrections
//   q <- q + RN(x - q*s) * r (the residual is exact with an FMA). The second
//   correction starts from a faithful quotient, which with a correctly rounded
//   reciprocal gives the correctly rounded quotient (Markstein's final-step
//   theorem); copysign restores the sign of a zero quotient. Used while s and
//   1/s are far from the float range ends ([2^-100, 2^100]); outside that the
//   plain IEEE division is used. On the device this agreed bit for bit with
//   IEEE division on 4.3e9 pairs drawn from the quantizer's domain wherever
//   |x/s| >= 2^-12, and on every resulting e4m3/int8 code.
template <bool UE>
struct Divider {
  float s, inv;
  bool fast;
  __device__ __forceinline__ explicit Divider(float s_) : s(s_) {
    if constexpr (UE) fast = s_ >= 1.17549435e-38f && s_ <= 8.5070592e37f;
    else fast = s_ >= 7.88860905e-31f && s_ <= 1.26765060e30f;
    inv = fast ? 1.0f / s_ : 0.0f;
  }
  // all eight elements of a vector under one branch on the (per-lane) path
  __device__ __forceinline__ void apply8(const float (&x)[8], float (&y)[8], float qmin,
                                         float qmax) const {
    if (__builtin_expect(fast, 1)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_fmed3f(fast_div(x[i]), qmin, qmax);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = __builtin_amdgcn_fmed3f(x[i] / s, qmin, qmax);
    }
  }
  __device__ __forceinline__ float fast_div(float x) const {
    if constexpr (UE) {
      return x * inv;
    } else {
      const float q0 = x * inv;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), inv, q0);
      return __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q1, s, x), inv, q1), x);
    }
  }
  __device__ __forceinline__ float operator()(float x, float qmin, float qmax) const {
    float y;
    if (!fast) {
      y = x / s;
    } else if constexpr (UE) {
      y = x * inv;
    } else {
      const float q0 = x * inv;
      const float q1 = __builtin_fmaf(__builtin_fmaf(-q0, s, x), inv, q0);
      y = __builtin_copysignf(__builtin_fmaf(__builtin_fmaf(-q1, s, x), inv, q1), x);
    }
    return __builtin_amdgcn_fmed3f(y, qmin, qmax);  // clamp (qmin <= qmax)
  }
};

// Scale store: UE = 2 keeps a UE8M0 scale as its E8M0 byte (the biased
// exponent; s = 2^(b - 127)), in a uint8 [M, K/g] buffer; otherwise float32.
template <int UE>
__device__ __forceinline__ void store_scale(float* s, int64_t i, float sc) {
  if constexpr (UE == 2) reinterpret_cast<uint8_t*>(s)[i] = (uint8_t)(__float_as_uint(sc) >> 23);
  else s[i] = sc;
}

template <bool FP8>
__device__ __forceinline__ uint32_t encode_pair_bytes(float a, float b) {
  if constexpr (FP8) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
  } else {
    int ia = (int)__builtin_rintf(a), ib = (int)__builtin_rintf(b);
    return ((uint32_t)ia & 0xFFu) | (((uint32_t)ib & 0xFFu) << 8);
  }
}

// Four codes in one dword, byte i from y[i]. FP8: the second convert writes
// its pair into the high half of the first one's result.
template <bool FP8>
__device__ __forceinline__ uint32_t encode4(float a, float b, float c, float d) {
  if constexpr (FP8) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
  } else {
    return encode_pair_bytes<false>(a, b) | (encode_pair_bytes<false>(c, d) << 16);
  }
}

template <bool FP8>
__device__ __forceinline__ uint2 encode8(const float (&y)[8]) {
  return uint2{encode4<FP8>(y[0], y[1], y[2], y[3]), encode4<FP8>(y[4], y[5], y[6], y[7])};
}

template <bool FP8>
__device__ __forceinline__ uint8_t encode1(float y) {
  return (uint8_t)(encode_pair_bytes<FP8>(y, 0.0f) & 0xFFu);
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max_xor(v, kWave);
  const int w = threadIdx.x / kWave, l = threadIdx.x % kWave;
  if (l == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / kWave; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---- kernels ---------------------------------------------------------------------
// Each lane handles EPL = 8 or 16 consecutive elements ("a vector": 16 or 32
// bytes of bf16 in, 8 or 16 bytes of codes out), and each thread kUnroll8 *
// 8 / EPL vectors, a grid-stride apart, issuing all of their loads before
// any math (a group's lanes stay adjacent in every slice). 16 elements per
// lane make every code store a full 16 bytes. 16 elements per thread was
// measured fastest on a [4096, 7168] bf16 input (32 and 64 put more bytes in
// flight and ran 8-12 % slower).
#ifndef Q8_QUANT_UNROLL8
#define Q8_QUANT_UNROLL8 2
#endif
constexpr int kUnroll8 = Q8_QUANT_UNROLL8;

template <int XT, bool FP8, int UE, int TPG, bool CONTIG, int EPL>
__global__ __launch_bounds__(kThreads) void quant_group_wave(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, float eps, float qmin, float qmax) {
  static_assert(EPL == 8 || EPL == 16, "8 or 16 elements per lane");
  constexpr int U = kUnroll8 * 8 / EPL;
  constexpr int H = EPL / 8;
  const uint32_t vpr = (uint32_t)(K / EPL);
  const uint32_t total = (uint32_t)(M * vpr);
  float f[U][H][8];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t v = (blockIdx.x + u * gridDim.x) * kThreads + threadIdx.x;
    // CONTIG: rows are ld_x = K apart, so vector v is elements [EPL v,
    // EPL v + EPL) of the flattened input; otherwise the row comes from a
    // 32-bit division (the host keeps M * K / 8 below 2^32). Groups are TPG
    // adjacent lanes aligned to TPG and total is a multiple of TPG, so a group
    // is wholly in range or wholly past the end; lanes past the end load the
    // last vector so every shuffle partner stays defined.
    const uint32_t vv = v < total ? v : total - 1;
    int64_t off;
    if constexpr (CONTIG) {
      off = (int64_t)vv * EPL;
    } else {
      const uint32_t row = vv / vpr;
      off = (int64_t)row * ld_x + (int64_t)(vv - row * vpr) * EPL;
    }
#pragma unroll
    for (int h = 0; h < H; ++h) load8<XT>(x, off + 8 * h, f[u][h]);
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const uint32_t v = (blockIdx.x + u * gridDim.x) * kThreads + threadIdx.x;
    float a = 0.0f;
#pragma unroll
    for (int h = 0; h < H; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[u][h][i]));
    a = wave_max_xor(a, TPG);
    const float sc = group_scale<(UE != 0)>(a, eps, qmax);
    if (v >= total) continue;
    const Divider<(UE != 0)> div(sc);
    // the output is contiguous in either case: vector v is bytes [EPL v,
    // EPL v + EPL) of q and group v / TPG of s
    if constexpr (EPL == 8) {
      float y[8];
      div.apply8(f[u][0], y, qmin, qmax);
      *reinterpret_cast<uint2*>(q + (int64_t)v * 8) = encode8<FP8>(y);
    } else {
      float y0[8], y1[8];
      div.apply8(f[u][0], y0, qmin, qmax);
      div.apply8(f[u][1], y1, qmin, qmax);
      const uint2 lo = encode8<FP8>(y0), hi = encode8<FP8>(y1);
      *reinterpret_cast<uint4*>(q + (int64_t)v * 16) = uint4{lo.x, lo.y, hi.x, hi.y};
    }
    if ((v & (TPG - 1)) == 0) store_scale<UE>(s, v / TPG, sc);
  }
}

template <int XT, bool FP8, int UE, bool VEC>
__global__ __launch_bounds__(kThreads) void quant_group_block(
    const void* __restrict__ x, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, int64_t g, float eps, float qmin, float qmax) {
  __shared__ float red[kThreads / kWave];
  const int64_t groups_per_row = K / g;
  const int64_t row = blockIdx.x / groups_per_row;
  const int64_t j = blockIdx.x - row * groups_per_row;
  const int64_t xb = row * ld_x + j * g;
  const int64_t qb = row * K + j * g;
  float a = 0.0f;
  if constexpr (VEC) {
    for (int64_t i = (int64_t)threadIdx.x * 8; i < g; i += kThreads * 8) {
      float f[8];
      load8<XT>(x, xb + i, f);
#pragma unroll
      for (int t = 0; t < 8; ++t) a = fmaxf(a, fabsf(f[t]));
    }
  } else {
    for (int64_t i = threadIdx.x; i < g; i += kThreads) a = fmaxf(a, fabsf(load1<XT>(x, xb + i)));
  }
  a = block_max(a, red);
  const float sc = group_scale<(UE != 0)>(a, eps, qmax);
  if (threadIdx.x == 0) store_scale<UE>(s, blockIdx.x, sc);
  const Divider<(UE != 0)> div(sc);
  if constexpr (VEC) {
    for (int64_t i = (int64_t)threadIdx.x * 8; i < g; i += kThreads * 8) {
      float f[8], y[8];
      load8<XT>(x, xb + i, f);
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = div(f[t], qmin, qmax);
      *reinterpret_cast<uint2*>(q + qb + i) = encode8<FP8>(y);
    }
  } else {
    for (int64_t i = threadIdx.x; i < g; i += kThreads)
      q[qb + i] = encode1<FP8>(div(load1<XT>(x, xb + i), qmin, qmax));
  }
}

// One workgroup per group of up to kThreads * 8 * NV elements (a per-token
// row, say) held in registers: one read of the input, a block reduction, then
// the codes, instead of re-reading the group after the reduction. Each thread
// owns NV slots of 8 consecutive elements and issues every slot's load before
// the first use, so all of them are in flight together; a slot past the end
// of the group re-reads the group's last 8 elements (repeats leave the maximum
// unchanged) and stores nothing.
template <int XT, bool FP8, int UE, int NV>
__global__ __launch_bounds__(kThreads) void quant_group_regs(
    const void* __restrict__ x, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, uint32_t g, uint32_t groups_per_row, float eps, float qmin,
    float qmax) {
  __shared__ float red[kThreads / kWave];
  const uint32_t row = blockIdx.x / groups_per_row;
  const uint32_t j = blockIdx.x - row * groups_per_row;
  const int64_t xb = (int64_t)row * ld_x + (int64_t)j * g;
  const int64_t qb = (int64_t)row * K + (int64_t)j * g;
  Vec8<XT> r[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t i = (v * kThreads + threadIdx.x) * 8;
    r[v].load(x, xb + (i < g ? i : g - 8));
  }
  float a = 0.0f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    float f[8];
    r[v].get(f);
#pragma unroll
    for (int t = 0; t < 8; ++t) a = fmaxf(a, fabsf(f[t]));
  }
  a = block_max(a, red);
  const float sc = group_scale<(UE != 0)>(a, eps, qmax);
  if (threadIdx.x == 0) store_scale<UE>(s, blockIdx.x, sc);
  const Divider<(UE != 0)> div(sc);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t i = (v * kThreads + threadIdx.x) * 8;
    if (i < g) {
      float f[8], y[8];
      r[v].get(f);
      div.apply8(f, y, qmin, qmax);
      *reinterpret_cast<uint2*>(q + qb + i) = encode8<FP8>(y);
    }
  }
}

// One wave per group of up to kWave * 8 * NV elements, any multiple of 8 (not
// only powers of two): lane l owns the 8-element slots l, l + 64, ... of the
// group, loads all of them before the first use (a slot past the end re-reads
// the group's last 8 elements and stores nothing), and the wave reduces the
// maximum with xor shuffles: no LDS, no barrier. A workgroup holds kThreads /
// kWave consecutive groups.
template <int XT, bool FP8, int UE, int NV>
__global__ __launch_bounds__(kThreads) void quant_group_rowwave(
    const void* __restrict__ x, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, uint32_t ngroups, uint32_t g, uint32_t groups_per_row, float eps,
    float qmin, float qmax) {
  const uint32_t lane = threadIdx.x % kWave;
  const uint32_t grp = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  if (grp >= ngroups) return;  // wave-uniform
  const uint32_t row = grp / groups_per_row;
  const uint32_t j = grp - row * groups_per_row;
  const int64_t xb = (int64_t)row * ld_x + (int64_t)j * g;
  const int64_t qb = (int64_t)row * K + (int64_t)j * g;
  Vec8<XT> r[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t i = (v * kWave + lane) * 8;
    r[v].load(x, xb + (i < g ? i : g - 8));
  }
  float a = 0.0f;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    float f[8];
    r[v].get(f);
#pragma unroll
    for (int t = 0; t < 8; ++t) a = fmaxf(a, fabsf(f[t]));
  }
  a = wave_max_xor(a, kWave);
  const float sc = group_scale<(UE != 0)>(a, eps, qmax);
  if (lane == 0) store_scale<UE>(s, grp, sc);
  const Divider<(UE != 0)> div(sc);
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    const uint32_t i = (v * kWave + lane) * 8;
    if (i < g) {
      float f[8], y[8];
      r[v].get(f);
      div.apply8(f, y, qmin, qmax);
      *reinterpret_cast<uint2*>(q + qb + i) = encode8<FP8>(y);
    }
  }
}

template <int XT, bool VEC>
__global__ __launch_bounds__(kThreads) void amax_partials(const void* __restrict__ x, int64_t M,
                                                         int64_t K, int64_t ld_x,
                                                         float* __restrict__ partial) {
  __shared__ float red[kThreads / kWave];
  float a = 0.0f;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if constexpr (VEC) {
    const int64_t vpr = K >> 3, total = M * vpr;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total; v += stride) {
      const int64_t row = v / vpr, cv = v - row * vpr;
      float f[8];
      load8<XT>(x, row * ld_x + cv * 8, f);
#pragma unroll
      for (int t = 0; t < 8; ++t) a = fmaxf(a, fabsf(f[t]));
    }
  } else {
    const int64_t total = M * K;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
      const int64_t row = e / K, c = e - row * K;
      a = fmaxf(a, fabsf(load1<XT>(x, row * ld_x + c)));
    }
  }
  a = block_max(a, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = a;
}

template <int XT, bool FP8, int UE, bool VEC, bool STATIC>
__global__ __launch_bounds__(kThreads) void quant_tensor(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, const float* __restrict__ partial, int nparts, float eps, float qmin,
    float qmax) {
  __shared__ float red[kThreads / kWave];
  float sc;
  if constexpr (STATIC) {
    sc = s[0];
  } else {
    float a = 0.0f;
    for (int i = threadIdx.x; i < nparts; i += kThreads) a = fmaxf(a, partial[i]);
    a = block_max(a, red);
    sc = group_scale<(UE != 0)>(a, eps, qmax);
    if (blockIdx.x == 0 && threadIdx.x == 0) store_scale<UE>(s, 0, sc);
  }
  const Divider<(UE != 0)> div(sc);
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  if constexpr (VEC) {
    const int64_t vpr = K >> 3, total = M * vpr;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < total; v += stride) {
      const int64_t row = v / vpr, cv = v - row * vpr;
      float f[8], y[8];
      load8<XT>(x, row * ld_x + cv * 8, f);
#pragma unroll
      for (int t = 0; t < 8; ++t) y[t] = div(f[t], qmin, qmax);
      *reinterpret_cast<uint2*>(q + row * K + cv * 8) = encode8<FP8>(y);
    }
  } else {
    const int64_t total = M * K;
    for (int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x; e < total; e += stride) {
      const int64_t row = e / K, c = e - row * K;
      q[row * K + c] = encode1<FP8>(div(load1<XT>(x, row * ld_x + c), qmin, qmax));
    }
  }
}

// ---- fused SiLU-and-mul and masked rows ---------------------------------------
// "Implementation: Sgl project Sglang GEMM Interface", Quantization Routines:
// the per-token-group quantizer's variant with a fused SiLU-and-mul and
// masked-M support. A row of the input is [gate | up] (2K wide); the value
// quantized is y = silu(gate) * up, evaluated in float32 as
//   e = exp(-g) (correctly rounded), d = 1 + e, h = g / d (IEEE), y = h * u,
// one rounding per step, so y (and the code decided from it) is unique.
// Masked rows: the M rows are E blocks of max_m; row r is processed only if
// r % max_m < masked_m[r / max_m], other rows are neither read nor written.

// Correctly rounded float32 exp. exp(x) = 2^k * exp(r) with k = rint(x / ln2)
// and r = x - k ln2 (ln2 split into two doubles, |r| <= ln2/2), exp(r) from
// its Taylor series to degree 13 in float64 (truncation below 2^-57, Horner
// rounding about 2^-52), then one rounding to float32: the result is the
// correctly rounded one unless exp(x) lies within ~2^-50 (relative) of a
// float32 rounding midpoint; the parity tests check every bf16 input.
// x is clamped to [-104, 89]: exp(89) overflows float32 and exp(-104) is below
// half the smallest subnormal, so the float64 -> float32 conversion of the
// clamped value gives +inf and +0 exactly as the unclamped value would.
__device__ __forceinline__ float exp_rn32(float x) {
  constexpr double kInvLn2 = 0x1.71547652b82fep+0;
  constexpr double kLn2Hi = 0x1.62e42fefa39efp-1;   // ln 2 rounded to double
  constexpr double kLn2Lo = 0x1.abc9e3b39803fp-56;  // ln 2 - kLn2Hi
  const double xd = (double)__builtin_amdgcn_fmed3f(x, -104.0f, 89.0f);
  const double k = __builtin_rint(xd * kInvLn2);
  double r = __builtin_fma(-k, kLn2Hi, xd);
  r = __builtin_fma(-k, kLn2Lo, r);
  // 1/n! for n = 13 .. 2, rounded to double
  double p = 0x1.6124613a86d09p-33;
  p = __builtin_fma(p, r, 0x1.1eed8eff8d898p-29);
  p = __builtin_fma(p, r, 0x1.ae64567f544e4p-26);
  p = __builtin_fma(p, r, 0x1.27e4fb7789f5cp-22);
  p = __builtin_fma(p, r, 0x1.71de3a556c734p-19);
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-16);
  p = __builtin_fma(p, r, 0x1.a01a01a01a01ap-13);
  p = __builtin_fma(p, r, 0x1.6c16c16c16c17p-10);
  p = __builtin_fma(p, r, 0x1.1111111111111p-7);
  p = __builtin_fma(p, r, 0x1.5555555555555p-5);
  p = __builtin_fma(p, r, 0x1.5555555555555p-3);
  p = __builtin_fma(p, r, 0.5);
  p = __builtin_fma(p, r, 1.0);
  p = __builtin_fma(p, r, 1.0);
  return (float)__builtin_ldexp(p, (int)k);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  const float d = 1.0f + exp_rn32(-g);
  const float h = g / d;  // IEEE division (correctly rounded)
  return h * u;
}

// Is row r live under the mask? (masked_m == nullptr: every row.)
__device__ __forceinline__ bool row_live(const int32_t* __restrict__ masked_m, uint32_t max_m,
                                         uint32_t row) {
  if (!masked_m) return true;
  const uint32_t e = row / max_m;
  return (int64_t)(row - e * max_m) < (int64_t)masked_m[e];
}

// Groups of 16 * TPG elements (16..512): each lane owns 16 consecutive outputs
// of one row (gate and up vectors loaded with 16-byte loads), the group's TPG
// lanes are adjacent and reduce their |max| with xor shuffles. Rows are
// addressed through ld_x (the input is [M, 2K] with SILU, [M, K] without),
// the codes and scales are contiguous. The host keeps M * K / 16 below 2^32.
template <int XT, bool FP8, int UE, int TPG, bool SILU>
__global__ __launch_bounds__(kThreads) void quant_fused_wave(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, const int32_t* __restrict__ masked_m, uint32_t max_m, float eps,
    float qmin, float qmax) {
  const uint32_t vpr = (uint32_t)(K / 16);
  const uint32_t total = (uint32_t)(M * vpr);
  const uint32_t v = blockIdx.x * kThreads + threadIdx.x;
  // lanes past the end stand in for the last vector (groups are wholly in or
  // out of range: total is a multiple of TPG)
  const uint32_t vv = v < total ? v : total - 1;
  const uint32_t row = vv / vpr;
  const bool live = v < total && row_live(masked_m, max_m, row);
  // a wave holds whole groups, so a wave with no live lane has nothing to do
  // (masked layouts are mostly dead rows)
  if (__ballot(live) == 0) return;
  float y[2][8];
  if (live) {
    const int64_t off = (int64_t)row * ld_x + (int64_t)(vv - row * vpr) * 16;
    load8<XT>(x, off, y[0]);
    load8<XT>(x, off + 8, y[1]);
    if constexpr (SILU) {
      float u[2][8];
      load8<XT>(x, off + K, u[0]);
      load8<XT>(x, off + K + 8, u[1]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) y[h][i] = silu_mul(y[h][i], u[h][i]);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i) y[h][i] = 0.0f;
  }
  float a = 0.0f;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(y[h][i]));
  a = wave_max_xor(a, TPG);  // every lane takes part; dead lanes add 0
  if (!live) return;
  const float sc = group_scale<(UE != 0)>(a, eps, qmax);
  const Divider<(UE != 0)> div(sc);
  float c0[8], c1[8];
  div.apply8(y[0], c0, qmin, qmax);
  div.apply8(y[1], c1, qmin, qmax);
  const uint2 lo = encode8<FP8>(c0), hi = encode8<FP8>(c1);
  *reinterpret_cast<uint4*>(q + (int64_t)v * 16) = uint4{lo.x, lo.y, hi.x, hi.y};
  if ((v & (TPG - 1)) == 0) store_scale<UE>(s, v / TPG, sc);
}

// Any group size: one workgroup per group, element-wise loads, a block
// reduction, then a second pass that recomputes y and writes the codes.
template <int XT, bool FP8, int UE, bool SILU>
__global__ __launch_bounds__(kThreads) void quant_fused_block(
    const void* __restrict__ x, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, int64_t g, const int32_t* __restrict__ masked_m, uint32_t max_m,
    float eps, float qmin, float qmax) {
  __shared__ float red[kThreads / kWave];
  const int64_t groups_per_row = K / g;
  const int64_t row = blockIdx.x / groups_per_row;
  const int64_t j = blockIdx.x - row * groups_per_row;
  if (!row_live(masked_m, max_m, (uint32_t)row)) return;  // uniform per workgroup
  const int64_t xb = row * ld_x + j * g;
  const int64_t qb = row * K + j * g;
  auto value = [&](int64_t i) -> float {
    const float gv = load1<XT>(x, xb + i);
    if constexpr (SILU) return silu_mul(gv, load1<XT>(x, xb + K + i));
    else return gv;
  };
  float a = 0.0f;
  for (int64_t i = threadIdx.x; i < g; i += kThreads) a = fmaxf(a, fabsf(value(i)));
  a = block_max(a, red);
  const float sc = group_scale<(UE != 0)>(a, eps, qmax);
  if (threadIdx.x == 0) store_scale<UE>(s, blockIdx.x, sc);
  const Divider<(UE != 0)> div(sc);
  for (int64_t i = threadIdx.x; i < g; i += kThreads) q[qb + i] = encode1<FP8>(div(value(i), qmin, qmax));
}

// bf16 gates: the float32 steps of silu_mul before the multiply by up,
// h(g) = g / (1 + exp(-g)), depend on the gate's 16 bits alone. For gates
// with 2^-25 <= |g| < 128 (biased exponent 102..133) h is tabulated in LDS,
// 2 signs x 32 exponents x 128 mantissas = 8192 float32, computed by each
// workgroup with the same float64 exp and IEEE division as silu_mul. Outside
// that range h has a closed form in the same float32 arithmetic:
//   |g| < 2^-25: exp(-g) rounds to 1, d = 2 and h = g / 2 = g * 0.5 (exact);
//   g >= 128:    exp(-g) < 2^-184 rounds to 0, d = 1 and h = g;
//   g <= -128:   exp(-g) > 2^184 overflows to +inf and h = g / inf = -0.
// Per element that leaves a table read, one multiply and the quantization.
constexpr int kSiluThreads = 1024;
constexpr int kSiluTable = 8192;
constexpr uint32_t kSiluExpLo = 102, kSiluExpHi = 134;  // table exponent range [lo, hi)

__device__ __forceinline__ float silu_h(float g) {
  const float d = 1.0f + exp_rn32(-g);
  return g / d;  // IEEE division (correctly rounded)
}

// One range test selects the table or, rarely, the closed forms.
__device__ __forceinline__ float silu_h_bf16(float g, const float* __restrict__ tab) {
  const uint32_t b = __float_as_uint(g) >> 16;  // the bf16 bits (g came from a bf16)
  const uint32_t e = (b >> 7) & 0xFFu;
  if (__builtin_expect(e - kSiluExpLo < kSiluExpHi - kSiluExpLo, 1))
    return tab[((b >> 15) << 12) | ((e - kSiluExpLo) << 7) | (b & 127u)];
  return e < kSiluExpLo ? g * 0.5f : ((b >> 15) ? -0.0f : g);
}

// Same work split as quant_fused_wave (16 outputs per lane, a group's TPG
// lanes adjacent in one wave), over a grid of at most two workgroups per CU
// striding in whole workgroups, so each workgroup builds the table once
// (two per CU measured 2 % faster than one at [4096, 2 x 7168]; two vectors
// per thread and iteration were 15 % slower). With a mask (E = M / max_m
// blocks, at most kSiluMaskMaxE) the workgroups stride over the live rows
// only: live row r is row r - pre[e] of block e, pre the exclusive prefix sum
// of the blocks' valid-row counts (clamped to [0, max_m]), found by a binary
// search of pre in LDS.
constexpr int kSiluMaskMaxE = 1024;
template <bool FP8, int UE, int TPG>
__global__ __launch_bounds__(kSiluThreads) void quant_silu_bf16_table(
    const void* __restrict__ x, int64_t M, int64_t K, int64_t ld_x, uint8_t* __restrict__ q,
    float* __restrict__ s, const int32_t* __restrict__ masked_m, uint32_t max_m, float eps,
    float qmin, float qmax) {
  __shared__ float tab[kSiluTable];
  __shared__ uint32_t pre[kSiluMaskMaxE + 1];
  for (int i = threadIdx.x; i < kSiluTable; i += kSiluThreads) {
    const uint32_t e = kSiluExpLo + ((uint32_t)i >> 7 & 31u);
    const uint32_t b = ((uint32_t)i >> 12 << 15) | (e << 7) | ((uint32_t)i & 127u);
    tab[i] = silu_h(__uint_as_float(b << 16));
  }
  const uint32_t vpr = (uint32_t)(K / 16);
  const uint32_t E = masked_m ? (uint32_t)(M / max_m) : 0u;
  if (masked_m && threadIdx.x < kWave) {
    // one wave: inclusive scan of 64 counts at a time
    const int lane = (int)threadIdx.x;
    uint32_t carry = 0;
    if (lane == 0) pre[0] = 0;
    for (uint32_t c = 0; c < E; c += kWave) {
      const uint32_t e = c + (uint32_t)lane;
      int32_t n = e < E ? masked_m[e] : 0;
      n = n < 0 ? 0 : ((uint32_t)n > max_m ? (int32_t)max_m : n);
      uint32_t incl = (uint32_t)n;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = (uint32_t)__shfl_up((int)incl, off, kWave);
        if (lane >= off) incl += y;
      }
      if (e < E) pre[e + 1] = carry + incl;
      carry += (uint32_t)__shfl((int)incl, kWave - 1, kWave);
    }
  }
  __syncthreads();
  const uint32_t rows = masked_m ? pre[E] : (uint32_t)M;
  const uint32_t total = rows * vpr;
  for (uint32_t base = blockIdx.x * kSiluThreads; base < total; base += gridDim.x * kSiluThreads) {
    const uint32_t vl = base + threadIdx.x;
    const bool live = vl < total;
    if (__ballot(live) == 0) continue;  // wave-uniform
    const uint32_t vc = live ? vl : total - 1;
    uint32_t row = vc / vpr;
    const uint32_t col = vc - row * vpr;
    if (masked_m) {
      // block e of live row `row`: the last e with pre[e] <= row
      uint32_t lo = 0, hi = E;  // pre[lo] <= row < pre[hi]
      while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        if (pre[mid] <= row) lo = mid;
        else hi = mid;
      }
      row = lo * max_m + (row - pre[lo]);
    }
    const uint32_t v = row * vpr + col;
    // dead lanes take part in the shuffles with a = 0; y is read on live
    // lanes only
    float y[2][8];
    float a = 0.0f;
    if (live) {
      const int64_t off = (int64_t)row * ld_x + (int64_t)col * 16;
      float u[2][8];
      load8<Q8_BF16>(x, off, y[0]);
      load8<Q8_BF16>(x, off + 8, y[1]);
      load8<Q8_BF16>(x, off + K, u[0]);
      load8<Q8_BF16>(x, off + K + 8, u[1]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          y[h][i] = silu_h_bf16(y[h][i], tab) * u[h][i];
          a = fmaxf(a, fabsf(y[h][i]));
        }
    }
    a = wave_max_xor(a, TPG);
    if (!live) continue;
    const float sc = group_scale<(UE != 0)>(a, eps, qmax);
    const Divider<(UE != 0)> div(sc);
    float c0[8], c1[8];
    div.apply8(y[0], c0, qmin, qmax);
    div.apply8(y[1], c1, qmin, qmax);
    const uint2 lo = encode8<FP8>(c0), hi = encode8<FP8>(c1);
    *reinterpret_cast<uint4*>(q + (int64_t)v * 16) = uint4{lo.x, lo.y, hi.x, hi.y};
    if ((v & (TPG - 1)) == 0) store_scale<UE>(s, v / TPG, sc);
  }
}

// The table pays for itself from a few million elements on (building it costs
// each workgroup about as much as 8192 elements of the direct evaluation).
constexpr int64_t kSiluTableMinElems = 1 << 22;

template <int XT, bool FP8, int UE, bool SILU>
hipError_t dispatch_fused(const QuantArgs& a, hipStream_t st) {
  const int esz = XT == Q8_F32 ? 4 : 2;
  const int64_t g = a.group_size;
  uint8_t* q = static_cast<uint8_t*>(a.q);
  const uint32_t max_m = a.masked_m ? (uint32_t)a.max_m : 1u;
  const dim3 blk(kThreads);
  const int64_t total = a.M * (a.K / 16);
  const bool wave = g >= 16 && g <= 512 && (g & (g - 1)) == 0 && total < 0xFFFF0000LL &&
                    (uintptr_t)a.x % 16 == 0 && (uintptr_t)q % 16 == 0 &&
                    (a.ld_x * esz) % 16 == 0 && (a.K * esz) % 16 == 0;
  const bool mask_fits = !a.masked_m || a.M / (int64_t)max_m <= kSiluMaskMaxE;
  if constexpr (SILU && XT == Q8_BF16) if (wave && mask_fits && a.M * a.K >= kSiluTableMinElems) {
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      return hipErrorInvalidDevice;
    const int64_t need = (total + kSiluThreads - 1) / kSiluThreads;
    const dim3 grid((unsigned)(need < 2 * cus ? need : 2 * cus)), tblk(kSiluThreads);
    switch (g / 16) {
#define Q8_SILU_TABLE_CASE(T)                                                                   \
  case T:                                                                                       \
    hipLaunchKernelGGL((quant_silu_bf16_table<FP8, UE, T>), grid, tblk, 0, st, a.x, a.M, a.K,   \
                       a.ld_x, q, a.s, a.masked_m, max_m, a.eps, a.qmin, a.qmax);               \
    break;
      Q8_SILU_TABLE_CASE(1) Q8_SILU_TABLE_CASE(2) Q8_SILU_TABLE_CASE(4) Q8_SILU_TABLE_CASE(8)
      Q8_SILU_TABLE_CASE(16) Q8_SILU_TABLE_CASE(32)
#undef Q8_SILU_TABLE_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  if (wave) {
    const dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
    switch (g / 16) {
#define Q8_FUSED_CASE(T)                                                                         \
  case T:                                                                                        \
    hipLaunchKernelGGL((quant_fused_wave<XT, FP8, UE, T, SILU>), grid, blk, 0, st, a.x, a.M, a.K, \
                       a.ld_x, q, a.s, a.masked_m, max_m, a.eps, a.qmin, a.qmax);                \
    break;
      Q8_FUSED_CASE(1) Q8_FUSED_CASE(2) Q8_FUSED_CASE(4) Q8_FUSED_CASE(8) Q8_FUSED_CASE(16)
      Q8_FUSED_CASE(32)
#undef Q8_FUSED_CASE
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int64_t ngroups = a.M * (a.K / g);
  if (ngroups > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((quant_fused_block<XT, FP8, UE, SILU>), dim3((unsigned)ngroups), blk, 0, st,
                     a.x, a.K, a.ld_x, q, a.s, g, a.masked_m, max_m, a.eps, a.qmin, a.qmax);
  return hipGetLastError();
}

// ---- host dispatch -------------------------------------------------------------
template <int XT, bool FP8, int UE>
hipError_t dispatch(const QuantArgs& a, hipStream_t st) {
  const int esz = XT == Q8_F32 ? 4 : 2;
  const bool vec = (a.K % 8 == 0) && (a.ld_x % (esz == 2 ? 8 : 4) == 0) &&
                   ((uintptr_t)a.x % 16 == 0) && ((uintptr_t)a.q % 8 == 0);
  uint8_t* q = static_cast<uint8_t*>(a.q);
  const dim3 blk(kThreads);
  if (a.mode == Q8_SCALE_PER_GROUP) {
    const int64_t g = a.group_size;
    const bool pow2 = g >= 8 && g <= 512 && (g & (g - 1)) == 0;
    const int64_t total = a.M * (a.K / 8);
    // 32-bit vector indices, with room for the grid's rounding up
    if (vec && pow2 && total < 0xFFFF0000LL) {
      const bool contig = a.ld_x == a.K;
      // 16 elements per lane when groups, rows and the code rows allow it
      const bool e16 = g >= 16 && a.K % 16 == 0 && (uintptr_t)a.q % 16 == 0 &&
                       (contig || a.ld_x % 16 == 0);
      const int epl = e16 ? 16 : 8;
      const int64_t per_block = (int64_t)kThreads * kUnroll8 * 8;  // elements
      const dim3 grid((unsigned)((a.M * a.K + per_block - 1) / per_block));
      switch ((int)(g / epl) * (e16 ? 1 : 1000)) {
#define Q8_WAVE_LAUNCH(T, C, E)                                                                   \
  hipLaunchKernelGGL((quant_group_wave<XT, FP8, UE, T, C, E>), grid, blk, 0, st, a.x, a.M, a.K, \
                     a.ld_x, q, a.s, a.eps, a.qmin, a.qmax)
#define Q8_WAVE_CASE_E(T, E, KEY)                                   \
  case KEY:                                                         \
    if (contig) Q8_WAVE_LAUNCH(T, true, E);                         \
    else Q8_WAVE_LAUNCH(T, false, E);                               \
    break;
#define Q8_WAVE_CASE(T) Q8_WAVE_CASE_E(T, 8, (T) * 1000)
#define Q8_WAVE_CASE16(T) Q8_WAVE_CASE_E(T, 16, T)
        Q8_WAVE_CASE16(1) Q8_WAVE_CASE16(2) Q8_WAVE_CASE16(4) Q8_WAVE_CASE16(8)
        Q8_WAVE_CASE16(16) Q8_WAVE_CASE16(32)
        Q8_WAVE_CASE(1) Q8_WAVE_CASE(2) Q8_WAVE_CASE(4) Q8_WAVE_CASE(8) Q8_WAVE_CASE(16)
        Q8_WAVE_CASE(32) Q8_WAVE_CASE(64)
#undef Q8_WAVE_CASE
#undef Q8_WAVE_CASE16
#undef Q8_WAVE_CASE_E
#undef Q8_WAVE_LAUNCH
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    const int64_t ngroups = a.M * (a.K / g);
    if (ngroups > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)ngroups);
    const uint32_t g32 = (uint32_t)g, gpr = (uint32_t)(a.K / g);
    if (vec && g % 8 == 0 && g <= kRowWaveMaxGroup) {
      const int nv = (int)((g + kWave * 8 - 1) / (kWave * 8));
      const dim3 wgrid((unsigned)((ngroups + kThreads / kWave - 1) / (kThreads / kWave)));
#define Q8_ROWWAVE_CASE(NV)                                                                     \
  case NV:                                                                                      \
    hipLaunchKernelGGL((quant_group_rowwave<XT, FP8, UE, NV>), wgrid, blk, 0, st, a.x, a.K,     \
                       a.ld_x, q, a.s, (uint32_t)ngroups, g32, gpr, a.eps, a.qmin, a.qmax);     \
    break;
      switch (nv <= 1 ? 1 : nv <= 2 ? 2 : 4) {
        Q8_ROWWAVE_CASE(1) Q8_ROWWAVE_CASE(2) Q8_ROWWAVE_CASE(4)
#undef Q8_ROWWAVE_CASE
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    if (vec && g % 8 == 0 && g <= kThreads * 8 * 4) {
      const int nv = (int)((g + kThreads * 8 - 1) / (kThreads * 8));
#define Q8_REGS_LAUNCH(NV)                                                                      \
  hipLaunchKernelGGL((quant_group_regs<XT, FP8, UE, NV>), grid, blk, 0, st, a.x, a.K, a.ld_x,   \
                     q, a.s, g32, gpr, a.eps, a.qmin, a.qmax)
      if (nv == 1) Q8_REGS_LAUNCH(1);
      else if (nv == 2) Q8_REGS_LAUNCH(2);
      else Q8_REGS_LAUNCH(4);
#undef Q8_REGS_LAUNCH
      return hipGetLastError();
    }
    if (vec && g % 8 == 0)
      hipLaunchKernelGGL((quant_group_block<XT, FP8, UE, true>), grid, blk, 0, st, a.x, a.K,
                         a.ld_x, q, a.s, g, a.eps, a.qmin, a.qmax);
    else
      hipLaunchKernelGGL((quant_group_block<XT, FP8, UE, false>), grid, blk, 0, st, a.x, a.K,
                         a.ld_x, q, a.s, g, a.eps, a.qmin, a.qmax);
    return hipGetLastError();
  }
  // per-tensor modes: grid-stride kernels
  const int64_t work = vec ? a.M * (a.K / 8) : a.M * a.K;
  int64_t blocks = (work + kThreads - 1) / kThreads;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  const dim3 grid((unsigned)blocks);
  float* partial = static_cast<float*>(a.workspace);
  if (a.mode == Q8_SCALE_PER_TENSOR_DYNAMIC) {
    const int np = (int)(blocks < kTensorPartials ? blocks : kTensorPartials);
    if (vec) {
      hipLaunchKernelGGL((amax_partials<XT, true>), dim3(np), blk, 0, st, a.x, a.M, a.K, a.ld_x,
                         partial);
      hipLaunchKernelGGL((quant_tensor<XT, FP8, UE, true, false>), grid, blk, 0, st, a.x, a.M,
                         a.K, a.ld_x, q, a.s, partial, np, a.eps, a.qmin, a.qmax);
    } else {
      hipLaunchKernelGGL((amax_partials<XT, false>), dim3(np), blk, 0, st, a.x, a.M, a.K, a.ld_x,
                         partial);
      hipLaunchKernelGGL((quant_tensor<XT, FP8, UE, false, false>), grid, blk, 0, st, a.x, a.M,
                         a.K, a.ld_x, q, a.s, partial, np, a.eps, a.qmin, a.qmax);
    }
  } else if (vec) {
    hipLaunchKernelGGL((quant_tensor<XT, FP8, false, true, true>), grid, blk, 0, st, a.x, a.M,
                       a.K, a.ld_x, q, a.s, nullptr, 0, a.eps, a.qmin, a.qmax);
  } else {
    hipLaunchKernelGGL((quant_tensor<XT, FP8, false, false, true>), grid, blk, 0, st, a.x, a.M,
                       a.K, a.ld_x, q, a.s, nullptr, 0, a.eps, a.qmin, a.qmax);
  }
  return hipGetLastError();
}

template <int XT, bool FP8, int UE>
hipError_t dispatch_any(const QuantArgs& a, hipStream_t st) {
  if (a.silu) return dispatch_fused<XT, FP8, UE, true>(a, st);
  if (a.masked_m) return dispatch_fused<XT, FP8, UE, false>(a, st);
  return dispatch<XT, FP8, UE>(a, st);
}

template <int XT, bool FP8>
hipError_t dispatch_ue(const QuantArgs& a, hipStream_t st) {
  const int ue = a.mode == Q8_SCALE_STATIC ? 0 : a.ue8m0;
  if (ue == 2) return dispatch_any<XT, FP8, 2>(a, st);
  if (ue == 1) return dispatch_any<XT, FP8, 1>(a, st);
  return dispatch_any<XT, FP8, 0>(a, st);
}

template <int XT>
hipError_t dispatch_q(const QuantArgs& a, hipStream_t st) {
  return a.q_dtype == Q8_E4M3FN ? dispatch_ue<XT, true>(a, st) : dispatch_ue<XT, false>(a, st);
}

}  // namespace

size_t quant_partials_count(int64_t, int64_t) { return kTensorPartials; }

hipError_t launch_quant(const QuantArgs& a, hipStream_t st) {
  switch (a.x_dtype) {
    case Q8_F32: return dispatch_q<Q8_F32>(a, st);
    case Q8_BF16: return dispatch_q<Q8_BF16>(a, st);
    case Q8_F16: return dispatch_q<Q8_F16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace q8
