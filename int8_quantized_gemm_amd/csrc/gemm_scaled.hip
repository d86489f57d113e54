// Per-tensor / per-token x per-channel scaled GEMMs for gfx950: INT8 W8A8
// and FP8 e4m3fn.
//
// vLLM scaled_mm page, AiterInt8ScaledMMLinearKernel.apply_weights: output =
// mm(scale_a * a, scale_b * b) with numpy broadcasting, a [M, K], weights
// [N, K]; per-tensor x per-tensor and per-token x per-channel scales (the
// other two combinations broadcast the same way here). "Implementation: Sgl
// project Sglang GEMM Interface", Scaled Matrix Multiplication: int8_scaled_mm
// and fp8_scaled_mm (per-tensor or per-row / per-column scales, optional
// bias, output dtype).
//
// With one scale per row and per column the whole K loop accumulates inside
// the matrix cores (INT8: v_mfma_i32_16x16x64_i8, exact int32; FP8:
// v_mfma_f32_16x16x128_f8f6f4, float32), with no per-block work; the scales
// and bias are applied once in the epilogue in float32 without FMA
// contraction: ((float)acc * sa) * sb + bias, then round to nearest even.
// gemm_scaled_pipe (K % 128 == 0) uses the block-FP8 tile kernel's pipeline;
// gemm_scaled_tile (register-staged loads, zero-filled partial last slab)
// covers K % 128 != 0.
#include "q8_internal.h"
#include "tile_common.h"

namespace q8 {
namespace {

struct ScaledParams {
  const uint8_t* A;
  const float* sa;
  const uint8_t* W;
  const float* sb;
  const void* bias;
  void* D;
  int64_t M, N, K;
  int sa_per_row, sb_per_col;
  int out_kind;  // 0 = int32 (INT8 only), 1 = bf16, 2 = f16
  int64_t tiles_m, tiles_n;
};

// Accumulator and MFMA per operand type. A 128-byte K slab is two
// 16x16x64 INT8 MFMAs or one 16x16x128 FP8 MFMA; lane group g supplies
// chunks g and g + 4 of the slab for both operands.
template <bool FP8>
struct Mma;
template <>
struct Mma<false> {
  typedef i32x4 acc_t;
  static __device__ __forceinline__ acc_t zero() { return i32x4{0, 0, 0, 0}; }
  static __device__ __forceinline__ acc_t slab(const i32x4& a0, const i32x4& a1, const i32x4& b0,
                                               const i32x4& b1, acc_t c) {
    c = __builtin_amdgcn_mfma_i32_16x16x64_i8(a0, b0, c, 0, 0, 0);
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a1, b1, c, 0, 0, 0);
  }
};
template <>
struct Mma<true> {
  typedef f32x4 acc_t;
  static __device__ __forceinline__ acc_t zero() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
  static __device__ __forceinline__ acc_t slab(const i32x4& a0, const i32x4& a1, const i32x4& b0,
                                               const i32x4& b1, acc_t c) {
    const i32x8 a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const i32x8 b = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    // cbsz = blgp = 0 (both e4m3), zero scale operands: the unscaled MFMA
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
};

template <int BM, int BN, int WM, int WN, bool FP8>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_scaled_tile(ScaledParams p) {
  typedef typename Mma<FP8>::acc_t acc_t;
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * 128];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;

  const int64_t t = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  int64_t tm, tn;
  grouped_order(t, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  const uint8_t* a_src[A_CH];
  const uint8_t* b_src[B_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int idx = tid + c * NT, r = idx >> 3, ch = idx & 7;
    const int64_t m = m0 + r < M ? m0 + r : M - 1;
    a_src[c] = p.A + m * K + ch * 16;
  }
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int idx = tid + c * NT, r = idx >> 3, ch = idx & 7;
    const int64_t n = n0 + r < N ? n0 + r : N - 1;
    b_src[c] = p.W + n * K + ch * 16;
  }

  uint4 ra[A_CH], rb[B_CH];
  // K is a multiple of 16 but not necessarily of 128: the last slab reads
  // only the chunks below K and zero-fills the rest.
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int ch = (tid + c * NT) & 7;
      ra[c] = k0 + ch * 16 < K ? *reinterpret_cast<const uint4*>(a_src[c] + k0) : uint4{0, 0, 0, 0};
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int ch = (tid + c * NT) & 7;
      rb[c] = k0 + ch * 16 < K ? *reinterpret_cast<const uint4*>(b_src[c] + k0) : uint4{0, 0, 0, 0};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) {
      const int idx = tid + c * NT;
      *reinterpret_cast<uint4*>(&sA[buf][swz(idx >> 3, idx & 7)]) = ra[c];
    }
#pragma unroll
    for (int c = 0; c < B_CH; ++c) {
      const int idx = tid + c * NT;
      *reinterpret_cast<uint4*>(&sB[buf][swz(idx >> 3, idx & 7)]) = rb[c];
    }
  };

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Mma<FP8>::zero();

  const int KT = (int)((K + 127) / 128);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload((int64_t)(kt + 1) * 128);
    i32x4 bf[2][FN];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bf[h][j] = *reinterpret_cast<const i32x4*>(&sB[buf][swz(wn * TN + j * 16 + r16, 4 * h + g)]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const i32x4 af0 = *reinterpret_cast<const i32x4*>(&sA[buf][swz(wm * TM + i * 16 + r16, g)]);
      const i32x4 af1 = *reinterpret_cast<const i32x4*>(&sA[buf][swz(wm * TM + i * 16 + r16, 4 + g)]);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = Mma<FP8>::slab(af0, af1, bf[0][j], bf[1][j], acc[i][j]);
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n0 + wn * TN + j * 16 + r16;
    if (col >= N) continue;
    float sbv = 0.f, bv = 0.f;
    if (p.out_kind != 0) {
      sbv = p.sb[p.sb_per_col ? col : 0];
      if (p.bias) {
        const uint16_t h = static_cast<const uint16_t*>(p.bias)[col];
        bv = p.out_kind == 1 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t row = m0 + wm * TM + i * 16 + 4 * g + rr;
        if (row >= M) continue;
        const auto v = acc[i][j][rr];
        if (!FP8 && p.out_kind == 0) {
          static_cast<int32_t*>(p.D)[row * N + col] = (int32_t)v;
        } else {
          const float sav = p.sa[p.sa_per_row ? row : 0];
          float o = __fmul_rn(__fmul_rn((float)v, sav), sbv);
          if (p.bias) o = __fadd_rn(o, bv);
          static_cast<uint16_t*>(p.D)[row * N + col] =
              (uint16_t)(p.out_kind == 1 ? f32_to_bf16_bits(o) : f32_to_f16_bits(o));
        }
      }
    }
  }
}

// K a multiple of 128: the FP8 tile kernel's pipeline (buffer -> LDS loads
// with scalar stage offsets, two LDS stages, one barrier per 128-byte K slab,
// conflict-free fragment layout) with the int32 accumulation kept inside the
// matrix cores. MFMA operand 0 is the weight fragment, so a lane's four
// accumulators are four consecutive output columns of one row.
template <int BM, int BN, int WM, int WN, bool FP8>
__global__ __launch_bounds__(WM * WN * 64) void gemm_scaled_pipe(ScaledParams p) {
  typedef typename Mma<FP8>::acc_t acc_t;
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_SLOTS = BM / 8, B_SLOTS = BN / 8;
  constexpr int A_PER = (A_SLOTS + NW - 1) / NW, B_PER = (B_SLOTS + NW - 1) / NW;
  static_assert(NW % 2 == 0 && TM % 16 == 0 && TN % 16 == 0, "tile");

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * 128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;

  const int64_t t = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
  int64_t tm, tn;
  grouped_order(t, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;

  // same load geometry as the FP8 tile kernel (rows past the end of A or W
  // read zeros from the buffer resource and are never stored)
  const uint32_t lane_off =
      (uint32_t)((lane >> 3) * K + (((lane & 7) ^ ((4 * (w & 1) + (lane >> 4)) & 7)) << 4));
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint32_t)(M * K));
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.W, (uint32_t)(N * K));
  const uint32_t a_base = (uint32_t)(m0 * K), b_base = (uint32_t)(n0 * K);
  auto issue_a = [&](int kt, uint8_t* __restrict__ la) {
#pragma unroll
    for (int c = 0; c < A_PER; ++c) {
      const int q = w + c * NW;
      if (A_SLOTS % NW == 0 || q < A_SLOTS)
        b2l16(rA, lane_off, a_base + (uint32_t)(8 * q) * (uint32_t)K + kt * 128, la + q * 1024);
    }
  };
  auto issue_w = [&](int kt, uint8_t* __restrict__ lb) {
#pragma unroll
    for (int c = 0; c < B_PER; ++c) {
      const int q = w + c * NW;
      if (B_SLOTS % NW == 0 || q < B_SLOTS)
        b2l16(rB, lane_off, b_base + (uint32_t)(8 * q) * (uint32_t)K + kt * 128, lb + q * 1024);
    }
  };
  auto issue = [&](int kt, uint8_t* __restrict__ la, uint8_t* __restrict__ lb) {
    issue_a(kt, la);
    issue_w(kt, lb);
  };

  acc_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = Mma<FP8>::zero();

  // lane group g holds 16-byte chunks g (first 64-wide K step) and g + 4
  // (second) of each row: the same K assignment for both operands
  auto compute = [&](const uint8_t* la, const uint8_t* lb, int wkt, uint8_t* __restrict__ wdst) {
    i32x4 bw[2][FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int row = wn * TN + j * 16 + r16;
      bw[0][j] = *reinterpret_cast<const i32x4*>(lb + swz(row, g));
      bw[1][j] = *reinterpret_cast<const i32x4*>(lb + swz(row, g + 4));
    }
    i32x4 av[2][2];
    av[0][0] = *reinterpret_cast<const i32x4*>(la + swz(wm * TM + r16, g));
    av[0][1] = *reinterpret_cast<const i32x4*>(la + swz(wm * TM + r16, g + 4));
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      // the next slab's weight rows go out here, after two row blocks (its
      // activation rows went out at the barrier): measured 2-5 % faster than
      // issuing both at the barrier, slower from the fourth row block on
      if (i == 2 && wkt >= 0) issue_w(wkt, wdst);
      if (i + 1 < FM) {
        const int row = wm * TM + (i + 1) * 16 + r16;
        av[(i + 1) & 1][0] = *reinterpret_cast<const i32x4*>(la + swz(row, g));
        av[(i + 1) & 1][1] = *reinterpret_cast<const i32x4*>(la + swz(row, g + 4));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = Mma<FP8>::slab(bw[0][j], bw[1][j], av[i & 1][0], av[i & 1][1], acc[i][j]);
    }
  };
  auto step = [&](int kt, bool refill, uint8_t* __restrict__ na, uint8_t* __restrict__ nb,
                  const uint8_t* __restrict__ la, const uint8_t* __restrict__ lb) {
    if (refill) issue_a(kt + 1, na);
    compute(la, lb, refill ? kt + 1 : -1, nb);
  };
  const int KT = (int)(K / 128);
  issue(0, sA0, sB0);
  for (int kt = 0; kt < KT; ++kt) {
    wait_vmem();
    __syncthreads();
    const bool odd = kt & 1;
    step(kt, kt + 1 < KT, odd ? sA0 : sA1, odd ? sB0 : sB1, odd ? sA1 : sA0, odd ? sB1 : sB0);
  }

  // epilogue: lane holds D[m, n .. n+3]. The row scales, column scales and
  // bias this lane needs are loaded once, up front (the output stores could
  // alias them, so the compiler would otherwise reload them before every
  // store, one round trip each).
  const bool scaled = FP8 || p.out_kind != 0;
  float sa_r[FM];
  f32x4 sb4[FN], b4[FN];
  if (scaled) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + wm * TM + i * 16 + r16;
      sa_r[i] = m < M ? p.sa[p.sa_per_row ? m : 0] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
      const bool in = n < N;  // N % 16 == 0: n .. n+3 all in range otherwise
#pragma unroll
      for (int r = 0; r < 4; ++r) sb4[j][r] = in ? p.sb[p.sb_per_col ? n + r : 0] : 0.0f;
      b4[j] = p.bias && in ? load_bias4(p.bias, n, N, p.out_kind == 1, true) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wm * TM + i * 16 + r16;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
      if (n >= N) continue;  // N % 16 == 0: n .. n+3 all in range otherwise
      const acc_t v = acc[i][j];
      if (!FP8 && p.out_kind == 0) {
        *reinterpret_cast<acc_t*>(static_cast<int32_t*>(p.D) + m * N + n) = v;
      } else {
        uint32_t o[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float f = __fmul_rn(__fmul_rn((float)v[r], sa_r[i]), sb4[j][r]);
          if (p.bias) f = __fadd_rn(f, b4[j][r]);
          o[r] = p.out_kind == 1 ? f32_to_bf16_bits(f) : f32_to_f16_bits(f);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.D) + m * N + n) =
            uint2{o[0] | (o[1] << 16), o[2] | (o[3] << 16)};
      }
    }
  }
}

constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;

}  // namespace

hipError_t launch_scaled(const ScaledGemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  ScaledParams p{};
  p.A = static_cast<const uint8_t*>(a.A); p.sa = a.sa;
  p.W = static_cast<const uint8_t*>(a.W); p.sb = a.sb;
  p.bias = a.bias; p.D = a.D;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.sa_per_row = a.sa_numel > 1 || (a.sa_numel == a.M && a.M == 1);
  p.sb_per_col = a.sb_numel > 1 || (a.sb_numel == a.N && a.N == 1);
  p.out_kind = a.out_dtype == Q8_I32 ? 0 : (a.out_dtype == Q8_BF16 ? 1 : 2);
  p.tiles_m = (a.M + kBM - 1) / kBM;
  p.tiles_n = (a.N + kBN - 1) / kBN;
  const int64_t tiles = p.tiles_m * p.tiles_n;
  if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // the pipelined kernel needs whole 128-byte K slabs and 16-byte aligned rows
  // of D (N % 16 == 0 always holds here)
  const bool pipe = a.K % 128 == 0 && (uintptr_t)a.D % 16 == 0 && (uintptr_t)a.bias % 8 == 0;
  const dim3 grid((unsigned)tiles), block(kWM * kWN * 64);
  if (a.fp8) {
    if (pipe) hipLaunchKernelGGL((gemm_scaled_pipe<kBM, kBN, kWM, kWN, true>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gemm_scaled_tile<kBM, kBN, kWM, kWN, true>), grid, block, 0, st, p);
  } else {
    if (pipe) hipLaunchKernelGGL((gemm_scaled_pipe<kBM, kBN, kWM, kWN, false>), grid, block, 0, st, p);
    else hipLaunchKernelGGL((gemm_scaled_tile<kBM, kBN, kWM, kWN, false>), grid, block, 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace q8
