// Block-scaled FP8 GEMM kernels for gfx950 (dense and expert-grouped).
//
// The block32 DeepGEMM PR for DeepSeek-V4.1 ("[SM90] Use native block32
// DeepGEMM for DeepSeek-V4.1"), Modifications: fp8_gemm_nt with recipe
// (1, bn, bk) — activation scale per (row, K block), weight scale per
// (bn x bk) tile — used for both prefill and decode:
//
//   D[m,n] = sum_kb As[m,kb] * Ws[n/bn,kb] * P_kb[m,n],
//   P_kb[m,n] = sum_{k in kb} A[m,k] * W[n,k]   (FP8 x FP8, float32 sum)
//
// Each K block's partial product comes out of the matrix cores on its own
// (a fresh MFMA accumulation), is multiplied by the row/tile scale product
// and added into float32 accumulators with one FMA per output element.
//
// gemm_tile   (M > 64) LDS-tiled: BM x BN output tile per workgroup, K slabs
//             of 128 bytes double-buffered in LDS (XOR-swizzled 16-byte
//             chunks), v_mfma_f32_16x16x128_f8f6f4 for 128-wide K blocks or
//             four v_mfma_f32_16x16x32_fp8_fp8 per slab for 32-wide blocks.
//             XCD-aware tile order. The grouped (MoE) variant walks
//             (expert, n tile, m tile) with row gather/scatter maps.
// gemm_skinny (M <= 64, decode; also the fallback when K is not a multiple of
//             128, one 64-row block per grid row) streams W once: each workgroup owns 16 W rows,
//             its waves split the K blocks, fragments are loaded straight
//             from global memory into MFMA registers (W in the first operand
//             slot, so a lane's four outputs share one activation row and
//             one scale product), and the waves' float32 partials are summed
//             in a fixed order through LDS (deterministic).
#include "q8_internal.h"
#include "tile_common.h"

namespace q8 {
namespace {

struct TileParams {
  const uint8_t* A;
  const float* As;
  const uint8_t* W;
  const float* Ws;
  const void* bias;
  void* D;
  int64_t M, N, K;
  int KB;         // K / bk
  int bn;
  int nbw;        // ceil(N / bn): weight-scale rows (per expert)
  int out_bf16;
  int64_t tiles_m, tiles_n;
  // expert-grouped variant
  const int32_t* offsets;  // [E+1] slot ranges per expert
  const int32_t* a_map;    // slot -> A row (nullable)
  const int32_t* c_inv;    // slot -> D row (nullable)
  int E;
};

__device__ __forceinline__ f32x4 fma4(f32x4 p, f32x4 s, f32x4 acc) {
  f32x4 r;
  r[0] = __builtin_fmaf(p[0], s[0], acc[0]);
  r[1] = __builtin_fmaf(p[1], s[1], acc[1]);
  r[2] = __builtin_fmaf(p[2], s[2], acc[2]);
  r[3] = __builtin_fmaf(p[3], s[3], acc[3]);
  return r;
}

__device__ __forceinline__ f32x4 fma4s(f32x4 p, float s, f32x4 acc) {
  f32x4 r;
  r[0] = __builtin_fmaf(p[0], s, acc[0]);
  r[1] = __builtin_fmaf(p[1], s, acc[1]);
  r[2] = __builtin_fmaf(p[2], s, acc[2]);
  r[3] = __builtin_fmaf(p[3], s, acc[3]);
  return r;
}

__device__ __forceinline__ f32x4 mfma_fp8_k128(const i32x8& a, const i32x8& b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  // cbsz = blgp = 0: both operands FP8 e4m3; zero scale operands select the
  // unscaled v_mfma_f32_16x16x128_f8f6f4.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_fp8_k32(long a, long b) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, b, z, 0, 0, 0);
}

__device__ __forceinline__ float load_out_f32(const void* p, int64_t i, bool bf16) {
  const uint16_t h = static_cast<const uint16_t*>(p)[i];
  return bf16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

__device__ __forceinline__ uint16_t to_out_bits(float v, bool bf16) {
  return (uint16_t)(bf16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v));
}

// ------------------------------------------------------------------------------
// LDS-tiled kernel
// ------------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int KS, bool GROUPED>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile(TileParams p) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KSUB = 128 / KS;
  constexpr int A_CH = BM * 8 / NT, B_CH = BN * 8 / NT;
  constexpr int S_TOT = BM * KSUB, S_PER = (S_TOT + NT - 1) / NT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile/thread mismatch");
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");

  __shared__ __attribute__((aligned(16))) uint8_t sA[2][BM * 128];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][BN * 128];
  __shared__ __attribute__((aligned(16))) float sS[2][KSUB][BM];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K;
  const int KB = p.KB;

  // ---- which tile
  int64_t m_lo, m_hi, n0;
  int e = 0;
  if constexpr (GROUPED) {
    int64_t total = 0;
    for (int x = 0; x < p.E; ++x) {
      const int64_t mt = (p.offsets[x + 1] - p.offsets[x] + BM - 1) / BM;
      total += mt * p.tiles_n;
    }
    if ((int64_t)blockIdx.x >= total) return;
    int64_t L = xcd_remap(blockIdx.x, total);
    int64_t mt = 0;
    for (e = 0; e < p.E; ++e) {
      mt = (p.offsets[e + 1] - p.offsets[e] + BM - 1) / BM;
      if (L < mt * p.tiles_n) break;
      L -= mt * p.tiles_n;
    }
    const int64_t tn = L / mt, tm = L - tn * mt;
    m_lo = p.offsets[e] + tm * BM;
    m_hi = m_lo + BM < p.offsets[e + 1] ? m_lo + BM : p.offsets[e + 1];
    n0 = tn * BN;
  } else {
    const int64_t t = xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n);
    int64_t tm, tn;
    grouped_order(t, p.tiles_m, p.tiles_n, 8, tm, tn);
    m_lo = tm * BM;
    m_hi = m_lo + BM < p.M ? m_lo + BM : p.M;
    n0 = tn * BN;
  }
  const uint8_t* Wb = p.W + (GROUPED ? (int64_t)e * N * K : 0);
  const float* Wsb = p.Ws + (GROUPED ? (int64_t)e * p.nbw * KB : 0);

  auto a_row = [&](int64_t slot) -> int64_t {
    if constexpr (GROUPED) return p.a_map ? (int64_t)p.a_map[slot] : slot;
    else return slot;
  };

  // ---- per-thread staging sources (rows past the end re-read the last valid
  // row; their results are never stored)
  const uint8_t* a_src[A_CH];
  const uint8_t* b_src[B_CH];
#pragma unroll
  for (int c = 0; c < A_CH; ++c) {
    const int idx = tid + c * NT, r = idx >> 3, ch = idx & 7;
    const int64_t slot = m_lo + r < m_hi ? m_lo + r : m_hi - 1;
    a_src[c] = p.A + a_row(slot) * K + ch * 16;
  }
#pragma unroll
  for (int c = 0; c < B_CH; ++c) {
    const int idx = tid + c * NT, r = idx >> 3, ch = idx & 7;
    const int64_t n = n0 + r < N ? n0 + r : N - 1;
    b_src[c] = Wb + n * K + ch * 16;
  }
  const float* s_src[S_PER];
  int s_dst[S_PER];
#pragma unroll
  for (int c = 0; c < S_PER; ++c) {
    const int idx = tid + c * NT;
    const int r = idx % BM, s = idx / BM;
    const int64_t slot = m_lo + r < m_hi ? m_lo + r : m_hi - 1;
    s_src[c] = p.As + a_row(slot) * KB + s;
    s_dst[c] = idx < S_TOT ? idx : -1;  // flat [KSUB][BM] index within a stage
  }

  uint4 ra[A_CH], rb[B_CH];
  float rs[S_PER];
  auto gload = [&](int kt) {
#pragma unroll
    for (int c = 0; c < A_CH; ++c) ra[c] = *reinterpret_cast<const uint4*>(a_src[c] + kt * 128);
#pragma unroll
    for (int c = 0; c < B_CH; ++c) rb[c] = *reinterpret_cast<const uint4*>(b_src[c] + kt * 128);
#pragma unroll
    for (int c = 0; c < S_PER; ++c)
      if (s_dst[c] >= 0) rs[c] = s_src[c][kt * KSUB];
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
#pragma unroll
    for (int c = 0; c < S_PER; ++c)
      if (s_dst[c] >= 0) (&sS[buf][0][0])[s_dst[c]] = rs[c];
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // weight-scale row for each 16-column block of this wave (clamped for
  // ragged N; those columns are never stored)
  const float* ws_row[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int64_t nb = (n0 + wn * TN + j * 16) / p.bn;
    if (nb > p.nbw - 1) nb = p.nbw - 1;
    ws_row[j] = Wsb + nb * KB;
  }

  const int KT = (int)(K / 128);
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint8_t* la = sA[buf];
    const uint8_t* lb = sB[buf];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const int kb = kt * KSUB + s;
      float wsc[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) wsc[j] = ws_row[j][kb];
      if constexpr (KS == 128) {
        i32x8 bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * TN + j * 16 + r16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(lb + swz(row, 2 * g));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(lb + swz(row, 2 * g + 1));
          bf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * TM + i * 16 + r16;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(la + swz(row, 2 * g));
          const i32x4 hi = *reinterpret_cast<const i32x4*>(la + swz(row, 2 * g + 1));
          const i32x8 af = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&sS[buf][s][wm * TM + i * 16 + 4 * g]);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f32x4 pr = mfma_fp8_k128(af, bf[j]);
            acc[i][j] = fma4(pr, sa * wsc[j], acc[i][j]);
          }
        }
      } else {
        long bf[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * TN + j * 16 + r16;
          bf[j] = *reinterpret_cast<const long*>(lb + swz(row, 2 * s + (g >> 1)) + (g & 1) * 8);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * TM + i * 16 + r16;
          const long af = *reinterpret_cast<const long*>(la + swz(row, 2 * s + (g >> 1)) + (g & 1) * 8);
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&sS[buf][s][wm * TM + i * 16 + 4 * g]);
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const f32x4 pr = mfma_fp8_k32(af, bf[j]);
            acc[i][j] = fma4(pr, sa * wsc[j], acc[i][j]);
          }
        }
      }
    }
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: (+ bias) -> 16-bit, MFMA layout: lane holds rows 4g..4g+3
  // of a 16 x 16 block at column r16
  const bool bf16 = p.out_bf16 != 0;
  uint16_t* D = static_cast<uint16_t*>(p.D);
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t col = n0 + wn * TN + j * 16 + r16;
    if (col >= N) continue;
    const float bv = p.bias ? load_out_f32(p.bias, col, bf16) : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int64_t slot = m_lo + wm * TM + i * 16 + 4 * g + rr;
        if (slot >= m_hi) continue;
        int64_t drow = slot;
        if constexpr (GROUPED) {
          drow = p.c_inv ? (int64_t)p.c_inv[slot] : slot;
          if (drow < 0 || drow >= p.M) continue;  // c_map was not a permutation
        }
        D[drow * N + col] = to_out_bits(acc[i][j][rr] + bv, bf16);
      }
    }
  }
}

// ------------------------------------------------------------------------------
// Skinny (decode) kernel
// ------------------------------------------------------------------------------
template <int KS>
struct Frag;
template <>
struct Frag<32> {
  long v;
  __device__ __forceinline__ void load(const uint8_t* p) { v = *reinterpret_cast<const long*>(p); }
};
template <>
struct Frag<128> {
  i32x8 v;
  __device__ __forceinline__ void load(const uint8_t* p) {
    const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
    v = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
};

template <int KS>
__device__ __forceinline__ f32x4 mfma_frag(const Frag<KS>& w, const Frag<KS>& a) {
  if constexpr (KS == 128) return mfma_fp8_k128(w.v, a.v);
  else return mfma_fp8_k32(w.v, a.v);
}

template <int KS, int MT, int NW, int U>
__global__ __launch_bounds__(NW * 64) void gemm_skinny(TileParams p) {
  __shared__ f32x4 red[NW][MT][64];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;
  const int KB = p.KB;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m_base = (int64_t)blockIdx.y * (MT * 16);

  // operand 0 = W rows n0 + r16, operand 1 = activation rows mb*16 + r16;
  // lane group g holds K bytes [g*KS/4, (g+1)*KS/4) of each block for both.
  const int64_t nrow = n0 + r16 < N ? n0 + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + g * (KS / 4);
  const uint8_t* ap[MT];
  const float* asp[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) {
    const int64_t m = m_base + mb * 16 + r16 < M ? m_base + mb * 16 + r16 : M - 1;
    ap[mb] = p.A + m * K + g * (KS / 4);
    asp[mb] = p.As + m * KB;
  }
  // n0 and bn are multiples of 16: one weight block covers all 16 rows
  const float* wsp = p.Ws + (n0 / p.bn) * KB;
  const int kb_b = (int)((int64_t)w * KB / NW), kb_e = (int)((int64_t)(w + 1) * KB / NW);

  f32x4 acc[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  Frag<KS> wf[2][U], af[2][U][MT];
  float sa[2][U][MT], sw[2][U];
  auto load_batch = [&](int b, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kb = kb0 + u < kb_e ? kb0 + u : kb_e - 1;
      wf[b][u].load(wp + (int64_t)kb * KS);
      sw[b][u] = wsp[kb];
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) {
        af[b][u][mb].load(ap[mb] + (int64_t)kb * KS);
        sa[b][u][mb] = asp[mb][kb];
      }
    }
  };
  auto compute_batch = [&](int b, int kb0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (kb0 + u < kb_e) {
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const f32x4 pr = mfma_frag<KS>(wf[b][u], af[b][u][mb]);
          acc[mb] = fma4s(pr, sa[b][u][mb] * sw[b][u], acc[mb]);
        }
      }
    }
  };

  if (kb_b < kb_e) {
    load_batch(0, kb_b);
    int b = 0;
    for (int kb0 = kb_b; kb0 < kb_e; kb0 += U) {
      if (kb0 + U < kb_e) load_batch(b ^ 1, kb0 + U);
      compute_batch(b, kb0);
      b ^= 1;
    }
  }

#pragma unroll
  for (int mb = 0; mb < MT; ++mb) red[w][mb][lane] = acc[mb];
  __syncthreads();

  // fixed-order sum over waves; lane' = (g', r16'): columns n0 + 4g' + rr,
  // activation row mb*16 + r16'
  const bool bf16 = p.out_bf16 != 0;
  uint16_t* D = static_cast<uint16_t*>(p.D);
  for (int idx = tid; idx < MT * 64; idx += NW * 64) {
    const int mb = idx >> 6, l2 = idx & 63;
    const int64_t m = m_base + mb * 16 + (l2 & 15);
    if (m >= M) continue;
    f32x4 s = red[0][mb][l2];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) s += red[ww][mb][l2];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int64_t n = n0 + 4 * (l2 >> 4) + rr;
      if (n >= N) continue;
      const float bv = p.bias ? load_out_f32(p.bias, n, bf16) : 0.0f;
      D[m * N + n] = to_out_bits(s[rr] + bv, bf16);
    }
  }
}

// ------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------
constexpr int kSkinnyMaxM = 64;

template <int KS, int MT>
hipError_t launch_skinny_mt(const TileParams& tp, hipStream_t st) {
  constexpr int NW = 8;
  constexpr int U = KS == 32 ? (MT <= 2 ? 8 : 4) : (MT <= 2 ? 2 : 1);
  const int64_t gy = (tp.M + MT * 16 - 1) / (MT * 16);
  if (gy > 65535 || (tp.N + 15) / 16 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((tp.N + 15) / 16), (unsigned)gy);
  hipLaunchKernelGGL((gemm_skinny<KS, MT, NW, U>), grid, dim3(NW * 64), 0, st, tp);
  return hipGetLastError();
}

template <int KS>
hipError_t launch_skinny(const TileParams& tp, hipStream_t st) {
  const int64_t mt = (tp.M + 15) / 16;  // > 4: several 64-row blocks on grid.y
  switch (mt) {
    case 1: return launch_skinny_mt<KS, 1>(tp, st);
    case 2: return launch_skinny_mt<KS, 2>(tp, st);
    case 3: return launch_skinny_mt<KS, 3>(tp, st);
    default: return launch_skinny_mt<KS, 4>(tp, st);
  }
}

constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;

template <int KS, bool GROUPED>
hipError_t launch_tile(const TileParams& tp, int64_t tiles, hipStream_t st) {
  if (tiles <= 0) return hipSuccess;
  if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm_tile<kBM, kBN, kWM, kWN, KS, GROUPED>), dim3((unsigned)tiles),
                     dim3(kWM * kWN * 64), 0, st, tp);
  return hipGetLastError();
}

TileParams make_params(const BlockGemmArgs& a) {
  TileParams tp{};
  tp.A = a.A; tp.As = a.As; tp.W = a.W; tp.Ws = a.Ws;
  tp.bias = a.bias; tp.D = a.D;
  tp.M = a.M; tp.N = a.N; tp.K = a.K;
  tp.KB = (int)(a.K / a.bk);
  tp.bn = a.bn;
  tp.nbw = (int)((a.N + a.bn - 1) / a.bn);
  tp.out_bf16 = a.out_dtype == Q8_BF16;
  tp.tiles_n = (a.N + kBN - 1) / kBN;
  tp.tiles_m = (a.M + kBM - 1) / kBM;
  tp.offsets = a.expert_offsets; tp.a_map = a.a_map; tp.c_inv = a.c_inv; tp.E = a.E;
  return tp;
}

__global__ void invert_permutation(const int32_t* __restrict__ perm, int64_t n,
                                   int32_t* __restrict__ inv) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) inv[perm[i]] = (int32_t)i;
}

}  // namespace

hipError_t launch_blockwise(const BlockGemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const TileParams tp = make_params(a);
  // decode-sized M, or a K that is not a whole number of 128-byte slabs
  if (a.M <= kSkinnyMaxM || a.K % 128 != 0)
    return a.bk == 128 ? launch_skinny<128>(tp, st) : launch_skinny<32>(tp, st);
  const int64_t tiles = tp.tiles_m * tp.tiles_n;
  return a.bk == 128 ? launch_tile<128, false>(tp, tiles, st) : launch_tile<32, false>(tp, tiles, st);
}

hipError_t launch_grouped(const BlockGemmArgs& a, int64_t total_m, int32_t* c_inv_ws,
                          const int32_t* c_map, hipStream_t st) {
  if (total_m == 0) return hipSuccess;
  BlockGemmArgs b = a;
  if (c_map) {
    const int threads = 256;
    hipLaunchKernelGGL(invert_permutation, dim3((unsigned)((total_m + threads - 1) / threads)),
                       dim3(threads), 0, st, c_map, total_m, c_inv_ws);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    b.c_inv = c_inv_ws;
  } else {
    b.c_inv = nullptr;
  }
  const TileParams tp = make_params(b);
  // upper bound on the number of (expert, m tile) pairs
  const int64_t tiles = ((total_m + kBM - 1) / kBM + a.E) * tp.tiles_n;
  return a.bk == 128 ? launch_tile<128, true>(tp, tiles, st) : launch_tile<32, true>(tp, tiles, st);
}

}  // namespace q8
