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
// Decode (M <= 64) kernels stream W once, its fragments loaded straight from
// global memory into MFMA registers (W in the first operand slot, so a lane's
// four outputs share one activation row and one scale product), and sum the
// waves' float32 partials in a fixed order through LDS (deterministic):
// gemm_stream     one workgroup per 16 W rows, waves splitting the K chunks;
// gemm_stream_pk  up to 2 rows (8 where the staged kernel does not fit),
//                 32-wide blocks: four rows' block partials per MFMA (column j
//                 of the activation operand is one row's block);
// gemm_stream_sa  3..16 rows with 32-wide blocks, 1..16 with 128-wide: the
//                 activation rows staged in LDS per workgroup;
// gemm_split_mid  17..64 rows: K split into ranges, 64 W rows per workgroup,
//                 the range's activation slice in LDS, float32 partials in the
//                 caller's workspace, summed in order by gemm_split_reduce;
// gemm_skinny     K not a multiple of 128 (8-byte fragments), one 64-row block
//                 per grid row.
#include <atomic>
#include <type_traits>

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
  int d_vec4;     // N % 4 == 0 and D (and bias) 8-byte aligned: 8-byte stores
  uint32_t a_bytes, as_bytes;  // extents of A and As (buffer resources)
  int64_t tiles_m, tiles_n;
  // expert-grouped variant
  const int32_t* offsets;  // [E+1] slot ranges per expert
  const int32_t* a_map;    // slot -> A row (nullable)
  const int32_t* c_inv;    // slot -> D row (nullable)
  int E;
  // dense tiles with the last, part-filled round split in K (gemm_tile with
  // SPLIT): tile j of that round is computed by an owner over K slabs
  // [0, split_k) and a helper over [split_k, K/128); the helper's float32
  // partial goes to part (fragment order, BM*BN floats per tile) and it then
  // writes token into flag[j]
  float* part;
  uint32_t* flag;
  uint32_t token;          // odd, new for every call
  int split_k;
  int64_t split_first;     // workgroups of the whole rounds (tiles not split)
  int64_t split_lead;      // helpers dispatched ahead of the owners
  int64_t split_tiles;     // tiles of the last round
  uint32_t part_bytes;     // extent of part (buffer resource)
  uint32_t split_wait;     // longest wait of an owner for its helper, in ticks
                           // of the 100 MHz real-time counter (0: no wait)
};

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
// 32-byte MFMA fragment of one row for lane group g: 16-byte chunks g and
// g + 4 of the row's 128-byte K slab. Any assignment of K bytes to lane groups
// gives the same product as long as both operands use it; this one makes the
// sixteen rows x four lane groups of a ds_read_b128 conflict free (measured on
// gfx950 with the swizzle of tile_common.h).
__device__ __forceinline__ i32x8 lds_frag32(const uint8_t* base, int row, int g) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + swz(row, g));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + swz(row, g + 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ long lds_frag8(const uint8_t* base, int row, int s, int g) {
  return *reinterpret_cast<const long*>(base + swz(row, 2 * s + (g >> 1)) + (g & 1) * 8);
}

// Store four consecutive outputs D[row, n .. n+3] as 16-bit values (any bias
// already added).
__device__ __forceinline__ void store4(const TileParams& p, int64_t row, int64_t n, f32x4 v,
                                       bool bf16, bool vec) {
  uint16_t* D = static_cast<uint16_t*>(p.D);
  const int64_t N = p.N;
  if (vec && n + 3 < N) {
    uint2 o;
    o.x = (uint32_t)to_out_bits(v[0], bf16) | ((uint32_t)to_out_bits(v[1], bf16) << 16);
    o.y = (uint32_t)to_out_bits(v[2], bf16) | ((uint32_t)to_out_bits(v[3], bf16) << 16);
    *reinterpret_cast<uint2*>(D + row * N + n) = o;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (n + r >= N) break;
      D[row * N + n + r] = to_out_bits(v[r], bf16);
    }
  }
}

// Shared memory of one workgroup: two stages of A rows, W rows and
// activation scales. Two stages in separate arrays: the compiler can then
// tell that the LDS reads of one stage never alias the in-flight
// global->LDS loads of the other and does not wait for those loads before
// computing.
struct TileSmem {
  uint8_t* a0; uint8_t* a1; uint8_t* b0; uint8_t* b1; float* s0; float* s1;
};

// BM x BN output tile [m_lo, m_hi) x [n0, n0 + BN) (of expert e) computed by
// one workgroup of WM x WN waves; each wave owns a (BM/WM) x (BN/WN) sub-tile
// made of 16 x 16 MFMA blocks. MFMA operand 0 is the weight fragment and
// operand 1 the activation fragment, so a lane's four accumulators are four
// consecutive output columns of one row: one activation-scale value per row
// block, and 8-byte output stores.
// WSU: every 16-column block of a wave lies in the same weight-scale block.
// sm holds stages of at least BM (A) and BN (W) rows; the activation-scale
// stages, [KSUB][WM][FM/4][16][4], let a lane read its FM row-block scales as
// FM/4 16-byte vectors, consecutive lanes 16 bytes apart (conflict free).
// SPLIT: role 0 computes the whole K range; role 1 (owner) K slabs
// [0, split_k), then adds the helper's partial of tile slot; role 2 (helper)
// slabs [split_k, K/128) into that partial.
template <int BM, int BN, int WM, int WN, int KS, bool GROUPED, bool WSU, bool BIAS, bool SPLIT>
__device__ __forceinline__ void tile_body(const TileParams& p, int64_t m_lo, int64_t m_hi, int64_t n0,
                                          int e, const TileSmem& sm, int role, int64_t slot) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KSUB = 128 / KS;
  constexpr int A_SLOTS = BM / 8, B_SLOTS = BN / 8;  // 1 KB (8 rows) per wave load
  constexpr int A_PER = (A_SLOTS + NW - 1) / NW, B_PER = (B_SLOTS + NW - 1) / NW;
  constexpr int S_SLOTS = BM * KSUB / 64;            // 64 scales per wave load
  constexpr int S_PER = (S_SLOTS + NW - 1) / NW;
  static_assert(TM % 16 == 0 && TN % 16 == 0 && FM % 4 == 0, "wave tile");
  static_assert(BM % 8 == 0 && BN % 8 == 0 && (BM * KSUB) % 64 == 0, "tile");
  uint8_t* const sA0 = sm.a0;
  uint8_t* const sA1 = sm.a1;
  uint8_t* const sB0 = sm.b0;
  uint8_t* const sB1 = sm.b1;
  float* const sS0 = sm.s0;
  float* const sS1 = sm.s1;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K;
  const int KB = p.KB;
  const uint8_t* Wb = p.W + (GROUPED ? (int64_t)e * N * K : 0);
  const float* Wsb = p.Ws + (GROUPED ? (int64_t)e * p.nbw * KB : 0);

  auto a_row = [&](int64_t slot) -> int64_t {
    const int64_t s = slot < m_hi ? slot : m_hi - 1;  // rows past the end re-read the last row
    if constexpr (GROUPED) return p.a_map ? (int64_t)p.a_map[s] : s;
    else return s;
  };

  // ---- per-lane global sources of this wave's LDS loads. Wave load q of a
  // stage fills rows 8q..8q+7; lane l writes physical chunk l%8 of row
  // 8q + l/8, which holds logical chunk (l%8) ^ (row%8).
  // 32-bit byte offsets into buffer resources (the host guarantees every
  // operand is below 4 GiB). Wave load q of a stage fills rows 8q..8q+7;
  // lane l writes physical chunk l%8 of row 8q + l/8, which holds logical
  // chunk (l%8) ^ swz_key(row), and swz_key(8q + l/8) = (4q + l/16) % 8
  // depends on q only through its parity, which is the wave's parity (NW is
  // even): one lane offset serves every load of the wave. The q and stage
  // parts of the offset are scalars. Rows past the end of A or W fall
  // outside the buffer and read as zeros (never stored).
  static_assert(NW % 2 == 0, "wave count must be even");
  const uint32_t lane_off =
      (uint32_t)((lane >> 3) * K + (((lane & 7) ^ ((4 * (w & 1) + (lane >> 4)) & 7)) << 4));
  // Grouped: the tile's gathered A rows differ per lane; their byte offsets
  // live in a small LDS table read at every stage (kept in registers they
  // would be spilled, and reloading a spill waits on every load in flight).
  __shared__ uint32_t sAoff[GROUPED ? BM : 1];
  if constexpr (GROUPED) {
    for (int r = tid; r < BM; r += NW * 64) sAoff[r] = (uint32_t)(a_row(m_lo + r) * K);
    __syncthreads();
  }
  // the lane's chunk within its row (grouped loads add the row from the table)
  auto chunk_off = [&]() -> uint32_t {
    uint32_t c = (uint32_t)(((lane & 7) ^ ((4 * (w & 1) + (lane >> 4)) & 7)) << 4);
    if constexpr (GROUPED) asm volatile("" : "+v"(c));  // recomputed per use, not held live
    return c;
  };
  uint32_t s_off[S_PER];
  // scale loads: waves past the last slot repeat an earlier slot (same bytes
  // to the same place), so every wave issues the same instruction stream
#pragma unroll
  for (int c = 0; c < S_PER; ++c) {
    const int q = (w + c * NW) % S_SLOTS;
    const int f = 64 * q + lane;
    const int s = f / BM, rem = f % BM;
    const int wmm = rem / TM, r2 = rem % TM;
    const int quad = r2 >> 2, i = (quad >> 4) * 4 + (r2 & 3), rr = quad & 15;
    const int row = wmm * TM + i * 16 + rr;
    s_off[c] = (uint32_t)((a_row(m_lo + row) * KB + s) * 4);
  }
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(Wb, (uint32_t)(N * K));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.As, p.as_bytes);
  const uint32_t a_base = GROUPED ? 0u : (uint32_t)(m_lo * K);
  const uint32_t b_base = (uint32_t)(n0 * K);
  // one slab's global->LDS copies, by operand: A rows, W rows, activation
  // scales. Grouped: one table index per lane, recomputed per call; the loads
  // add constant offsets to it (entry 8q + l/8 for q = w + c*NW)
  auto issue_a = [&](int kt, uint8_t* __restrict__ la) {
    uint32_t tix = (uint32_t)(8 * w + (lane >> 3));
    if constexpr (GROUPED) asm volatile("" : "+v"(tix));
#pragma unroll
    for (int c = 0; c < A_PER; ++c) {
      const int q = w + c * NW;
      if (A_SLOTS % NW == 0 || q < A_SLOTS) {
        if constexpr (GROUPED)
          b2l16(rA, sAoff[tix + 8 * NW * c] + chunk_off(), kt * 128, la + q * 1024);
        else
          b2l16(rA, lane_off, a_base + (uint32_t)(8 * q) * (uint32_t)K + kt * 128, la + q * 1024);
      }
    }
  };
  auto issue_w = [&](int kt, uint8_t* __restrict__ lb) {
#pragma unroll
    for (int c = 0; c < B_PER; ++c) {
      const int q = w + c * NW;
      if (B_SLOTS % NW == 0 || q < B_SLOTS)
        b2l16(rB, GROUPED ? (uint32_t)((lane >> 3) * K) + chunk_off() : lane_off,
              b_base + (uint32_t)(8 * q) * (uint32_t)K + kt * 128, lb + q * 1024);
    }
  };
  auto issue_s = [&](int kt, float* __restrict__ ls) {
#pragma unroll
    for (int c = 0; c < S_PER; ++c) b2l4(rS, s_off[c], kt * KSUB * 4, ls + ((w + c * NW) % S_SLOTS) * 64);
  };
  auto issue = [&](int kt, uint8_t* __restrict__ la, uint8_t* __restrict__ lb, float* __restrict__ ls) {
    issue_a(kt, la);
    issue_w(kt, lb);
    issue_s(kt, ls);
  };

  // weight-scale rows of this wave's 16-column blocks (clamped for ragged N);
  // wave-uniform, kept in scalar registers
  int ws_idx[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    int64_t nb = (n0 + wn * TN + j * 16) / p.bn;
    if (nb > p.nbw - 1) nb = p.nbw - 1;
    ws_idx[j] = __builtin_amdgcn_readfirstlane((int)(nb * KB));
  }

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Weight scales of stage kt are loaded (into registers) before the loads of
  // stage kt+1 are issued, so using them never waits on those loads (vector
  // memory completes in order).
  float wsv[KSUB][FN];
  auto load_ws = [&](int kt) {
#pragma unroll
    for (int s = 0; s < KSUB; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) wsv[s][j] = (WSU && j > 0) ? 0.0f : Wsb[ws_idx[j] + kt * KSUB + s];
  };
  auto compute = [&](const uint8_t* la, const uint8_t* lb, const float* ls, const float (&wv)[KSUB][FN]) {
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      float ws[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) ws[j] = WSU ? wv[s][0] : wv[s][j];
      // activation scales of four row blocks at a time (one 16-byte read)
      auto sa_quad = [&](int i4) {
        return *reinterpret_cast<const f32x4*>(ls + s * BM + wm * TM + (i4 * 16 + r16) * 4);
      };
      if constexpr (KS == 128) {
        // Software pipeline over the FM row blocks: the next activation
        // fragment is read from LDS while this block's MFMAs run, and the
        // MFMA results of block i are folded into the accumulators only after
        // block i+1's MFMAs are issued (hides the MFMA result latency).
        i32x8 bw[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bw[j] = lds_frag32(lb, wn * TN + j * 16 + r16, g);
        i32x8 av[2];
        f32x4 pr[2][FN];
        av[0] = lds_frag32(la, wm * TM + r16, g);
        f32x4 saq = sa_quad(0);
        float sa_prev = 0.0f;
        // The two waves sharing a SIMD both run this loop; the issue arbiter
        // favours the older one, which would finish its slab first and idle at
        // the barrier while the younger one runs alone. Each wave drops its
        // priority halfway through the slab, so the one ahead yields to the
        // one behind (measured: prefill 4096x7168x7168 -1.7 %).
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          if (i == FM / 2) __builtin_amdgcn_s_setprio(0);
          if (i + 1 < FM) av[(i + 1) & 1] = lds_frag32(la, wm * TM + (i + 1) * 16 + r16, g);
#pragma unroll
          for (int j = 0; j < FN; ++j) pr[i & 1][j] = mfma_fp8_k128(bw[j], av[i & 1]);
          if (i > 0) {
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i - 1][j] = fma4s(pr[(i - 1) & 1][j], sa_prev * ws[j], acc[i - 1][j]);
          }
          sa_prev = saq[i & 3];
          if ((i & 3) == 3 && i + 1 < FM) saq = sa_quad((i + 1) >> 2);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[FM - 1][j] = fma4s(pr[(FM - 1) & 1][j], sa_prev * ws[j], acc[FM - 1][j]);
      } else {
        float sa[FM];
#pragma unroll
        for (int i4 = 0; i4 < FM / 4; ++i4) {
          const f32x4 v = sa_quad(i4);
          sa[4 * i4] = v[0]; sa[4 * i4 + 1] = v[1]; sa[4 * i4 + 2] = v[2]; sa[4 * i4 + 3] = v[3];
        }
        long bw[FN];
#pragma unroll
        for (int j = 0; j < FN; ++j) bw[j] = lds_frag8(lb, wn * TN + j * 16 + r16, s, g);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const long av = lds_frag8(la, wm * TM + i * 16 + r16, s, g);
          f32x4 pr[FN];
#pragma unroll
          for (int j = 0; j < FN; ++j) pr[j] = mfma_fp8_k32(bw[j], av);
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = fma4s(pr[j], sa[i] * ws[j], acc[i][j]);
        }
      }
    }
  };

  // Stage kt lives in buffer kt % 2; one barrier per stage: after it, stage kt
  // has landed for every wave and stage kt-1 (the other buffer) is no longer
  // read, so it is refilled while stage kt is computed. The refill and the
  // compute go through restrict-qualified pointers of one inlined step, which
  // tells the compiler that the LDS reads never alias the in-flight
  // global->LDS writes (otherwise it waits for those loads before every read).
  auto step = [&](int kt, bool refill, uint8_t* __restrict__ na, uint8_t* __restrict__ nb,
                  float* __restrict__ ns, const uint8_t* __restrict__ la,
                  const uint8_t* __restrict__ lb, const float* __restrict__ ls) {
    float wcur[KSUB][FN];
#pragma unroll
    for (int s = 0; s < KSUB; ++s)
#pragma unroll
      for (int j = 0; j < FN; ++j) wcur[s][j] = wsv[s][j];
    if (refill) {
      load_ws(kt + 1);
      issue(kt + 1, na, nb, ns);
    }
    compute(la, lb, ls, wcur);
  };
  const int KT = (int)(K / 128);
  // K slabs [ka, kb) into the accumulators. The loop used for K blocks of
  // 128, one weight-scale block per wave and up to 64 K blocks; every other
  // case takes the general loop below
  auto general_loop = [&](int ka, int kb) {
    load_ws(ka);
    issue(ka, sA0, sB0, sS0);
    for (int kt = ka; kt < kb; ++kt) {
      wait_vmem();
      __syncthreads();
      const bool odd = (kt - ka) & 1;
      step(kt, kt + 1 < kb, odd ? sA0 : sA1, odd ? sB0 : sB1, odd ? sS0 : sS1,
           odd ? sA1 : sA0, odd ? sB1 : sB0, odd ? sS1 : sS0);
    }
  };
  auto run = [&](int ka, int kb) {
  if constexpr (!(KS == 128 && WSU)) {
    general_loop(ka, kb);
  } else if (KB > 64) {
    general_loop(ka, kb);
  } else {
    // 128-wide K blocks: the last row block of each slab is computed after
    // the slab barrier, behind the LDS reads of the next slab's weight
    // fragments and first activation fragment (issued right after the
    // barrier into a second set of registers), so those reads are in flight
    // while the matrix cores work instead of before the first MFMA of the
    // slab. MFMA results are folded into the accumulators two MFMAs after
    // issue through a ring of three, which frees the registers for the second
    // fragment set. Slabs alternate between stage 0 and stage 1 with the loop
    // unrolled by two, so every LDS address names its stage array and the
    // compiler sees that the refill of one stage never aliases reads of the
    // other.
    constexpr int NT = FM * FN;  // MFMAs per slab and wave
    struct SlabRegs {
      i32x8 bw[FN];
      float sa[FM];
      float ws[1];
    };
    SlabRegs R0, R1;
    i32x8 av[2];
    f32x4 pr[3];
    // the wave's weight scales of all K blocks, one per lane (KB <= 64),
    // loaded once: slab kt takes lane kt's with a readlane, so no load of a
    // scale (and no wait for one) sits in the slab loop
    const float wsl = Wsb[ws_idx[0] + (lane < KB ? lane : KB - 1)];
    auto slab_start = [&](SlabRegs& r, int kt, const uint8_t* __restrict__ lb,
                          const float* __restrict__ ls) {
#pragma unroll
      for (int j = 0; j < FN; ++j) r.bw[j] = lds_frag32(lb, wn * TN + j * 16 + r16, g);
#pragma unroll
      for (int i4 = 0; i4 < FM / 4; ++i4) {
        const f32x4 q = *reinterpret_cast<const f32x4*>(ls + wm * TM + (i4 * 16 + r16) * 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) r.sa[4 * i4 + c] = q[c];
      }
      r.ws[0] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsl), kt));
    };
    auto fold = [&](const SlabRegs& r, int n) {
      const int i = n / FN, j = n % FN;
      acc[i][j] = fma4s(pr[n % 3], r.sa[i] * r.ws[0], acc[i][j]);
      // pins the fold here: otherwise it is sunk past the slab barrier, to its
      // next use, and every MFMA result of the slab stays live until then
      asm volatile("" : "+v"(acc[i][j]));
    };
    // B0, E0: std::integral_constant bounds, so the loop is unrolled with
    // every register index a constant; wkt >= 0 issues the W rows of slab
    // wkt into wdst at step W_STEP (wkt < 0: none)
    constexpr int W_STEP = 12;
    static_assert(W_STEP < NT - FN, "the W refill must go out before the slab barrier");
    auto rows = [&](const SlabRegs& r, const uint8_t* __restrict__ la, auto B0, auto E0, int wkt,
                    uint8_t* __restrict__ wdst) {
      constexpr int n0_ = decltype(B0)::value, n1_ = decltype(E0)::value;
#pragma unroll
      for (int n = n0_; n < n1_; ++n) {
        const int i = n / FN, j = n % FN;
        if (n == W_STEP && wkt >= 0) issue_w(wkt, wdst);
        if (j == 0 && i + 1 < FM) av[(i + 1) & 1] = lds_frag32(la, wm * TM + (i + 1) * 16 + r16, g);
        pr[n % 3] = mfma_fp8_k128(r.bw[j], av[i & 1]);
        if (n >= 2) fold(r, n - 2);
        // keep this order: hoisting the MFMAs ahead of the folds would keep
        // every result live at once
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // one slab: rows 0 .. FM-2, the barrier and the next slab's first reads
    // (plus the refill of this slab's stage with slab kt + 2), then row FM-1
    auto slab = [&](int kt, SlabRegs& cur, SlabRegs& nxt, uint8_t* __restrict__ la,
                    uint8_t* __restrict__ lb, float* __restrict__ ls, const uint8_t* __restrict__ na,
                    const uint8_t* __restrict__ nb, const float* __restrict__ ns) {
      // dense tiles: the W rows of slab kt + 1 go out mid-slab (its A rows and
      // scales went out at the last barrier); grouped tiles refill whole slabs
      rows(cur, la, std::integral_constant<int, 0>{}, std::integral_constant<int, NT - FN>{},
           !GROUPED && kt >= ka + 1 && kt + 1 < kb ? kt + 1 : -1, const_cast<uint8_t*>(nb));
      if (kt + 1 < kb) {
        __builtin_amdgcn_sched_barrier(0);
        wait_vmem();
        __syncthreads();
        // grouped tiles: the refill first (its row-table lookups then retire
        // before the fragment registers fill up)
        if constexpr (GROUPED) {
          if (kt + 2 < kb) issue(kt + 2, la, lb, ls);
        }
        slab_start(nxt, kt + 1, nb, ns);
        av[0] = lds_frag32(na, wm * TM + r16, g);
        if constexpr (!GROUPED) {
          if (kt + 2 < kb) {
            issue_a(kt + 2, la);
            issue_s(kt + 2, ls);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      rows(cur, la, std::integral_constant<int, NT - FN>{}, std::integral_constant<int, NT>{}, -1, nullptr);
      fold(cur, NT - 2);
      fold(cur, NT - 1);
    };
    issue(ka, sA0, sB0, sS0);
    wait_vmem();
    __syncthreads();
    slab_start(R0, ka, sB0, sS0);
    av[0] = lds_frag32(sA0, wm * TM + r16, g);
    if (kb - ka > 1) issue(ka + 1, sA1, sB1, sS1);
    for (int kt = ka; kt < kb; kt += 2) {
      slab(kt, R0, R1, sA0, sB0, sS0, sA1, sB1, sS1);
      if (kt + 1 < kb) slab(kt + 1, R1, R0, sA1, sB1, sS1, sA0, sB0, sS0);
    }
  }
  };

  // Split tiles: the helper's partial lives in part in fragment order (wave,
  // row block, column block, lane: 1 KB per store instruction). Its stores
  // and the owner's loads are agent-coherent (sc1: written through to and
  // read from past the XCD's L2, which is not coherent with the other XCDs'
  // L2s), and the helper publishes the partial by writing the call's token
  // into its flag word once every store has completed.
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(SPLIT ? p.part : nullptr, SPLIT ? p.part_bytes : 0u);
  const uint32_t p_off = (uint32_t)slot * (uint32_t)(BM * BN * 4) + (uint32_t)(w * FM * FN * 1024 + lane * 16);
  uint32_t* const flag = SPLIT ? p.flag + slot : nullptr;
  if constexpr (!SPLIT) {
    run(0, KT);
  } else {
    // The owner trusts the flag only if it changes to this call's token
    // while the owner runs: whatever the word held before (a token of an
    // earlier call, leftovers of other data) can then never pass for the
    // helper's signal, and the workspace needs no initialisation.
    __shared__ uint32_t sReady;
    uint32_t v0 = 0;
    if (role == 1 && w == 0)
      v0 = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    run(role == 2 ? p.split_k : 0, role == 1 ? p.split_k : KT);
    bool ready = false;
    if (role == 1) {
      // wave 0 waits for the helper, at most split_wait ticks of the 100 MHz
      // real-time counter; a helper that is not done by then (it could not
      // get a compute unit, say) leaves the owner to compute the rest of K
      // itself (the general slab loop: the same products folded in the same
      // order as the unsplit kernel's, so such a tile comes out as unsplit)
      if (w == 0) {
        const bool ok = split_owner_wait(flag, p.token, v0, p.split_wait);
        if (lane == 0) sReady = ok ? 1u : 0u;
      }
      __syncthreads();
      ready = sReady != 0;
      if (!ready) general_loop(p.split_k, KT);
    }
    if (role == 2) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          __builtin_amdgcn_raw_buffer_store_b128(acc[i][j], rP, p_off, (uint32_t)((i * FN + j) * 1024), kSc1);
      wait_vmem();
      __syncthreads();
      if (tid == 0) __hip_atomic_store(flag, p.token, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      return;
    }
    if (role == 1) {
      if (ready) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] += __builtin_amdgcn_raw_buffer_load_b128(rP, p_off, (uint32_t)((i * FN + j) * 1024), kSc1);
      }
      // the word goes back to zero for the next call (a graph replay passes
      // the same token again)
      if (tid == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- epilogue: lane holds D[row, n .. n+3], row = block row r16
  const bool bf16 = p.out_bf16 != 0;
  const bool vec = p.d_vec4 != 0;
  // Everything the stores need from memory is loaded once, up front: this
  // lane's bias columns (an instance of its own, so the kernel without a bias
  // carries none of this) and, grouped, its output rows. The stores could
  // alias these arrays, so loads left between them would each wait for every
  // store before them to complete.
  static_assert(!(GROUPED && BIAS), "the grouped entry point has no bias");
  f32x4 bias4[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
    bias4[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BIAS) {
      if (n < N) bias4[j] = load_bias4(p.bias, n, N, bf16, vec && n + 3 < N);
    }
  }
  int64_t drow[FM];  // output row of block row i, -1 for none
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t slot = m_lo + wm * TM + i * 16 + r16;
    drow[i] = slot < m_hi ? slot : -1;
    if constexpr (GROUPED) {
      if (slot < m_hi && p.c_inv) drow[i] = p.c_inv[slot];
      if (drow[i] >= p.M) drow[i] = -1;  // c_map was not a permutation
    }
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (drow[i] < 0) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
      if (n >= N) continue;
      store4(p, drow[i], n, BIAS ? acc[i][j] + bias4[j] : acc[i][j], bf16, vec);
    }
  }
}

#define Q8_TILE_SMEM(BM, BN, KSUB)                                        \
  __shared__ __attribute__((aligned(1024))) uint8_t sA0_[(BM) * 128];     \
  __shared__ __attribute__((aligned(1024))) uint8_t sA1_[(BM) * 128];     \
  __shared__ __attribute__((aligned(1024))) uint8_t sB0_[(BN) * 128];     \
  __shared__ __attribute__((aligned(1024))) uint8_t sB1_[(BN) * 128];     \
  __shared__ __attribute__((aligned(16))) float sS0_[(KSUB) * (BM)];      \
  __shared__ __attribute__((aligned(16))) float sS1_[(KSUB) * (BM)];      \
  const TileSmem sm{sA0_, sA1_, sB0_, sB1_, sS0_, sS1_}

// One tile shape over the whole output (dense), or over the experts' row
// ranges (GROUPED). SPLIT (dense): after split_first workgroups of whole
// tiles come split_lead helpers, then the owners of the split_tiles tiles of
// the last round, then the remaining helpers; helpers ahead of the owners are
// dispatched first, and the later ones take the compute units that the early
// helpers free while the owners still run.
template <int BM, int BN, int WM, int WN, int KS, bool GROUPED, bool WSU, bool BIAS, bool SPLIT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile(TileParams p) {
  Q8_TILE_SMEM(BM, BN, 128 / KS);
  const int lane = threadIdx.x & 63;
  int64_t m_lo, m_hi, n0;
  int e = 0;
  int role = 0;
  int64_t slot = 0;
  if constexpr (GROUPED) {
    // (expert, m tile, n tile) of this workgroup from the experts' row
    // offsets, 64 experts at a time across the lanes of every wave (a serial
    // walk over the experts would cost one dependent load per expert): a
    // reduction gives the number of tiles, an inclusive scan and a ballot
    // find the expert whose tiles contain this one. The host keeps the tile
    // count below 2^31.
    auto tiles_of = [&](int x) -> int {
      if (x >= p.E) return 0;
      return ((p.offsets[x + 1] - p.offsets[x] + BM - 1) / BM) * (int)p.tiles_n;
    };
    int total = 0;
    for (int c = 0; c < p.E; c += 64) {
      int t = tiles_of(c + lane);
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off, 64);
      total += t;
    }
    total = __builtin_amdgcn_readfirstlane(total);
    if ((int)blockIdx.x >= total) return;
    int L = (int)xcd_remap(blockIdx.x, total);
    int base = 0, mt = 1;
    for (int c = 0; c < p.E; c += 64) {
      const int t = tiles_of(c + lane);
      int incl = t;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const int chunk = __shfl(incl, 63, 64);
      if (L < base + chunk) {
        const int le = __builtin_ctzll(__ballot(base + incl > L));
        e = c + le;
        L -= base + __shfl(incl - t, le, 64);
        mt = __shfl(t, le, 64) / (int)p.tiles_n;
        break;
      }
      base += chunk;
    }
    e = __builtin_amdgcn_readfirstlane(e);
    L = __builtin_amdgcn_readfirstlane(L);
    mt = __builtin_amdgcn_readfirstlane(mt);
    const int64_t tn = L / mt, tm = L - tn * mt;
    m_lo = p.offsets[e] + tm * BM;
    m_hi = m_lo + BM < p.offsets[e + 1] ? m_lo + BM : p.offsets[e + 1];
    n0 = tn * BN;
  } else {
    int64_t b = blockIdx.x;
    if constexpr (SPLIT) {
      // split tile j takes the tile that workgroup split_first + j would
      // take unsplit (same XCD when the counts are multiples of 8)
      const int64_t c = b - p.split_first;
      if (c >= 0) {
        if (c < p.split_lead) { role = 2; slot = c; }
        else if (c < p.split_lead + p.split_tiles) { role = 1; slot = c - p.split_lead; }
        else { role = 2; slot = c - p.split_tiles; }
        b = p.split_first + slot;
      }
    }
    const int64_t t = xcd_remap(b, p.tiles_m * p.tiles_n);
    int64_t tm, tn;
    // four tile-rows per group (measured against eight: 4096x18432x7168
    // 3 % faster, 4096x7168x7168 and 2048x7168x7168 0.5-1 %; sixteen slower)
    grouped_order(t, p.tiles_m, p.tiles_n, 4, tm, tn);
    m_lo = tm * BM;
    m_hi = m_lo + BM < p.M ? m_lo + BM : p.M;
    n0 = tn * BN;
  }
  tile_body<BM, BN, WM, WN, KS, GROUPED, WSU, BIAS, SPLIT>(p, m_lo, m_hi, n0, e, sm, role, slot);
}

// ------------------------------------------------------------------------------
// Skinny (decode) kernel
// ------------------------------------------------------------------------------
// A 16x16x128 fragment (lane group g: chunk bytes [16g, 16g+16) in dwords
// 0..3, [64+16g, 64+16g+16) in dwords 4..7) regrouped into four 16x16x32
// operands, one per 32-wide K block: v_permlane32_swap exchanges the upper
// 32 lanes of its first operand with the lower 32 lanes of its second, so
// swapping dwords 0, 1, 4, 5 with dwords 2, 3, 6, 7 that way leaves in dwords
// 2s and 2s + 1 of lane group g the chunk bytes [32s + 16 (g & 1) +
// 8 (g >> 1), +8): each block's 32 bytes spread over the four lane groups.
// The other operand must hold the same bytes per lane group.
__device__ __forceinline__ void regroup_blocks(i32x8& f) {
  constexpr int lo[4] = {0, 1, 4, 5};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d = lo[i];
    const auto r = __builtin_amdgcn_permlane32_swap(f[d], f[d + 2], false, false);
    f[d] = (int)r[0];
    f[d + 2] = (int)r[1];
  }
}

// 16x16x32 operand of block s from a regrouped fragment
__device__ __forceinline__ long dword_pair(const i32x8& f, int s) {
  return (long)(uint32_t)f[2 * s] | ((long)(uint32_t)f[2 * s + 1] << 32);
}

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
// Streaming (decode) kernel: K a multiple of 128
// ------------------------------------------------------------------------------
__device__ __forceinline__ i32x8 gload32(const uint8_t* p) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 16);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Fragment layout of gemm_stream_sel and gemm_stream_sa: lane group g holds bytes [16g, 16g+16)
// (first half) and [64+16g, 64+16g+16) (second half) of each 128-byte chunk,
// so each load instruction reads a contiguous 64-byte half of sixteen weight
// rows (measured: M = 16 10.9 -> 10.5 us against 32-byte lane pieces).
__device__ __forceinline__ i32x8 gload_halves(const uint8_t* p) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 64);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// One workgroup per 16 weight rows (x one 16*MT-row activation block); its
// NW waves split the 128-byte K chunks and issue every load of their share
// before any math, so the whole weight slice is in flight at once. Lane group
// g of both operands holds bytes [32g, 32g+32) of a chunk — exactly one
// 32-wide K block — so for bk = 32 each block's partial sum is the
// 16x16x128 product with the activation fragment zeroed outside lane group s
// (compute is idle at decode sizes; the weight bytes are read once, 32 per
// lane per chunk). Partials are summed over the waves in a fixed order.
template <int KS, int MT, int NW, int R>
__global__ __launch_bounds__(NW * 64) void gemm_stream(TileParams p) {
  constexpr int KSUB = 128 / KS;
  static_assert(R * KSUB <= 64, "round scales must fit one wave");
  __shared__ f32x4 red[NW][MT][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;
  const int KB = p.KB;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t m_base = (int64_t)blockIdx.y * (MT * 16);
  const int NC = (int)(K / 128);
  const int c_b = (int)((int64_t)w * NC / NW), c_e = (int)((int64_t)(w + 1) * NC / NW);

  const int64_t nrow = n0 + r16 < N ? n0 + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + 32 * g;
  const uint8_t* ap[MT];
  const float* asp[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) {
    const int64_t m = m_base + mb * 16 + r16 < M ? m_base + mb * 16 + r16 : M - 1;
    ap[mb] = p.A + m * K + 32 * g;
    asp[mb] = p.As + m * KB;
  }
  const float* wsp = p.Ws + (n0 / p.bn) * KB;  // n0, bn multiples of 16: one block

  f32x4 acc[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  for (int c0 = c_b; c0 < c_e; c0 += R) {
    i32x8 wf[R], af[R][MT];
    float sa[R][KSUB][MT];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int c = c0 + u < c_e ? c0 + u : c_e - 1;
      wf[u] = gload32(wp + (int64_t)c * 128);
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) {
        af[u][mb] = gload32(ap[mb] + (int64_t)c * 128);
#pragma unroll
        for (int s = 0; s < KSUB; ++s) sa[u][s][mb] = asp[mb][c * KSUB + s];
      }
    }
    // this round's weight scales, one per lane, broadcast with readlane
    const int kb_l = c0 * KSUB + lane < KB ? c0 * KSUB + lane : KB - 1;
    const float wsl = wsp[kb_l];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (c0 + u >= c_e) break;
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsl), u * KSUB + s));
#pragma unroll
        for (int mb = 0; mb < MT; ++mb) {
          const i32x8 a = (KS == 128 || g == s) ? af[u][mb] : zero8;
          const f32x4 pr = mfma_fp8_k128(wf[u], a);
          acc[mb] = fma4s(pr, sa[u][s][mb] * ws, acc[mb]);
        }
      }
    }
  }

#pragma unroll
  for (int mb = 0; mb < MT; ++mb) red[w][mb][lane] = acc[mb];
  __syncthreads();
  const bool bf16 = p.out_bf16 != 0;
  const bool vec = p.d_vec4 != 0;
  for (int idx = tid; idx < MT * 64; idx += NW * 64) {
    const int mb = idx >> 6, l2 = idx & 63;
    const int64_t m = m_base + mb * 16 + (l2 & 15);
    if (m >= M) continue;
    f32x4 sum = red[0][mb][l2];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][mb][l2];
    const int64_t n = n0 + 4 * (l2 >> 4);
    if (n < N) store4(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec && n + 3 < N) : sum, bf16, vec);
  }
}

// ------------------------------------------------------------------------------
// Streaming (decode) kernel for 32-wide K blocks and few activation rows
// ------------------------------------------------------------------------------
// One 16x16x128 MFMA over a 128-byte chunk yields every 32-wide block partial
// of four activation rows at once: column j of the activation operand carries
// row m = 4t + j/4 restricted to K block b = j%4 of the chunk (zero outside
// it), so D[n, j] = P_b[n, m]. Lane group g holds bytes [32g, 32g+32) of the
// chunk for both operands — block g — so column j's lane in group g loads its
// 32 activation bytes only when g == j%4 and is zero otherwise. MT4 MFMAs per
// chunk cover 4*MT4 activation rows (against one MFMA per block and 16-row
// block for a dense activation operand). A lane's four outputs share (m, b):
// one scale product As[m, kb] * Ws[n/bn, kb] per MFMA. After the K loop the
// four block residues b of a row are summed across the adjacent lanes (a fixed
// pairing, so every lane holds the same bits), then over the waves in a fixed
// order.
template <int MT4, int NW, int R>
__global__ __launch_bounds__(NW * 64) void gemm_stream_pk(TileParams p) {
  __shared__ f32x4 red[NW][MT4][16];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int b = r16 & 3, q = r16 >> 2;
  const int64_t N = p.N, K = p.K, M = p.M;
  const int KB = p.KB;  // K / 32
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int NC = (int)(K / 128);
  const int c_b = (int)((int64_t)w * NC / NW), c_e = (int)((int64_t)(w + 1) * NC / NW);

  const int64_t nrow = n0 + r16 < N ? n0 + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + 32 * g;
  const float* wsp = p.Ws + (n0 / p.bn) * KB + b;  // n0, bn multiples of 16: one block
  const uint8_t* ap[MT4];
  const float* asp[MT4];
  bool act[MT4], has[MT4];
#pragma unroll
  for (int t = 0; t < MT4; ++t) {
    const int64_t m = 4 * t + q;
    has[t] = m < M;
    act[t] = has[t] && g == b;
    const int64_t mc = has[t] ? m : M - 1;
    ap[t] = p.A + mc * K + 32 * g;
    asp[t] = p.As + mc * KB + b;
  }

  f32x4 acc[MT4];
#pragma unroll
  for (int t = 0; t < MT4; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  const i32x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};

  for (int c0 = c_b; c0 < c_e; c0 += R) {
    i32x8 wf[R], af[R][MT4];
    float sa[R][MT4], ws[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int c = c0 + u < c_e ? c0 + u : c_e - 1;
      wf[u] = gload32(wp + (int64_t)c * 128);
#pragma unroll
      for (int t = 0; t < MT4; ++t) af[u][t] = act[t] ? gload32(ap[t] + (int64_t)c * 128) : zero8;
      ws[u] = wsp[4 * c];
#pragma unroll
      for (int t = 0; t < MT4; ++t) sa[u][t] = has[t] ? asp[t][4 * c] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (c0 + u >= c_e) break;
#pragma unroll
      for (int t = 0; t < MT4; ++t) {
        const f32x4 pr = mfma_fp8_k128(wf[u], af[u][t]);
        acc[t] = fma4s(pr, sa[u][t] * ws[u], acc[t]);
      }
    }
  }

  // sum the four block residues of each activation row: (b0 + b1) + (b2 + b3)
#pragma unroll
  for (int t = 0; t < MT4; ++t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = acc[t][i];
      v += __shfl_xor(v, 1, 64);
      v += __shfl_xor(v, 2, 64);
      acc[t][i] = v;
    }
    if (b == 0) red[w][t][4 * g + q] = acc[t];
  }
  __syncthreads();
  // fixed-order sum over the waves; entry e = 4g + q holds W rows n0 + 4g ..
  // n0 + 4g + 3 of activation row 4t + q
  const bool bf16 = p.out_bf16 != 0;
  const bool vec = p.d_vec4 != 0;
  for (int idx = tid; idx < MT4 * 16; idx += NW * 64) {
    const int t = idx >> 4, e = idx & 15;
    const int64_t m = 4 * t + (e & 3);
    if (m >= M) continue;
    f32x4 sum = red[0][t][e];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][t][e];
    const int64_t n = n0 + 4 * (e >> 2);
    if (n < N) store4(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec && n + 3 < N) : sum, bf16, vec);
  }
}

// ------------------------------------------------------------------------------
// Streaming (decode) kernel with shared activations: M <= 16, K a multiple of 1024
// ------------------------------------------------------------------------------

// Activation rows and their scales -> LDS, the rows at a pitch of a_pitch
// bytes (rows are K bytes, K a multiple of 1024, so no 1 KB load crosses a
// row); the scale copy is rounded up to whole 1 KB loads, the tail reading
// zeros from the resource's range check. Wave w of NW issues every NW-th load.
template <int NW>
__device__ __forceinline__ void stage_rows(const TileParams& p, uint32_t a_pitch, uint32_t s_bytes,
                                           uint8_t* sA, uint8_t* sS, int w, int lane) {
  const int64_t M = p.M, K = p.K;
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint32_t)(M * K));
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.As, s_bytes);
  const int per_row = (int)(K / 1024), a_loads = (int)M * per_row;
  for (int i = w; i < a_loads; i += NW) {
    const int row = i / per_row, col = (i - row * per_row) * 1024;
    b2l16(rA, (uint32_t)lane * 16, (uint32_t)i * 1024, sA + row * a_pitch + col);
  }
  const int s_loads = (int)((s_bytes + 1023u) >> 10);
  for (int i = w; i < s_loads; i += NW) b2l16(rS, (uint32_t)lane * 16, (uint32_t)i * 1024, sS + i * 1024);
}

// Every workgroup needs all M activation rows and their scales. Read from L2
// by every wave, those few lines are requested by thousands of waves at once
// and serialise on their L2 channels; here one linear pass per workgroup
// copies them into LDS (buffer->LDS, 1 KB per load) while the weight loads of
// every wave are already in flight, and the waves read them from LDS.
// LDS: activation rows at a pitch of K + 16 bytes (sixteen lanes reading one
// K offset of sixteen rows hit sixteen bank groups), then the scale rows,
// then the waves' partials.
// DA: weight chunks a wave issues before its first MFMA; each later chunk is
// issued while the one DA before it is computed (DA = R: all up front).
template <int KS, int NW, int R, int DA>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(1, NW / 4)))
void gemm_stream_sa(TileParams p) {
  constexpr int KSUB = 128 / KS;
  static_assert(R * KSUB <= 64, "round scales must fit one wave");
  static_assert(KSUB == 1 || KSUB == 4, "128- or 32-wide K blocks");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;  // M <= 16
  const int KB = p.KB;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int NC = (int)(K / 128);
  const int c_b = (int)((int64_t)w * NC / NW), c_e = (int)((int64_t)(w + 1) * NC / NW);
  const uint32_t a_pitch = (uint32_t)K + 16;
  const uint32_t s_bytes = (uint32_t)(M * KB * 4);
  uint8_t* sA = smem;
  uint8_t* sS = smem + M * a_pitch;
  f32x4* red = reinterpret_cast<f32x4*>(sS + ((s_bytes + 1023u) & ~1023u));  // [NW][64]

  stage_rows<NW>(p, a_pitch, s_bytes, sA, sS, w, lane);
  // this wave's weight scales (one per lane) and weight chunks, issued after
  // the LDS copies so that waiting for the copies leaves them in flight
  const float* wsp = p.Ws + (n0 / p.bn) * KB;  // n0, bn multiples of 16: one block
  const int kb_l = c_b * KSUB + lane < KB ? c_b * KSUB + lane : KB - 1;
  const float wsl = wsp[kb_l];
  asm volatile("" ::: "memory");
  const int64_t nrow = n0 + r16 < N ? n0 + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + 16 * g;
  static_assert(DA >= 1 && DA <= R, "chunks issued ahead");
  i32x8 wf[R];
  auto issue_w = [&](int u) {
    // unconditional (clamped) loads: exactly 2 DA of them follow the copies
    const int c = c_b + u < NC - 1 ? c_b + u : NC - 1;
    wf[u] = gload_halves(wp + (int64_t)c * 128);
  };
#pragma unroll
  for (int u = 0; u < DA; ++u) issue_w(u);
  // the copies were issued before the 2 DA weight loads, and loads complete
  // in order: at most 2 DA outstanding means this wave's copies have landed.
  // The bare barrier (no fence) keeps the weight loads in flight across it.
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DA) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = r16 < M ? r16 : (int)M - 1;  // rows past M repeat the last (never stored)
  // 32-wide blocks: the regrouped weight fragment's bytes of every block,
  // 8 at 32s + 16 (g & 1) + 8 (g >> 1) per lane group
  const uint8_t* al = sA + arow * a_pitch + (KS == 32 ? 16 * (g & 1) + 8 * (g >> 1) : 16 * g);
  const float* sl = reinterpret_cast<const float*>(sS) + arow * KB;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int c = c_b + u;
    if (c >= c_e) break;
    if (u + DA < R) issue_w(u + DA);
    i32x8 af;
    if constexpr (KS == 32) {
      regroup_blocks(wf[u]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int2 v = *reinterpret_cast<const int2*>(al + c * 128 + 32 * q);
        af[2 * q] = v.x;
        af[2 * q + 1] = v.y;
      }
    } else {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(al + c * 128);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(al + c * 128 + 64);
      af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    f32x4 sa;
    if constexpr (KSUB == 4) sa = *reinterpret_cast<const f32x4*>(sl + c * 4);
    else sa[0] = sl[c];
#pragma unroll
    for (int s = 0; s < KSUB; ++s) {
      const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsl), u * KSUB + s));
      const f32x4 pr = KS == 128 ? mfma_fp8_k128(wf[u], af) : mfma_fp8_k32(dword_pair(wf[u], s), dword_pair(af, s));
      acc = fma4s(pr, sa[s] * ws, acc);
    }
  }

  red[w * 64 + lane] = acc;
  __syncthreads();
  // fixed-order sum over the waves, one output per thread
  const bool bf16 = p.out_bf16 != 0;
  uint16_t* D = static_cast<uint16_t*>(p.D);
  const float* redf = reinterpret_cast<const float*>(red);
  for (int idx = tid; idx < 256; idx += NW * 64) {
    const int l2 = idx >> 2, rr = idx & 3;
    const int64_t m = l2 & 15;
    const int64_t n = n0 + 4 * (l2 >> 4) + rr;
    if (m >= M || n >= N) continue;
    float sum = redf[l2 * 4 + rr];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += redf[(ww * 64 + l2) * 4 + rr];
    if (p.bias) sum += load_out_f32(p.bias, n, bf16);
    D[m * N + n] = to_out_bits(sum, bf16);
  }
}

// ------------------------------------------------------------------------------
// Split-K streaming kernel for decode batches of 17..64 activation rows
// ------------------------------------------------------------------------------
// A workgroup that owns 16 weight rows for all of K needs the whole activation
// (M x K bytes) from L2: at 64 rows that is four times the weight bytes it
// streams, and those L2 reads, not the HBM stream, set the time. Here a
// workgroup owns 64 weight rows (four 16-row blocks) and one of S K ranges of
// Kc = K/S bytes: it copies the activation slice [M, Kc] and its scales into
// LDS once (buffer->LDS, so the copies are in flight with the weight loads),
// streams its 64 x Kc weight bytes (each wave keeps one 128-byte chunk, two
// above 32 rows, in flight ahead of its MFMAs; 128-wide blocks up to 32 rows
// issue all of them up front), and writes its float32 partial [M, 64] for
// that K range;
// gemm_split_reduce then sums the S partials of every output in a fixed
// order (deterministic), adds the bias and rounds.
// MFMA columns: sixteen activation rows per MFMA (one 16x16x128 MFMA per
// chunk and 16-row block for 128-wide K blocks; for 32-wide blocks four
// 16x16x32 MFMAs, one per block, on the regrouped weight fragment), so a
// lane's four outputs share one scale product.
// LDS activation slice: dense [M, Kc], 16-byte piece j of row m stored at
// piece position j ^ (m & 15) (Kc a multiple of 256 bytes keeps every row's
// pieces inside the row); sixteen lanes reading one piece of sixteen rows
// then hit sixteen different bank groups. The XOR is applied through the
// source address of the copies, whose LDS side is contiguous.
constexpr int kMidRows = 64;   // weight rows per workgroup
constexpr int kMidNW = 8;      // waves: 4 row blocks x 2 chunk parities

template <int KS, int MT, int R>
__global__ __launch_bounds__(kMidNW * 64) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_split_mid(TileParams p, float* __restrict__ part, int Kc) {
  constexpr int KSUB = 128 / KS;
  constexpr int NP = kMidNW / 4;  // chunk parities (waves per row block)
  static_assert(R * KSUB <= 64, "a wave's weight scales fit one register");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = w & 3, h = w >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;
  const int KB = p.KB;
  const int s_idx = blockIdx.y;
  const int64_t k0 = (int64_t)s_idx * Kc;
  const int kb0 = (int)(k0 / KS);
  const int kbc = Kc / KS;          // K blocks in the slice
  const int ncc = Kc / 128;         // chunks in the slice
  const int pr = Kc / 16;           // 16-byte pieces per activation row
  const int64_t n0 = (int64_t)blockIdx.x * kMidRows;
  uint8_t* sA = smem;
  const uint32_t a_bytes = (uint32_t)(((M * Kc) + 1023) & ~1023LL);
  float* sS = reinterpret_cast<float*>(smem + a_bytes);

  // ---- activation slice and its scales -> LDS
  {
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, (uint32_t)(M * K));
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.As, (uint32_t)(M * KB * 4));
    // Piece pc = 64 i + lane of the slice is (row, j) = divmod(pc, pr); a
    // lane's pieces advance by 64 kMidNW per step, so (row, j) is stepped by
    // the constant quotient and remainder of that stride with one carry
    // instead of a division per piece (likewise for the scales).
    const int pieces = (int)M * pr;
    {
      constexpr int kStride = 64 * kMidNW;
      const int dq = kStride / pr, dr = kStride - dq * pr;
      int pc = w * 64 + lane;
      int row = pc / pr, j = pc - row * pr;
      for (int i = w; i * 64 < pieces; i += kMidNW) {
        // slot (row, j) holds piece j ^ key(row); lanes past the slice read
        // zeros (offset beyond the resource) into the padding
        const uint32_t src = pc < pieces ? (uint32_t)(row * K + k0 + 16 * (j ^ (row & 15))) : 0xFFFFFFF0u;
        b2l16(rA, src, 0, sA + i * 1024);
        pc += kStride;
        row += dq;
        j += dr;
        if (j >= pr) {
          j -= pr;
          ++row;
        }
      }
    }
    const int nsc = (int)M * kbc;
    if constexpr (KS == 32) {
      // 32-wide blocks: a row's kbc scales are 16-byte aligned (KB and kb0
      // multiples of 4), copied as 16-byte pieces: a quarter of the copy
      // instructions of 4-byte pieces (N = 4096, K = 7168, M = 17 / 64:
      // 11.29 / 14.62 -> 11.19 / 14.32 us; the buffer->LDS copies are partly
      // bound by their instruction count)
      const int spr = kbc / 4, nsp = (int)M * spr;
      constexpr int kStride = 64 * kMidNW;
      const int dq = kStride / spr, dr = kStride - dq * spr;
      int f = w * 64 + lane;
      int row = f / spr, c = f - row * spr;
      for (int i = w; i * 64 < nsp; i += kMidNW) {
        const uint32_t src = f < nsp ? (uint32_t)((row * KB + kb0 + 4 * c) * 4) : 0xFFFFFFF0u;
        b2l16(rS, src, 0, sS + i * 256);
        f += kStride;
        row += dq;
        c += dr;
        if (c >= spr) {
          c -= spr;
          ++row;
        }
      }
    } else {
      constexpr int kStride = 64 * kMidNW;
      const int dq = kStride / kbc, dr = kStride - dq * kbc;
      int f = w * 64 + lane;
      int row = f / kbc, c = f - row * kbc;
      for (int i = w; i * 64 < nsc; i += kMidNW) {
        const uint32_t src = f < nsc ? (uint32_t)((row * KB + kb0 + c) * 4) : 0xFFFFFFF0u;
        b2l4(rS, src, 0, sS + i * 64);
        f += kStride;
        row += dq;
        c += dr;
        if (c >= kbc) {
          c -= kbc;
          ++row;
        }
      }
    }
  }
  // ---- this wave's weight chunks (row block rb, chunks h, h + NP, ...); lane
  // group g holds bytes [16g, 16g+16) and [64+16g, 64+16g+16) of each chunk
  // (the 16x16x128 MFMA's K order; regrouped per 32-wide block for the
  // 16x16x32 MFMAs)
  const int64_t nrow = n0 + 16 * rb + r16 < N ? n0 + 16 * rb + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + k0 + 16 * g;
  int64_t nb = (n0 + 16 * rb) / p.bn;
  if (nb > p.nbw - 1) nb = p.nbw - 1;
  // this row block's weight scales of the slice, one per lane (wave-uniform
  // per block): lane i holds block kb0 + (chunk h + (i / KSUB) * NP) * KSUB + i % KSUB
  const int li = lane < R * KSUB ? lane : R * KSUB - 1;
  const int lc = h + (li / KSUB) * NP;
  const float wsl = p.Ws[nb * KB + kb0 + (lc < ncc ? lc : ncc - 1) * KSUB + li % KSUB];
  asm volatile("" ::: "memory");
  // The first DA chunks are issued here, each later one while the chunk DA
  // before it is computed: issued all up front, the loads stalled the wave at
  // issue until most of their bytes had arrived, so the MFMA work only began
  // after the weight stream (N = 4096, K = 7168, 32-wide blocks, M = 17 / 24
  // / 48 / 64: 12.85 / 13.02 / 14.55 / 16.11 us all up front, 11.75 / 12.06 /
  // 13.61 / 14.68 us one ahead, 11.90 / 12.28 / 13.03 / 14.20 us two ahead).
  // 128-wide blocks have a quarter of the MFMA work: up to 32 rows all up
  // front is faster there (M = 32: 12.00 against 12.20 us one ahead), at 64
  // rows two ahead (13.83 -> 13.35 us).
  constexpr int DA0 = MT > 2 ? 2 : (KS == 32 ? 1 : R);
  constexpr int DA = DA0 < R ? DA0 : R;
  i32x8 wf[R];
  auto issue_w = [&](int u) {
    const int cc0 = h + u * NP;
    const int cc = cc0 < ncc ? cc0 : ncc - 1;
    wf[u] = gload_halves(wp + (int64_t)cc * 128);
  };
#pragma unroll
  for (int u = 0; u < DA; ++u) issue_w(u);
  // the copies were issued first and loads complete in order: once at most
  // 2 DA (weight halves) + 1 (scales) remain, this wave's copies have landed;
  // the barrier without a fence keeps the weight loads in flight across it
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * DA + 1) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // LDS byte offsets of this lane's fragment pieces and scales for its
  // first chunk (h), per 16-row block t. 128-wide blocks: the two 16-byte
  // pieces x = 8h + 4f + g of the 16x16x128 fragment. 32-wide blocks: the
  // four 8-byte halves (g >> 1) of pieces x = 8h + 2s + (g & 1), block s's
  // bytes of lane group g in the regrouped weight fragment. Chunk h + NP u
  // (NP = 2) adds 256 u bytes to every offset: piece (8 cc + x) ^ key with
  // x < 16 and key < 16 is 16 u + (x ^ key). Rows past M repeat the last
  // row (never stored).
  static_assert(NP == 2, "piece offsets assume two chunk parities");
  constexpr int NA = KS == 32 ? 4 : 2;
  uint32_t aoff[MT][NA], soff[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + r16 < M ? 16 * t + r16 : (int)M - 1;
    const int key = m & 15;
#pragma unroll
    for (int f = 0; f < NA; ++f)
      aoff[t][f] = KS == 32 ? (uint32_t)(m * Kc + 16 * ((8 * h + 2 * f + (g & 1)) ^ key) + 8 * (g >> 1))
                            : (uint32_t)(m * Kc + 16 * ((8 * h + 4 * f + g) ^ key));
    soff[t] = (uint32_t)((m * kbc + h * KSUB) * 4);
  }
  const uint8_t* sSb = reinterpret_cast<const uint8_t*>(sS);
  // fragments of (u, t) read one step ahead of their MFMAs
  i32x8 afb[2];
  f32x4 sab[2];
  auto load = [&](int u, int t, int b) {
    if constexpr (KS == 32) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int2 v = *reinterpret_cast<const int2*>(sA + aoff[t][q] + 256 * u);
        afb[b][2 * q] = v.x;
        afb[b][2 * q + 1] = v.y;
      }
    } else {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(sA + aoff[t][0] + 256 * u);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(sA + aoff[t][1] + 256 * u);
      afb[b] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    if constexpr (KSUB == 4) sab[b] = *reinterpret_cast<const f32x4*>(sSb + soff[t] + 32 * u);
    else sab[b][0] = *reinterpret_cast<const float*>(sSb + soff[t] + 8 * u);
  };
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (h < ncc) load(0, 0, 0);
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int cc = h + u * NP;
    if (cc >= ncc) break;
    if (u + DA < R) issue_w(u + DA);
    if constexpr (KS == 32) regroup_blocks(wf[u]);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const int b = (u * MT + t) & 1;
      if (t + 1 < MT) load(u, t + 1, b ^ 1);
      else if (u + 1 < R && cc + NP < ncc) load(u + 1, 0, b ^ 1);
#pragma unroll
      for (int s = 0; s < KSUB; ++s) {
        const float ws = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wsl), u * KSUB + s));
        const f32x4 pr = KS == 32 ? mfma_fp8_k32(dword_pair(wf[u], s), dword_pair(afb[b], s))
                                  : mfma_fp8_k128(wf[u], afb[b]);
        acc[t] = fma4s(pr, sab[b][s] * ws, acc[t]);
      }
    }
  }
  // the NP waves of a row block -> one partial, summed in parity order
  __syncthreads();  // every wave is done with the activation slice
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [kMidNW][MT][64]
#pragma unroll
  for (int t = 0; t < MT; ++t) red[(w * MT + t) * 64 + lane] = acc[t];
  __syncthreads();
  if (h == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4 v = red[(rb * MT + t) * 64 + lane];
#pragma unroll
      for (int hh = 1; hh < NP; ++hh) v += red[((rb + 4 * hh) * MT + t) * 64 + lane];
      const int64_t m = 16 * t + r16;
      const int64_t n = n0 + 16 * rb + 4 * g;
      if (m < M && n < N) *reinterpret_cast<f32x4*>(part + ((int64_t)s_idx * M + m) * N + n) = v;
    }
  }
}

// D[m, n .. n+3] = sum_s part[s][m][n .. n+3] (s ascending) + bias, rounded.
__global__ __launch_bounds__(256) void gemm_split_reduce(TileParams p, const float* __restrict__ part,
                                                         int S) {
  const int64_t N = p.N, M = p.M;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nv = N / 4;
  if (v >= M * nv) return;
  const int64_t m = v / nv, n = (v - m * nv) * 4;
  f32x4 sum = *reinterpret_cast<const f32x4*>(part + m * N + n);
  for (int s = 1; s < S; ++s) sum += *reinterpret_cast<const f32x4*>(part + ((int64_t)s * M + m) * N + n);
  const bool bf16 = p.out_bf16 != 0;
  const bool vec = p.d_vec4 != 0;
  store4(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec) : sum, bf16, vec);
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

template <int KS, int MT>
hipError_t launch_stream_mt(const TileParams& tp, hipStream_t st) {
  constexpr int NW = 16;
  constexpr int R = MT == 1 ? 4 : 2;
  const int64_t gy = (tp.M + MT * 16 - 1) / (MT * 16);
  if (gy > 65535 || (tp.N + 15) / 16 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const dim3 grid((unsigned)((tp.N + 15) / 16), (unsigned)gy);
  hipLaunchKernelGGL((gemm_stream<KS, MT, NW, R>), grid, dim3(NW * 64), 0, st, tp);
  return hipGetLastError();
}

constexpr int64_t kLdsBytes = 160 * 1024;
// gemm_stream_sa: eight waves, each with all of its chunks' loads in flight
// (against sixteen waves of up to four chunks, one process, launches
// interleaved, 32-wide blocks, N = 4096, K = 7168: M = 5 / 8 / 12 / 16
// 9.09 / 9.15 / 9.75 / 10.26 -> 8.21 / 8.52 / 8.93 / 9.40 us)
constexpr int kStreamSaNW = 8;
constexpr int kStreamSaMaxR = 8;

// dynamic LDS of gemm_stream_sa
inline int64_t stream_sa_lds(int64_t M, int64_t K, int KB) {
  return M * (K + 16) + ((M * KB * 4 + 1023) & ~1023LL) + (int64_t)kStreamSaNW * 64 * 16;
}

// M <= 16, K a multiple of 1024, at most kStreamSaMaxR chunks of 128 per wave,
// and the staged activations fit in LDS
inline bool stream_sa_fits(int64_t M, int64_t K, int KB) {
  return M <= 16 && K % 1024 == 0 && (K / 128 + kStreamSaNW - 1) / kStreamSaNW <= kStreamSaMaxR &&
         stream_sa_lds(M, K, KB) <= kLdsBytes;
}

// Raises a kernel's dynamic-LDS limit to the whole 160 KB on the current
// device, once per (kernel, device): `done` holds one bit per device. Threads
// racing on a first call may both make the (idempotent) attribute call; the
// bit is set only after it succeeded. Devices past the 64th set it every call.
hipError_t raise_lds_limit(const void* kern, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? 1ull << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kLdsBytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

template <int KS, int R>
hipError_t launch_stream_sa_r(const TileParams& tp, hipStream_t st) {
  // from 8 rows on (16 with 128-wide blocks, a quarter of the MFMA work),
  // one chunk issued ahead of the MFMAs instead of all up front (N = 4096,
  // K = 7168, 32-wide blocks: M = 8 / 16 8.28 / 9.25 -> 8.02 / 8.68 us;
  // 128-wide blocks M = 16 8.67 -> 8.48 us); with fewer rows the MFMA work is
  // too short to hide and all up front is faster (128-wide M = 1 / 4 / 8:
  // 7.33 / 7.47 / 7.77 us against 7.75 / 7.82 / 7.92 us)
  const bool ahead = tp.M >= (KS == 32 ? 8 : 16);
  const auto kern = ahead ? gemm_stream_sa<KS, kStreamSaNW, R, 1> : gemm_stream_sa<KS, kStreamSaNW, R, R>;
  static std::atomic<uint64_t> lds_raised[2]{};
  const hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), lds_raised[ahead]);
  if (e != hipSuccess) return e;
  if ((tp.N + 15) / 16 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  const unsigned lds = (unsigned)stream_sa_lds(tp.M, tp.K, tp.KB);
  hipLaunchKernelGGL(kern, dim3((unsigned)((tp.N + 15) / 16)), dim3(kStreamSaNW * 64), lds, st, tp);
  return hipGetLastError();
}

// R: the fewest of 2, 4, 7 or 8 chunks per wave that covers K
template <int KS>
hipError_t launch_stream_sa(const TileParams& tp, hipStream_t st) {
  const int64_t per = (tp.K / 128 + kStreamSaNW - 1) / kStreamSaNW;
  if (per <= 2) return launch_stream_sa_r<KS, 2>(tp, st);
  if (per <= 4) return launch_stream_sa_r<KS, 4>(tp, st);
  if (per <= 7) return launch_stream_sa_r<KS, 7>(tp, st);
  return launch_stream_sa_r<KS, 8>(tp, st);
}

template <int MT4>
hipError_t launch_stream_pk_mt(const TileParams& tp, hipStream_t st) {
  // eight waves of seven chunks each (K = 7168: every load of the workgroup
  // in flight at once; measured M = 1 8.3 -> 8.0 us and M = 4 9.0 -> 8.3 us
  // against sixteen waves of four)
  constexpr int NW = 8, R = 7;
  if ((tp.N + 15) / 16 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((gemm_stream_pk<MT4, NW, R>), dim3((unsigned)((tp.N + 15) / 16)), dim3(NW * 64), 0, st, tp);
  return hipGetLastError();
}

// 32-wide K blocks, M <= 8: MFMAs packing four activation rows each
hipError_t launch_stream_pk(const TileParams& tp, hipStream_t st) {
  return tp.M <= 4 ? launch_stream_pk_mt<1>(tp, st) : launch_stream_pk_mt<2>(tp, st);
}

template <int KS>
hipError_t launch_stream(const TileParams& tp, hipStream_t st) {
  const int64_t mt = (tp.M + 15) / 16;
  switch (mt) {
    case 1: return launch_stream_mt<KS, 1>(tp, st);
    case 2: return launch_stream_mt<KS, 2>(tp, st);
    case 3: return launch_stream_mt<KS, 3>(tp, st);
    default: return launch_stream_mt<KS, 4>(tp, st);
  }
}

// ---- split-K decode for 17..64 rows ----------------------------------------------
struct MidPlan {
  int S = 0;      // K ranges (grid.y)
  int Kc = 0;     // bytes of K per range
  int mt = 0;     // 16-row activation blocks
  int R = 0;      // chunks per wave (loads issued up front)
  int64_t lds = 0;
};

// K ranges: the fewest that give 256 workgroups, each range a multiple of 256
// bytes and at most 2048 (so a wave's chunks fit its registers); none fits ->
// not this kernel.
inline bool mid_plan(int64_t M, int64_t N, int64_t K, int bk, MidPlan& pl) {
  if (M < 17 || M > kSkinnyMaxM || N % 4 != 0) return false;
  const int64_t groups = (N + kMidRows - 1) / kMidRows;
  int best = 0;
  for (int S = 1; S <= 32; S *= 2) {
    if (K % (256LL * S) != 0) continue;
    if (K / S > 2048) continue;
    best = S;
    if (groups * S >= 256) break;
  }
  if (!best || groups * best > 0x7FFFFFFFLL) return false;
  pl.S = best;
  pl.Kc = (int)(K / best);
  const int ncc = pl.Kc / 128;
  const int need = (ncc + kMidNW / 4 - 1) / (kMidNW / 4);
  // chunks per wave rounded up to 4, 7 or 8 (a clamped duplicate load for
  // each chunk short: M = 24 / 48 / 64 at K = 7168, 7 chunks, 13.98 / 16.19 /
  // 18.60 us with R = 8, 13.45 / 15.77 / 17.84 us with R = 7)
  pl.R = need <= 4 ? 4 : (need <= 7 ? 7 : 8);
  pl.mt = (int)((M + 15) / 16);
  const int64_t kbc = pl.Kc / bk;
  const int64_t a_bytes = ((M * pl.Kc) + 1023) & ~1023LL;
  // scale copies: whole 256-byte (4-byte pieces) or 1 KB (16-byte pieces) loads
  const int64_t s_bytes = bk == 32 ? ((M * kbc * 4 + 1023) / 1024) * 1024 : ((M * kbc + 63) / 64) * 64 * 4;
  const int64_t red_bytes = (int64_t)kMidNW * pl.mt * 64 * 16;
  pl.lds = a_bytes + s_bytes > red_bytes ? a_bytes + s_bytes : red_bytes;
  return pl.lds <= kLdsBytes;
}

template <int KS, int MT, int R>
hipError_t launch_mid_inst(const TileParams& tp, const MidPlan& pl, float* part, hipStream_t st) {
  const auto kern = gemm_split_mid<KS, MT, R>;
  static std::atomic<uint64_t> lds_raised{0};
  hipError_t e = raise_lds_limit(reinterpret_cast<const void*>(kern), lds_raised);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((tp.N + kMidRows - 1) / kMidRows), (unsigned)pl.S);
  hipLaunchKernelGGL(kern, grid, dim3(kMidNW * 64), (unsigned)pl.lds, st, tp, part, pl.Kc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t vecs = tp.M * (tp.N / 4);
  hipLaunchKernelGGL(gemm_split_reduce, dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, st, tp,
                     (const float*)part, pl.S);
  return hipGetLastError();
}

template <int KS, int MT>
hipError_t launch_mid_r(const TileParams& tp, const MidPlan& pl, float* part, hipStream_t st) {
  return pl.R == 4 ? launch_mid_inst<KS, MT, 4>(tp, pl, part, st)
         : pl.R == 7 ? launch_mid_inst<KS, MT, 7>(tp, pl, part, st)
                     : launch_mid_inst<KS, MT, 8>(tp, pl, part, st);
}

template <int KS>
hipError_t launch_mid_ks(const TileParams& tp, const MidPlan& pl, float* part, hipStream_t st) {
  switch (pl.mt) {
    case 2: return launch_mid_r<KS, 2>(tp, pl, part, st);
    case 3: return launch_mid_r<KS, 3>(tp, pl, part, st);
    default: return launch_mid_r<KS, 4>(tp, pl, part, st);
  }
}

hipError_t launch_mid(const TileParams& tp, const MidPlan& pl, int bk, float* part, hipStream_t st) {
  return bk == 32 ? launch_mid_ks<32>(tp, pl, part, st) : launch_mid_ks<128>(tp, pl, part, st);
}

constexpr int kBM = 256, kBN = 256, kWM = 2, kWN = 4;

// grid: workgroups (tiles, or for SPLIT the whole-round tiles plus an owner
// and a helper per split tile)
template <int KS, bool GROUPED, bool SPLIT = false>
hipError_t launch_tile(const TileParams& tp, int64_t grid_n, hipStream_t st) {
  static_assert(!(GROUPED && SPLIT), "the grouped kernel is not split");
  if (grid_n <= 0) return hipSuccess;
  if (grid_n > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  constexpr int TN = kBN / kWN;
  // every 16-column block of a wave shares one weight-scale block when the
  // wave's column range never crosses a bn boundary
  const bool wsu = tp.bn % TN == 0;
  const dim3 grid((unsigned)grid_n), block(kWM * kWN * 64);
  if (!GROUPED && tp.bias) {
    constexpr bool B = !GROUPED;
    if (wsu)
      hipLaunchKernelGGL((gemm_tile<kBM, kBN, kWM, kWN, KS, GROUPED, true, B, SPLIT>), grid, block, 0, st, tp);
    else
      hipLaunchKernelGGL((gemm_tile<kBM, kBN, kWM, kWN, KS, GROUPED, false, B, SPLIT>), grid, block, 0, st, tp);
  } else if (wsu) {
    hipLaunchKernelGGL((gemm_tile<kBM, kBN, kWM, kWN, KS, GROUPED, true, false, SPLIT>), grid, block, 0, st, tp);
  } else {
    hipLaunchKernelGGL((gemm_tile<kBM, kBN, kWM, kWN, KS, GROUPED, false, false, SPLIT>), grid, block, 0, st, tp);
  }
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
  tp.d_vec4 = a.N % 4 == 0 && (uintptr_t)a.D % 8 == 0 && (uintptr_t)a.bias % 8 == 0;
  // A / As extents: the dense call knows M; the grouped call addresses A rows
  // through a_map, so the extent is only bounded by the 4 GiB limit
  const bool dense = a.expert_offsets == nullptr;
  tp.a_bytes = dense ? (uint32_t)(a.M * a.K) : 0xFFFFFFFFu;
  tp.as_bytes = dense ? (uint32_t)(a.M * (a.K / a.bk) * 4) : 0xFFFFFFFFu;
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

// Compute units of the current device (0 when there is none), cached per
// device.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) {
      (void)hipGetLastError();
      return 0;
    }
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

// Split of the last round. With one 256x256 workgroup per compute unit, an
// unsplit launch of T tiles on C units ends with a round of R = T mod C
// tiles while C - R units idle (4096 x 18432: 1152 tiles, 128 in the fifth
// round on 256 units). When R <= C / 2 each of those tiles is split in K:
// its owner takes slabs [0, k), a helper [k, K/128) on one of the idle
// units. Measured on 4096 x 18432 x 7168: 573 -> 548 us. A fuller last round
// gains nothing: the chip already runs at its power limit there, and filling
// the idle units lowers the clock of all (4096 x 7168 x 7168, 192 of 256: 208
// us unsplit, 219-231 us split with helpers taking up to three tiles each).
bool split_plan(int64_t tiles, int KT, int cus, SplitPlan& sp) {
  if (cus <= 0 || KT < 8 || tiles <= 0) return false;
  const int64_t R = tiles % cus;
  if (R == 0 || 2 * R > cus) return false;
  sp.first = tiles - R;
  sp.lead = R;
  sp.tiles = R;
  sp.k = KT / 2 + 1;
  return true;
}
namespace {
std::atomic<uint32_t> g_split_wait_ticks{20000};  // 200 us
}  // namespace

size_t split_part_bytes(int64_t R) { return (size_t)R * 256 * 256 * sizeof(float); }
size_t split_bytes(int64_t R) { return (split_part_bytes(R) + (size_t)R * 4 + 255) / 256 * 256; }

void set_split_wait_ticks(uint32_t ticks) { g_split_wait_ticks.store(ticks, std::memory_order_relaxed); }

uint32_t split_wait_ticks() { return g_split_wait_ticks.load(std::memory_order_relaxed); }

uint32_t next_split_token() {
  static std::atomic<uint32_t> calls{0};
  return (calls.fetch_add(1, std::memory_order_relaxed) << 1) | 1u;
}

size_t blockwise_workspace_bytes(int64_t M, int64_t N, int64_t K, int bn, int bk) {
  (void)bn;
  if (K % 128 != 0) return 0;
  MidPlan pl;
  if (!mid_plan(M, N, K, bk, pl)) return 0;
  return (size_t)pl.S * (size_t)M * (size_t)N * sizeof(float);
}

size_t blockwise_split_bytes(int64_t M, int64_t N, int64_t K, int bn, int bk) {
  (void)bn; (void)bk;
  if (M <= kSkinnyMaxM || K % 128 != 0 || N < 1) return 0;
  SplitPlan sp;
  const int64_t tiles = ((M + kBM - 1) / kBM) * ((N + kBN - 1) / kBN);
  if (!split_plan(tiles, (int)(K / 128), device_cus(), sp)) return 0;
  return split_bytes(sp.tiles);
}

hipError_t launch_blockwise(const BlockGemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  const TileParams tp = make_params(a);
  if (a.K % 128 != 0)  // only the 8-byte-fragment kernel handles partial slabs
    return a.bk == 128 ? launch_skinny<128>(tp, st) : launch_skinny<32>(tp, st);
  // the streaming kernel reads a chunk's four 32-wide activation scales as
  // one 16-byte vector
  if (a.M <= kSkinnyMaxM) {
    // 17..64 rows: split-K over 64-row workgroups, partials in the workspace
    MidPlan pl;
    if (mid_plan(a.M, a.N, a.K, a.bk, pl) && a.workspace && (uintptr_t)a.workspace % 16 == 0 &&
        (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.As % 16 == 0)
      return launch_mid(tp, pl, a.bk, static_cast<float*>(a.workspace), st);
    // staging the activation rows once per workgroup beats every wave reading
    // them from L2 at any row count with 128-wide blocks (N = 4096, K = 7168,
    // M = 1 / 2 / 4 / 7: 8.03 / 8.69 / 8.99 / 9.74 us unstaged, 7.28 / 7.35 /
    // 7.55 / 7.76 us staged), and with 32-wide blocks (16x16x32 MFMAs) beats
    // the packed kernel below at any row count too (M = 1 / 2: 7.87 / 7.97 us
    // packed, 7.67 / 7.70 us staged)
    if (stream_sa_fits(a.M, a.K, tp.KB) && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.As % 16 == 0)
      return a.bk == 128 ? launch_stream_sa<128>(tp, st) : launch_stream_sa<32>(tp, st);
    // 32-wide blocks, up to 8 rows, where the staged kernel does not apply
    // (K not a multiple of 1024): four rows' block partials per MFMA
    if (a.bk == 32 && a.M <= 8) return launch_stream_pk(tp, st);
    return a.bk == 128 ? launch_stream<128>(tp, st) : launch_stream<32>(tp, st);
  }
  const int64_t tiles = tp.tiles_m * tp.tiles_n;
  SplitPlan sp;
  if (a.workspace && (uintptr_t)a.workspace % 16 == 0 &&
      split_plan(tiles, (int)(a.K / 128), device_cus(), sp) && a.workspace_bytes >= split_bytes(sp.tiles)) {
    TileParams ts = tp;
    ts.part = static_cast<float*>(a.workspace);
    ts.flag = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.workspace) + split_part_bytes(sp.tiles));
    ts.token = next_split_token();
    ts.split_k = sp.k;
    ts.split_first = sp.first;
    ts.split_lead = sp.lead;
    ts.split_tiles = sp.tiles;
    ts.part_bytes = (uint32_t)split_part_bytes(sp.tiles);
    ts.split_wait = split_wait_ticks();
    const int64_t grid_n = sp.first + 2 * sp.tiles;
    return a.bk == 128 ? launch_tile<128, false, true>(ts, grid_n, st) : launch_tile<32, false, true>(ts, grid_n, st);
  }
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
