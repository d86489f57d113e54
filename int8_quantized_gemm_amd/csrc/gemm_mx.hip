// Block-scaled FP8 GEMM with power-of-two (E8M0) block scales on both
// operands, applied by gfx950's MX-scaled matrix instruction.
//
// The block32 DeepGEMM PR for DeepSeek-V4.1 ("[SM90] Use native block32
// DeepGEMM for DeepSeek-V4.1"): recipe (1, bn, 32) with UE8M0 activation
// scales; the vLLM scaled_mm page (XPUFp8BlockScaledMMKernel): weight scales
// stored as float8_e8m0fnu bytes. An E8M0 byte b is the scale 2^(b - 127):
//
//   D[m,n] = sum_kb 2^(As[m,kb]-127) 2^(Ws[n/bn,kb]-127) sum_{k in kb} A[m,k] W[n,k]
//
// over 32-wide K blocks kb (+ bias[n], then RNE to bf16/f16).
//
// v_mfma_scale_f32_16x16x128_f8f6f4 takes one E8M0 byte per lane for each
// operand. In its K numbering (measured on gfx950 with single non-zero
// registers) lane group g = l / 16 holds K elements [16g, 16g + 16) in its
// first four registers and [64 + 16g, 64 + 16g + 16) in its last four, for
// row l % 16; the scale of 32-wide block kb (K elements [32kb, 32kb + 32)) of
// row r is the byte supplied by lane r + 16 kb. With the K bytes of a
// 128-byte slab laid out that way, the block scales are applied inside the
// matrix core and the K loop accumulates in the MFMA accumulators: no VALU
// work per K block, unlike the float32-scale kernel, which adds every block's
// partial product with an FMA.
//
// gemm_tile_mx   (M > 64) 256 x 256 output tiles, 128-byte K slabs
//                double-buffered in LDS through direct buffer -> LDS loads, as
//                the float32-scale tile kernel, whose fragment (16-byte chunks
//                g and g + 4 of the slab for lane group g) is already that
//                layout. Scale dwords (four blocks of one row) are loaded from
//                global memory one slab ahead.
// gemm_stream_mx (M <= 64) streams W once, one workgroup per 16 weight rows,
//                lane group g loading bytes [16g, 16g + 16) and
//                [64 + 16g, 64 + 16g + 16) of each 128-byte chunk.
// gemm_stream_mx_sa (M <= 16, K a multiple of 1024) as gemm_stream_mx, with
//                the activation rows and their scale bytes copied into LDS
//                once per workgroup instead of read from L2 by every wave
//                (measured against reading them per wave: M = 1 7.90 -> 7.62,
//                M = 4 8.94 -> 7.97, M = 16 11.7 -> 9.1 us at N=4096, K=7168).
// gemm_split_mx  (17 <= M <= 64, with a workspace) K split into ranges: a
//                workgroup owns 64 weight rows of one range, copies the range's
//                activation slice and its scale dwords into LDS once, streams
//                its weights, and writes float32 partials that
//                gemm_split_reduce_mx sums over the ranges in a fixed order.
#include <atomic>

#include "q8_internal.h"
#include "tile_common.h"

namespace q8 {
namespace {

struct MxParams {
  const uint8_t* A;
  const uint8_t* As;
  const uint8_t* W;
  const uint8_t* Ws;
  const void* bias;
  void* D;
  int64_t M, N, K;
  int KB;   // K / 32: bytes per scale row
  int bn;
  int nbw;  // ceil(N / bn)
  int out_bf16;
  int d_vec4;
  uint32_t a_bytes, as_bytes;
  int64_t tiles_m, tiles_n;
  // last round split in K (gemm_tile_mx with SPLIT): the first split_first
  // workgroups take whole tiles, then split_lead helpers, the owners of the
  // split_tiles tiles of the last round, and the remaining helpers; owners
  // take K slabs [0, split_k), helpers the rest, their float32 partials going
  // to part (fragment order, 256 * 256 floats per tile) and published by
  // writing token into the tile's flag word
  float* part;
  uint32_t* flag;
  uint32_t token;
  int split_k;
  int64_t split_first, split_lead, split_tiles;
  uint32_t part_bytes;
  uint32_t split_wait;  // longest wait of an owner, in 100 MHz ticks (0: none)
};

__device__ __forceinline__ f32x4 mfma_mx(const i32x8& w, const i32x8& a, const f32x4& c,
                                         uint32_t sw, uint32_t sa) {
  // operand 0 = weight rows, operand 1 = activation rows, both FP8 e4m3
  // (format codes 0); byte 0 of each scale register is used
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, c, 0, 0, 0, (int)sw, 0, (int)sa);
}

__device__ __forceinline__ i32x8 lds_frag_mx(const uint8_t* base, int row, int g) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(base + swz(row, g));
  const i32x4 hi = *reinterpret_cast<const i32x4*>(base + swz(row, g + 4));
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Fragment of lane group g from global memory: p points at byte 16g of a
// 128-byte chunk; bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16).
__device__ __forceinline__ i32x8 gload_mx(const uint8_t* p) {
  const i32x4 lo = *reinterpret_cast<const i32x4*>(p);
  const i32x4 hi = *reinterpret_cast<const i32x4*>(p + 64);
  return i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

__device__ __forceinline__ uint32_t out_bits(float v, bool bf16) {
  return bf16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
}

// D[row, n .. n+3] as 16-bit values (any bias already added)
__device__ __forceinline__ void store4_mx(const MxParams& p, int64_t row, int64_t n, f32x4 v,
                                          bool bf16, bool vec) {
  uint16_t* D = static_cast<uint16_t*>(p.D);
  const int64_t N = p.N;
  if (vec && n + 3 < N) {
    uint2 o;
    o.x = out_bits(v[0], bf16) | (out_bits(v[1], bf16) << 16);
    o.y = out_bits(v[2], bf16) | (out_bits(v[3], bf16) << 16);
    *reinterpret_cast<uint2*>(D + row * N + n) = o;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (n + r >= N) break;
      D[row * N + n + r] = (uint16_t)out_bits(v[r], bf16);
    }
  }
}

// ------------------------------------------------------------------------------
// SPLIT: the launch splits the tiles of its last round in K (see MxParams);
// an owner that stops waiting for its helper runs on through the rest of K,
// so that tile comes out exactly as unsplit.
template <int BM, int BN, int WM, int WN, bool SPLIT>
__global__ __launch_bounds__(WM * WN * 64) void gemm_tile_mx(MxParams p) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int A_SLOTS = BM / 8, B_SLOTS = BN / 8;  // 1 KB (8 rows) per wave load
  constexpr int A_PER = (A_SLOTS + NW - 1) / NW, B_PER = (B_SLOTS + NW - 1) / NW;
  static_assert(TM % 16 == 0 && TN % 16 == 0 && NW % 2 == 0, "tile");

  __shared__ __attribute__((aligned(1024))) uint8_t sA0[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sA1[BM * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB0[BN * 128];
  __shared__ __attribute__((aligned(1024))) uint8_t sB1[BN * 128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = w / WN, wn = w % WN;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int KB = p.KB;

  const int KT = (int)(K / 128);
  int64_t b = blockIdx.x;
  int role = 0, ka = 0, kb = KT;  // role 0: whole K, 1: owner, 2: helper
  int64_t slot = 0;
  if constexpr (SPLIT) {
    // split tile j takes the tile that workgroup split_first + j would take
    // unsplit (same XCD when the counts are multiples of 8)
    const int64_t c = b - p.split_first;
    if (c >= 0) {
      if (c < p.split_lead) { role = 2; slot = c; }
      else if (c < p.split_lead + p.split_tiles) { role = 1; slot = c - p.split_lead; }
      else { role = 2; slot = c - p.split_tiles; }
      b = p.split_first + slot;
      if (role == 1) kb = p.split_k;
      else ka = p.split_k;
    }
  }
  const int64_t t = xcd_remap(b, p.tiles_m * p.tiles_n);
  int64_t tm, tn;
  grouped_order(t, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int64_t m_lo = tm * BM, n0 = tn * BN;

  // Wave load q fills rows 8q..8q+7 of a stage; lane l writes physical chunk
  // l % 8 of row 8q + l / 8, which holds chunk c = (l % 8) ^ key of the row's
  // slab, key = swz_key(row) = (4q + l / 16) % 8 (the wave's parity fixes q's).
  const int key = (4 * (w & 1) + (lane >> 4)) & 7;
  const uint32_t lane_off = (uint32_t)((lane >> 3) * K + (((lane & 7) ^ key) << 4));
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, p.a_bytes);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(p.W, (uint32_t)(N * K));
  const uint32_t a_base = (uint32_t)(m_lo * K), b_base = (uint32_t)(n0 * K);
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

  // Scale dwords (the four 32-wide blocks of a slab for one row) are staged
  // in LDS with the slab, one 4-byte buffer -> LDS load per wave: waves
  // 0..NW/2-1 fetch activation rows, the others weight rows. Table layouts
  // follow the lanes that read them: activation position (wm*16 + r16)*FM + i
  // holds row wm*TM + i*16 + r16, weight position (wn*16 + r16)*FN + j holds
  // row wn*TN + j*16 + r16, so a lane reads its FM (FN) dwords contiguously.
  // Rows past the end of As / Ws read as zero (their outputs are never stored).
  static_assert(WM * 16 * FM == BM && WN * 16 * FN == BN && BM == BN && BM == NW / 2 * 64,
                "one scale load per wave covers the tile's rows");
  __shared__ __attribute__((aligned(16))) uint32_t sSA[2][BM];
  __shared__ __attribute__((aligned(16))) uint32_t sSW[2][BN];
  const __amdgpu_buffer_rsrc_t rAs = make_rsrc(p.As, p.as_bytes);
  const __amdgpu_buffer_rsrc_t rWs = make_rsrc(p.Ws, (uint32_t)(p.nbw * KB));
  const bool a_side = w < NW / 2;
  const int pos0 = (a_side ? w : w - NW / 2) * 64;
  uint32_t vo_s;
  if (a_side) {
    const int pos = pos0 + lane;
    const int wm_ = pos / (16 * FM), r_ = (pos / FM) % 16, i_ = pos % FM;
    vo_s = (uint32_t)((m_lo + wm_ * TM + i_ * 16 + r_) * KB);
  } else {
    const int pos = pos0 + lane;
    const int wn_ = pos / (16 * FN), r_ = (pos / FN) % 16, j_ = pos % FN;
    const int64_t n = n0 + wn_ * TN + j_ * 16 + r_;
    vo_s = (uint32_t)((n < N ? n / p.bn : (int64_t)p.nbw) * KB);
  }
  auto issue_scales = [&](int kt, int stage) {
    if (a_side) b2l4(rAs, vo_s, 4 * kt, &sSA[stage][pos0]);
    else b2l4(rWs, vo_s, 4 * kt, &sSW[stage][pos0]);
  };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Slab kt lives in stage st (0 or 1, alternating from the first slab run).
  // The refill of the other stage with slab kt + 1 is split: activation rows
  // and scales at the top of the slab, weight rows after its first half of
  // MFMAs (4096 x 18432 x 7168 514.8 -> 486.1 us, 4096 x 7168 x 7168 and
  // 2048 x 7168 x 7168 unchanged; after 8 or 12 MFMAs the same or slower).
  auto step = [&](int kt, int st, bool refill, uint8_t* __restrict__ na, uint8_t* __restrict__ nb,
                  const uint8_t* __restrict__ la, const uint8_t* __restrict__ lb) {
    if (refill) {
      issue_a(kt + 1, na);
      issue_scales(kt + 1, st ^ 1);
    }
    // this slab's scale bytes for lane group g (block 4 kt + g), shifted to byte 0
    uint32_t sa[FM], sw[FN];
#pragma unroll
    for (int i4 = 0; i4 < FM / 4; ++i4) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(&sSA[st][(wm * 16 + r16) * FM + 4 * i4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sa[4 * i4 + e] = (uint32_t)v[e] >> (8 * g);
    }
#pragma unroll
    for (int j4 = 0; j4 < FN / 4; ++j4) {
      const i32x4 v = *reinterpret_cast<const i32x4*>(&sSW[st][(wn * 16 + r16) * FN + 4 * j4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) sw[4 * j4 + e] = (uint32_t)v[e] >> (8 * g);
    }
    i32x8 bw[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) bw[j] = lds_frag_mx(lb, wn * TN + j * 16 + r16, g);
    i32x8 av[2];
    av[0] = lds_frag_mx(la, wm * TM + r16, g);
    // the wave ahead yields to the one behind halfway through the slab (see
    // the float32-scale tile kernel)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if (i == FM / 2) __builtin_amdgcn_s_setprio(0);
      if (i == FM / 2 && refill) issue_w(kt + 1, nb);
      if (i + 1 < FM) av[(i + 1) & 1] = lds_frag_mx(la, wm * TM + (i + 1) * 16 + r16, g);
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = mfma_mx(bw[j], av[i & 1], acc[i][j], sw[j], sa[i]);
    }
  };

  // K slabs [k0, k1) into the accumulators
  auto run = [&](int k0, int k1) {
    issue(k0, sA0, sB0);
    issue_scales(k0, 0);
    for (int kt = k0; kt < k1; ++kt) {
      wait_vmem();
      __syncthreads();
      const int odd = (kt - k0) & 1;
      step(kt, odd, kt + 1 < k1, odd ? sA0 : sA1, odd ? sB0 : sB1, odd ? sA1 : sA0, odd ? sB1 : sB0);
    }
  };
  if constexpr (!SPLIT) {
    run(0, KT);
  } else {
    // The partial of a split tile lives in part in fragment order (wave, row
    // block, column block, lane: 1 KB per store instruction), written and
    // read coherently at agent scope (sc1).
    __shared__ uint32_t sReady;
    uint32_t* const flag = p.flag + slot;
    uint32_t v0 = 0;
    if (role == 1 && w == 0)
      v0 = (uint32_t)__builtin_amdgcn_readfirstlane(
          (int)__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    // An owner whose helper is not done in time runs on through the rest of
    // K (a second pass of the same loop): the same MFMA chain as the unsplit
    // kernel, so the tile comes out exactly as unsplit.
    bool ready = false;
    int k0 = ka, k1 = kb;
    for (;;) {
      run(k0, k1);
      if (role != 1 || k1 == KT) break;
      if (w == 0) {
        const bool ok = split_owner_wait(flag, p.token, v0, p.split_wait);
        if (lane == 0) sReady = ok ? 1u : 0u;
      }
      __syncthreads();
      ready = sReady != 0;
      if (ready) break;
      k0 = kb;
      k1 = KT;
    }
    const __amdgpu_buffer_rsrc_t rP = make_rsrc(p.part, p.part_bytes);
    const uint32_t p_off = (uint32_t)slot * (uint32_t)(BM * BN * 4) + (uint32_t)(w * FM * FN * 1024 + lane * 16);
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
        // one row block's partials at a time (all of them in flight at once
        // would need 128 more registers)
#pragma unroll
        for (int i = 0; i < FM; ++i) {
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] += __builtin_amdgcn_raw_buffer_load_b128(rP, p_off, (uint32_t)((i * FN + j) * 1024), kSc1);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // the word goes back to zero for the next call (a graph replay passes
      // the same token again)
      if (tid == 0) __hip_atomic_store(flag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  const bool bf16 = p.out_bf16 != 0, vec = p.d_vec4 != 0;
  // this lane's bias columns, loaded once (the output stores could alias the
  // bias, so the compiler would otherwise reload it before every store)
  f32x4 bias4[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
    bias4[j] = p.bias && n < N ? load_bias4(p.bias, n, N, bf16, vec && n + 3 < N) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t row = m_lo + wm * TM + i * 16 + r16;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = n0 + wn * TN + j * 16 + 4 * g;
      if (n >= N) continue;
      store4_mx(p, row, n, p.bias ? acc[i][j] + bias4[j] : acc[i][j], bf16, vec);
    }
  }
}

// ------------------------------------------------------------------------------
// One workgroup per 16 weight rows (x a 16*MT-row activation block); its NW
// waves split the 128-byte K chunks, issue a round of R chunks' loads, then
// one scaled MFMA per chunk and activation block; float32 partials of the
// waves are summed through LDS in a fixed order (deterministic).
template <int MT, int NW, int R>
__global__ __launch_bounds__(NW * 64) void gemm_stream_mx(MxParams p) {
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
  const uint8_t* wp = p.W + nrow * K + 16 * g;
  const uint32_t* wsr = reinterpret_cast<const uint32_t*>(p.Ws + (nrow / p.bn) * KB);
  const uint8_t* ap[MT];
  const uint32_t* asr[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) {
    const int64_t m = m_base + mb * 16 + r16 < M ? m_base + mb * 16 + r16 : M - 1;
    ap[mb] = p.A + m * K + 16 * g;
    asr[mb] = reinterpret_cast<const uint32_t*>(p.As + m * KB);
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mb = 0; mb < MT; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int c0 = c_b; c0 < c_e; c0 += R) {
    i32x8 wf[R], af[R][MT];
    uint32_t sw[R], sa[R][MT];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int c = c0 + u < c_e ? c0 + u : c_e - 1;
      wf[u] = gload_mx(wp + (int64_t)c * 128);
      sw[u] = wsr[c];
#pragma unroll
      for (int mb = 0; mb < MT; ++mb) {
        af[u][mb] = gload_mx(ap[mb] + (int64_t)c * 128);
        sa[u][mb] = asr[mb][c];
      }
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      if (c0 + u >= c_e) break;
#pragma unroll
      for (int mb = 0; mb < MT; ++mb)
        acc[mb] = mfma_mx(wf[u], af[u][mb], acc[mb], sw[u] >> (8 * g), sa[u][mb] >> (8 * g));
    }
  }

#pragma unroll
  for (int mb = 0; mb < MT; ++mb) red[w][mb][lane] = acc[mb];
  __syncthreads();
  const bool bf16 = p.out_bf16 != 0, vec = p.d_vec4 != 0;
  for (int idx = tid; idx < MT * 64; idx += NW * 64) {
    const int mb = idx >> 6, l2 = idx & 63;
    const int64_t m = m_base + mb * 16 + (l2 & 15);
    if (m >= M) continue;
    f32x4 sum = red[0][mb][l2];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww][mb][l2];
    const int64_t n = n0 + 4 * (l2 >> 4);
    if (n < N) store4_mx(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec && n + 3 < N) : sum, bf16, vec);
  }
}

// ---- up to 16 rows: activations staged in LDS once per workgroup ---------------
// eight waves, each with all of its chunks' loads in flight (against sixteen
// waves of up to four chunks, N = 4096, K = 7168: M = 1 / 4 / 8 / 16
// 7.64 / 7.88 / 8.18 / 8.98 -> 7.46 / 7.64 / 7.87 / 8.62 us)
constexpr int kMxSaNW = 8, kMxSaMaxR = 8;

// dynamic LDS: activation rows (pitch K + 16), scale bytes rounded up to whole
// 1 KB copies, and the waves' partials
inline int64_t stream_mx_sa_lds(int64_t M, int64_t K) {
  return M * (K + 16) + ((M * (K / 32) + 1023) & ~1023LL) + (int64_t)kMxSaNW * 64 * 16;
}

inline bool stream_mx_sa_fits(int64_t M, int64_t K) {
  return M >= 1 && M <= 16 && K % 1024 == 0 && (K / 128 + kMxSaNW - 1) / kMxSaNW <= kMxSaMaxR &&
         stream_mx_sa_lds(M, K) <= 160 * 1024;
}

// One workgroup per 16 weight rows; its waves split the 128-byte K chunks.
// The activation rows and their scale bytes are copied into LDS first
// (buffer->LDS, 1 KB per wave instruction), then each wave issues its weight
// loads and waits for its copies with vmcnt(2R + 1) and a barrier without a
// fence, so the weight loads stay in flight across it. One MX-scaled MFMA per
// chunk (sixteen activation rows), partials summed over the waves in a fixed
// order.
template <int NW, int R>
__global__ __launch_bounds__(NW * 64) void gemm_stream_mx_sa(MxParams p) {
  static_assert(R <= 64, "a wave's weight-scale dwords fit one register");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;  // M <= 16
  const int KB = p.KB;                      // scale bytes per row
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int NC = (int)(K / 128);
  const int c_b = (int)((int64_t)w * NC / NW), c_e = (int)((int64_t)(w + 1) * NC / NW);
  const uint32_t a_pitch = (uint32_t)K + 16;
  const uint32_t s_bytes = (uint32_t)(M * KB);
  uint8_t* sA = smem;
  uint8_t* sS = smem + M * a_pitch;
  f32x4* red = reinterpret_cast<f32x4*>(sS + ((s_bytes + 1023u) & ~1023u));  // [NW][64]
  {
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.As, s_bytes);
    const int per_row = (int)(K / 1024), a_loads = (int)M * per_row;
    for (int i = w; i < a_loads; i += NW) {
      const int row = i / per_row, col = (i - row * per_row) * 1024;
      b2l16(rA, (uint32_t)lane * 16, (uint32_t)i * 1024, sA + row * a_pitch + col);
    }
    // the tail of the last 1 KB reads zeros from the resource's range check
    const int s_loads = (int)((s_bytes + 1023u) >> 10);
    for (int i = w; i < s_loads; i += NW) b2l16(rS, (uint32_t)lane * 16, (uint32_t)i * 1024, sS + i * 1024);
  }
  // the wave's weight-scale dwords (lane u: chunk c_b + u; the 16 rows share
  // one scale row since n0 and bn are multiples of 16) and weight chunks,
  // issued after the copies (clamped, so exactly 2R loads follow the dword)
  const int64_t nrow = n0 + r16 < N ? n0 + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + 16 * g;
  const int wc = c_b + lane < NC ? c_b + lane : NC - 1;
  const uint32_t wsl = reinterpret_cast<const uint32_t*>(p.Ws + (nrow / p.bn) * KB)[wc];
  asm volatile("" ::: "memory");
  i32x8 wf[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int c = c_b + u < NC - 1 ? c_b + u : NC - 1;
    wf[u] = gload_mx(wp + (int64_t)c * 128);
  }
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * R + 1) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  const int arow = r16 < M ? r16 : (int)M - 1;  // rows past M repeat the last (never stored)
  const uint8_t* al = sA + arow * a_pitch + 16 * g;
  const uint8_t* sl = sS + arow * KB;
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int c = c_b + u;
    if (c >= c_e) break;
    const i32x4 lo = *reinterpret_cast<const i32x4*>(al + c * 128);
    const i32x4 hi = *reinterpret_cast<const i32x4*>(al + c * 128 + 64);
    const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const uint32_t as = *reinterpret_cast<const uint32_t*>(sl + 4 * c) >> (8 * g);
    const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wsl, u) >> (8 * g);
    acc = mfma_mx(wf[u], af, acc, ws, as);
  }
  red[w * 64 + lane] = acc;
  __syncthreads();
  const bool bf16 = p.out_bf16 != 0, vec = p.d_vec4 != 0;
  for (int idx = tid; idx < 64; idx += NW * 64) {
    const int64_t m = idx & 15;
    if (m >= M) continue;
    f32x4 sum = red[idx];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) sum += red[ww * 64 + idx];
    const int64_t n = n0 + 4 * (idx >> 4);
    if (n < N) store4_mx(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec && n + 3 < N) : sum, bf16, vec);
  }
}

// ---- split K for 17..64 rows ---------------------------------------------------
constexpr int kMxMidRows = 64;  // weight rows per workgroup (four 16-row blocks)
constexpr int kMxMidNW = 8;     // waves: four row blocks x two chunk parities

// Workgroup (n block of 64 weight rows, K range s): all waves copy the range's
// activation slice (M rows x Kc bytes, 16-byte pieces, piece j of row m at
// slot j ^ (m & 15), so that the sixteen rows of a fragment read hit distinct
// banks) and the rows' scale dwords (four 32-wide blocks per 128-byte chunk)
// into LDS, then issue every weight load of their chunks (row block w & 3,
// chunks of parity w >> 2) before waiting for the copies. Each chunk and
// 16-row activation block is one MX-scaled MFMA accumulating across K (block
// scales applied in the matrix core); the two parities' sums meet in LDS and
// one float32 partial per output goes to part[s][m][n].
template <int MT, int R>
__global__ __launch_bounds__(kMxMidNW * 64) void gemm_split_mx(MxParams p, float* __restrict__ part, int Kc) {
  constexpr int NP = kMxMidNW / 4;
  static_assert(NP == 2 && R <= 64, "two chunk parities; a wave's scale dwords fit one register");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rb = w & 3, h = w >> 2;
  const int g = lane >> 4, r16 = lane & 15;
  const int64_t N = p.N, K = p.K, M = p.M;
  const int KB = p.KB;
  const int s_idx = blockIdx.y;
  const int64_t k0 = (int64_t)s_idx * Kc;
  const int ncc = Kc / 128;  // chunks in the range
  const int pr = Kc / 16;    // 16-byte pieces per activation row
  const int64_t n0 = (int64_t)blockIdx.x * kMxMidRows;
  uint8_t* sA = smem;
  const uint32_t a_bytes = (uint32_t)(((M * Kc) + 1023) & ~1023LL);
  uint32_t* sS = reinterpret_cast<uint32_t*>(smem + a_bytes);  // [M][ncc] scale dwords

  {
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(p.A, p.a_bytes);
    const __amdgpu_buffer_rsrc_t rS = make_rsrc(p.As, p.as_bytes);
    constexpr int kStride = 64 * kMxMidNW;
    // piece pc = 64 i + lane is (row, j) = divmod(pc, pr), stepped by the
    // stride's quotient and remainder with one carry (no division per piece)
    const int pieces = (int)M * pr;
    {
      const int dq = kStride / pr, dr = kStride - dq * pr;
      int pc = w * 64 + lane;
      int row = pc / pr, j = pc - row * pr;
      for (int i = w; i * 64 < pieces; i += kMxMidNW) {
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
    // scale dword (row, c): bytes kb0 + 4c .. kb0 + 4c + 3 of the row
    const int nsd = (int)M * ncc;
    {
      const int dq = kStride / ncc, dr = kStride - dq * ncc;
      int f = w * 64 + lane;
      int row = f / ncc, c = f - row * ncc;
      for (int i = w; i * 64 < nsd; i += kMxMidNW) {
        const uint32_t src = f < nsd ? (uint32_t)(row * KB + k0 / 32 + 4 * c) : 0xFFFFFFF0u;
        b2l4(rS, src, 0, sS + i * 64);
        f += kStride;
        row += dq;
        c += dr;
        if (c >= ncc) {
          c -= ncc;
          ++row;
        }
      }
    }
  }
  // the wave's weight rows and their scale dwords (row block rb shares one
  // weight-scale row: bn is a multiple of 16); lane u holds the dword of the
  // wave's u-th chunk
  const int64_t nrow = n0 + 16 * rb + r16 < N ? n0 + 16 * rb + r16 : N - 1;
  const uint8_t* wp = p.W + nrow * K + k0 + 16 * g;
  int64_t nb = (n0 + 16 * rb) / p.bn;
  if (nb > p.nbw - 1) nb = p.nbw - 1;
  const int li = lane < R ? lane : R - 1;
  const int lc = h + li * NP < ncc ? h + li * NP : ncc - 1;
  const uint32_t wsl = reinterpret_cast<const uint32_t*>(p.Ws + nb * KB + k0 / 32)[lc];
  asm volatile("" ::: "memory");
  i32x8 wf[R];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int cc0 = h + u * NP;
    const int cc = cc0 < ncc ? cc0 : ncc - 1;
    wf[u] = gload_mx(wp + (int64_t)cc * 128);
  }
  // loads complete in order: with at most 2R (weight halves) + 1 (scale
  // dword) outstanding, this wave's copies have landed; the barrier carries
  // no fence, so the weight loads stay in flight across it
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * R + 1) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // LDS offsets of this lane's pieces for its first chunk (h), per 16-row
  // block t; chunk h + NP u adds 256 u bytes (see the float32-scale kernel)
  uint32_t aoff[MT][2], soff[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int m = 16 * t + r16 < M ? 16 * t + r16 : (int)M - 1;
    const int key = m & 15;
#pragma unroll
    for (int f = 0; f < 2; ++f) aoff[t][f] = (uint32_t)(m * Kc + 16 * ((8 * h + 4 * f + g) ^ key));
    soff[t] = (uint32_t)((m * ncc + h) * 4);
  }
  const uint8_t* sSb = reinterpret_cast<const uint8_t*>(sS);
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const int cc = h + u * NP;
    if (cc >= ncc) break;
    const uint32_t ws = (uint32_t)__builtin_amdgcn_readlane((int)wsl, u) >> (8 * g);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const i32x4 lo = *reinterpret_cast<const i32x4*>(sA + aoff[t][0] + 256 * u);
      const i32x4 hi = *reinterpret_cast<const i32x4*>(sA + aoff[t][1] + 256 * u);
      const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      const uint32_t as = *reinterpret_cast<const uint32_t*>(sSb + soff[t] + 8 * u) >> (8 * g);
      acc[t] = mfma_mx(wf[u], af, acc[t], ws, as);
    }
  }
  __syncthreads();  // every wave is done with the slice
  f32x4* red = reinterpret_cast<f32x4*>(smem);  // [kMxMidNW][MT][64]
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
__global__ __launch_bounds__(256) void gemm_split_reduce_mx(MxParams p, const float* __restrict__ part,
                                                            int S) {
  const int64_t N = p.N, M = p.M;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t nv = N / 4;
  if (v >= M * nv) return;
  const int64_t m = v / nv, n = (v - m * nv) * 4;
  f32x4 sum = *reinterpret_cast<const f32x4*>(part + m * N + n);
  for (int s = 1; s < S; ++s) sum += *reinterpret_cast<const f32x4*>(part + ((int64_t)s * M + m) * N + n);
  const bool bf16 = p.out_bf16 != 0, vec = p.d_vec4 != 0;
  store4_mx(p, m, n, p.bias ? sum + load_bias4(p.bias, n, N, bf16, vec) : sum, bf16, vec);
}

struct MxMidPlan {
  int S = 0, Kc = 0, mt = 0, R = 0;
  int64_t lds = 0;
};

// K ranges: the fewest that give 256 workgroups, each a multiple of 256 bytes
// and at most 2048 (a wave's chunks then fit its registers); none fits -> not
// this kernel.
bool mx_mid_plan(int64_t M, int64_t N, int64_t K, MxMidPlan& pl) {
  if (M < 17 || M > 64 || N % 4 != 0) return false;
  const int64_t groups = (N + kMxMidRows - 1) / kMxMidRows;
  int best = 0;
  for (int S = 1; S <= 32; S *= 2) {
    if (K % (256LL * S) != 0 || K / S > 2048) continue;
    best = S;
    if (groups * S >= 256) break;
  }
  if (!best || groups * best > 0x7FFFFFFFLL) return false;
  pl.S = best;
  pl.Kc = (int)(K / best);
  const int ncc = pl.Kc / 128;
  // chunks per wave rounded up to 4, 7 or 8 (as for the float32-scale split;
  // M = 24 / 48 / 64 at K = 7168: 11.79 / 13.00 / 14.32 us with R = 8,
  // 11.41 / 12.67 / 14.05 us with R = 7)
  const int need = (ncc + 1) / 2;
  pl.R = need <= 4 ? 4 : (need <= 7 ? 7 : 8);
  pl.mt = (int)((M + 15) / 16);
  const int64_t a_bytes = ((M * pl.Kc) + 1023) & ~1023LL;
  const int64_t s_bytes = ((M * ncc + 63) / 64) * 64 * 4;
  const int64_t red_bytes = (int64_t)kMxMidNW * pl.mt * 64 * 16;
  pl.lds = a_bytes + s_bytes > red_bytes ? a_bytes + s_bytes : red_bytes;
  return pl.lds <= 160 * 1024;
}

// dynamic LDS above 64 KiB needs the kernel's limit raised, once per device
hipError_t raise_lds_limit_mx(const void* kern, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  const uint64_t bit = 1ull << dev;
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

template <int MT, int R>
hipError_t launch_split_mx_inst(const MxParams& p, const MxMidPlan& pl, float* part, hipStream_t st) {
  const auto kern = gemm_split_mx<MT, R>;
  static std::atomic<uint64_t> lds_raised{0};
  hipError_t e = raise_lds_limit_mx(reinterpret_cast<const void*>(kern), lds_raised);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((p.N + kMxMidRows - 1) / kMxMidRows), (unsigned)pl.S);
  hipLaunchKernelGGL(kern, grid, dim3(kMxMidNW * 64), (unsigned)pl.lds, st, p, part, pl.Kc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t vecs = p.M * (p.N / 4);
  hipLaunchKernelGGL(gemm_split_reduce_mx, dim3((unsigned)((vecs + 255) / 256)), dim3(256), 0, st, p,
                     (const float*)part, pl.S);
  return hipGetLastError();
}

template <int R>
hipError_t launch_stream_mx_sa_r(const MxParams& p, hipStream_t st) {
  const auto kern = gemm_stream_mx_sa<kMxSaNW, R>;
  static std::atomic<uint64_t> lds_raised{0};
  const hipError_t e = raise_lds_limit_mx(reinterpret_cast<const void*>(kern), lds_raised);
  if (e != hipSuccess) return e;
  if ((p.N + 15) / 16 > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3((unsigned)((p.N + 15) / 16)), dim3(kMxSaNW * 64),
                     (unsigned)stream_mx_sa_lds(p.M, p.K), st, p);
  return hipGetLastError();
}

// R: the fewest of 2, 4, 7 or 8 chunks per wave that covers K
hipError_t launch_stream_mx_sa(const MxParams& p, hipStream_t st) {
  const int64_t per = (p.K / 128 + kMxSaNW - 1) / kMxSaNW;
  if (per <= 2) return launch_stream_mx_sa_r<2>(p, st);
  if (per <= 4) return launch_stream_mx_sa_r<4>(p, st);
  if (per <= 7) return launch_stream_mx_sa_r<7>(p, st);
  return launch_stream_mx_sa_r<8>(p, st);
}

template <int MT>
hipError_t launch_split_mx_r(const MxParams& p, const MxMidPlan& pl, float* part, hipStream_t st) {
  return pl.R == 4   ? launch_split_mx_inst<MT, 4>(p, pl, part, st)
         : pl.R == 7 ? launch_split_mx_inst<MT, 7>(p, pl, part, st)
                     : launch_split_mx_inst<MT, 8>(p, pl, part, st);
}

hipError_t launch_split_mx(const MxParams& p, const MxMidPlan& pl, float* part, hipStream_t st) {
  switch (pl.mt) {
    case 2: return launch_split_mx_r<2>(p, pl, part, st);
    case 3: return launch_split_mx_r<3>(p, pl, part, st);
    default: return launch_split_mx_r<4>(p, pl, part, st);
  }
}

constexpr int kMxBM = 256, kMxBN = 256, kMxWM = 2, kMxWN = 4;
constexpr int kMxStreamNW = 16;

template <int MT>
hipError_t launch_stream_mx(const MxParams& p, hipStream_t st) {
  const dim3 grid((unsigned)((p.N + 15) / 16), (unsigned)((p.M + MT * 16 - 1) / (MT * 16)));
  constexpr int R = MT == 1 ? 4 : 2;
  hipLaunchKernelGGL((gemm_stream_mx<MT, kMxStreamNW, R>), grid, dim3(kMxStreamNW * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

size_t blockwise_e8m0_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (K % 128 != 0) return 0;
  MxMidPlan pl;
  if (!mx_mid_plan(M, N, K, pl)) return 0;
  return (size_t)pl.S * (size_t)M * (size_t)N * sizeof(float);
}

size_t blockwise_e8m0_split_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 64 || K % 128 != 0 || N < 1) return 0;
  SplitPlan sp;
  const int64_t tiles = ((M + kMxBM - 1) / kMxBM) * ((N + kMxBN - 1) / kMxBN);
  if (!split_plan(tiles, (int)(K / 128), device_cus(), sp)) return 0;
  return split_bytes(sp.tiles);
}

hipError_t launch_blockwise_e8m0(const MxGemmArgs& a, hipStream_t st) {
  if (a.M == 0) return hipSuccess;
  MxParams p{};
  p.A = a.A; p.As = a.As; p.W = a.W; p.Ws = a.Ws; p.bias = a.bias; p.D = a.D;
  p.M = a.M; p.N = a.N; p.K = a.K;
  p.KB = (int)(a.K / 32);
  p.bn = a.bn;
  p.nbw = (int)((a.N + a.bn - 1) / a.bn);
  p.out_bf16 = a.out_dtype == Q8_BF16;
  p.d_vec4 = a.N % 4 == 0 && (uintptr_t)a.D % 8 == 0 && (uintptr_t)a.bias % 8 == 0;
  p.a_bytes = (uint32_t)(a.M * a.K);
  p.as_bytes = (uint32_t)(a.M * (a.K / 32));
  p.tiles_m = (a.M + kMxBM - 1) / kMxBM;
  p.tiles_n = (a.N + kMxBN - 1) / kMxBN;
  if (a.M <= 64) {
    // 17..64 rows: split K, partials in the workspace
    MxMidPlan pl;
    if (mx_mid_plan(a.M, a.N, a.K, pl) && a.workspace && (uintptr_t)a.workspace % 16 == 0 &&
        (uintptr_t)a.A % 16 == 0)
      return launch_split_mx(p, pl, static_cast<float*>(a.workspace), st);
    // up to 16 rows: the activations staged in LDS once per workgroup
    if (stream_mx_sa_fits(a.M, a.K) && (uintptr_t)a.A % 16 == 0 && (uintptr_t)a.As % 16 == 0)
      return launch_stream_mx_sa(p, st);
    const int mt = (int)((a.M + 15) / 16);
    switch (mt) {
      case 1: return launch_stream_mx<1>(p, st);
      case 2: return launch_stream_mx<2>(p, st);
      case 3: return launch_stream_mx<3>(p, st);
      default: return launch_stream_mx<4>(p, st);
    }
  }
  const int64_t tiles = p.tiles_m * p.tiles_n;
  if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  SplitPlan sp;
  if (a.workspace && (uintptr_t)a.workspace % 16 == 0 && split_plan(tiles, (int)(a.K / 128), device_cus(), sp) &&
      a.workspace_bytes >= split_bytes(sp.tiles)) {
    p.part = static_cast<float*>(a.workspace);
    p.flag = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(a.workspace) + split_part_bytes(sp.tiles));
    p.token = next_split_token();
    p.split_k = sp.k;
    p.split_first = sp.first;
    p.split_lead = sp.lead;
    p.split_tiles = sp.tiles;
    p.part_bytes = (uint32_t)split_part_bytes(sp.tiles);
    p.split_wait = split_wait_ticks();
    hipLaunchKernelGGL((gemm_tile_mx<kMxBM, kMxBN, kMxWM, kMxWN, true>),
                       dim3((unsigned)(sp.first + 2 * sp.tiles)), dim3(kMxWM * kMxWN * 64), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((gemm_tile_mx<kMxBM, kMxBN, kMxWM, kMxWN, false>), dim3((unsigned)tiles),
                     dim3(kMxWM * kMxWN * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace q8
