// MoE routing-table construction and row gather for gfx950.
//
// "Implementation: Sgl project Sglang CUTLASS MoE", Description: from the
// router's topk_ids build expert_offsets, per-expert problem sizes and the
// input/output permutations around the grouped GEMM; "Implementation: Sgl
// project Sglang GEMM Interface", Utility: shuffle_rows (destination-to-
// source row permutation).
//
// Routing is a stable counting sort over the flat choices i = t*topk + j:
//   1. moe_count  — one workgroup per chunk of 256 flat entries builds the
//                   chunk's per-expert histogram in LDS (counts are order
//                   independent);
//   2. moe_scan   — the experts' counts are scanned over the chunks
//                   (exclusive, from LDS slabs), then the per-expert totals
//                   are scanned over the experts into expert_offsets and
//                   problem sizes, and the chunk bases are shifted by the
//                   expert offsets;
//   3. moe_scatter — each entry's slot = its chunk's base for its expert plus
//                   the number of earlier entries of the same expert inside
//                   the chunk (counted from an LDS copy of the chunk), so
//                   slots ascend with the flat index inside every expert and
//                   the tables are deterministic.
#include <atomic>
#include <mutex>

#include "q8_internal.h"
#include "q8_device.h"

namespace q8 {
namespace {

constexpr int kChunk = 256;
constexpr int kScanThreads = 1024;

__global__ __launch_bounds__(kChunk) void moe_count(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, int32_t* __restrict__ counts) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < E; e += kChunk) hist[e] = 0;
  __syncthreads();
  const int64_t i = (int64_t)blockIdx.x * kChunk + threadIdx.x;
  if (i < n) atomicAdd(&hist[ids[i]], 1);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kChunk) counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// Chunk counts are staged through LDS a slab at a time (coalesced loads by
// every thread) so that each expert's column is scanned from LDS instead of
// through dependent global loads. A count matrix that fits one slab (up to
// 8192 counts: 4096 tokens x top-8 over 64 experts) stays in LDS until the
// experts' offsets are added and is written once, and each expert's column
// is scanned by P = 1024 / E threads (P = 16 for 64 experts): every thread
// sums its run of rows, the runs' sums are added up in order for its base,
// and it rewrites its rows as exclusive prefixes, so the chain of dependent
// LDS accesses is a run of rows long instead of a whole column. Larger
// matrices go slab by slab, one thread per expert (the split scan's extra
// barrier per slab measured slower there). A slab's loads all go out before
// the first LDS store. Measured for the three routing kernels: 4096 x top-8
// of 64 experts 18.3 -> 16.4 us (split scan) -> 15.0 us (batched loads);
// 16384 x top-8 of 256 (16 slabs) 89.6 -> 69.4 us.
constexpr int kSlabInts = 8192;  // 32 KB of LDS

// counts[0, n) -> slab, every thread's loads in flight together (n <=
// kSlabInts: at most eight per thread)
__device__ __forceinline__ void load_slab(const int32_t* __restrict__ src, int64_t n, int32_t* slab) {
  constexpr int U = kSlabInts / kScanThreads;
  int32_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = (int64_t)u * kScanThreads + threadIdx.x;
    v[u] = i < n ? src[i] : 0;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = (int64_t)u * kScanThreads + threadIdx.x;
    if (i < n) slab[i] = v[u];
  }
}

__global__ __launch_bounds__(kScanThreads) void moe_scan(int32_t* __restrict__ counts,
                                                         int64_t nchunks, int E, int64_t nk,
                                                         int64_t kk, int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ ps1,
                                                         int32_t* __restrict__ ps2) {
  __shared__ int32_t tot[kScanThreads];
  __shared__ int32_t carry[kScanThreads];    // per expert: its total count
  __shared__ int32_t part_sum[kScanThreads];  // [part][expert]
  __shared__ int32_t slab[kSlabInts];
  const int tid = threadIdx.x;
  const int64_t rows_per_slab = kSlabInts / E;
  const bool one_slab = nchunks <= rows_per_slab;
  // pass 1: per-expert exclusive scan over the chunks (relative bases)
  if (one_slab) {
    const int parts = kScanThreads / E;  // E <= kScanThreads
    const int e = tid % E, part = tid / E;
    const bool active = part < parts;
    const int64_t rows = nchunks;
    load_slab(counts, rows * E, slab);
    __syncthreads();
    const int64_t rpp = (rows + parts - 1) / parts;
    const int64_t r0 = part * rpp, r1 = r0 + rpp < rows ? r0 + rpp : rows;
    int32_t sum = 0;
    if (active)
      for (int64_t r = r0; r < r1; ++r) sum += slab[r * E + e];
    if (active) part_sum[part * E + e] = sum;
    __syncthreads();
    if (active) {
      int32_t run = 0;
      for (int q = 0; q < part; ++q) run += part_sum[q * E + e];
      for (int64_t r = r0; r < r1; ++r) {
        const int32_t v = slab[r * E + e];
        slab[r * E + e] = run;
        run += v;
      }
    }
    if (tid < E) {
      int32_t t = 0;
      for (int q = 0; q < parts; ++q) t += part_sum[q * E + tid];
      carry[tid] = t;
    }
    __syncthreads();
  } else {
    int32_t run = 0;
    for (int64_t c0 = 0; c0 < nchunks; c0 += rows_per_slab) {
      const int64_t rows = nchunks - c0 < rows_per_slab ? nchunks - c0 : rows_per_slab;
      load_slab(counts + c0 * E, rows * E, slab);
      __syncthreads();
      if (tid < E) {
        for (int64_t r = 0; r < rows; ++r) {
          const int32_t v = slab[r * E + tid];
          slab[r * E + tid] = run;
          run += v;
        }
      }
      __syncthreads();
      for (int64_t i = tid; i < rows * E; i += kScanThreads) counts[c0 * E + i] = slab[i];
      __syncthreads();
    }
    if (tid < E) carry[tid] = run;
    __syncthreads();
  }
  const int32_t run = tid < E ? carry[tid] : 0;  // the expert's total
  tot[tid] = run;
  __syncthreads();
  // inclusive Hillis-Steele scan over the per-expert totals
  for (int off = 1; off < E; off <<= 1) {
    const int32_t v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    const int32_t base = tot[tid] - run;  // exclusive prefix
    offsets[tid] = base;
    if (tid == E - 1) offsets[E] = tot[tid];
    ps1[3 * tid + 0] = run; ps1[3 * tid + 1] = (int32_t)nk; ps1[3 * tid + 2] = (int32_t)kk;
    ps2[3 * tid + 0] = run; ps2[3 * tid + 1] = (int32_t)kk; ps2[3 * tid + 2] = (int32_t)nk;
  }
  __shared__ int32_t base_of[kScanThreads];
  if (tid < E) base_of[tid] = tot[tid] - run;
  __syncthreads();
  // pass 2: shift every chunk base by its expert's offset (coalesced)
  if (one_slab) {
    for (int64_t i = tid; i < nchunks * E; i += kScanThreads) counts[i] = slab[i] + base_of[i % E];
  } else {
    for (int64_t i = tid; i < nchunks * E; i += kScanThreads) counts[i] += base_of[i % E];
  }
}

__global__ __launch_bounds__(kChunk) void moe_scatter(const int32_t* __restrict__ ids, int64_t n,
                                                      int topk, int E,
                                                      const int32_t* __restrict__ bases,
                                                      int32_t* __restrict__ in_perm,
                                                      int32_t* __restrict__ out_perm) {
  __shared__ int32_t sid[kChunk];
  const int64_t i0 = (int64_t)blockIdx.x * kChunk;
  const int64_t i = i0 + threadIdx.x;
  const int32_t id = i < n ? ids[i] : -1;
  sid[threadIdx.x] = id;
  __syncthreads();
  if (i >= n) return;
  int32_t rank = 0;
  for (int t = 0; t < (int)threadIdx.x; ++t) rank += sid[t] == id;
  const int32_t slot = bases[(int64_t)blockIdx.x * E + id] + rank;
  in_perm[slot] = (int32_t)(i / topk);
  out_perm[i] = slot;
}

__global__ void shuffle_rows_vec(const uint4* __restrict__ src, int64_t row_vecs,
                                 const int32_t* __restrict__ map, int64_t rows,
                                 uint4* __restrict__ dst) {
  const int64_t total = rows * row_vecs;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / row_vecs, c = v - r * row_vecs;
    dst[v] = src[(int64_t)map[r] * row_vecs + c];
  }
}

__global__ void shuffle_rows_bytes(const uint8_t* __restrict__ src, int64_t row_bytes,
                                   const int32_t* __restrict__ map, int64_t rows,
                                   uint8_t* __restrict__ dst) {
  const int64_t total = rows * row_bytes;
  for (int64_t v = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = v / row_bytes, c = v - r * row_bytes;
    dst[v] = src[(int64_t)map[r] * row_bytes + c];
  }
}

}  // namespace

size_t moe_workspace_ints(int64_t T, int topk, int E) {
  const int64_t n = T * topk;
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  return (size_t)(nchunks * E);
}

// ---- finalize: weight each token's top-k expert rows and sum them ----------------
// out[t, n] = sum_{j < topk} w[t, j] * D[row(t, j), n], in float32 in ascending
// j with one FMA per term, then rounded to the 16-bit output type; row(t, j)
// = perm[t * topk + j] (D in expert-sorted order) or t * topk + j. One
// workgroup row of threads per token, eight columns (16 bytes) per thread.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(256) void moe_finalize_k(const uint16_t* __restrict__ D,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ perm,
                                                      int64_t T, int topk, int64_t N,
                                                      uint16_t* __restrict__ out) {
  constexpr int E = VEC ? 8 : 1;
  const int64_t t = blockIdx.y;
  const int64_t c = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) * E;
  if (c >= N) return;
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.0f;
  for (int j = 0; j < topk; ++j) {
    const int64_t i = t * topk + j;
    const int64_t row = perm ? (int64_t)perm[i] : i;
    const float wt = w ? w[i] : 1.0f;
    if constexpr (VEC) {
      const uint4 v = *reinterpret_cast<const uint4*>(D + row * N + c);
      const uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = BF16 ? bf16_bits_to_f32(h[q] & 0xFFFFu) : f16_bits_to_f32(h[q] & 0xFFFFu);
        const float hi = BF16 ? bf16_bits_to_f32(h[q] >> 16) : f16_bits_to_f32(h[q] >> 16);
        acc[2 * q] = __builtin_fmaf(wt, lo, acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wt, hi, acc[2 * q + 1]);
      }
    } else {
      const uint16_t h = D[row * N + c];
      acc[0] = __builtin_fmaf(wt, BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h), acc[0]);
    }
  }
  if constexpr (VEC) {
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = BF16 ? f32_to_bf16_bits(acc[2 * q]) : f32_to_f16_bits(acc[2 * q]);
      const uint32_t hi = BF16 ? f32_to_bf16_bits(acc[2 * q + 1]) : f32_to_f16_bits(acc[2 * q + 1]);
      o[q] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(out + t * N + c) = uint4{o[0], o[1], o[2], o[3]};
  } else {
    out[t * N + c] = (uint16_t)(BF16 ? f32_to_bf16_bits(acc[0]) : f32_to_f16_bits(acc[0]));
  }
}

hipError_t launch_moe_mm_data(const int32_t* ids, int64_t T, int topk, int E, int64_t nk,
                              int64_t kk, int32_t* offsets, int32_t* ps1, int32_t* ps2,
                              int32_t* in_perm, int32_t* out_perm, int32_t* ws,
                              hipStream_t st) {
  const int64_t n = T * topk;
  const int64_t nchunks = (n + kChunk - 1) / kChunk;
  if (nchunks > 0) {
    hipLaunchKernelGGL(moe_count, dim3((unsigned)nchunks), dim3(kChunk), E * sizeof(int32_t), st,
                       ids, n, E, ws);
  }
  hipLaunchKernelGGL(moe_scan, dim3(1), dim3(kScanThreads), 0, st, ws, nchunks, E, nk, kk,
                     offsets, ps1, ps2);
  if (nchunks > 0) {
    hipLaunchKernelGGL(moe_scatter, dim3((unsigned)nchunks), dim3(kChunk), 0, st, ids, n, topk,
                       E, ws, in_perm, out_perm);
  }
  return hipGetLastError();
}

// ---- allocation-free routing ----------------------------------------------------
// moe_mm_data_noalloc keeps its per-chunk expert counts (the only memory the
// three routing kernels use besides their inputs and outputs) in this
// file-scope array instead of a caller workspace: kNoAllocInts ints per device,
// held until the process ends. In host code `scratch` is only a host-side
// stand-in for the symbol; its device address on each GPU comes from
// hipGetSymbolAddress, looked up once per device with that device current and
// kept in scratch_on[]. moe_count overwrites every count a call reads, so
// nothing has to start at zero; two calls that overlap on one device share the
// array and race.
static __device__ __align__(256) int32_t scratch[kNoAllocInts];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int32_t*> scratch_on[kMaxDevices];
std::mutex scratch_mu;
}  // namespace

hipError_t noalloc_scratch(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int32_t* p = scratch_on[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_on[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = static_cast<int32_t*>(addr);
      scratch_on[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_moe_mm_data_noalloc(const int32_t* ids, int64_t T, int topk, int E, int64_t nk,
                                      int64_t kk, int32_t* offsets, int32_t* ps1, int32_t* ps2,
                                      int32_t* in_perm, int32_t* out_perm, hipStream_t st) {
  if (moe_workspace_ints(T, topk, E) > (size_t)kNoAllocInts) return hipErrorInvalidValue;
  int32_t* ws = nullptr;
  const hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  return launch_moe_mm_data(ids, T, topk, E, nk, kk, offsets, ps1, ps2, in_perm, out_perm, ws, st);
}

hipError_t launch_shuffle_rows(const void* src, int64_t row_bytes, const int32_t* map,
                               int64_t rows, void* dst, hipStream_t st) {
  if (rows == 0 || row_bytes == 0) return hipSuccess;
  const int threads = 256;
  const bool vec = row_bytes % 16 == 0 && (uintptr_t)src % 16 == 0 && (uintptr_t)dst % 16 == 0;
  const int64_t work = vec ? rows * (row_bytes / 16) : rows * row_bytes;
  int64_t blocks = (work + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  if (vec)
    hipLaunchKernelGGL(shuffle_rows_vec, dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const uint4*>(src), row_bytes / 16, map, rows,
                       static_cast<uint4*>(dst));
  else
    hipLaunchKernelGGL(shuffle_rows_bytes, dim3((unsigned)blocks), dim3(threads), 0, st,
                       static_cast<const uint8_t*>(src), row_bytes, map, rows,
                       static_cast<uint8_t*>(dst));
  return hipGetLastError();
}

hipError_t launch_moe_finalize(const void* D, bool bf16, const float* w, const int32_t* perm,
                               int64_t T, int topk, int64_t N, void* out, hipStream_t st) {
  if (T == 0 || N == 0) return hipSuccess;
  const bool vec = N % 8 == 0 && (uintptr_t)D % 16 == 0 && (uintptr_t)out % 16 == 0;
  const int64_t per_thread = vec ? 8 : 1;
  const int64_t bx = (N + 256 * per_thread - 1) / (256 * per_thread);
  if (T > 65535 * 1024LL || bx > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
  // grid.y is limited to 65535: tokens beyond it go in further launches
  for (int64_t t0 = 0; t0 < T; t0 += 65535) {
    const int64_t nt = T - t0 < 65535 ? T - t0 : 65535;
    const dim3 grid((unsigned)bx, (unsigned)nt);
    const uint16_t* d = static_cast<const uint16_t*>(D);
    const float* wt = w ? w + t0 * topk : nullptr;
    const int32_t* pm = perm ? perm + t0 * topk : nullptr;
    uint16_t* o = static_cast<uint16_t*>(out) + t0 * N;
#define Q8_FIN(B, V) hipLaunchKernelGGL((moe_finalize_k<B, V>), grid, dim3(256), 0, st, \
                                        perm ? d : d + t0 * topk * N, wt, pm, nt, topk, N, o)
    if (bf16) { if (vec) Q8_FIN(true, true); else Q8_FIN(true, false); }
    else { if (vec) Q8_FIN(false, true); else Q8_FIN(false, false); }
#undef Q8_FIN
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace q8
