/*
 * q8gemm — scaled 8-bit GEMM for LLM linear layers on AMD Instinct MI355X
 * (gfx950 / CDNA4). C ABI.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every pointer argument is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *   tensor's data_ptr), unless a comment says otherwise. The caller owns and
 *   allocates every buffer, outputs and workspace included; outputs are
 *   written in place. The library never allocates or frees memory and may be
 *   called from several threads at once. Its process-wide state: per-device
 *   records that a kernel's LDS limit was raised and of the compute-unit
 *   count, for the one allocation-free entry point (moe_mm_data_noalloc) a
 *   fixed device array per GPU and its device address, looked up once per
 *   device; a call counter (blockwise_scaled_mm tokens) and the setting of
 *   q8gemm_set_split_wait_us. All of it is thread-safe.
 * - Every matrix is row-major and contiguous unless a leading dimension is
 *   passed. Weights are [N, K] with K contiguous (the "nt" layout: a
 *   column-major [K, N] weight is the same bytes).
 * - All calls are asynchronous on `stream` (0 = the null stream).
 * - Return value: Q8_OK (0) or a negative Q8_E* code. Every argument is
 *   validated on the host before any HIP call, so an invalid call touches
 *   neither the device nor the stream. q8gemm_last_error() then returns a
 *   message for the calling thread. Device-side preconditions (for example
 *   expert ids in range) are documented per call and are not checked.
 * - FP8 means OCP float8 e4m3fn (torch.float8_e4m3fn): largest finite 448,
 *   no infinities, codes 0x7F/0xFF are NaN.
 */
#ifndef Q8GEMM_H
#define Q8GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  Q8_OK = 0,
  Q8_EINVAL = -1,        /* null pointer, bad dtype or enum value          */
  Q8_ESHAPE = -2,        /* a size or divisibility rule is broken          */
  Q8_EUNSUPPORTED = -3,  /* a valid request the library does not implement */
  Q8_EWORKSPACE = -4,    /* workspace missing or smaller than required     */
  Q8_EHIP = -5           /* a HIP call (kernel launch) failed              */
};

typedef enum {
  Q8_F32 = 0,
  Q8_BF16 = 1,
  Q8_F16 = 2,
  Q8_E4M3FN = 3,
  Q8_I8 = 4,
  Q8_I32 = 5
} q8_dtype;

typedef enum {
  Q8_SCALE_PER_GROUP = 0,          /* s[M, K/group_size], one per token group */
  Q8_SCALE_PER_TENSOR_DYNAMIC = 1, /* s[1] from the whole tensor's |max|      */
  Q8_SCALE_STATIC = 2              /* s[1] is an INPUT scale                  */
} q8_scale_mode;

/* Message describing the last failed call on this thread ("" if none). */
const char* q8gemm_last_error(void);

/*
 * Longest time the first part of a split tile (blockwise_scaled_mm and
 * blockwise_scaled_mm_e8m0 with more than 64 rows and a workspace) waits for
 * its second part, in
 * microseconds, for later calls of this process: default 200, at most
 * 100000. A first part whose second part is not done by then (its
 * workgroup did not get a compute unit in time) computes the rest of K
 * itself. 0: first parts never wait, so every tile's outputs equal the
 * unsplit kernel's bit for bit (testing). Q8_EINVAL outside [0, 100000].
 */
int q8gemm_set_split_wait_us(int microseconds);

/*
 * 8-bit activation quantization.
 * "Implementation: Sgl project Sglang GEMM Interface", Description >
 * Quantization Routines: sgl_per_token_group_quant_8bit (per token, per
 * group of group_size consecutive K elements, FP8 or INT8, epsilon,
 * clipping range, optional UE8M0 scale), sgl_per_token_quant_fp8 (one group
 * per row: group_size = K) and sgl_per_tensor_quant_fp8 (static or dynamic
 * per-tensor scale); the INT8 flavour is the symmetric dynamic/static
 * quantization of the vLLM scaled_mm page (AiterInt8ScaledMMLinearKernel).
 *
 * x       [M, K] of x_dtype (Q8_F32, Q8_BF16 or Q8_F16), row stride ld_x >= K
 *         elements ([M, 2K], ld_x >= 2K, with fuse_silu_and_mul).
 * q       [M, K] of q_dtype (Q8_E4M3FN or Q8_I8), contiguous (row stride K).
 * s       Q8_SCALE_PER_GROUP: output, [M, K/group_size] float32 row-major.
 *         Q8_SCALE_PER_TENSOR_DYNAMIC: output, s[0].
 *         Q8_SCALE_STATIC: input, s[0] (must be > 0; read on the device).
 * Per group (all float32, round to nearest even):
 *   a = max|x|; s = max(a, eps) / qmax; UE8M0: s rounded up to a power of
 *   two; y = clamp(x / s, qmin, qmax) with a true division; FP8: nearest
 *   e4m3fn code, ties to even, sign kept (-0 -> 0x80); INT8: rint(y).
 * group_size must divide K (PER_GROUP); it is ignored by the other modes.
 * eps > 0 floors a (an all-zero group gets s = eps/qmax and zero codes).
 * Typical ranges: FP8 qmin=-448, qmax=448; INT8 qmin=-128, qmax=127.
 * scale_ue8m0: 0 plain float32 scales; 1 UE8M0-rounded scales stored as
 * float32; 2 UE8M0-rounded scales stored packed as their E8M0 byte (the
 * biased exponent b, s = 2^(b - 127); the float8_e8m0fnu scale dtype of the
 * vLLM scaled_mm page), s then being a uint8 buffer of the same shape
 * ([M, K/group_size] or [1]) passed through this float* argument.
 * scale_ue8m0 must be 0 with Q8_SCALE_STATIC.
 *
 * Fused SiLU-and-mul and masked rows (the same page names a second version of
 * the per-token-group quantizer that fuses the gated activation and honours
 * a per-expert row count; Q8_SCALE_PER_GROUP only, else Q8_EUNSUPPORTED):
 * fuse_silu_and_mul = 1: x is [M, 2K] (row stride ld_x >= 2K), each row
 *   [gate | up]; the value quantized is y = silu(gate) * up, evaluated in
 *   float32 one rounding per step: e = exp(-g) correctly rounded, d = 1 + e,
 *   h = g / d (true division), y = h * u. q and s are [M, K] and
 *   [M, K/group_size] as above. 0 quantizes x itself.
 * masked_m != NULL: the M rows are E = M / max_m blocks of max_m rows (a
 *   [E, max_m, .] tensor) and masked_m [E] int32 (device) holds the number
 *   of valid leading rows of each block; row r is quantized only if
 *   r % max_m < masked_m[r / max_m]. Other rows of q and s are not written
 *   and their inputs are not read. Needs max_m >= 1 dividing M, M < 2^32.
 *   Device precondition: 0 <= masked_m[e] <= max_m (larger values act as
 *   max_m, negative values as 0). max_m is ignored when masked_m is NULL.
 *
 * workspace: Q8_SCALE_PER_TENSOR_DYNAMIC needs quant_8bit_workspace_size()
 * bytes (partial maxima); other modes need none (NULL, 0 allowed).
 * M == 0 or K == 0 is a no-op.
 */
size_t quant_8bit_workspace_size(int64_t M, int64_t K, q8_scale_mode mode);
int quant_8bit(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, int64_t ld_x,
               void* q, q8_dtype q_dtype, float* s, int64_t group_size,
               q8_scale_mode mode, float eps, float qmin, float qmax,
               int scale_ue8m0, int fuse_silu_and_mul, const int32_t* masked_m,
               int64_t max_m, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with bf16/f16 output.
 * The block32 DeepGEMM PR for DeepSeek-V4.1 ("[SM90] Use native block32
 * DeepGEMM for DeepSeek-V4.1"), Modifications: fp8_gemm_nt((Aq, As), (Wq, Ws),
 * D, recipe=(1, bn, bk)) with [32,32] or [128,128] weight blocks; weight
 * scale layout [n_blocks, k_blocks] from the vLLM scaled_mm page
 * (XPUFp8BlockScaledMMKernel).
 *
 *   D[m,n] = sum_kb As[m,kb] * Ws[n/bn, kb] * sum_{k in kb} A[m,k] * W[n,k]
 *            (+ bias[n]), rounded to nearest even into out_dtype.
 *
 * A   [M, K] e4m3fn, As [M, K/bk] float32 (activation groups of 1 x bk).
 * W   [N, K] e4m3fn, Ws [ceil(N/bn), K/bk] float32.
 * bias [N] of out_dtype, or NULL.   D [M, N] of out_dtype (Q8_BF16, Q8_F16).
 * Rules: bk in {32, 128}; bn a positive multiple of 16; K % bk == 0
 * (ragged K is rejected, as the vLLM XPU kernel does); any M >= 0, N >= 1;
 * A, W and As each below 4 GiB (Q8_EUNSUPPORTED otherwise).
 * Accumulation: FP8 products summed in float32 per K block, scaled and
 * summed in float32.
 * workspace: blockwise_scaled_mm_workspace_size() bytes, 16-byte aligned.
 * - 17..64 rows: float32 split-K partials (S x M x N floats, S the number of
 *   K ranges; 4 MiB for 64 x 4096 x 7168); required (Q8_EWORKSPACE if
 *   missing or short).
 * - more than 64 rows, K a multiple of 128 and at least 1024: optional. The
 *   LDS-tiled kernel runs one 256 x 256 tile per compute unit at a time; when
 *   the tile count T leaves a last round of R = T mod C tiles on the device's
 *   C compute units with 0 < R <= C / 2, those R tiles are each split in K
 *   between two workgroups (idle units run the second parts), which needs R
 *   float32 tile partials and R flag words (32 MiB for 4096 x 18432 on 256
 *   units; 4096 x 7168, R = 192, is not split). Without a workspace of that
 *   size every tile runs whole. A
 *   split tile adds two float32 partial sums, so its outputs can differ from
 *   the unsplit ones in the last bits; each way is deterministic (a tile's
 *   first part comes out as unsplit when its second part is late, see
 *   q8gemm_set_split_wait_us). The size depends on the current device.
 * - 0 for every other shape (then NULL is allowed).
 * The contents need no initialisation (flag words hold any value between
 * calls) and are overwritten. Calls that may overlap in time (other streams)
 * must not share a workspace.
 */
size_t blockwise_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K, int bn, int bk);
int blockwise_scaled_mm(const void* A, const float* As, const void* W, const float* Ws,
                        const void* bias, void* D, q8_dtype out_dtype,
                        int64_t M, int64_t N, int64_t K, int bn, int bk,
                        void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Block-scaled FP8 GEMM with power-of-two (E8M0) block scales on both
 * operands, applied by the matrix cores (gfx950 MX-scaled MFMA).
 * The block32 DeepGEMM PR for DeepSeek-V4.1 ("[SM90] Use native block32
 * DeepGEMM for DeepSeek-V4.1"), Modifications: recipe (1, bn, 32) with UE8M0
 * activation scales; vLLM scaled_mm page (XPUFp8BlockScaledMMKernel): weight
 * scales stored as float8_e8m0fnu bytes. A byte b is the scale 2^(b - 127).
 *
 *   D[m,n] = sum_kb 2^(As[m,kb]-127) * 2^(Ws[n/bn,kb]-127)
 *            * sum_{k in kb} A[m,k] * W[n,k]   (+ bias[n]), RNE to out_dtype
 *
 * over 32-wide K blocks kb.
 * A   [M, K] e4m3fn, As [M, K/32] uint8 E8M0 (quant_8bit with
 *     scale_ue8m0 = 2 and group_size 32 writes this).
 * W   [N, K] e4m3fn, Ws [ceil(N/bn), K/32] uint8 E8M0.
 * bias [N] of out_dtype, or NULL.   D [M, N] of out_dtype (Q8_BF16, Q8_F16).
 * Rules: K a positive multiple of 128; bn a positive multiple of 16; any
 * M >= 0, N >= 1; As and Ws 4-byte aligned; A and W each below 4 GiB.
 * Byte 255 (NaN) is not a valid scale (documented, not checked).
 * Accumulation: FP8 products scaled and summed in float32 inside the matrix
 * cores (order unspecified); for 17..64 rows with a workspace, K is split into
 * ranges whose float32 partials are summed in ascending range order.
 * workspace: blockwise_scaled_mm_e8m0_workspace_size() bytes, 16-byte
 * aligned.
 * - 17..64 rows: the split-K partials (S x M x N floats; 4 MiB for 64 x 4096
 *   x 7168); required (Q8_EWORKSPACE if missing or short).
 * - more than 64 rows, K at least 1024: optional, as for blockwise_scaled_mm:
 *   a last round of 256 x 256 tiles that fills at most half of the device's
 *   compute units is split in K between two workgroups each, with R float32
 *   tile partials and R flag words. A split tile adds two float32 partial
 *   sums (its outputs can differ from the unsplit ones in the last bits);
 *   with q8gemm_set_split_wait_us(0) every tile equals the unsplit kernel's
 *   bit for bit. The size depends on the current device.
 * - 0 for every other shape (then NULL is allowed).
 * The contents need no initialisation and are overwritten; calls that may
 * overlap in time must not share a workspace. Caller owns all buffers;
 * asynchronous on stream.
 */
size_t blockwise_scaled_mm_e8m0_workspace_size(int64_t M, int64_t N, int64_t K, int bn);
int blockwise_scaled_mm_e8m0(const void* A, const uint8_t* As, const void* W, const uint8_t* Ws,
                             const void* bias, void* D, q8_dtype out_dtype,
                             int64_t M, int64_t N, int64_t K, int bn,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * INT8 W8A8 scaled GEMM.
 * vLLM scaled_mm page, AiterInt8ScaledMMLinearKernel.apply_weights: output =
 * mm(scale_a * a, scale_b * b) with numpy-style broadcasting, weights [N, K],
 * N and K multiples of 16, bias [N] of the output dtype; "Implementation: Sgl
 * project Sglang GEMM Interface", int8_scaled_mm (scales and optional bias).
 *
 * A [M, K] int8, W [N, K] int8. acc[m,n] = sum_k A[m,k] * W[n,k] in int32
 * (exact: |acc| <= 128*128*K < 2^31 for K <= 131071).
 * out_dtype Q8_BF16 / Q8_F16: D = ((float)acc * sa[m or 0]) * sb[n or 0]
 *   (+ (float)bias[n]) in float32 without contraction, then RNE.
 *   sa_numel in {1, M}, sb_numel in {1, N}; all four combinations broadcast.
 * out_dtype Q8_I32: D receives acc itself; sa, sb and bias must be NULL.
 * Rules: N % 16 == 0, K % 16 == 0, K <= 131071, A and W each below 4 GiB.
 */
int scaled_mm_int8(const int8_t* A, const float* sa, int64_t sa_numel,
                   const int8_t* W, const float* sb, int64_t sb_numel,
                   const void* bias, void* D, q8_dtype out_dtype,
                   int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * FP8 e4m3fn scaled GEMM with per-tensor or per-row / per-column scales.
 * "Implementation: Sgl project Sglang GEMM Interface", Description > Scaled
 * Matrix Multiplication (fp8_scaled_mm: per-tensor scales, optional bias,
 * output dtype) and its usage example (scales of shape (1,) or per row of A /
 * per column of B); vLLM scaled_mm page, the per-tensor x per-tensor and
 * per-token x per-channel rule, broadcast here to all four combinations.
 *
 * A [M, K] e4m3fn, W [N, K] e4m3fn (row-major, K contiguous; the pages' (K, N)
 * mat_b is the transposed view of this W). acc[m,n] = sum_k A[m,k] * W[n,k]
 * accumulated in float32 inside the matrix cores (order unspecified).
 * D = ((acc * sa[m or 0]) * sb[n or 0]) (+ (float)bias[n]) in float32 without
 * contraction, then RNE to out_dtype (Q8_BF16 or Q8_F16); bias [N] of the
 * output dtype or NULL. sa_numel in {1, M}, sb_numel in {1, N}.
 * Rules: N % 16 == 0, K % 16 == 0, A and W each below 4 GiB. Caller owns all
 * buffers; asynchronous on stream; errors as for scaled_mm_int8.
 */
int scaled_mm_fp8(const void* A, const float* sa, int64_t sa_numel,
                  const void* W, const float* sb, int64_t sb_numel,
                  const void* bias, void* D, q8_dtype out_dtype,
                  int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * MoE routing tables from the router's top-k expert ids.
 * "Implementation: Sgl project Sglang CUTLASS MoE", Description and I/O
 * Contract (get_cutlass_w4a8_moe_mm_data): expert offsets, per-expert problem
 * sizes, and the input/output permutations around the grouped GEMM.
 *
 * topk_ids [T, topk] int32, values in [0, E) (device precondition).
 * With flat index i = t * topk + j:
 *   expert_offsets [E+1]: exclusive prefix sum of the per-expert counts,
 *                         expert_offsets[E] = T * topk;
 *   problem_sizes1 [E, 3] = (m_e, n, k); problem_sizes2 [E, 3] = (m_e, k, n);
 *   input_permutation  [T*topk]: token row feeding sorted slot p;
 *   output_permutation [T*topk]: sorted slot holding flat choice i.
 * Within one expert, slots follow ascending flat index (stable), so the
 * result is deterministic and unique.
 * Rules: T >= 0, 1 <= topk, 1 <= E <= 1024, T * topk < 2^31.
 * workspace: moe_mm_data_workspace_size() bytes.
 */
size_t moe_mm_data_workspace_size(int64_t T, int topk, int E);
int moe_mm_data(const int32_t* topk_ids, int64_t T, int topk, int E, int64_t n, int64_t k,
                int32_t* expert_offsets, int32_t* problem_sizes1, int32_t* problem_sizes2,
                int32_t* input_permutation, int32_t* output_permutation,
                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_mm_data without a workspace, for callers that cannot allocate device
 * memory around the call: code under HIP graph capture, serving loops that
 * must not allocate per step, harnesses that forbid hipMalloc.
 * Same arguments, tables and errors as moe_mm_data, minus the workspace. The
 * per-chunk expert counts go to a device array inside the library,
 * Q8_MOE_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, reserved when the library is
 * loaded on that GPU and held until the process ends; its address is looked
 * up once per device on the first call (with the stream's device current).
 * The call never allocates or frees. Requests whose counts do not fit
 * (moe_mm_data_workspace_size(T, topk, E) above the limit, e.g. E = 1024 with
 * T * topk above 262144) return Q8_EUNSUPPORTED before any HIP call. Every
 * call on one GPU uses that GPU's one array: calls that overlap in time on one
 * device (several streams or threads) race and must be serialised by the
 * caller; calls in sequence on a stream are fine (each rewrites every count it
 * reads).
 */
#define Q8_MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_mm_data_noalloc(const int32_t* topk_ids, int64_t T, int topk, int E, int64_t n, int64_t k,
                        int32_t* expert_offsets, int32_t* problem_sizes1, int32_t* problem_sizes2,
                        int32_t* input_permutation, int32_t* output_permutation,
                        hipStream_t stream);

/*
 * Expert-grouped block-scaled FP8 GEMM.
 * "Implementation: Sgl project Sglang CUTLASS MoE" (cutlass_w4a8_moe_mm:
 * grouped GEMM over expert segments given by expert_offsets and
 * problem_sizes), here with FP8 weights in [bn, bk] blocks as in
 * blockwise_scaled_mm.
 *
 * For each expert e and sorted slot p in [expert_offsets[e], expert_offsets[e+1]):
 *   row(p) = a_map ? a_map[p] : p            (fused input gather)
 *   Dsorted[p, :] = blockwise(A[row(p)], As[row(p)], W[e], Ws[e])
 * and Dsorted[p] is stored at D row p when c_map is NULL, otherwise at every
 * row i with c_map[i] == p — pass output_permutation to un-permute into the
 * [T*topk, N] order of the flat choices (fused output scatter; c_map must be
 * a permutation of [0, total_m), and the library uses its inverse, so
 * c_map's row count must equal total_m).
 * A [*, K] e4m3fn (rows addressed through a_map), As [*, K/bk] float32,
 * W [E, N, K] e4m3fn, Ws [E, ceil(N/bn), K/bk] float32, D [total_m, N].
 * problem_sizes [E, 3] (m_e, N, K) must agree with expert_offsets (device
 * precondition; the kernels take the row ranges from expert_offsets).
 * Rules as blockwise_scaled_mm; total_m = expert_offsets[E] (host value).
 * workspace: grouped_blockwise_scaled_mm_workspace_size() bytes (the inverse
 * of c_map).
 */
size_t grouped_blockwise_scaled_mm_workspace_size(int E, int64_t total_m, int64_t N, int64_t K,
                                                  int bn, int bk);
int grouped_blockwise_scaled_mm(const void* A, const float* As, const void* W, const float* Ws,
                                void* D, q8_dtype out_dtype,
                                const int32_t* expert_offsets, const int32_t* problem_sizes,
                                const int32_t* a_map, const int32_t* c_map,
                                int E, int64_t total_m, int64_t N, int64_t K, int bn, int bk,
                                void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * MoE finalize: weight every routed row by its top-k gate weight and sum each
 * token's top-k rows.
 * "Implementation: Sgl project Sglang Fused MoE Marlin", I/O Contract:
 * topk_weights (the router's gate weight of each chosen expert), mul_topk_weights
 * (multiply the output by them) and the reduction of the routed outputs
 * (use_atomic_add, use_fp32_reduce). Here the reduction is deterministic.
 *
 * D [T*topk, N] (dtype Q8_BF16 or Q8_F16), out [T, N] of the same dtype,
 * topk_weights [T, topk] float32 or NULL (every weight 1: a plain sum).
 * output_permutation NULL: row (t, j) of D is t*topk + j (un-permuted GEMM
 * output); otherwise D is in expert-sorted order and row (t, j) is
 * output_permutation[t*topk + j] (the table moe_mm_data builds), which fuses
 * the un-permute into this pass.
 * out[t, n] = RNE( sum_{j < topk} w[t, j] * (float)D[row(t, j), n] ), summed
 * in float32 in ascending j with one fused multiply-add per term.
 * Rules: T*topk < 2^31. Rows named by output_permutation must be in D
 * (documented, not checked). Caller owns all buffers; asynchronous on stream.
 */
int moe_finalize(const void* D, q8_dtype dtype, const float* topk_weights,
                 const int32_t* output_permutation, int64_t T, int topk, int64_t N,
                 void* out, hipStream_t stream);

/*
 * Row gather.
 * "Implementation: Sgl project Sglang GEMM Interface", Utility: shuffle_rows
 * (permute rows by a destination-to-source map).
 * dst[i, :] = src[dst2src[i], :] for 0 <= i < dst_rows; rows are row_bytes
 * bytes (any dtype). dst2src values must index valid src rows (device
 * precondition). src and dst must not overlap.
 */
int shuffle_rows(const void* src, int64_t row_bytes, const int32_t* dst2src, int64_t dst_rows,
                 void* dst, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* Q8GEMM_H */
