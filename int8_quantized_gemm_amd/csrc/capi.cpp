// C-ABI front end: argument validation (host only, before any HIP call),
// thread-local error messages, and dispatch to the kernel launchers.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "q8_internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return Q8_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(Q8_EHIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool is_16bit_out(q8_dtype t) { return t == Q8_BF16 || t == Q8_F16; }

constexpr int64_t kMaxI32 = 0x7FFFFFFFLL;
constexpr int64_t kFourGiB = 0x100000000LL;

// Shared validation of the block-scaled FP8 GEMM shape rules.
int check_block_shape(const char* fn, int64_t M, int64_t N, int64_t K, int bn, int bk) {
  if (M < 0 || N < 1 || K < 1) return fail(Q8_ESHAPE, "%s: need M >= 0, N >= 1, K >= 1", fn);
  if (bk != 32 && bk != 128) return fail(Q8_EUNSUPPORTED, "%s: bk must be 32 or 128 (got %d)", fn, bk);
  if (bn < 16 || bn % 16 != 0)
    return fail(Q8_EUNSUPPORTED, "%s: bn must be a positive multiple of 16 (got %d)", fn, bn);
  if (K % bk != 0) return fail(Q8_ESHAPE, "%s: K (%lld) must be a multiple of bk (%d)", fn, (long long)K, bk);
  if (K / bk > kMaxI32 || (N + bn - 1) / bn > kMaxI32)
    return fail(Q8_ESHAPE, "%s: too many blocks", fn);
  // the kernels address every operand with 32-bit byte offsets
  if (M * K >= kFourGiB || N * K >= kFourGiB || M * (K / bk) * 4 >= kFourGiB)
    return fail(Q8_EUNSUPPORTED, "%s: an operand (A, W or As) reaches 4 GiB", fn);
  return Q8_OK;
}

}  // namespace

extern "C" {

const char* q8gemm_last_error(void) { return g_last_error.c_str(); }

int q8gemm_set_split_wait_us(int microseconds) {
  if (microseconds < 0 || microseconds > 100000)
    return fail(Q8_EINVAL, "q8gemm_set_split_wait_us: %d outside [0, 100000]", microseconds);
  q8::set_split_wait_ticks((uint32_t)microseconds * 100u);
  return ok();
}

size_t quant_8bit_workspace_size(int64_t M, int64_t K, q8_scale_mode mode) {
  if (mode != Q8_SCALE_PER_TENSOR_DYNAMIC) return 0;
  return q8::quant_partials_count(M, K) * sizeof(float);
}

int quant_8bit(const void* x, q8_dtype x_dtype, int64_t M, int64_t K, int64_t ld_x, void* q,
               q8_dtype q_dtype, float* s, int64_t group_size, q8_scale_mode mode, float eps,
               float qmin, float qmax, int scale_ue8m0, int fuse_silu_and_mul,
               const int32_t* masked_m, int64_t max_m, void* workspace, size_t workspace_bytes,
               hipStream_t stream) {
  static const char* fn = "quant_8bit";
  if (fuse_silu_and_mul != 0 && fuse_silu_and_mul != 1)
    return fail(Q8_EINVAL, "%s: fuse_silu_and_mul must be 0 or 1", fn);
  if ((fuse_silu_and_mul || masked_m) && mode != Q8_SCALE_PER_GROUP)
    return fail(Q8_EUNSUPPORTED, "%s: fuse_silu_and_mul and masked_m need per-group scales", fn);
  if (x_dtype != Q8_F32 && x_dtype != Q8_BF16 && x_dtype != Q8_F16)
    return fail(Q8_EINVAL, "%s: x_dtype must be F32, BF16 or F16", fn);
  if (q_dtype != Q8_E4M3FN && q_dtype != Q8_I8)
    return fail(Q8_EINVAL, "%s: q_dtype must be E4M3FN or I8", fn);
  if (mode != Q8_SCALE_PER_GROUP && mode != Q8_SCALE_PER_TENSOR_DYNAMIC && mode != Q8_SCALE_STATIC)
    return fail(Q8_EINVAL, "%s: unknown scale mode %d", fn, (int)mode);
  if (M < 0 || K < 0) return fail(Q8_ESHAPE, "%s: negative size", fn);
  if (ld_x < (fuse_silu_and_mul ? 2 * K : K))
    return fail(Q8_ESHAPE, "%s: ld_x (%lld) < input row width (%lld)", fn, (long long)ld_x,
                (long long)(fuse_silu_and_mul ? 2 * K : K));
  if (masked_m) {
    if (max_m < 1 || M % max_m != 0)
      return fail(Q8_ESHAPE, "%s: masked_m needs max_m >= 1 dividing M (M=%lld, max_m=%lld)", fn,
                  (long long)M, (long long)max_m);
    if (max_m > 0x7FFFFFFFLL || M > 0xFFFFFFFFLL)
      return fail(Q8_ESHAPE, "%s: masked rows are indexed in 32 bits", fn);
  }
  if (!(qmax > 0.0f) || !(qmin < 0.0f))
    return fail(Q8_EINVAL, "%s: need qmin < 0 < qmax", fn);
  if (q_dtype == Q8_E4M3FN && (qmax > 448.0f || qmin < -448.0f))
    return fail(Q8_EINVAL, "%s: FP8 clip range must lie within [-448, 448]", fn);
  if (q_dtype == Q8_I8 && (qmax > 127.0f || qmin < -128.0f))
    return fail(Q8_EINVAL, "%s: INT8 clip range must lie within [-128, 127]", fn);
  if (mode != Q8_SCALE_STATIC && !(eps > 0.0f)) return fail(Q8_EINVAL, "%s: eps must be > 0", fn);
  if (scale_ue8m0 < 0 || scale_ue8m0 > 2)
    return fail(Q8_EINVAL, "%s: scale_ue8m0 must be 0, 1 or 2", fn);
  if (mode == Q8_SCALE_STATIC && scale_ue8m0)
    return fail(Q8_EINVAL, "%s: scale_ue8m0 applies to computed scales, not a static scale", fn);
  if (mode == Q8_SCALE_PER_GROUP) {
    if (group_size < 1) return fail(Q8_ESHAPE, "%s: group_size must be >= 1", fn);
    if (K % group_size != 0)
      return fail(Q8_ESHAPE, "%s: group_size (%lld) must divide K (%lld)", fn, (long long)group_size,
                  (long long)K);
  }
  if (M == 0 || K == 0) return ok();
  if (!x || !q || !s) return fail(Q8_EINVAL, "%s: null pointer", fn);
  const size_t need = quant_8bit_workspace_size(M, K, mode);
  if (need && (!workspace || workspace_bytes < need))
    return fail(Q8_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  q8::QuantArgs a{x, x_dtype, M, K, ld_x, q, q_dtype, s, group_size, mode, eps, qmin, qmax,
                  scale_ue8m0, workspace, fuse_silu_and_mul, masked_m, masked_m ? max_m : 0};
  return hip_status(q8::launch_quant(a, stream), fn);
}

size_t blockwise_scaled_mm_workspace_size(int64_t M, int64_t N, int64_t K, int bn, int bk) {
  if (M < 0 || N < 1 || K < 1 || (bk != 32 && bk != 128) || bn < 16 || bn % 16 != 0 || K % bk != 0)
    return 0;
  return q8::blockwise_workspace_bytes(M, N, K, bn, bk) + q8::blockwise_split_bytes(M, N, K, bn, bk);
}

int blockwise_scaled_mm(const void* A, const float* As, const void* W, const float* Ws,
                        const void* bias, void* D, q8_dtype out_dtype, int64_t M, int64_t N,
                        int64_t K, int bn, int bk, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  static const char* fn = "blockwise_scaled_mm";
  if (!is_16bit_out(out_dtype)) return fail(Q8_EINVAL, "%s: out_dtype must be BF16 or F16", fn);
  int r = check_block_shape(fn, M, N, K, bn, bk);
  if (r != Q8_OK) return r;
  if (M == 0) return ok();
  if (!A || !As || !W || !Ws || !D) return fail(Q8_EINVAL, "%s: null pointer", fn);
  // the decode split needs its workspace; the split of a last round of tiles
  // (M > 64) uses one when it is given and large enough
  const size_t need = q8::blockwise_workspace_bytes(M, N, K, bn, bk);
  const size_t want = need ? 0 : q8::blockwise_split_bytes(M, N, K, bn, bk);
  if (need && (!workspace || workspace_bytes < need))
    return fail(Q8_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const bool use_ws = need || (want && workspace && workspace_bytes >= want);
  if (use_ws && (uintptr_t)workspace % 16 != 0)
    return fail(Q8_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  q8::BlockGemmArgs a{};
  a.A = static_cast<const uint8_t*>(A); a.As = As;
  a.W = static_cast<const uint8_t*>(W); a.Ws = Ws;
  a.bias = bias; a.D = D; a.out_dtype = out_dtype;
  a.M = M; a.N = N; a.K = K; a.bn = bn; a.bk = bk;
  a.workspace = use_ws ? workspace : nullptr;
  a.workspace_bytes = use_ws ? workspace_bytes : 0;
  return hip_status(q8::launch_blockwise(a, stream), fn);
}

size_t blockwise_scaled_mm_e8m0_workspace_size(int64_t M, int64_t N, int64_t K, int bn) {
  if (M < 0 || N < 1 || K < 1 || bn < 16 || bn % 16 != 0 || K % 128 != 0) return 0;
  return q8::blockwise_e8m0_workspace_bytes(M, N, K) + q8::blockwise_e8m0_split_bytes(M, N, K);
}

int blockwise_scaled_mm_e8m0(const void* A, const uint8_t* As, const void* W, const uint8_t* Ws,
                             const void* bias, void* D, q8_dtype out_dtype, int64_t M, int64_t N,
                             int64_t K, int bn, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  static const char* fn = "blockwise_scaled_mm_e8m0";
  if (!is_16bit_out(out_dtype)) return fail(Q8_EINVAL, "%s: out_dtype must be BF16 or F16", fn);
  if (M < 0 || N < 1 || K < 1) return fail(Q8_ESHAPE, "%s: need M >= 0, N >= 1, K >= 1", fn);
  if (bn < 16 || bn % 16 != 0)
    return fail(Q8_EUNSUPPORTED, "%s: bn must be a positive multiple of 16 (got %d)", fn, bn);
  if (K % 128 != 0)
    return fail(Q8_ESHAPE, "%s: K (%lld) must be a multiple of 128", fn, (long long)K);
  if (M * K >= (int64_t)1 << 32 || N * K >= (int64_t)1 << 32)
    return fail(Q8_EUNSUPPORTED, "%s: A and W must each be below 4 GiB", fn);
  if (M == 0) return ok();
  if (!A || !As || !W || !Ws || !D) return fail(Q8_EINVAL, "%s: null pointer", fn);
  if ((uintptr_t)As % 4 != 0 || (uintptr_t)Ws % 4 != 0)
    return fail(Q8_EINVAL, "%s: As and Ws must be 4-byte aligned", fn);
  // the decode split needs its workspace; the split of a last round of tiles
  // (M > 64) uses one when it is given and large enough
  const size_t need = q8::blockwise_e8m0_workspace_bytes(M, N, K);
  const size_t want = need ? 0 : q8::blockwise_e8m0_split_bytes(M, N, K);
  if (need && (!workspace || workspace_bytes < need))
    return fail(Q8_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  const bool use_ws = need || (want && workspace && workspace_bytes >= want);
  if (use_ws && (uintptr_t)workspace % 16 != 0)
    return fail(Q8_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  q8::MxGemmArgs a{static_cast<const uint8_t*>(A), As, static_cast<const uint8_t*>(W), Ws,
                   bias, D, out_dtype, M, N, K, bn, use_ws ? workspace : nullptr,
                   use_ws ? workspace_bytes : 0};
  return hip_status(q8::launch_blockwise_e8m0(a, stream), fn);
}

int scaled_mm_int8(const int8_t* A, const float* sa, int64_t sa_numel, const int8_t* W,
                   const float* sb, int64_t sb_numel, const void* bias, void* D,
                   q8_dtype out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  static const char* fn = "scaled_mm_int8";
  if (out_dtype != Q8_BF16 && out_dtype != Q8_F16 && out_dtype != Q8_I32)
    return fail(Q8_EINVAL, "%s: out_dtype must be BF16, F16 or I32", fn);
  if (M < 0 || N < 1 || K < 1) return fail(Q8_ESHAPE, "%s: need M >= 0, N >= 1, K >= 1", fn);
  if (N % 16 != 0 || K % 16 != 0)
    return fail(Q8_ESHAPE, "%s: N (%lld) and K (%lld) must be multiples of 16", fn, (long long)N,
                (long long)K);
  if (K > 131071) return fail(Q8_ESHAPE, "%s: K above 131071 could overflow int32", fn);
  if (M * K >= kFourGiB || N * K >= kFourGiB)
    return fail(Q8_EUNSUPPORTED, "%s: an operand (A or W) reaches 4 GiB", fn);
  if (out_dtype == Q8_I32) {
    if (sa || sb || bias) return fail(Q8_EINVAL, "%s: I32 output takes no scales and no bias", fn);
  } else {
    if (!sa || !sb) return fail(Q8_EINVAL, "%s: null scale pointer", fn);
    if (!(sa_numel == 1 || sa_numel == M))
      return fail(Q8_EUNSUPPORTED, "%s: scales_a numel %lld is neither 1 nor M", fn, (long long)sa_numel);
    if (!(sb_numel == 1 || sb_numel == N))
      return fail(Q8_EUNSUPPORTED, "%s: scales_b numel %lld is neither 1 nor N", fn, (long long)sb_numel);
  }
  if (M == 0) return ok();
  if (!A || !W || !D) return fail(Q8_EINVAL, "%s: null pointer", fn);
  q8::ScaledGemmArgs a{A, sa, sa_numel, W, sb, sb_numel, bias, D, out_dtype, M, N, K, false};
  return hip_status(q8::launch_scaled(a, stream), fn);
}

int scaled_mm_fp8(const void* A, const float* sa, int64_t sa_numel, const void* W,
                  const float* sb, int64_t sb_numel, const void* bias, void* D,
                  q8_dtype out_dtype, int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  static const char* fn = "scaled_mm_fp8";
  if (out_dtype != Q8_BF16 && out_dtype != Q8_F16)
    return fail(Q8_EINVAL, "%s: out_dtype must be BF16 or F16", fn);
  if (M < 0 || N < 1 || K < 1) return fail(Q8_ESHAPE, "%s: need M >= 0, N >= 1, K >= 1", fn);
  if (N % 16 != 0 || K % 16 != 0)
    return fail(Q8_ESHAPE, "%s: N (%lld) and K (%lld) must be multiples of 16", fn, (long long)N,
                (long long)K);
  if (M * K >= kFourGiB || N * K >= kFourGiB)
    return fail(Q8_EUNSUPPORTED, "%s: an operand (A or W) reaches 4 GiB", fn);
  if (!sa || !sb) return fail(Q8_EINVAL, "%s: null scale pointer", fn);
  if (!(sa_numel == 1 || sa_numel == M))
    return fail(Q8_EUNSUPPORTED, "%s: scales_a numel %lld is neither 1 nor M", fn, (long long)sa_numel);
  if (!(sb_numel == 1 || sb_numel == N))
    return fail(Q8_EUNSUPPORTED, "%s: scales_b numel %lld is neither 1 nor N", fn, (long long)sb_numel);
  if (M == 0) return ok();
  if (!A || !W || !D) return fail(Q8_EINVAL, "%s: null pointer", fn);
  q8::ScaledGemmArgs a{A, sa, sa_numel, W, sb, sb_numel, bias, D, out_dtype, M, N, K, true};
  return hip_status(q8::launch_scaled(a, stream), fn);
}

size_t moe_mm_data_workspace_size(int64_t T, int topk, int E) {
  if (T < 0 || topk < 1 || E < 1) return 0;
  return q8::moe_workspace_ints(T, topk, E) * sizeof(int32_t);
}

}  // extern "C"

namespace {
// Shared argument rules of moe_mm_data and moe_mm_data_noalloc.
int check_moe_args(const char* fn, const int32_t* topk_ids, int64_t T, int topk, int E, int64_t n,
                   int64_t k, const int32_t* expert_offsets, const int32_t* problem_sizes1,
                   const int32_t* problem_sizes2, const int32_t* input_permutation,
                   const int32_t* output_permutation) {
  if (T < 0 || topk < 1) return fail(Q8_ESHAPE, "%s: need T >= 0 and topk >= 1", fn);
  if (E < 1 || E > 1024) return fail(Q8_EUNSUPPORTED, "%s: E must be in [1, 1024]", fn);
  if (T * (int64_t)topk >= kMaxI32) return fail(Q8_ESHAPE, "%s: T * topk must be below 2^31", fn);
  if (n < 0 || k < 0 || n > kMaxI32 || k > kMaxI32) return fail(Q8_ESHAPE, "%s: n, k out of int32 range", fn);
  if (!expert_offsets || !problem_sizes1 || !problem_sizes2)
    return fail(Q8_EINVAL, "%s: null pointer", fn);
  if (T > 0 && (!topk_ids || !input_permutation || !output_permutation))
    return fail(Q8_EINVAL, "%s: null pointer", fn);
  return Q8_OK;
}
}  // namespace

extern "C" {

int moe_mm_data(const int32_t* topk_ids, int64_t T, int topk, int E, int64_t n, int64_t k,
                int32_t* expert_offsets, int32_t* problem_sizes1, int32_t* problem_sizes2,
                int32_t* input_permutation, int32_t* output_permutation, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "moe_mm_data";
  const int r = check_moe_args(fn, topk_ids, T, topk, E, n, k, expert_offsets, problem_sizes1,
                               problem_sizes2, input_permutation, output_permutation);
  if (r != Q8_OK) return r;
  const size_t need = moe_mm_data_workspace_size(T, topk, E);
  if (need && (!workspace || workspace_bytes < need))
    return fail(Q8_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  return hip_status(q8::launch_moe_mm_data(topk_ids, T, topk, E, n, k, expert_offsets,
                                           problem_sizes1, problem_sizes2, input_permutation,
                                           output_permutation, static_cast<int32_t*>(workspace),
                                           stream),
                    fn);
}

int moe_mm_data_noalloc(const int32_t* topk_ids, int64_t T, int topk, int E, int64_t n,
                        int64_t k, int32_t* expert_offsets, int32_t* problem_sizes1,
                        int32_t* problem_sizes2, int32_t* input_permutation,
                        int32_t* output_permutation, hipStream_t stream) {
  static const char* fn = "moe_mm_data_noalloc";
  const int r = check_moe_args(fn, topk_ids, T, topk, E, n, k, expert_offsets, problem_sizes1,
                               problem_sizes2, input_permutation, output_permutation);
  if (r != Q8_OK) return r;
  const size_t need = moe_mm_data_workspace_size(T, topk, E);
  if (need > (size_t)Q8_MOE_NOALLOC_SCRATCH_BYTES)
    return fail(Q8_EUNSUPPORTED,
                "%s: these routing tables need %zu bytes of scratch, above the %u bytes the "
                "allocation-free entry point holds per device (call moe_mm_data with a workspace)",
                fn, need, (unsigned)Q8_MOE_NOALLOC_SCRATCH_BYTES);
  static_assert((size_t)Q8_MOE_NOALLOC_SCRATCH_BYTES == q8::kNoAllocInts * sizeof(int32_t),
                "header limit and device array agree");
  return hip_status(q8::launch_moe_mm_data_noalloc(topk_ids, T, topk, E, n, k, expert_offsets,
                                                   problem_sizes1, problem_sizes2,
                                                   input_permutation, output_permutation, stream),
                    fn);
}

size_t grouped_blockwise_scaled_mm_workspace_size(int E, int64_t total_m, int64_t, int64_t, int,
                                                  int) {
  (void)E;
  if (total_m < 0) return 0;
  return (size_t)total_m * sizeof(int32_t);
}

int grouped_blockwise_scaled_mm(const void* A, const float* As, const void* W, const float* Ws,
                                void* D, q8_dtype out_dtype, const int32_t* expert_offsets,
                                const int32_t* problem_sizes, const int32_t* a_map,
                                const int32_t* c_map, int E, int64_t total_m, int64_t N,
                                int64_t K, int bn, int bk, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  static const char* fn = "grouped_blockwise_scaled_mm";
  (void)problem_sizes;
  if (!is_16bit_out(out_dtype)) return fail(Q8_EINVAL, "%s: out_dtype must be BF16 or F16", fn);
  if (E < 1 || E > 65536) return fail(Q8_EUNSUPPORTED, "%s: E must be in [1, 65536]", fn);
  if (total_m < 0 || total_m >= kMaxI32) return fail(Q8_ESHAPE, "%s: total_m out of range", fn);
  int r = check_block_shape(fn, total_m, N, K, bn, bk);
  if (r != Q8_OK) return r;
  if (!expert_offsets) return fail(Q8_EINVAL, "%s: null expert_offsets", fn);
  if (total_m == 0) return ok();
  if (!A || !As || !W || !Ws || !D) return fail(Q8_EINVAL, "%s: null pointer", fn);
  const size_t need = c_map ? grouped_blockwise_scaled_mm_workspace_size(E, total_m, N, K, bn, bk) : 0;
  if (need && (!workspace || workspace_bytes < need))
    return fail(Q8_EWORKSPACE, "%s: workspace needs %zu bytes", fn, need);
  q8::BlockGemmArgs a{};
  a.A = static_cast<const uint8_t*>(A); a.As = As;
  a.W = static_cast<const uint8_t*>(W); a.Ws = Ws;
  a.bias = nullptr; a.D = D; a.out_dtype = out_dtype;
  a.M = total_m; a.N = N; a.K = K; a.bn = bn; a.bk = bk;
  a.expert_offsets = expert_offsets; a.a_map = a_map; a.c_inv = nullptr; a.E = E;
  return hip_status(q8::launch_grouped(a, total_m, static_cast<int32_t*>(workspace), c_map, stream), fn);
}

int moe_finalize(const void* D, q8_dtype dtype, const float* topk_weights,
                 const int32_t* output_permutation, int64_t T, int topk, int64_t N, void* out,
                 hipStream_t stream) {
  static const char* fn = "moe_finalize";
  if (dtype != Q8_BF16 && dtype != Q8_F16) return fail(Q8_EINVAL, "%s: dtype must be BF16 or F16", fn);
  if (T < 0 || topk < 1 || N < 0) return fail(Q8_ESHAPE, "%s: need T >= 0, topk >= 1, N >= 0", fn);
  if (T * (int64_t)topk >= kMaxI32) return fail(Q8_ESHAPE, "%s: T * topk must be below 2^31", fn);
  if (T == 0 || N == 0) return ok();
  if (!D || !out) return fail(Q8_EINVAL, "%s: null pointer", fn);
  return hip_status(q8::launch_moe_finalize(D, dtype == Q8_BF16, topk_weights, output_permutation,
                                            T, topk, N, out, stream), fn);
}

int shuffle_rows(const void* src, int64_t row_bytes, const int32_t* dst2src, int64_t dst_rows,
                 void* dst, hipStream_t stream) {
  static const char* fn = "shuffle_rows";
  if (row_bytes < 0 || dst_rows < 0) return fail(Q8_ESHAPE, "%s: negative size", fn);
  if (row_bytes == 0 || dst_rows == 0) return ok();
  if (!src || !dst2src || !dst) return fail(Q8_EINVAL, "%s: null pointer", fn);
  return hip_status(q8::launch_shuffle_rows(src, row_bytes, dst2src, dst_rows, dst, stream), fn);
}

}  // extern "C"
