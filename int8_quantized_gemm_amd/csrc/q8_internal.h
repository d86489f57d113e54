// Internal declarations shared by the C-ABI front end (capi.cpp) and the
// kernel translation units. Launchers assume their arguments were validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/q8gemm.h"

namespace q8 {

// ---- quantization -----------------------------------------------------------
struct QuantArgs {
  const void* x; q8_dtype x_dtype; int64_t M, K, ld_x;
  void* q; q8_dtype q_dtype; float* s; int64_t group_size;
  q8_scale_mode mode; float eps, qmin, qmax; int ue8m0;
  void* workspace;
  int silu;                  // x rows are [gate | up], 2K wide
  const int32_t* masked_m;   // [M / max_m] valid rows per block, or null
  int64_t max_m;
};
size_t quant_partials_count(int64_t M, int64_t K);
hipError_t launch_quant(const QuantArgs& a, hipStream_t stream);

// ---- block-scaled FP8 GEMM --------------------------------------------------
struct BlockGemmArgs {
  const uint8_t* A; const float* As; const uint8_t* W; const float* Ws;
  const void* bias; void* D; q8_dtype out_dtype;
  int64_t M, N, K; int bn, bk;
  // grouped / MoE extensions (null for the dense call)
  const int32_t* expert_offsets;  // [E+1]
  const int32_t* a_map;           // sorted slot -> A row
  const int32_t* c_inv;           // sorted slot -> D row
  int E;
  int64_t w_expert_stride;        // bytes between experts in W
  int64_t ws_expert_stride;       // floats between experts in Ws
  void* workspace;                // split-K partials (dense call), or null
  size_t workspace_bytes;
};
// workspace bytes the dense call needs for this shape (0: none)
size_t blockwise_workspace_bytes(int64_t M, int64_t N, int64_t K, int bn, int bk);
// workspace bytes with which the dense call splits the tiles of a last,
// part-filled round of workgroups on the current device (0: no split); optional
size_t blockwise_split_bytes(int64_t M, int64_t N, int64_t K, int bn, int bk);
// longest wait of a split tile's owner for its helper (100 MHz ticks; 0: none)
void set_split_wait_ticks(uint32_t ticks);
uint32_t split_wait_ticks();
// odd, new for every call
uint32_t next_split_token();
// compute units of the current device (0 without one), cached per device
int device_cus();
// Split of the last round of 256 x 256 tiles (both block-scaled tile
// kernels): the R = tiles mod C tiles of a last round that fills at most half
// of the C compute units are each split in K between an owner (slabs
// [0, k)), and a helper (the rest).
struct SplitPlan {
  int64_t first, lead, tiles;
  int k;
};
bool split_plan(int64_t tiles, int KT, int cus, SplitPlan& sp);
size_t split_part_bytes(int64_t R);  // float32 partials of R tiles
size_t split_bytes(int64_t R);       // the partials and R flag words
hipError_t launch_blockwise(const BlockGemmArgs& a, hipStream_t stream);
hipError_t launch_grouped(const BlockGemmArgs& a, int64_t total_m, int32_t* c_inv_ws,
                          const int32_t* c_map, hipStream_t stream);

// ---- block-scaled FP8 GEMM, E8M0 scales (MX-scaled MFMA) ---------------------
struct MxGemmArgs {
  const uint8_t* A; const uint8_t* As; const uint8_t* W; const uint8_t* Ws;
  const void* bias; void* D; q8_dtype out_dtype;
  int64_t M, N, K; int bn;
  void* workspace;  // split-K partials (17..64 rows), or null
  size_t workspace_bytes;
};
// workspace bytes the E8M0 call needs for this shape (0: none)
size_t blockwise_e8m0_workspace_bytes(int64_t M, int64_t N, int64_t K);
// workspace bytes with which the E8M0 call splits a last, half-empty round of
// tiles on the current device (0: no split); optional
size_t blockwise_e8m0_split_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_blockwise_e8m0(const MxGemmArgs& a, hipStream_t stream);

// ---- INT8 GEMM ----------------------------------------------------------------
struct ScaledGemmArgs {
  const void* A; const float* sa; int64_t sa_numel;
  const void* W; const float* sb; int64_t sb_numel;
  const void* bias; void* D; q8_dtype out_dtype;
  int64_t M, N, K;
  bool fp8;  // e4m3fn operands (else int8)
};
hipError_t launch_scaled(const ScaledGemmArgs& a, hipStream_t stream);

// ---- MoE routing + row gather -------------------------------------------------
size_t moe_workspace_ints(int64_t T, int topk, int E);
hipError_t launch_moe_mm_data(const int32_t* topk_ids, int64_t T, int topk, int E,
                              int64_t n, int64_t k, int32_t* offsets, int32_t* ps1,
                              int32_t* ps2, int32_t* in_perm, int32_t* out_perm,
                              int32_t* ws, hipStream_t stream);
// allocation-free variant: the counts live in a file-scope device array of
// kNoAllocInts ints per device (the front end rejects larger requests)
constexpr int64_t kNoAllocInts = 1 << 20;
hipError_t launch_moe_mm_data_noalloc(const int32_t* topk_ids, int64_t T, int topk, int E,
                                      int64_t n, int64_t k, int32_t* offsets, int32_t* ps1,
                                      int32_t* ps2, int32_t* in_perm, int32_t* out_perm,
                                      hipStream_t stream);
hipError_t launch_moe_finalize(const void* D, bool bf16, const float* w, const int32_t* perm,
                               int64_t T, int topk, int64_t N, void* out, hipStream_t stream);
hipError_t launch_shuffle_rows(const void* src, int64_t row_bytes, const int32_t* dst2src,
                               int64_t dst_rows, void* dst, hipStream_t stream);

}  // namespace q8
