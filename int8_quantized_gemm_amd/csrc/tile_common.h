// Shared pieces of the LDS-tiled MFMA GEMM kernels (FP8 block-scaled and INT8).
//
// LDS tile layout: a [rows x 128 B] K-slab per stage, one 128-byte line per
// row, split into eight 16-byte chunks. The LDS serves 256 bytes (64 banks of
// 4 bytes) per cycle, so a pair of rows spans the banks once: an even row
// sits in the lower 128 bytes of the bank space and an odd row in the upper.
// Chunk c of row r is stored at chunk position c ^ ((r >> 1) & 7); sixteen
// lanes reading the same logical chunk of sixteen consecutive rows then hit
// sixteen different 16-byte bank groups (conflict-free ds_read_b128, and
// ds_read_b64 of either half), while the row-contiguous global loads stay
// fully coalesced.
#pragma once

#include "q8_device.h"

namespace q8 {

__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int chunk) { return row * 128 + ((chunk ^ swz_key(row)) << 4); }

#define Q8_AS1 __attribute__((address_space(1)))
#define Q8_AS3 __attribute__((address_space(3)))

// Direct global -> LDS loads (no staging registers): lane l of the wave writes
// its 16 (or 4) bytes at lds + 16*l (4*l); lds must be wave-uniform.
__device__ __forceinline__ void g2l16(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((Q8_AS1 void*)g, (Q8_AS3 void*)lds, 16, 0, 0);
}
__device__ __forceinline__ void g2l4(const void* g, void* lds) {
  __builtin_amdgcn_global_load_lds((Q8_AS1 void*)g, (Q8_AS3 void*)lds, 4, 0, 0);
}
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Raw buffer resource over [base, base + bytes) and buffer -> LDS loads:
// a 32-bit per-lane offset (VGPR) plus a wave-uniform offset (SGPR); lane l
// writes lds + 16*l (or 4*l). Out-of-range lanes read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void b2l16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (Q8_AS3 void*)lds, 16, voff, soff, 0, 0);
}
__device__ __forceinline__ void b2l4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (Q8_AS3 void*)lds, 4, voff, soff, 0, 0);
}

// Blocks of a launch are spread round-robin over the 8 XCDs (each with its
// own L2). Renumber them so that consecutive logical tiles land on the same
// XCD: block b runs on XCD b % 8, and logical ids are handed out to XCDs in
// contiguous runs. Bijective on [0, total).
__device__ __forceinline__ int64_t xcd_remap(int64_t b, int64_t total) {
  constexpr int kXcd = 8;
  const int64_t base = total / kXcd, rem = total % kXcd;
  const int64_t x = b % kXcd, i = b / kXcd;
  return x < rem ? x * (base + 1) + i : rem * (base + 1) + (x - rem) * base + i;
}

// Cache-policy operand of the raw buffer load / store builtins: sc1, coherent
// at agent scope (written through past, and read from past, the XCD's L2,
// which is not coherent with the other XCDs' L2s).
constexpr int kSc1 = 16;

// Split tiles of a last round (the tile kernels' SPLIT instances): the owner
// of a tile read its flag word (v0) when it started; after its own K slabs it
// takes the helper's partial only if the word changes to this call's token
// while it waits, at most wait_ticks of the 100 MHz real-time counter (0: it
// never waits). Called by one wave; the result is wave-uniform.
__device__ __forceinline__ bool split_owner_wait(uint32_t* flag, uint32_t token, uint32_t v0,
                                                 uint32_t wait_ticks) {
  if (wait_ticks == 0 || v0 == token) return false;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  for (;;) {
    const uint32_t f = (uint32_t)__builtin_amdgcn_readfirstlane(
        (int)__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    if (f == token) return true;
    if (__builtin_amdgcn_s_memrealtime() - t0 > wait_ticks) return false;
    __builtin_amdgcn_s_sleep(2);
  }
}

// Logical tile id -> (tm, tn), walking GM tile-rows at a time so that the
// tiles resident together share A rows and W rows in L2.
__device__ __forceinline__ void grouped_order(int64_t t, int64_t tiles_m, int64_t tiles_n, int gm,
                                              int64_t& tm, int64_t& tn) {
  const int64_t per_group = (int64_t)gm * tiles_n;
  const int64_t group = t / per_group;
  const int64_t first_m = group * gm;
  const int64_t rows = tiles_m - first_m < gm ? tiles_m - first_m : gm;
  const int64_t r = t - group * per_group;
  tm = first_m + r % rows;
  tn = r / rows;
}

}  // namespace q8
