"""CPU oracle for the scaled 8-bit GEMM hot path — TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct numpy implementations of what the GPU library
computes, written from the pages' descriptions of each operation:

* ``e4m3``  — the OCP float8 e4m3fn code (torch ``float8_e4m3fn``, named in
  the block32 DeepGEMM PR review) decoded exactly and encoded with
  round-to-nearest-even;
* ``quant`` — per-token-group 8-bit activation quantization
  ("Implementation: Sgl project Sglang GEMM Interface", Description ›
  Quantization Routines: sgl_per_token_group_quant_8bit, per-tensor and
  per-token variants);
* ``gemm``  — the block-scaled FP8 matmul (the block32 DeepGEMM PR,
  "Modifications": fp8_gemm_nt with recipe (1, 32, 32)) and the INT8 W8A8
  scaled matmul (vLLM scaled_mm API page, AiterInt8ScaledMMLinearKernel
  apply_weights);
* ``moe``   — MoE routing tables and the expert-grouped GEMM
  ("Implementation: Sgl project Sglang CUTLASS MoE", Description).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The GPU library shares no code with it, and nothing here
ever consumes a value produced by the GPU library.

Floating point: quantization runs in float32, the precision of the scales the
pages store (fp32 ``[M, K/g]`` group scales), so both sides take every
rounding decision in the same precision. Matmuls decode codes exactly and
accumulate in float64 (exact for the per-block partial sums, see ``gemm``).
"""
from . import e4m3, quant, gemm, moe  # noqa: F401
