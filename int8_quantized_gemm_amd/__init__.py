"""Python binding of libq8gemm (scaled 8-bit GEMM for MI355X / gfx950).

Argument marshalling only: each function checks that torch tensors are on the
GPU and laid out as the C ABI expects (``include/q8gemm.h``), then passes raw
pointers, sizes and the current HIP stream to the library. Every step of the
computation runs in the library's HIP kernels; there is no fallback, and
importing this package fails loudly when ``libq8gemm.so`` is missing (build it
with ``python -m int8_quantized_gemm_amd.build``).

Names and argument orders follow the pages' wrappers: sgl-kernel's
``sgl_per_token_group_quant_8bit``, ``fp8_blockwise_scaled_mm``,
``int8_scaled_mm`` and ``shuffle_rows`` ("Implementation: Sgl project Sglang
GEMM Interface", Signature), and ``get_cutlass_w4a8_moe_mm_data`` /
``cutlass_w4a8_moe_mm`` ("Implementation: Sgl project Sglang CUTLASS MoE",
Signature).
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libq8gemm.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m int8_quantized_gemm_amd.build` "
        "(there is no CPU fallback)")

_lib = ctypes.CDLL(LIB_PATH)

# status codes and enums of include/q8gemm.h
Q8_OK, Q8_EINVAL, Q8_ESHAPE, Q8_EUNSUPPORTED, Q8_EWORKSPACE, Q8_EHIP = 0, -1, -2, -3, -4, -5
Q8_F32, Q8_BF16, Q8_F16, Q8_E4M3FN, Q8_I8, Q8_I32 = 0, 1, 2, 3, 4, 5
SCALE_PER_GROUP, SCALE_PER_TENSOR_DYNAMIC, SCALE_STATIC = 0, 1, 2

EXPORTS = (
    "q8gemm_last_error", "q8gemm_set_split_wait_us",
    "quant_8bit_workspace_size", "quant_8bit",
    "blockwise_scaled_mm_workspace_size", "blockwise_scaled_mm",
    "blockwise_scaled_mm_e8m0_workspace_size", "blockwise_scaled_mm_e8m0",
    "scaled_mm_int8",
    "scaled_mm_fp8",
    "moe_finalize",
    "moe_mm_data_workspace_size", "moe_mm_data", "moe_mm_data_noalloc",
    "grouped_blockwise_scaled_mm_workspace_size", "grouped_blockwise_scaled_mm",
    "shuffle_rows",
)

_p, _i64, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_size_t


def _sig(name, res, *args):
    fn = getattr(_lib, name)
    fn.restype = res
    fn.argtypes = list(args)
    return fn


_lib_last_error = _sig("q8gemm_last_error", ctypes.c_char_p)
_split_wait = _sig("q8gemm_set_split_wait_us", _i, _i)
_quant_ws = _sig("quant_8bit_workspace_size", _sz, _i64, _i64, _i)
_quant = _sig("quant_8bit", _i, _p, _i, _i64, _i64, _i64, _p, _i, _p, _i64, _i, _f, _f, _f, _i, _i,
              _p, _i64, _p, _sz, _p)
_bmm_ws = _sig("blockwise_scaled_mm_workspace_size", _sz, _i64, _i64, _i64, _i, _i)
_bmm = _sig("blockwise_scaled_mm", _i, _p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i, _i, _p,
            _sz, _p)
_bmm8_ws = _sig("blockwise_scaled_mm_e8m0_workspace_size", _sz, _i64, _i64, _i64, _i)
_bmm8 = _sig("blockwise_scaled_mm_e8m0", _i, _p, _p, _p, _p, _p, _p, _i, _i64, _i64, _i64, _i, _p,
             _sz, _p)
_imm = _sig("scaled_mm_int8", _i, _p, _p, _i64, _p, _p, _i64, _p, _p, _i, _i64, _i64, _i64, _p)
_fin = _sig("moe_finalize", _i, _p, _i, _p, _p, _i64, _i, _i64, _p, _p)
_fmm = _sig("scaled_mm_fp8", _i, _p, _p, _i64, _p, _p, _i64, _p, _p, _i, _i64, _i64, _i64, _p)
_moe_ws = _sig("moe_mm_data_workspace_size", _sz, _i64, _i, _i)
_moe = _sig("moe_mm_data", _i, _p, _i64, _i, _i, _i64, _i64, _p, _p, _p, _p, _p, _p, _sz, _p)
_moe_na = _sig("moe_mm_data_noalloc", _i, _p, _i64, _i, _i, _i64, _i64, _p, _p, _p, _p, _p, _p)
_gmm_ws = _sig("grouped_blockwise_scaled_mm_workspace_size", _sz, _i, _i64, _i64, _i64, _i, _i)
_gmm = _sig("grouped_blockwise_scaled_mm", _i, _p, _p, _p, _p, _p, _i, _p, _p, _p, _p, _i, _i64,
            _i64, _i64, _i, _i, _p, _sz, _p)
_shuf = _sig("shuffle_rows", _i, _p, _i64, _p, _i64, _p, _p)


class Q8Error(RuntimeError):
    """A library call returned a non-zero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


def last_error() -> str:
    return _lib_last_error().decode()


def _check(status: int) -> None:
    if status != Q8_OK:
        raise Q8Error(status, last_error())


def set_split_wait_us(microseconds: int) -> None:
    """Longest wait of a split tile's first part for its second part (see
    ``blockwise_scaled_mm``); 0 makes every tile come out as unsplit."""
    _check(_split_wait(int(microseconds)))


_DT = {
    torch.float32: Q8_F32, torch.bfloat16: Q8_BF16, torch.float16: Q8_F16,
    torch.float8_e4m3fn: Q8_E4M3FN, torch.uint8: Q8_E4M3FN, torch.int8: Q8_I8,
    torch.int32: Q8_I32,
}


def _dt(t: torch.dtype) -> int:
    if t not in _DT:
        raise TypeError(f"unsupported dtype {t}")
    return _DT[t]


def _ptr(t: torch.Tensor | None):
    return None if t is None else t.data_ptr()


def _dev(*ts) -> int:
    """Index of the one GPU every given tensor lives on (integer indices: the
    launch path runs once per kernel, and torch.device objects cost time)."""
    dev = -1
    for t in ts:
        if t is None:
            continue
        d = t.get_device()
        if d < 0:
            raise ValueError("every tensor must be on the GPU")
        if dev < 0:
            dev = d
        elif d != dev:
            raise ValueError("tensors on different devices")
    return dev


def _contig(*ts) -> None:
    for t in ts:
        if t is not None and not t.is_contiguous():
            raise ValueError("tensor must be contiguous")


def _need(cond: bool, msg: str) -> None:
    """Host-side argument check: raised before any device work, so a tensor
    too small for what the kernels write or read is never handed to them."""
    if not cond:
        raise ValueError(msg)


_FP8 = (torch.float8_e4m3fn, torch.uint8)
_OUT16 = (torch.bfloat16, torch.float16)
_BYTE_SCALE = tuple(t for t in (torch.uint8, getattr(torch, "float8_e8m0fnu", None)) if t is not None)


def _check_bias(bias, N: int, out_dtype) -> None:
    if bias is not None:
        _need(bias.dtype == out_dtype, f"bias dtype {bias.dtype} must be the output dtype {out_dtype}")
        _need(bias.numel() == N, f"bias must have N = {N} elements (has {bias.numel()})")


def _check_out(out, M: int, N: int, dtypes) -> None:
    _need(tuple(out.shape) == (M, N), f"out must be [{M}, {N}] (is {list(out.shape)})")
    _need(out.dtype in dtypes, f"out dtype {out.dtype} not supported")


def _stream(dev: int) -> int:
    """Raw handle of torch's current stream on device ``dev`` (no Stream object)."""
    return torch._C._cuda_getCurrentRawStream(dev)


_ws_cache: dict = {}


_ws_sizes: dict = {}


def _ws_size(fn, *args) -> int:
    """A workspace-size query of the library, memoised per shape (each query is
    a ctypes call, which costs about a microsecond on the launch path)."""
    key = (fn.__name__, args)
    n = _ws_sizes.get(key)
    if n is None:
        n = fn(*args)
        if len(_ws_sizes) < 4096:
            _ws_sizes[key] = n
    return n


def _workspace(dev, nbytes: int):
    """Device workspace cached per (device, stream); grows, never shrinks."""
    if nbytes == 0:
        return None, 0
    key = (dev, _stream(dev))
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        _ws_cache[key] = buf
    return buf.data_ptr(), buf.numel()


def _workspace_for(dev, nbytes: int, own):
    """(pointer, size, owner): the shared cached workspace; with ``own`` True a
    buffer of its own (the cache may be reallocated by a later, larger call);
    with ``own`` a uint8 device tensor, that tensor (at least ``nbytes``)."""
    if own is False:
        return (*_workspace(dev, nbytes), None)
    if nbytes == 0:
        return None, 0, None
    if own is True:
        own = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _need(own.dtype == torch.uint8 and own.is_contiguous() and own.numel() >= nbytes
          and own.device == torch.device("cuda", dev),
          f"workspace must be a contiguous uint8 tensor of at least {nbytes} bytes on the same device")
    return own.data_ptr(), own.numel(), own


def _bound(fn, args, keep):
    def call():
        _check(fn(*args))
    call.keep = keep
    return call


# ---------------------------------------------------------------------------
def quant_8bit(input: torch.Tensor, output_q: torch.Tensor, output_s: torch.Tensor,
               group_size: int, eps: float = 1e-10, fp8_min: float = -448.0,
               fp8_max: float = 448.0, scale_ue8m0: bool = False, mode: int = SCALE_PER_GROUP,
               fuse_silu_and_mul: bool = False, masked_m: torch.Tensor | None = None) -> None:
    """Per-token-group (or per-tensor) 8-bit quantization, in place.

    ``input`` [M, K] (fp32/bf16/f16, unit column stride), ``output_q`` [M, K]
    float8_e4m3fn/uint8 codes or int8, ``output_s`` [M, K // group_size]
    float32 (``[1]`` for the per-tensor modes; an input for SCALE_STATIC).
    For INT8 pass ``fp8_min=-128, fp8_max=127``. ``scale_ue8m0=2`` stores the
    UE8M0 scales as their E8M0 bytes (``output_s`` uint8).

    ``fuse_silu_and_mul``: ``input`` is [..., 2K] (rows [gate | up]) and the
    codes are of ``silu(gate) * up``. ``masked_m`` (int32 [E]): ``input`` is
    3-D [E, max_m, .] and only the first ``masked_m[e]`` rows of block ``e``
    are quantized; the other rows of the outputs are left as they were.
    """
    max_m = 0
    if masked_m is not None:
        if input.dim() != 3 or masked_m.dtype != torch.int32 or masked_m.numel() != input.shape[0]:
            raise ValueError("masked_m needs a 3-D input [E, max_m, .] and int32 masked_m [E]")
        _contig(masked_m)
        E, max_m = input.shape[0], input.shape[1]
        if input.stride(1) * max_m != input.stride(0) and E > 1:
            raise ValueError("masked input blocks must be evenly strided rows")
        input = input.reshape(E * max_m, input.shape[2]) if input.is_contiguous() else \
            input.as_strided((E * max_m, input.shape[2]), (input.stride(1), input.stride(2)))
        output_q = output_q.reshape(E * max_m, -1)
        output_s = output_s.reshape(E * max_m, -1)
    if input.dim() != 2 or input.stride(1) != 1:
        raise ValueError("input must be 2-D with unit column stride")
    _contig(output_q, output_s)
    M, Kin = input.shape
    K = Kin // 2 if fuse_silu_and_mul else Kin
    if fuse_silu_and_mul and Kin % 2:
        raise ValueError("fuse_silu_and_mul needs an even input width")
    if tuple(output_q.shape) != (M, K):
        raise ValueError("output_q must be [M, K] (K = half the input width when fused)")
    _need(input.dtype in (torch.float32, torch.bfloat16, torch.float16), "input must be fp32, bf16 or f16")
    _need(output_q.dtype in _FP8 + (torch.int8,), "output_q must be float8_e4m3fn, uint8 or int8")
    ue = int(scale_ue8m0)
    if ue == 2:
        _need(output_s.dtype in _BYTE_SCALE, "scale_ue8m0=2 stores one E8M0 byte per scale (uint8)")
    else:
        _need(output_s.dtype == torch.float32, "output_s must be float32")
    if mode == SCALE_PER_GROUP:
        if group_size >= 1 and K % group_size == 0:
            _need(output_s.numel() == M * (K // group_size),
                  f"output_s must hold M * K / group_size = {M * (K // group_size)} scales "
                  f"(has {output_s.numel()})")
    else:
        _need(output_s.numel() == 1, "per-tensor modes take a one-element output_s")
    dev = _dev(input, output_q, output_s, masked_m)
    ws, wsb = _workspace(dev, _ws_size(_quant_ws, M, K, mode))
    _check(_quant(_ptr(input), _dt(input.dtype), M, K, input.stride(0) if M > 1 else Kin,
                  _ptr(output_q), _dt(output_q.dtype), _ptr(output_s), group_size, mode, eps,
                  fp8_min, fp8_max, ue, int(fuse_silu_and_mul), _ptr(masked_m),
                  max_m, ws, wsb, _stream(dev)))


def blockwise_scaled_mm(mat_a: torch.Tensor, mat_b: torch.Tensor, scales_a: torch.Tensor,
                        scales_b: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                        bias: torch.Tensor | None = None, block=(128, 128),
                        out: torch.Tensor | None = None, *, _own_workspace=False) -> torch.Tensor:
    """Block-scaled FP8 GEMM ``D = A @ W.T`` with per-(row, K block) ``scales_a``
    [M, K/bk] and per-(bn x bk tile) ``scales_b`` [ceil(N/bn), K/bk]."""
    _contig(mat_a, mat_b, scales_a, scales_b, bias)
    M, K = mat_a.shape
    N = mat_b.shape[0]
    if mat_b.shape[1] != K:
        raise ValueError("mat_b must be [N, K]")
    bn, bk = block
    _need(mat_a.dtype in _FP8 and mat_b.dtype in _FP8, "mat_a and mat_b must be float8_e4m3fn (or uint8 codes)")
    _need(scales_a.dtype == torch.float32 and scales_b.dtype == torch.float32, "scales must be float32")
    if bk >= 1 and bn >= 1 and K % bk == 0:
        _need(scales_a.numel() == M * (K // bk), f"scales_a must be [M, K/bk] = [{M}, {K // bk}]")
        _need(scales_b.numel() == -(-N // bn) * (K // bk),
              f"scales_b must be [ceil(N/bn), K/bk] = [{-(-N // bn)}, {K // bk}]")
    _check_bias(bias, N, out.dtype if out is not None else out_dtype)
    if out is not None:
        _check_out(out, M, N, _OUT16)
    dev = _dev(mat_a, mat_b, scales_a, scales_b, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _contig(out)
    ws, wsb, keep = _workspace_for(dev, _ws_size(_bmm_ws, M, N, K, bn, bk), _own_workspace)
    args = (_ptr(mat_a), _ptr(scales_a), _ptr(mat_b), _ptr(scales_b), _ptr(bias), _ptr(out),
            _dt(out.dtype), M, N, K, bn, bk, ws, wsb, _stream(dev))
    if _own_workspace is not False:
        return _bound(_bmm, args, (keep, mat_a, mat_b, scales_a, scales_b, bias, out))
    _check(_bmm(*args))
    return out


def blockwise_scaled_mm_e8m0(mat_a: torch.Tensor, mat_b: torch.Tensor, scales_a: torch.Tensor,
                             scales_b: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                             bias: torch.Tensor | None = None, block_n: int = 32,
                             out: torch.Tensor | None = None, *, _own_workspace=False) -> torch.Tensor:
    """Block-scaled FP8 GEMM with E8M0 (power-of-two) scales on both operands:
    ``scales_a`` [M, K/32] and ``scales_b`` [ceil(N/block_n), K/32] as uint8
    (or torch.float8_e8m0fnu) bytes, 32-wide K blocks."""
    _contig(mat_a, mat_b, scales_a, scales_b, bias)
    M, K = mat_a.shape
    N = mat_b.shape[0]
    if mat_b.shape[1] != K:
        raise ValueError("mat_b must be [N, K]")
    for t in (scales_a, scales_b):
        if t.element_size() != 1:
            raise ValueError("E8M0 scales are one byte each")
    _need(mat_a.dtype in _FP8 and mat_b.dtype in _FP8, "mat_a and mat_b must be float8_e4m3fn (or uint8 codes)")
    if K % 32 == 0 and block_n >= 1:
        _need(scales_a.numel() == M * (K // 32), f"scales_a must be [M, K/32] = [{M}, {K // 32}]")
        _need(scales_b.numel() == -(-N // block_n) * (K // 32),
              f"scales_b must be [ceil(N/block_n), K/32] = [{-(-N // block_n)}, {K // 32}]")
    _check_bias(bias, N, out.dtype if out is not None else out_dtype)
    if out is not None:
        _check_out(out, M, N, _OUT16)
    dev = _dev(mat_a, mat_b, scales_a, scales_b, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _contig(out)
    ws, wsb, keep = _workspace_for(dev, _ws_size(_bmm8_ws, M, N, K, block_n), _own_workspace)
    args = (_ptr(mat_a), _ptr(scales_a), _ptr(mat_b), _ptr(scales_b), _ptr(bias), _ptr(out),
            _dt(out.dtype), M, N, K, block_n, ws, wsb, _stream(dev))
    if _own_workspace is not False:
        return _bound(_bmm8, args, (keep, mat_a, mat_b, scales_a, scales_b, bias, out))
    _check(_bmm8(*args))
    return out


def blockwise_scaled_mm_workspace_size(M: int, N: int, K: int, bn: int, bk: int) -> int:
    """Bytes of device workspace ``blockwise_scaled_mm`` takes for these sizes
    on the current device (0: none)."""
    return _ws_size(_bmm_ws, M, N, K, bn, bk)


def blockwise_scaled_mm_e8m0_workspace_size(M: int, N: int, K: int, block_n: int = 32) -> int:
    """Bytes of device workspace ``blockwise_scaled_mm_e8m0`` takes for these
    sizes on the current device (0: none)."""
    return _ws_size(_bmm8_ws, M, N, K, block_n)


def bind_blockwise_scaled_mm(mat_a, mat_b, scales_a, scales_b, out, bias=None, block=(128, 128),
                             workspace=None):
    """Checks and marshals one ``blockwise_scaled_mm`` call once and returns a
    function of no arguments that repeats exactly that C call (same buffers,
    the stream current at bind time): for timing loops, where the per-call
    host-side checks would otherwise be timed with kernels of a few
    microseconds. ``workspace``: a uint8 device tensor of at least
    ``blockwise_scaled_mm_workspace_size`` bytes (calls bound to one tensor
    share it and must run in one stream's order), or None for a buffer of
    the call's own. The returned function keeps the tensors alive; their
    contents may change between calls."""
    return blockwise_scaled_mm(mat_a, mat_b, scales_a, scales_b, out.dtype, bias, block, out,
                               _own_workspace=True if workspace is None else workspace)


def bind_blockwise_scaled_mm_e8m0(mat_a, mat_b, scales_a, scales_b, out, bias=None, block_n=32,
                                  workspace=None):
    """``bind_blockwise_scaled_mm`` for ``blockwise_scaled_mm_e8m0``."""
    return blockwise_scaled_mm_e8m0(mat_a, mat_b, scales_a, scales_b, out.dtype, bias, block_n, out,
                                    _own_workspace=True if workspace is None else workspace)


def scaled_mm_int8(mat_a: torch.Tensor, mat_b: torch.Tensor, scales_a: torch.Tensor | None,
                   scales_b: torch.Tensor | None, out_dtype: torch.dtype = torch.bfloat16,
                   bias: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """INT8 W8A8: ``mat_a`` [M, K] int8; ``mat_b`` [N, K] int8 (or its ``.t()``
    view [K, N]); ``out_dtype=torch.int32`` returns the raw accumulators."""
    _contig(mat_a, scales_a, scales_b, bias)
    _need(mat_a.dtype == torch.int8 and mat_b.dtype == torch.int8, "mat_a and mat_b must be int8")
    for t in (scales_a, scales_b):
        _need(t is None or t.dtype == torch.float32, "scales must be float32")
    M, K = mat_a.shape
    if mat_b.is_contiguous() and mat_b.shape[1] == K:
        N = mat_b.shape[0]
    elif mat_b.shape[0] == K and mat_b.stride() == (1, K):
        N = mat_b.shape[1]  # transposed view of a contiguous [N, K]
    else:
        raise ValueError("mat_b must be [N, K] contiguous or the .t() view of one")
    _check_bias(bias, N, out.dtype if out is not None else out_dtype)
    if out is not None:
        _check_out(out, M, N, _OUT16 + (torch.int32,))
    dev = _dev(mat_a, mat_b, scales_a, scales_b, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _contig(out)
    _check(_imm(_ptr(mat_a), _ptr(scales_a), 0 if scales_a is None else scales_a.numel(),
                _ptr(mat_b), _ptr(scales_b), 0 if scales_b is None else scales_b.numel(),
                _ptr(bias), _ptr(out), _dt(out.dtype), M, N, K, _stream(dev)))
    return out


def scaled_mm_fp8(mat_a: torch.Tensor, mat_b: torch.Tensor, scales_a: torch.Tensor,
                  scales_b: torch.Tensor, out_dtype: torch.dtype = torch.bfloat16,
                  bias: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """FP8 per-tensor / per-token x per-channel: ``mat_a`` [M, K] e4m3fn;
    ``mat_b`` [N, K] e4m3fn (or its ``.t()`` view [K, N]); ``scales_a`` numel 1
    or M, ``scales_b`` numel 1 or N (float32)."""
    _contig(mat_a, scales_a, scales_b, bias)
    _need(mat_a.dtype in _FP8 and mat_b.dtype in _FP8, "mat_a and mat_b must be float8_e4m3fn (or uint8 codes)")
    _need(scales_a.dtype == torch.float32 and scales_b.dtype == torch.float32, "scales must be float32")
    M, K = mat_a.shape
    if mat_b.is_contiguous() and mat_b.shape[1] == K:
        N = mat_b.shape[0]
    elif mat_b.shape[0] == K and mat_b.stride() == (1, K):
        N = mat_b.shape[1]  # transposed view of a contiguous [N, K]
    else:
        raise ValueError("mat_b must be [N, K] contiguous or the .t() view of one")
    _check_bias(bias, N, out.dtype if out is not None else out_dtype)
    if out is not None:
        _check_out(out, M, N, _OUT16)
    dev = _dev(mat_a, mat_b, scales_a, scales_b, bias, out)
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=dev)
    _contig(out)
    _check(_fmm(_ptr(mat_a), _ptr(scales_a), scales_a.numel(), _ptr(mat_b), _ptr(scales_b),
                scales_b.numel(), _ptr(bias), _ptr(out), _dt(out.dtype), M, N, K, _stream(dev)))
    return out


def moe_mm_data(topk_ids: torch.Tensor, expert_offsets: torch.Tensor,
                problem_sizes1: torch.Tensor, problem_sizes2: torch.Tensor,
                input_permutation: torch.Tensor, output_permutation: torch.Tensor,
                num_experts: int, n: int, k: int) -> None:
    """MoE routing tables from ``topk_ids`` [T, topk] int32, in place."""
    _contig(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
            output_permutation)
    for t in (topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
              output_permutation):
        if t.dtype != torch.int32:
            raise TypeError("routing tensors are int32")
    T, topk = topk_ids.shape
    if expert_offsets.numel() < num_experts + 1 or problem_sizes1.numel() < 3 * num_experts \
            or problem_sizes2.numel() < 3 * num_experts \
            or input_permutation.numel() < T * topk or output_permutation.numel() < T * topk:
        raise ValueError("an output tensor is too small")
    dev = _dev(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
               output_permutation)
    ws, wsb = _workspace(dev, _moe_ws(T, topk, num_experts))
    _check(_moe(_ptr(topk_ids), T, topk, num_experts, n, k, _ptr(expert_offsets),
                _ptr(problem_sizes1), _ptr(problem_sizes2), _ptr(input_permutation),
                _ptr(output_permutation), ws, wsb, _stream(dev)))


def moe_mm_data_noalloc(topk_ids: torch.Tensor, expert_offsets: torch.Tensor,
                        problem_sizes1: torch.Tensor, problem_sizes2: torch.Tensor,
                        input_permutation: torch.Tensor, output_permutation: torch.Tensor,
                        num_experts: int, n: int, k: int) -> None:
    """``moe_mm_data`` without a workspace (nothing is allocated: the counts go
    to the library's own per-device scratch array, 4 MiB). For callers that
    cannot allocate, such as code under graph capture; calls overlapping on one
    device race."""
    _contig(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
            output_permutation)
    for t in (topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
              output_permutation):
        if t.dtype != torch.int32:
            raise TypeError("routing tensors are int32")
    T, topk = topk_ids.shape
    if expert_offsets.numel() < num_experts + 1 or problem_sizes1.numel() < 3 * num_experts \
            or problem_sizes2.numel() < 3 * num_experts \
            or input_permutation.numel() < T * topk or output_permutation.numel() < T * topk:
        raise ValueError("an output tensor is too small")
    dev = _dev(topk_ids, expert_offsets, problem_sizes1, problem_sizes2, input_permutation,
               output_permutation)
    _check(_moe_na(_ptr(topk_ids), T, topk, num_experts, n, k, _ptr(expert_offsets),
                   _ptr(problem_sizes1), _ptr(problem_sizes2), _ptr(input_permutation),
                   _ptr(output_permutation), _stream(dev)))


def moe_finalize(d: torch.Tensor, topk_weights: torch.Tensor | None, topk: int,
                 output_permutation: torch.Tensor | None = None,
                 out: torch.Tensor | None = None) -> torch.Tensor:
    """``out[t] = sum_j topk_weights[t, j] * d[row(t, j)]`` -> ``[T, N]``.

    ``d`` [T*topk, N] bf16/f16, un-permuted, or expert-sorted with
    ``output_permutation`` (int32 [T*topk]) naming the row of each choice.
    """
    _contig(d, topk_weights, output_permutation)
    rows, N = d.shape
    if rows % topk:
        raise ValueError("d must have T * topk rows")
    T = rows // topk
    if topk_weights is not None and (topk_weights.dtype != torch.float32 or topk_weights.numel() != rows):
        raise ValueError("topk_weights must be float32 [T, topk]")
    if output_permutation is not None and (output_permutation.dtype != torch.int32
                                           or output_permutation.numel() != rows):
        raise ValueError("output_permutation must be int32 [T * topk]")
    _need(d.dtype in _OUT16, "d must be bf16 or f16")
    if out is not None:
        _check_out(out, T, N, (d.dtype,))
    dev = _dev(d, topk_weights, output_permutation, out)
    if out is None:
        out = torch.empty((T, N), dtype=d.dtype, device=dev)
    _contig(out)
    _check(_fin(_ptr(d), _dt(d.dtype), _ptr(topk_weights), _ptr(output_permutation), T, topk, N,
                _ptr(out), _stream(dev)))
    return out


def grouped_blockwise_scaled_mm(d: torch.Tensor, a: torch.Tensor, b: torch.Tensor,
                                a_scales: torch.Tensor, b_scales: torch.Tensor,
                                expert_offsets: torch.Tensor, problem_sizes: torch.Tensor,
                                a_map: torch.Tensor | None = None,
                                c_map: torch.Tensor | None = None, block=(128, 128)) -> None:
    """Expert-grouped block-FP8 GEMM into ``d`` [total_m, N] (in place).

    ``b`` [E, N, K] e4m3fn, ``b_scales`` [E, ceil(N/bn), K/bk]; ``a``/``a_scales``
    rows are addressed through ``a_map`` (input_permutation) when given;
    ``c_map`` (output_permutation) un-permutes the result rows.
    """
    _contig(d, a, b, a_scales, b_scales, expert_offsets, problem_sizes, a_map, c_map)
    E, N, K = b.shape
    total_m = d.shape[0]
    if d.shape[1] != N or a.shape[1] != K:
        raise ValueError("shape mismatch")
    bn, bk = block
    _need(a.dtype in _FP8 and b.dtype in _FP8, "a and b must be float8_e4m3fn (or uint8 codes)")
    _need(d.dtype in _OUT16, "d must be bf16 or f16")
    _need(a_scales.dtype == torch.float32 and b_scales.dtype == torch.float32, "scales must be float32")
    for t, name in ((expert_offsets, "expert_offsets"), (problem_sizes, "problem_sizes"),
                    (a_map, "a_map"), (c_map, "c_map")):
        _need(t is None or t.dtype == torch.int32, f"{name} must be int32")
    _need(expert_offsets.numel() == E + 1, f"expert_offsets must have E + 1 = {E + 1} entries")
    _need(problem_sizes.numel() == 3 * E, f"problem_sizes must be [E, 3] = [{E}, 3]")
    if bk >= 1 and K % bk == 0 and bn >= 1:
        _need(a_scales.dim() == 2 and tuple(a_scales.shape) == (a.shape[0], K // bk),
              f"a_scales must be [rows of a, K/bk] = [{a.shape[0]}, {K // bk}]")
        _need(b_scales.numel() == E * -(-N // bn) * (K // bk),
              f"b_scales must be [E, ceil(N/bn), K/bk] = [{E}, {-(-N // bn)}, {K // bk}]")
    if a_map is not None:
        _need(a_map.numel() == total_m, f"a_map must have total_m = {total_m} entries")
    else:
        _need(a.shape[0] >= total_m, "without a_map, a must hold total_m sorted rows")
    if c_map is not None:
        _need(c_map.numel() == total_m, f"c_map must have total_m = {total_m} entries")
    dev = _dev(d, a, b, a_scales, b_scales, expert_offsets, problem_sizes, a_map, c_map)
    ws, wsb = _workspace(dev, _gmm_ws(E, total_m, N, K, bn, bk) if c_map is not None else 0)
    _check(_gmm(_ptr(a), _ptr(a_scales), _ptr(b), _ptr(b_scales), _ptr(d), _dt(d.dtype),
                _ptr(expert_offsets), _ptr(problem_sizes), _ptr(a_map), _ptr(c_map), E, total_m,
                N, K, bn, bk, ws, wsb, _stream(dev)))


def shuffle_rows(input_tensor: torch.Tensor, dst2src_map: torch.Tensor,
                 output_tensor_shape) -> torch.Tensor:
    """``out[i] = input_tensor[dst2src_map[i]]`` for a row-major tensor."""
    dev = _dev(input_tensor, dst2src_map)
    _contig(input_tensor, dst2src_map)
    out = torch.empty(output_tensor_shape, dtype=input_tensor.dtype, device=dev)
    rows = dst2src_map.numel()
    row_bytes = input_tensor[0].numel() * input_tensor.element_size() if input_tensor.shape[0] else 0
    if out.numel() * out.element_size() != rows * row_bytes:
        raise ValueError("output shape does not match the map")
    _check(_shuf(_ptr(input_tensor), row_bytes, _ptr(dst2src_map), rows, _ptr(out), _stream(dev)))
    return out
