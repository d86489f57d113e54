"""Helpers shared by the GPU parity tests (import only from tests)."""
import numpy as np
import torch

DEV = "cuda:0"


def q8():
    import int8_quantized_gemm_amd as m
    return m


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def codes(t: torch.Tensor) -> np.ndarray:
    """GPU e4m3/int8 tensor -> numpy uint8/int8 codes."""
    t = t.detach().cpu()
    if t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t.numpy()


def assert_gemm_close(d_gpu: torch.Tensor, d_ref: np.ndarray, what: str = ""):
    """|D - D_ref| <= 1e-2 |D_ref| + 1e-3 rms(D_ref), element by element."""
    d = d_gpu.detach().cpu().double().numpy()
    ref = np.asarray(d_ref, dtype=np.float64)
    assert d.shape == ref.shape, (d.shape, ref.shape)
    assert np.all(np.isfinite(d)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(d - ref)
    bound = 1e-2 * np.abs(ref) + 1e-3 * rms
    bad = err > bound
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; first at {tuple(i)}: "
            f"gpu={d[tuple(i)]!r} ref={ref[tuple(i)]!r} bound={bound[tuple(i)]!r}")


def sync():
    torch.cuda.synchronize()
