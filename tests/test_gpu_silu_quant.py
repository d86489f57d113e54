"""GPU parity: fused SiLU-and-mul quantization and masked rows (quant_8bit with
fuse_silu_and_mul / masked_m) against the CPU oracle, bit for bit.

The exhaustive sweep runs every finite bf16 gate value through the library
with group size 1 and clipping range [-1, 1]: the stored scale is then
max(|y|, eps) exactly, so it exposes y = silu(gate) * up itself (the correctly
rounded exp, the division and the product) for all 65280 gate values.
"""
import numpy as np
import pytest
import torch

from gpu_util import DEV, codes, q8, sync
from oracle import quant as oq
import synth

pytestmark = pytest.mark.gpu
EPS = 1e-10


def _qdt(int8):
    return torch.int8 if int8 else torch.float8_e4m3fn


def _run(x_dev, K, g, ue=False, int8=False, qmin=None, qmax=None, masked_m=None, silu=True,
         fill=True):
    lead = x_dev.shape[:-1]
    q = torch.empty(lead + (K,), dtype=_qdt(int8), device=DEV)
    s = torch.empty(lead + (K // g,), dtype=torch.float32, device=DEV)
    if fill:  # sentinels: rows the library must not touch keep them
        q.view(torch.uint8).fill_(0x5A) if not int8 else q.fill_(90)
        s.fill_(-7.0)
    lo = (-128.0 if int8 else -448.0) if qmin is None else qmin
    hi = (127.0 if int8 else 448.0) if qmax is None else qmax
    m = q8()
    m.quant_8bit(x_dev, q, s, g, EPS, lo, hi, ue, fuse_silu_and_mul=silu, masked_m=masked_m)
    sync()
    return codes(q), s.cpu().numpy()


def _oracle(x_cpu, g, ue=False, int8=False, qmin=None, qmax=None, silu=True, masked_m=None,
            max_m=None):
    lo = (-128.0 if int8 else -448.0) if qmin is None else qmin
    hi = (127.0 if int8 else 448.0) if qmax is None else qmax
    x = x_cpu.float().numpy()
    return oq.per_token_group_fused(x.reshape(-1, x.shape[-1]), g, EPS, lo, hi, ue,
                                    "i8" if int8 else "e4m3", silu, masked_m, max_m)


def _all_finite_bf16(n):
    v = (np.arange(65536, dtype=np.uint32) << 16).view(np.float32)
    v = v[np.isfinite(v)]
    out = np.zeros(n, dtype=np.float32)
    out[:v.size] = v
    return torch.from_numpy(out).to(torch.bfloat16)


@pytest.mark.parametrize("up", ["one", "random"])
def test_every_bf16_gate_exactly(up):
    M, K = 256, 256
    gate = _all_finite_bf16(M * K).reshape(M, K)
    if up == "one":
        u = torch.ones(M, K, dtype=torch.bfloat16)
    else:
        # |up| <= 1 keeps every product finite (the largest bf16 gate is 3.4e38)
        u = torch.clamp(synth.activations(M, K, "bf16", sigma=0.5, seed=21), -1.0, 1.0)
    x = torch.cat([gate, u], dim=1)
    qg, sg = _run(x.to(DEV), K, 1, qmin=-1.0, qmax=1.0)
    qo, so, _ = _oracle(x, 1, qmin=-1.0, qmax=1.0)
    bad = sg.view(np.uint32) != so.view(np.uint32)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} scales differ; first gate={float(gate[tuple(i)])} "
                             f"gpu={sg[tuple(i)]!r} oracle={so[tuple(i)]!r}")
    assert np.array_equal(qg, qo)


@pytest.mark.parametrize("up", ["one", "random"])
def test_every_bf16_gate_table_path(up):
    """The bf16 path of large inputs reads h(g) = g / (1 + exp(-g)) from a
    table (and closed forms outside it). Groups of 16 equal elements with
    clipping range [-1, 1] make every stored scale |y| exactly; every finite
    bf16 gate appears in its own group, the sweep repeated four times to
    reach the table path's size (2^22 elements)."""
    K = 1024
    gates = _all_finite_bf16(65536).float().numpy()
    gx = np.repeat(gates, 16).reshape(-1, K)                  # 1024 rows
    if up == "one":
        ux = np.ones_like(gx)
    else:
        r = np.clip(synth.activations(65536, 1, "bf16", sigma=0.5, seed=22).float().numpy()[:, 0],
                    -1.0, 1.0)
        ux = np.repeat(r, 16).reshape(-1, K)
    x = torch.from_numpy(np.concatenate([gx, ux], axis=1)).to(torch.bfloat16).repeat(4, 1)
    assert x.shape[0] * K == 1 << 22
    qg, sg = _run(x.to(DEV), K, 16, qmin=-1.0, qmax=1.0, fill=False)
    qo, so, _ = _oracle(x, 16, qmin=-1.0, qmax=1.0)
    bad = sg.view(np.uint32) != so.view(np.uint32)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{int(bad.sum())} scales differ; first group {tuple(i)}: "
                             f"gpu={sg[tuple(i)]!r} oracle={so[tuple(i)]!r}")
    assert np.array_equal(qg, qo)


def test_masked_rows_table_path():
    """Masked layout large enough for the table path (8 x 1024 rows of 2 x 512)."""
    E, max_m, K, g = 8, 1024, 512, 128
    mm = np.array([0, 1024, 7, 513, 1, 1000, 64, 300], dtype=np.int32)
    x = synth.activations(E * max_m, 2 * K, "bf16", seed=17).reshape(E, max_m, -1)
    qg, sg = _run(x.to(DEV), K, g, masked_m=torch.from_numpy(mm).to(DEV))
    qo, so, valid = _oracle(x, g, masked_m=mm, max_m=max_m)
    qg, sg = qg.reshape(E * max_m, K), sg.reshape(E * max_m, -1)
    assert np.array_equal(qg[valid], qo[valid]) and np.array_equal(sg[valid], so[valid])
    assert np.all(qg[~valid].view(np.uint8) == 0x5A) and np.all(sg[~valid] == -7.0)


@pytest.mark.parametrize("E,max_m", [(300, 16), (1100, 4)])
def test_masked_many_blocks_table_path(E, max_m):
    """Many masked blocks on the table path: more than one 64-count chunk of
    the live-row prefix sum (300 blocks), counts above the block size, zero
    and negative counts, and more blocks than the live-row table holds (1100:
    the kernel that tests every row). Untouched rows keep their bytes."""
    K, g = 1024, 128
    rng = np.random.default_rng(E)
    mm = rng.integers(-3, max_m + 4, size=E).astype(np.int32)
    mm[:4] = [0, max_m, max_m + 5, -1]
    x = synth.activations(E * max_m, 2 * K, "bf16", seed=E).reshape(E, max_m, -1)
    qg, sg = _run(x.to(DEV), K, g, masked_m=torch.from_numpy(mm).to(DEV))
    qo, so, valid = _oracle(x, g, masked_m=np.clip(mm, 0, max_m), max_m=max_m)
    qg, sg = qg.reshape(E * max_m, K), sg.reshape(E * max_m, -1)
    assert np.array_equal(qg[valid], qo[valid]) and np.array_equal(sg[valid], so[valid])
    assert np.all(qg[~valid].view(np.uint8) == 0x5A) and np.all(sg[~valid] == -7.0)


@pytest.mark.parametrize("xdt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("g,ue,int8", [(128, False, False), (32, True, False), (16, False, False),
                                       (512, False, False), (128, False, True), (96, False, False),
                                       (1024, True, False)])
def test_fused_matches_oracle(xdt, g, ue, int8):
    M, K = 67, 1536 if g == 96 else 2048
    x = synth.activations(M, 2 * K, xdt, sigma=3.0, seed=g)
    qg, sg = _run(x.to(DEV), K, g, ue, int8)
    qo, so, _ = _oracle(x, g, ue, int8)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)


def test_fused_strided_rows():
    """The [gate | up] rows are a view into a wider buffer (row stride > 2K)."""
    M, K, g = 40, 1024, 128
    full = synth.activations(M, 2 * K + 64, "bf16", seed=3)
    x = full[:, :2 * K]
    qg, sg = _run(full.to(DEV)[:, :2 * K], K, g)
    qo, so, _ = _oracle(x.contiguous(), g)
    assert np.array_equal(qg, qo) and np.array_equal(sg, so)


@pytest.mark.parametrize("silu", [True, False])
@pytest.mark.parametrize("g", [128, 64, 48])
def test_masked_rows(silu, g):
    E, max_m, K = 5, 24, 768
    mm = np.array([0, 24, 7, 1, 13], dtype=np.int32)
    x = synth.activations(E * max_m, (2 if silu else 1) * K, "bf16", seed=7).reshape(E, max_m, -1)
    qg, sg = _run(x.to(DEV), K, g, masked_m=torch.from_numpy(mm).to(DEV), silu=silu)
    qo, so, valid = _oracle(x, g, silu=silu, masked_m=mm, max_m=max_m)
    qg, sg = qg.reshape(E * max_m, K), sg.reshape(E * max_m, -1)
    assert np.array_equal(qg[valid], qo[valid]) and np.array_equal(sg[valid], so[valid])
    assert np.all(qg[~valid].view(np.uint8) == 0x5A) and np.all(sg[~valid] == -7.0)


def test_masked_count_above_block_acts_as_block():
    E, max_m, K = 3, 8, 256
    mm = np.array([9, 100, 8], dtype=np.int32)  # beyond max_m: every row of the block
    x = synth.activations(E * max_m, 2 * K, "bf16", seed=8).reshape(E, max_m, -1)
    qg, sg = _run(x.to(DEV), K, 128, masked_m=torch.from_numpy(mm).to(DEV))
    qo, so, valid = _oracle(x, 128, masked_m=np.minimum(mm, max_m), max_m=max_m)
    assert valid.all()
    assert np.array_equal(qg.reshape(-1, K), qo) and np.array_equal(sg.reshape(E * max_m, -1), so)


def test_prefill_size_fused():
    """[4096, 2 x 7168] bf16 -> [4096, 7168] codes, group 128 (the size the
    benchmark times), compared with the oracle on every element."""
    M, K = 4096, 7168
    x = synth.activations(M, 2 * K, "bf16", seed=0)
    qg, sg = _run(x.to(DEV), K, 128, fill=False)
    qo, so, _ = _oracle(x, 128)
    assert np.array_equal(sg.view(np.uint32), so.view(np.uint32))
    assert np.array_equal(qg, qo)


def test_fused_empty():
    m = q8()
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q = torch.empty((0, 128), dtype=torch.float8_e4m3fn, device=DEV)
    s = torch.empty((0, 1), dtype=torch.float32, device=DEV)
    m.quant_8bit(x, q, s, 128, EPS, -448.0, 448.0, False, fuse_silu_and_mul=True)
    sync()
