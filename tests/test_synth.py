"""The seeded generators are deterministic and give the documented shapes."""
import numpy as np
import torch

import synth


def test_activations_deterministic_and_outliers():
    a = synth.activations(8, 256, "bf16", outlier_frac=0.01, seed=0)
    b = synth.activations(8, 256, "bf16", outlier_frac=0.01, seed=0)
    assert a.dtype == torch.bfloat16 and torch.equal(a, b)
    c = synth.activations(8, 256, "bf16", seed=1)
    assert not torch.equal(a, c)
    big = synth.activations(64, 7168, "f32", outlier_frac=0.01, seed=0)
    frac = (big.abs() > 6).float().mean().item()
    assert 0.003 < frac < 0.02


def test_block_weights_shapes_and_range():
    wq, ws = synth.fp8_block_weights(100, 256, 32, 128, seed=0)
    assert wq.shape == (100, 256) and wq.dtype == torch.uint8
    assert ws.shape == (4, 2) and ws.dtype == torch.float32
    v = wq.view(torch.float8_e4m3fn).float()
    assert torch.isfinite(v).all() and v.abs().max() <= 448
    # every tile reaches the top of the code range (its amax maps to 448)
    for nb in range(4):
        for kb in range(2):
            t = v[nb * 32:(nb + 1) * 32, kb * 128:(kb + 1) * 128]
            assert t.abs().max() == 448
    w2, s2 = synth.fp8_block_weights(100, 256, 32, 128, seed=0)
    assert torch.equal(wq, w2) and torch.equal(ws, s2)
    we, se = synth.fp8_block_weights(64, 128, 32, 32, experts=3, seed=0)
    assert we.shape == (3, 64, 128) and se.shape == (3, 2, 4)


def test_int8_weights():
    q, s = synth.int8_weights(32, 64, per_channel=True)
    assert q.dtype == torch.int8 and s.shape == (32,)
    assert (q.abs().max(dim=1).values == 127).all()
    q1, s1 = synth.int8_weights(32, 64, per_channel=False)
    assert s1.shape == (1,) and q1.abs().max() == 127
