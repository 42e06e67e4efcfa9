"""The seeded input generator: deterministic, and shaped as its recipe says."""

import numpy as np
import torch

from exact_tiled_attention_23_amd.workloads import WORKLOADS, HEADLINE, generate, softmax_scale


def test_deterministic_and_dtype():
    a = generate(2, 3, 17, 64, "bf16", causal=True, seed=7)
    b = generate(2, 3, 17, 64, "bf16", causal=True, seed=7)
    c = generate(2, 3, 17, 64, "bf16", causal=True, seed=8)
    for x, y in ((a.q, b.q), (a.k, b.k), (a.v, b.v)):
        assert x.dtype == torch.bfloat16 and x.shape == (2, 3, 17, 64) and torch.equal(x, y)
    assert not torch.equal(a.q, c.q)
    assert a.kv_len is None and a.scale == float(np.float32(1 / 8))


def test_padding_and_row_scale():
    x = generate(8, 2, 100, 64, "f16", causal=True, seed=5, padding=True, q_row_scale=True)
    assert x.kv_len.dtype == np.int32 and x.kv_len.shape == (8,)
    assert (x.kv_len >= 0).all() and (x.kv_len <= 100).all()
    assert x.kv_len[x.meta["zero_batch"]] == 0
    # |Q| reaches far beyond a standard normal draw once rows are scaled by factors up to 100.
    assert x.q.abs().max().item() > 50


def test_scale_is_float32_exact():
    for D in (64, 128):
        s = softmax_scale(D)
        assert float(np.float32(s)) == s and abs(s - 1 / np.sqrt(D)) < 1e-8


def test_named_workloads():
    assert HEADLINE in WORKLOADS
    shapes = {(w.B, w.H, w.N, w.D, w.dtype, w.causal) for w in WORKLOADS.values()}
    assert (2, 32, 8192, 128, "bf16", False) in shapes
    assert len(WORKLOADS) == 5
