"""The CPU oracle against its pins: brute force, closed forms, invariants, block-size invariance.

No GPU needed. The pins themselves live in ``oracle_pins.py``.
"""

import numpy as np
import pytest

import oracle
from oracle_pins import ALL_PINS, _close


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_naive_oracle_pin(pin):
    pin(oracle.attention)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_tiled_model_pin(pin):
    """The float64 tiled model meets every pin the naive definition meets."""
    pin(lambda q, k, v, scale, causal=False, kv_len=None:
        oracle.tiled_attention(q, k, v, scale, causal=causal, kv_len=kv_len, block_q=3, block_kv=2))


def _inputs(seed, B, H, N, D, span=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    v = rng.standard_normal((B, H, N, D))
    if span:
        # Rows whose logits span more than 1e6 in magnitude across the tensor
        # (js-flash-attention-tiled-online-softmax-exactness, Verification: span >= 1e6).
        q *= 10.0 ** rng.uniform(-3.0, 3.5, size=(B, H, N, 1))
    return q, k, v


BLOCK_Q = (2, 3, 5, 8, 16, 32, 64)


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_invariance_small(causal):
    """B=2 H=3 N=8 D=16 (vectorized-flash-attention-kernel, Evidence table, multi-head batched):
    every block size from 2 to 64 gives the naive result to 5e-10 (the pages' bound); we ask 1e-12."""
    q, k, v = _inputs(21, 2, 3, 8, 16)
    want = oracle.attention(q, k, v, 0.25, causal=causal)
    for bq in BLOCK_Q:
        for bk in range(2, 65):
            got = oracle.tiled_attention(q, k, v, 0.25, causal=causal, block_q=bq, block_kv=bk)
            _close(got[0], want[0], 1e-12, 1e-12, f"O bq={bq} bk={bk}")
            _close(got[1], want[1], 1e-12, 1e-12, f"LSE bq={bq} bk={bk}")


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_invariance_ragged_padded(causal):
    """Ragged N with per-batch padding, one batch fully masked; every kv block size 2..64."""
    q, k, v = _inputs(22, 3, 2, 67, 8)
    kv = np.array([40, 0, 67])
    scale = float(np.float32(1 / np.sqrt(8)))
    want = oracle.attention(q, k, v, scale, causal=causal, kv_len=kv)
    for bk in range(2, 65):
        for bq in (5, 64):
            got = oracle.tiled_attention(q, k, v, scale, causal=causal, kv_len=kv, block_q=bq, block_kv=bk)
            _close(got[0], want[0], 1e-12, 1e-12, f"O bq={bq} bk={bk}")
            _close(got[1], want[1], 1e-12, 1e-12, f"LSE bq={bq} bk={bk}")
    for bq in BLOCK_Q:
        got = oracle.tiled_attention(q, k, v, scale, causal=causal, kv_len=kv, block_q=bq, block_kv=7)
        _close(got[0], want[0], 1e-12, 1e-12, f"O bq={bq}")


@pytest.mark.parametrize("causal", [False, True])
def test_block_size_invariance_wide_span(causal):
    """Logits spanning more than 1e6: relative error at most 1e-9 (the pages' bound)."""
    q, k, v = _inputs(23, 1, 2, 40, 16, span=True)
    s = np.abs(np.einsum("bhid,bhjd->bhij", q, k) * 0.25)
    assert s.max() / max(s[s > 0].min(), 1e-300) > 1e6
    want = oracle.attention(q, k, v, 0.25, causal=causal)
    for bk in (2, 3, 7, 16, 33, 64):
        for bq in (3, 16):
            got = oracle.tiled_attention(q, k, v, 0.25, causal=causal, block_q=bq, block_kv=bk)
            _close(got[0], want[0], 1e-9, 1e-12, f"O bq={bq} bk={bk}")
            _close(got[1], want[1], 1e-9, 1e-9, f"LSE bq={bq} bk={bk}")


def test_merge_split_and_associativity():
    """Partial states over disjoint key ranges merge into the full state (Paper: FlashAttention,
    Objectives: partial softmax states merge associatively, with an identity element)."""
    q, k, v = _inputs(24, 2, 2, 12, 6)
    full = oracle.attention(q, k, v, 0.3)
    part = [_range_state(q, k, v, 0.3, a, b) for a, b in ((0, 4), (4, 9), (9, 12))]
    ab_c = oracle.merge_states(*oracle.merge_states(*part[0], *part[1]), *part[2])
    a_bc = oracle.merge_states(*part[0], *oracle.merge_states(*part[1], *part[2]))
    for got in (ab_c, a_bc):
        _close(got[0], full[0], 1e-13, 1e-14, "merged O")
        _close(got[1], full[1], 1e-13, 1e-14, "merged LSE")


def _range_state(q, k, v, scale, a, b):
    """State over keys [a, b) for every query row: non-causal attention over that key slice."""
    return oracle.attention(q, _front(k, a, b), _front(v, a, b), scale, kv_len=np.full(q.shape[0], b - a))


def _front(x, a, b):
    """Keys [a, b) moved to the front, followed by the rest (masked by kv_len = b - a)."""
    idx = np.r_[np.arange(a, b), np.arange(0, a), np.arange(b, x.shape[2])]
    return x[:, :, idx]


def test_merge_identity_and_empty():
    q, k, v = _inputs(25, 1, 2, 5, 4)
    o, lse = oracle.attention(q, k, v, 0.5, causal=True)
    zo, zl = np.zeros_like(o), np.full_like(lse, -np.inf)
    for got in (oracle.merge_states(o, lse, zo, zl), oracle.merge_states(zo, zl, o, lse)):
        assert np.array_equal(got[0], o) and np.array_equal(got[1], lse)
    eo, el = oracle.merge_states(zo, zl, zo, zl)
    assert not eo.any() and (el == -np.inf).all()


def test_rows_subset_matches_full():
    """Computing selected query rows gives the same rows as the full computation."""
    q, k, v = _inputs(26, 2, 2, 30, 4)
    kv = np.array([17, 30])
    full = oracle.attention(q, k, v, 0.5, causal=True, kv_len=kv)
    rows = np.array([29, 0, 16, 17, 3])
    sub = oracle.attention(q, k, v, 0.5, causal=True, kv_len=kv, rows=rows, row_chunk=2)
    _close(sub[0], full[0][:, :, rows], 1e-14, 1e-15, "row subset O")
    _close(sub[1], full[1][:, :, rows], 1e-14, 1e-15, "row subset LSE")
    par = oracle.attention(q, k, v, 0.5, causal=True, kv_len=kv, workers=3)
    assert np.array_equal(par[0], full[0]) and np.array_equal(par[1], full[1])
