"""The gradient oracle against its pins, the tiled recomputing backward against the
definition at every block size, and one-line mutants of both. CPU only."""

import numpy as np
import pytest

import oracle
import oracle.backward
from oracle_grad_pins import ALL_GRAD_PINS, failing_grad_pins
from oracle_pins import _close
from test_oracle_mutants import _mutant


def _tiled_grad(block_q, block_kv, module=oracle.backward):
    def grad(q, k, v, do, scale, causal=False, kv_len=None):
        o, lse = oracle.attention(q, k, v, scale, causal=causal, kv_len=kv_len)
        return module.tiled_backward(q, k, v, o, lse, do, scale, causal=causal, kv_len=kv_len,
                                     block_q=block_q, block_kv=block_kv)
    return grad


@pytest.mark.parametrize("pin", ALL_GRAD_PINS, ids=lambda p: p.__name__)
def test_grad_oracle_pin(pin):
    pin(oracle.attention_grad)


@pytest.mark.parametrize("pin", ALL_GRAD_PINS, ids=lambda p: p.__name__)
def test_tiled_backward_pin(pin):
    pin(_tiled_grad(3, 2))


def _inputs(seed, B, H, N, D, span=False):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    if span:
        q *= 10.0 ** rng.uniform(-2.0, 1.5, size=(B, H, N, 1))
    return q, k, v, do


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_backward_block_size_invariance(causal):
    """Ragged N, per-batch padding with a fully padded batch, logits of widely varying size:
    the recomputing backward equals the definition at every block shape to 1e-12."""
    q, k, v, do = _inputs(51, 3, 2, 37, 8, span=True)
    kv = np.array([23, 0, 37])
    scale = float(np.float32(1 / np.sqrt(8)))
    want = oracle.attention_grad(q, k, v, do, scale, causal=causal, kv_len=kv)
    o, lse = oracle.attention(q, k, v, scale, causal=causal, kv_len=kv)
    for bq in (1, 2, 5, 16, 37, 64):
        for bk in (1, 3, 8, 13, 64):
            got = oracle.tiled_backward(q, k, v, o, lse, do, scale, causal=causal, kv_len=kv, block_q=bq, block_kv=bk)
            for name, a, b in zip(("dQ", "dK", "dV"), got, want):
                scale_ref = np.abs(b).max()
                _close(a, b, 1e-12, 1e-12 * scale_ref, f"{name} bq={bq} bk={bk}")


def test_rowsum_identity():
    """rowsum(dP o P) = rowsum(dO o O) for every row ("Paper: FlashAttention", Objectives, Math &
    data structures), with P from the definition and O from the forward oracle."""
    q, k, v, do = _inputs(52, 1, 2, 30, 6)
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, 0.4, causal=causal)
        for h in range(2):
            s = 0.4 * q[0, h] @ k[0, h].T
            if causal:
                s = np.where(np.tril(np.ones((30, 30), bool)), s, -np.inf)
            p = np.exp(s - s.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do[0, h] @ v[0, h].T
            _close((dp * p).sum(axis=1), (do[0, h] * o[0, h]).sum(axis=1), 1e-12, 1e-12, f"identity h={h}")


def test_grad_rows_subset():
    q, k, v, do = _inputs(53, 2, 2, 50, 8)
    kv = np.array([31, 50])
    rows = np.array([0, 7, 30, 31, 49])
    for causal in (False, True):
        full = oracle.attention_grad(q, k, v, do, 0.3, causal=causal, kv_len=kv)[0]
        part = oracle.attention_grad_rows(q, k, v, do, 0.3, rows, causal=causal, kv_len=kv)
        _close(part, full[:, :, rows], 1e-13, 1e-14, f"rows causal={causal}")


GRAD_MUTANTS = {
    "drop-delta": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))", "ds = p * dp"),
    "delta-wrong-axis": ("ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))",
                         "ds = p * (dp - (p * dp).sum(axis=0, keepdims=True))"),
    "dk-unscaled": ("dk = scale * (ds.T @ q)", "dk = ds.T @ q"),
    "dq-from-q": ("dq = scale * (ds @ k)", "dq = scale * (ds @ q)"),
    "dk-untransposed": ("dk = scale * (ds.T @ q)", "dk = scale * (ds @ q)"),
    "dv-untransposed": ("dv = p.T @ do", "dv = p @ do"),
    "dp-from-k": ("dp = do @ v.T", "dp = do @ k[:, :do.shape[1]].T if k.shape[1] >= do.shape[1] else do @ v.T"),
    "mask-dropped": ("w = np.exp(np.where(valid, s - m[:, None], 0.0)) * valid",
                     "w = np.exp(np.where(valid, s - m[:, None], 0.0))"),
    "causal-off-by-one": ("valid &= keys[None, :] <= pos[:, None]", "valid &= keys[None, :] < pos[:, None]"),
    "unnormalised-p": ("p = w / np.where(has, l, 1.0)[:, None]", "p = w"),
}


def test_grad_oracle_query_padding_pin():
    from oracle_grad_pins import pin_grad_query_padding
    pin_grad_query_padding(oracle.attention_grad)


GRAD_QUERY_PADDING_MUTANTS = {
    "padding-dO-kept": ("    q = _drop_padding_queries(q, q_len)\n    do = _drop_padding_queries(do, q_len)\n    dq = np.zeros_like(q)",
                        "    q = _drop_padding_queries(q, q_len)\n    dq = np.zeros_like(q)"),
    "padding-q-kept": ("    q = _drop_padding_queries(q, q_len)\n    do = _drop_padding_queries(do, q_len)\n    dq = np.zeros_like(q)",
                       "    do = _drop_padding_queries(do, q_len)\n    dq = np.zeros_like(q)"),
    "padding-off-by-one": ("        x[b, :, pos >= int(q_len[b])] = 0.0", "        x[b, :, pos > int(q_len[b])] = 0.0"),
    "padding-rows-not-zeroed": ("        x[b, :, pos >= int(q_len[b])] = 0.0", "        pass"),
}


@pytest.mark.parametrize("name", sorted(GRAD_QUERY_PADDING_MUTANTS))
def test_grad_query_padding_mutant_is_caught(name):
    from oracle_grad_pins import pin_grad_query_padding
    mod = _mutant(oracle.backward, *GRAD_QUERY_PADDING_MUTANTS[name])
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pin_grad_query_padding(mod.attention_grad)


@pytest.mark.parametrize("name", sorted(GRAD_MUTANTS))
def test_grad_mutant_is_caught(name):
    mod = _mutant(oracle.backward, *GRAD_MUTANTS[name])
    assert failing_grad_pins(mod.attention_grad), f"mutant {name} passes every pin"


def test_unmutated_grad_passes_every_pin():
    assert failing_grad_pins(oracle.attention_grad) == []


TILED_GRAD_MUTANTS = {
    "delta-from-do-only": ("delta = (do * o).sum(axis=-1)", "delta = do.sum(axis=-1)"),
    "no-lse-subtraction": ("s - np.where(live_row, lse_b, 0.0)", "s"),
    "masked-keys-weighted": ("p = np.where(dead | ~live_row, 0.0,", "p = np.where(~live_row, 0.0,"),
    "causal-skip-too-early": ("if causal and q1 - 1 < k0:", "if causal and q1 - 1 <= k0:"),
    "dq-missing-scale": ("dq[:, :, q0:q1] += scale * np.matmul(ds, k[:, :, k0:k1])",
                         "dq[:, :, q0:q1] += np.matmul(ds, k[:, :, k0:k1])"),
    "ds-sign": ("ds = p * (dp - delta[:, :, q0:q1, None])", "ds = p * (delta[:, :, q0:q1, None] - dp)"),
    "padding-ignored": ("dead = cols[None, None, None, :] >= L[:, None, None, None]",
                        "dead = cols[None, None, None, :] >= N"),
}


@pytest.mark.parametrize("name", sorted(TILED_GRAD_MUTANTS))
def test_tiled_grad_mutant_is_caught(name):
    mod = _mutant(oracle.backward, *TILED_GRAD_MUTANTS[name])
    assert failing_grad_pins(_tiled_grad(3, 2, module=mod)), f"mutant {name} passes every pin"
