"""One-line mutants of the oracle: each planted mistake must break at least one pin.

The mutants are made on the CPU from the oracle's own source text (a single
substring replaced), so they are plausible slips in the code as written: a
dropped term, a wrong sign or bound, a swapped operand. The tiled-model
mutants include the slips that the exercise on breaking an online-softmax
kernel on purpose asks about ("Paper: FlashAttention", Exercises): the sum or
the accumulator left unrescaled, the causal mask off by one, the guard for an
empty row dropped, the division by the sum done inside the loop, and more.
"""

import inspect
import types

import numpy as np
import pytest

import oracle
import oracle.naive
import oracle.tiled
from oracle_pins import _close, failing_pins


def _mutant(module, old, new):
    src = inspect.getsource(module)
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    mod = types.ModuleType(module.__name__ + "_mutant")
    exec(compile(src.replace(old, new), module.__file__ + ":mutant", "exec"), mod.__dict__)
    return mod


NAIVE_MUTANTS = {
    "causal-drops-diagonal": ("counts = np.minimum(counts, positions + 1)", "counts = np.minimum(counts, positions)"),
    "padding-ignored": ("min(int(kv_len_b), int(n_keys))", "max(int(kv_len_b), int(n_keys))"),
    "scale-dropped": ("s = scale * (q @ k[:kmax].T)", "s = (q @ k[:kmax].T)"),
    "scale-squared": ("s = scale * (q @ k[:kmax].T)", "s = scale * scale * (q @ k[:kmax].T)"),
    "no-max-subtraction": ("m = np.where(has, m, 0.0)", "m = np.where(has, 0.0, 0.0)"),
    "max-over-masked-keys": ("m = np.max(s, axis=1, where=valid, initial=-np.inf)",
                             "m = np.max(s, axis=1, initial=-np.inf)"),
    "masked-keys-weighted": ("w = np.exp(np.where(valid, s - m[:, None], 0.0)) * valid",
                             "w = np.exp(np.where(valid, s - m[:, None], 0.0))"),
    "mask-off-by-one": ("valid = np.arange(kmax)[None, :] < counts[:, None]",
                        "valid = np.arange(kmax)[None, :] <= counts[:, None]"),
    "no-normalisation": ("o[has] = (w[has] @ v[:kmax]) / l[has, None]", "o[has] = (w[has] @ v[:kmax])"),
    "keys-for-values": ("o[has] = (w[has] @ v[:kmax]) / l[has, None]", "o[has] = (w[has] @ k[:kmax]) / l[has, None]"),
    "lse-drops-max": ("lse[has] = m[has] + np.log(l[has])", "lse[has] = np.log(l[has])"),
    "lse-sign": ("lse[has] = m[has] + np.log(l[has])", "lse[has] = m[has] - np.log(l[has])"),
    "empty-row-lse-zero": ("lse = np.full(n_rows, -np.inf)", "lse = np.full(n_rows, 0.0)"),
    "softmax-wrong-axis": ("l = w.sum(axis=1)", "l = w.sum(axis=0)[:n_rows] if w.shape[1] >= n_rows else w.sum(axis=1)"),
}


@pytest.mark.parametrize("name", sorted(NAIVE_MUTANTS))
def test_naive_mutant_is_caught(name):
    mod = _mutant(oracle.naive, *NAIVE_MUTANTS[name])
    assert failing_pins(mod.attention), f"mutant {name} passes every pin"


def test_unmutated_naive_passes_every_pin():
    assert failing_pins(oracle.attention) == []


QUERY_PADDING_MUTANTS = {
    "query-padding-off-by-one": ("counts = np.where(positions < int(q_len_b), counts, 0)",
                                 "counts = np.where(positions <= int(q_len_b), counts, 0)"),
    "query-padding-ignored": ("counts = np.where(positions < int(q_len_b), counts, 0)", "counts = counts"),
    "query-padding-inverted": ("counts = np.where(positions < int(q_len_b), counts, 0)",
                               "counts = np.where(positions < int(q_len_b), 0, counts)"),
}


def test_oracle_query_padding_pin():
    from oracle_pins import pin_query_padding
    pin_query_padding(oracle.attention)


@pytest.mark.parametrize("name", sorted(QUERY_PADDING_MUTANTS))
def test_query_padding_mutant_is_caught(name):
    from oracle_pins import pin_query_padding
    mod = _mutant(oracle.naive, *QUERY_PADDING_MUTANTS[name])
    with pytest.raises(AssertionError):
        with np.errstate(all="ignore"):
            pin_query_padding(mod.attention)


TILED_MUTANTS = {
    "no-rescale-l": ("f1 * l1 + f2 * l2", "l1 + f2 * l2"),
    "no-rescale-acc": ("f1[..., None] * a1 + f2[..., None] * a2", "a1 + f2[..., None] * a2"),
    "causal-mask-drops-diagonal": ("(cols[None, :] <= rows[:, None])", "(cols[None, :] < rows[:, None])"),
    "no-inf-guard": ("m_sub = np.where(m > -np.inf, m, 0.0)", "m_sub = m"),
    "normalise-in-loop": ("            m, l, a = _merge(m, l, a, *_block_state(s, valid, v[:, :, k0:k1]))\n",
                          "            m, l, a = _merge(m, l, a, *_block_state(s, valid, v[:, :, k0:k1]))\n"
                          "            a = a / np.where(l > 0, l, 1.0)[..., None]\n"),
    "skip-diagonal-block": ("if causal and k0 > q1 - 1:", "if causal and k0 >= q1 - 1:"),
    "correction-sign": ("f1 = np.exp(m1 - m_sub)", "f1 = np.exp(m_sub - m1)"),
    "stale-max": ("return m, f1 * l1", "return m1, f1 * l1"),
    "masked-keys-weighted": ("np.where(valid, s - np.where(seen, m, 0.0)[..., None], -np.inf)",
                             "s - np.where(seen, m, 0.0)[..., None]"),
    "padding-ignored": ("valid = cols[None, None, None, :] < L[:, None, None, None]",
                        "valid = cols[None, None, None, :] < N"),
}


def _tiled_vs_naive(tiled):
    """The check a tiled model must pass: naive results at several block sizes, with masked rows."""
    rng = np.random.default_rng(31)
    q = 2.0 * rng.standard_normal((2, 2, 23, 8))
    k = rng.standard_normal((2, 2, 23, 8))
    v = rng.standard_normal((2, 2, 23, 8))
    kv = np.array([0, 19])
    for causal in (False, True):
        want = oracle.attention(q, k, v, 0.35, causal=causal, kv_len=kv)
        for bq, bk in ((3, 5), (8, 8), (16, 7), (23, 2)):
            with np.errstate(all="ignore"):
                got = tiled(q, k, v, 0.35, causal=causal, kv_len=kv, block_q=bq, block_kv=bk)
            _close(got[0], want[0], 1e-12, 1e-12, f"O causal={causal} bq={bq} bk={bk}")
            _close(got[1], want[1], 1e-12, 1e-12, f"LSE causal={causal} bq={bq} bk={bk}")


@pytest.mark.parametrize("name", sorted(TILED_MUTANTS))
def test_tiled_mutant_is_caught(name):
    mod = _mutant(oracle.tiled, *TILED_MUTANTS[name])
    with pytest.raises(AssertionError):
        _tiled_vs_naive(mod.tiled_attention)


def test_unmutated_tiled_passes():
    _tiled_vs_naive(oracle.tiled_attention)
