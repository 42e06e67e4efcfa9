"""Pins for attention gradients with the signature
``grad(q, k, v, do, scale, causal=False, kv_len=None) -> (dq, dk, dv)`` (float64).

None of them re-runs the gradient formula under test. They compare against:
central finite differences of the pinned forward oracle (``oracle.attention``),
float64 autograd of an independently written masked-softmax attention in torch,
and invariants that the mathematics fixes (shift invariance of the softmax,
the weights of each row summing to one, the q/k rescaling symmetry), plus the
exactly known special cases (one key, no key, padding keys).
"""

import numpy as np
import torch

import oracle
from oracle_pins import _close


def _inputs(seed, B, H, N, D, Dv=None, scale_q=1.0):
    rng = np.random.default_rng(seed)
    Dv = D if Dv is None else Dv
    q = scale_q * rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    v = rng.standard_normal((B, H, N, Dv))
    do = rng.standard_normal((B, H, N, Dv))
    return q, k, v, do


def _loss(q, k, v, do, scale, causal, kv_len, q_len=None):
    o, _ = oracle.attention(q, k, v, scale, causal=causal, kv_len=kv_len, q_len=q_len)
    return float((o * do).sum())


def finite_difference(q, k, v, do, scale, causal, kv_len, h=1e-6, q_len=None):
    """Central differences of sum(dO o O) through the forward oracle, one element at a time."""
    grads = []
    args = [q.copy(), k.copy(), v.copy()]
    for t in range(3):
        g = np.zeros_like(args[t])
        for idx in np.ndindex(*args[t].shape):
            keep = args[t][idx]
            args[t][idx] = keep + h
            up = _loss(*args, do, scale, causal, kv_len, q_len)
            args[t][idx] = keep - h
            dn = _loss(*args, do, scale, causal, kv_len, q_len)
            args[t][idx] = keep
            g[idx] = (up - dn) / (2 * h)
        grads.append(g)
    return grads


def pin_grad_finite_difference(grad):
    """Every element of dQ, dK, dV against central differences of the forward: every causal
    flag, padding that cuts the keys, a fully padded batch, Dv != D, B and H above one."""
    q, k, v, do = _inputs(41, 2, 2, 4, 3, Dv=2)
    for causal in (False, True):
        for kv in (None, np.array([2, 4]), np.array([0, 3])):
            want = finite_difference(q, k, v, do, 0.7, causal, kv)
            got = grad(q, k, v, do, 0.7, causal=causal, kv_len=kv)
            for name, a, b in zip(("dQ", "dK", "dV"), got, want):
                _close(a, b, 1e-7, 1e-8, f"finite difference {name} causal={causal} kv={kv}")


def torch_autograd(q, k, v, do, scale, causal, kv_len):
    """float64 autograd of a plainly written masked-softmax attention (torch, CPU)."""
    B, H, N, D = q.shape
    qt, kt, vt = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    keys = torch.arange(N)
    L = torch.full((B,), N) if kv_len is None else torch.as_tensor(np.asarray(kv_len), dtype=torch.int64)
    valid = (keys[None, None, :] < L[:, None, None]).expand(B, N, N)
    if causal:
        valid = valid & (keys[None, :] <= keys[:, None])[None]
    valid = valid[:, None]                        # [B, 1, N, N]
    has = valid.any(dim=-1, keepdim=True)         # rows with at least one key
    s = scale * torch.matmul(qt, kt.transpose(-1, -2))
    s = torch.where(valid, s, torch.tensor(float("-inf"), dtype=torch.float64))
    s = torch.where(has, s, torch.zeros((), dtype=torch.float64))   # empty rows: finite, weight 0 below
    p = torch.softmax(s, dim=-1) * has
    o = torch.matmul(p, vt)
    (o * torch.tensor(do)).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


def pin_grad_torch_autograd(grad):
    q, k, v, do = _inputs(42, 2, 3, 9, 5, Dv=4)
    for causal in (False, True):
        for kv in (None, np.array([6, 0])):
            for scale in (0.45, -0.45, 0.0):   # the scale carries no sign restriction
                want = torch_autograd(q, k, v, do, scale, causal, kv)
                got = grad(q, k, v, do, scale, causal=causal, kv_len=kv)
                for name, a, b in zip(("dQ", "dK", "dV"), got, want):
                    _close(a, b, 1e-11, 1e-12, f"autograd {name} causal={causal} kv={kv} scale={scale}")


def pin_grad_invariants(grad):
    """Per (b, h): sum_j dK_j = 0 (adding one vector to every key shifts each row's logits by a
    constant); sum_j dV_j = sum of dO over rows with a key (each row's weights sum to one);
    sum_i <q_i, dQ_i> = sum_j <k_j, dK_j> (scaling q by t and k by 1/t changes nothing)."""
    q, k, v, do = _inputs(43, 2, 2, 40, 8, scale_q=2.0)
    for causal in (False, True):
        for kv in (None, np.array([17, 40])):
            dq, dk, dv = grad(q, k, v, do, 0.5, causal=causal, kv_len=kv)
            L = np.full(2, 40) if kv is None else kv
            for b in range(2):
                rows_with_key = np.full(40, L[b] > 0)     # with a key, row i always sees key 0
                for h in range(2):
                    tag = f"causal={causal} kv={kv} b={b} h={h}"
                    _close(dk[b, h].sum(axis=0), np.zeros(8), 0, 1e-11, "sum dK " + tag)
                    _close(dv[b, h].sum(axis=0), do[b, h][rows_with_key].sum(axis=0), 0, 1e-11, "sum dV " + tag)
                    lhs = (q[b, h] * dq[b, h]).sum()
                    rhs = (k[b, h] * dk[b, h]).sum()
                    _close(lhs, rhs, 0, 1e-10, "q.dQ = k.dK " + tag)
                    assert (dk[b, h, L[b]:] == 0).all() and (dv[b, h, L[b]:] == 0).all(), "padding keys " + tag


def pin_grad_special_cases(grad):
    """One key: O = v_0 whatever q and k are, so dQ = dK = 0 (to rounding: a recomputing backward
    forms dP - rowsum(dO o O) from two differently rounded products) and dV = dO. No valid key
    (kv_len 0): every gradient is 0. Causal: row 0 sees only key 0, so dQ_0 = 0."""
    q, k, v, do = _inputs(44, 1, 2, 1, 4)
    for causal in (False, True):
        dq, dk, dv = grad(q, k, v, do, 0.9, causal=causal, kv_len=None)
        _close(dq, np.zeros_like(dq), 0, 1e-14, "single key dQ")
        _close(dk, np.zeros_like(dk), 0, 1e-14, "single key dK")
        _close(dv, do, 0, 0, "single key dV")
    q, k, v, do = _inputs(45, 2, 1, 6, 3)
    for causal in (False, True):
        dq, dk, dv = grad(q, k, v, do, 0.9, causal=causal, kv_len=np.array([0, 6]))
        assert (dq[0] == 0).all() and (dk[0] == 0).all() and (dv[0] == 0).all(), "kv_len 0"
        assert np.abs(dq[1]).max() > 0
    dq, dk, dv = grad(q, k, v, do, 0.9, causal=True, kv_len=None)
    _close(dq[:, :, 0], np.zeros_like(dq[:, :, 0]), 0, 1e-14, "causal row 0")


ALL_GRAD_PINS = [pin_grad_finite_difference, pin_grad_torch_autograd, pin_grad_invariants, pin_grad_special_cases]


def pin_grad_query_padding(grad):
    """Query padding (q_len): every element of dQ, dK, dV against central differences of the
    pinned forward with the same q_len (its padding rows are the constant 0, so their dO drops
    out); NaN in the padding rows of Q and dO changes nothing, and their dQ rows are exactly 0."""
    q, k, v, do = _inputs(46, 2, 2, 4, 3, Dv=2)
    for causal in (False, True):
        for kv in (None, np.array([3, 4])):
            for ql in (np.array([2, 4]), np.array([0, 3])):
                want = finite_difference(q, k, v, do, 0.7, causal, kv, q_len=ql)
                got = grad(q, k, v, do, 0.7, causal=causal, kv_len=kv, q_len=ql)
                tag = f"causal={causal} kv={kv} q_len={ql}"
                for name, a, b in zip(("dQ", "dK", "dV"), got, want):
                    _close(a, b, 1e-7, 1e-8, f"finite difference {name} " + tag)
                qn, don = q.copy(), do.copy()
                for b in range(2):
                    qn[b, :, ql[b]:] = np.nan
                    don[b, :, ql[b]:] = np.nan
                got_nan = grad(qn, k, v, don, 0.7, causal=causal, kv_len=kv, q_len=ql)
                for name, a, b in zip(("dQ", "dK", "dV"), got_nan, got):
                    assert np.array_equal(a, b), f"NaN padding rows change {name} " + tag
                for b in range(2):
                    assert (got_nan[0][b, :, ql[b]:] == 0).all(), "padding dQ rows " + tag


def failing_grad_pins(grad):
    """Names of the pins that the implementation breaks (AssertionError or an exception)."""
    bad = []
    for pin in ALL_GRAD_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(grad)
        except Exception:
            bad.append(pin.__name__)
    return bad
