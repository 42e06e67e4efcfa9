"""Elementwise rounding bound for the attention gradients of the bf16/f16 backward.

Derived from the arithmetic (the forward's bound is stated for outputs of unit scale;
gradients vary in scale from one position to the next, most of all under the causal mask).
The kernels round P and dS to the working type before the products that take them, use the
forward's O, itself rounded, in Delta = rowsum(dO o O), accumulate in float32 and round the
results once. With unit roundoff u (2^-8 bf16, 2^-11 f16), a (the f16 subnormal spacing's half,
2^-25; 0 for bf16) and gamma = D 2^-24 for a float32 dot product of length D, the first-order
error of each result is at most, elementwise, with P, dS, O from the definition:

    e_i   = u sum_d |dO_id||O_id| + gamma sum_d |dO_id| (|O_id| + max_j |v_jd|)   (Delta, dP)
    T(dV) = (u P + a)^T |dO|
    T(dQ) = |scale| (u |dS| + a + P e) |K|
    T(dK) = |scale| (u |dS| + a + P e)^T |Q|

and a result passes when |gpu - ref| <= 2 T + u |ref| + 1e-6 (the last term: output rounding
and exact zeros). On CPU emulations of these rounding points the error stays under 0.6 of this
bound, while dropping Delta from dS exceeds it 1.4x to 580x.

Test infrastructure: used by the GPU tests and the smoke check, never by the product path.
"""

import numpy as np
import torch


UNIT = {"bf16": (2.0 ** -8, 0.0), "f16": (2.0 ** -11, 2.0 ** -25)}
DTYPE_NAME = {torch.bfloat16: "bf16", torch.float16: "f16"}


def rounding_bound(q, k, v, do, scale, causal, kv_len, dtype, rows=None):
    """T(dQ), T(dK), T(dV) of the module docstring (float64 inputs [B, H, N, D]); with `rows`,
    only T(dQ) for those query positions (T(dK) and T(dV) need every row)."""
    u, a = UNIT[dtype]
    B, H, N, D = q.shape
    gamma = D * 2.0 ** -24
    pos = np.arange(N) if rows is None else np.asarray(rows)
    tq = np.zeros((B, H, pos.size, D))
    tk = np.zeros_like(k) if rows is None else None
    tv = np.zeros_like(v) if rows is None else None
    for b in range(B):
        L = N if kv_len is None else int(kv_len[b])
        valid = np.broadcast_to(np.arange(N)[None, :] < L, (pos.size, N)).copy()
        if causal:
            valid &= np.arange(N)[None, :] <= pos[:, None]
        has = valid.any(axis=1)
        for h in range(H):
            kk, vv = k[b, h], v[b, h]
            s = scale * (q[b, h, pos] @ kk.T)
            m = np.where(has, np.max(np.where(valid, s, -np.inf), axis=1), 0.0)
            w = np.where(valid, np.exp(np.where(valid, s - m[:, None], 0.0)), 0.0)
            P = w / np.where(has, w.sum(axis=1), 1.0)[:, None]
            o = P @ vv
            dp = do[b, h, pos] @ vv.T
            ds = P * (dp - (P * dp).sum(axis=1, keepdims=True))
            dabs = np.abs(do[b, h, pos])
            e = u * (dabs * np.abs(o)).sum(axis=1) + gamma * (dabs * (np.abs(o) + np.abs(vv).max(axis=0))).sum(axis=1)
            g = u * np.abs(ds) + a * valid + P * e[:, None]
            tq[b, h] = abs(scale) * (g @ np.abs(kk))
            if rows is None:
                tk[b, h] = abs(scale) * (g.T @ np.abs(q[b, h]))
                tv[b, h] = (u * P + a * valid).T @ dabs
    return tq, tk, tv


def compare_grad(got, ref, bound_t, dtype, what):
    """|got - ref| <= 2 T + u |ref| + 1e-6 elementwise; returns the worst err / bound."""
    g = got.detach().float().cpu().double().numpy()
    assert not np.isnan(g).any(), f"{what}: NaN"
    err = np.abs(g - ref)
    bound = 2.0 * bound_t + UNIT[dtype][0] * np.abs(ref) + 1e-6
    ratio = err / bound
    worst = float(ratio.max(initial=0.0))
    if not (err <= bound).all():
        i = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: err/bound {worst:.2f} at {i}: got {g[i]:.6g} ref {ref[i]:.6g} T {bound_t[i]:.3g}")
    return worst
