"""The pages' tiled forward pass with online softmax, in float64.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

What this model is: the recurrence the GPU kernel runs, kept in float64, so that
it must reach the naive definition up to the order of rounding. The method it
follows is the one of "vectorized-flash-attention-kernel" (Core algorithm; Key
design decisions 1, 3 and 4) and "js-flash-attention-tiled-online-softmax-
exactness" (Root causes addressed 1 and 2).

In short: every query row carries a small state while the key blocks go by, its
largest scaled logit so far, the sum of its exponentials taken relative to that
largest value, and the matching weighted sum of value rows. A new key block
contributes its own exponentials; when it raises the row's largest logit, the
state held so far is first brought to the new reference by one exponential
factor, which keeps every exponential at most 1 and so nothing overflows. A key
after the query (causal mask) or at or past kv_len contributes nothing. A row
that has not yet seen a valid key keeps the empty state, so the factor is never
formed from two infinities. At the end the weighted sum is divided by the sum
(exact zeros for an empty row, whose sum is exactly zero) and the two row
statistics are returned folded into one number, LSE = largest logit + ln(sum).

A key/value block is skipped when it lies wholly in the future of the query
block (its first key index exceeds the block's last query index), and blocks
wholly past every batch's kv_len are skipped too. All (b, h) are processed at
once with array arithmetic; the two loops are the block loops.
"""

import numpy as np


def tiled_attention(q, k, v, scale, causal=False, kv_len=None, block_q=64, block_kv=64):
    """Tiled online-softmax attention in float64. Returns (o [B,H,N,Dv], lse [B,H,N])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    Dv = v.shape[3]
    if block_q < 1 or block_kv < 1:
        raise ValueError("block sizes must be positive")
    L = np.full(B, N, dtype=np.int64) if kv_len is None else np.clip(np.asarray(kv_len).reshape(-1), 0, N)
    o = np.zeros((B, H, N, Dv))
    lse = np.full((B, H, N), -np.inf)
    for q0 in range(0, N, block_q):
        q1 = min(q0 + block_q, N)
        rows = np.arange(q0, q1)
        m = np.full((B, H, q1 - q0), -np.inf)
        l = np.zeros((B, H, q1 - q0))
        acc = np.zeros((B, H, q1 - q0, Dv))
        for k0 in range(0, N, block_kv):
            k1 = min(k0 + block_kv, N)
            if causal and k0 > q1 - 1:
                continue
            if k0 >= L.max():
                continue
            cols = np.arange(k0, k1)
            s = scale * np.matmul(q[:, :, q0:q1], np.swapaxes(k[:, :, k0:k1], -1, -2))
            masked = cols[None, None, None, :] >= L[:, None, None, None]
            if causal:
                masked = masked | (cols[None, :] > rows[:, None])[None, None]
            s = np.where(masked, -np.inf, s)
            m_new = np.maximum(m, s.max(axis=-1))
            live = m_new > -np.inf
            m_sub = np.where(live, m_new, 0.0)
            correction = np.where(live, np.exp(m - m_sub), 1.0)
            p = np.exp(s - m_sub[..., None])
            l = correction * l + p.sum(axis=-1)
            acc = correction[..., None] * acc + np.matmul(p, v[:, :, k0:k1])
            m = m_new
        has = ~(l == 0)
        safe_l = np.where(has, l, 1.0)
        o[:, :, q0:q1] = np.where(has[..., None], acc / safe_l[..., None], 0.0)
        lse[:, :, q0:q1] = np.where(has, m + np.log(safe_l), -np.inf)
    return o, lse
