"""The pages' tiled forward pass with online softmax, in float64.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

This is the recurrence the GPU kernel runs, written as the pages give it and
kept in float64 so that it must agree with the naive definition to rounding
order ("vectorized-flash-attention-kernel", Core algorithm; Key design
decision 1, online softmax; decision 3, causal masking with whole-block skip).
For each query block every row starts with m = -inf, l = 0, O = 0; for each
key/value block:

  1. S = scale * Q_block K_block^T;
  2. masked scores (key after query under the causal mask, or key at or past
     kv_len) become -inf;
  3. m_new = max(m_old, max_j S_ij); correction = exp(m_old - m_new);
     l = correction * l + sum_j exp(S_ij - m_new);
     O = correction * O + sum_j exp(S_ij - m_new) V_j;
     a row whose m_new is still -inf has seen no valid key and is left as it
     is ("js-flash-attention-tiled-online-softmax-exactness", Root causes
     addressed 2: exp(-inf - -inf) would be NaN);

then O /= l, with exact zeros where l == 0 (Root causes addressed 2 tests l
for zero, so a NaN that escaped the guard stays visible), and the per-row
statistics are returned in compressed form as LSE = m + ln l (Key design
decision 4 keeps the row max and row sum for the backward pass).

A key/value block is skipped when it lies wholly in the future of the query
block: its first key index is greater than the block's last query index.
Blocks wholly past every batch's kv_len are skipped too. All (b, h) are
processed at once with array arithmetic; the loops are the pages' block loops.
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
