"""The tiled forward pass with online softmax, in float64, as merges of per-block partial states.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

What this model is: the computation the GPU kernel runs, block by block, kept in
float64, so that it must reach the naive definition up to the order of rounding.
The pages describe it as a running per-row state updated by each key block
("vectorized-flash-attention-kernel", Core algorithm; Key design decisions 1 and
3; "js-flash-attention-tiled-online-softmax-exactness", Root causes addressed 1
and 2), and the course module names the structure behind that update: partial
softmax states form a monoid ("Paper: FlashAttention", Objectives, Math & data
structures). This model is written in the second form.

A partial state of one query row over a set of keys is a triple (m, l, a): m is
the largest scaled logit among the keys, l the sum of exp(logit - m) over them,
and a the same sum with each term multiplying the key's value row. The empty set
has (-inf, 0, 0). Two states merge into the state of the union by bringing both
to the larger of the two m, each scaled by exp(its m - the larger m), and adding
l and a. The merge is associative, so walking the key blocks in order and
merging each block's own state into the running one gives the state of all keys,
whatever the block size. An empty block or an empty running state has m = -inf;
its scale factor is taken as 0, never formed from two infinities. At the end the
row's output is a / l (exact zeros when l is zero: the row saw no key) and its
LSE is m + ln(l).

Keys after the query (causal mask) or at or past kv_len belong to no block's
state. A key block is skipped when it lies wholly in the future of the query
block (its first key index exceeds the block's last query index), and blocks
wholly past every batch's kv_len are skipped too. All (b, h) are processed at
once with array arithmetic; the two loops are the block loops.
"""

import numpy as np


def _block_state(s, valid, v_block):
    """Partial state (m, l, a) of each row over one key block: s the scaled logits [B,H,R,C],
    valid the visible keys, v_block [B,H,C,Dv]."""
    m = np.max(np.where(valid, s, -np.inf), axis=-1)
    seen = m > -np.inf
    w = np.exp(np.where(valid, s - np.where(seen, m, 0.0)[..., None], -np.inf))
    return m, w.sum(axis=-1), np.matmul(w, v_block)


def _merge(m1, l1, a1, m2, l2, a2):
    """State of the union of two disjoint key sets from their two states."""
    m = np.maximum(m1, m2)
    m_sub = np.where(m > -np.inf, m, 0.0)   # both empty: factors exp(-inf) = 0, not exp(nan)
    f1 = np.exp(m1 - m_sub)
    f2 = np.exp(m2 - m_sub)
    return m, f1 * l1 + f2 * l2, f1[..., None] * a1 + f2[..., None] * a2


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
        a = np.zeros((B, H, q1 - q0, Dv))
        for k0 in range(0, N, block_kv):
            k1 = min(k0 + block_kv, N)
            if causal and k0 > q1 - 1:
                continue
            if k0 >= L.max():
                continue
            cols = np.arange(k0, k1)
            s = scale * np.matmul(q[:, :, q0:q1], np.swapaxes(k[:, :, k0:k1], -1, -2))
            valid = cols[None, None, None, :] < L[:, None, None, None]
            if causal:
                valid = valid & (cols[None, :] <= rows[:, None])[None, None]
            m, l, a = _merge(m, l, a, *_block_state(s, valid, v[:, :, k0:k1]))
        seen = l != 0   # exactly when the row saw no key (a NaN from a slip stays visible)
        o[:, :, q0:q1] = np.where(seen[..., None], a / np.where(seen, l, 1.0)[..., None], 0.0)
        lse[:, :, q0:q1] = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)
    return o, lse
