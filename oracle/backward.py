"""Gradients of exact attention, in float64.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

The forward is the one in ``naive.py``: per (batch, head) and query row i, the
valid keys J_i, P_ij = softmax_j(scale * <q_i, k_j>) over J_i (P_ij = 0 for j
outside J_i, and a whole row of zeros when J_i is empty), O_i = sum_j P_ij v_j.
Given the output gradient dO, the chain rule through O = P V and through the
row softmax (whose Jacobian is diag(p) - p p^T) gives

    dV   = P^T dO
    dP   = dO V^T
    dS   = P o (dP - rowsum(P o dP))          (o: elementwise product)
    dQ   = scale * dS K
    dK   = scale * dS^T Q

``attention_grad`` is that definition written out. ``tiled_backward`` is the
recomputing backward the pages describe ("Paper: FlashAttention", Objectives,
Math & data structures: the backward pass by recomputation, with the identity
rowsum(dP o P) = rowsum(dO o O); "vectorized-flash-attention-kernel", Key design
decision 4: the forward keeps per-row statistics so that any block of S and P
can be rebuilt later, and the backward uses them for dQ, dK, dV). It never
holds a full row of P: it rebuilds each block P_ij = exp(S_ij - LSE_i) from the
saved LSE, and uses Delta_i = rowsum(dO_i o O_i) in place of rowsum(P o dP).
A row with no valid key (LSE = -inf) gets P = 0: its output is the constant 0.

With query padding (q_len), a row at or past q_len[b] is not part of the batch element: its
output is the constant 0 and its rows of Q and dO are not inputs at all, so they are replaced
by zeros before the definition is applied. That alone gives the padding rows dP = dO V^T = 0,
hence dS = P o (0 - 0) = 0: their dQ rows are exactly 0 and they add nothing to dK or dV,
whatever Q and dO held there (NaN included).
"""

import numpy as np


def _valid_mask(n_rows, n_keys, causal, kv_len_b, rows=None):
    """valid[i, j]: key j is in J_i for query position rows[i] (all positions by default)."""
    pos = np.arange(n_rows) if rows is None else np.asarray(rows)
    keys = np.arange(n_keys)
    valid = np.broadcast_to(keys[None, :] < min(int(kv_len_b), n_keys), (pos.size, n_keys)).copy()
    if causal:
        valid &= keys[None, :] <= pos[:, None]
    return valid


def _drop_padding_queries(x, q_len, rows=None):
    """Copy of x [B, H, R, ...] with the rows of padding queries (position >= q_len[b]) zeroed."""
    if q_len is None:
        return x
    x = x.copy()
    q_len = np.asarray(q_len).reshape(-1)
    pos = np.arange(x.shape[2]) if rows is None else np.asarray(rows)
    for b in range(x.shape[0]):
        x[b, :, pos >= int(q_len[b])] = 0.0
    return x


def _probs_and_ds(q, k, v, do, scale, valid):
    """P and dS for some query rows of one (batch, head): q [R, D], do [R, Dv] (those rows),
    k [N, D], v [N, Dv], valid [R, N]."""
    s = scale * (q @ k.T)
    has = valid.any(axis=1)
    m = np.max(s, axis=1, where=valid, initial=-np.inf)
    m = np.where(has, m, 0.0)
    w = np.exp(np.where(valid, s - m[:, None], 0.0)) * valid
    l = w.sum(axis=1)
    p = w / np.where(has, l, 1.0)[:, None]
    dp = do @ v.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return p, ds


def _grad_one_head(q, k, v, do, scale, valid):
    """The definition for one (batch, head): q [N, D], k [N, D], v [N, Dv], do [N, Dv]."""
    p, ds = _probs_and_ds(q, k, v, do, scale, valid)
    dv = p.T @ do
    dq = scale * (ds @ k)
    dk = scale * (ds.T @ q)
    return dq, dk, dv


def attention_grad(q, k, v, do, scale, causal=False, kv_len=None, q_len=None):
    """Gradients (dq, dk, dv) of sum(dO o O) for exact attention, by the definition.

    q, k: [B, H, N, D]; v, do: [B, H, N, Dv]; kv_len: None or ints [B] (keys at or past
    kv_len[b] are padding); q_len: None or ints [B] (query rows at or past q_len[b] are
    padding). Returns float64 arrays shaped like q, k, v.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, D = q.shape
    if k.shape != (B, H, N, D) or v.shape[:3] != (B, H, N) or do.shape != v.shape:
        raise ValueError("q, k, v, do shapes disagree")
    q = _drop_padding_queries(q, q_len)
    do = _drop_padding_queries(do, q_len)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        L = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        valid = _valid_mask(N, N, causal, L)
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _grad_one_head(q[b, h], k[b, h], v[b, h], do[b, h], float(scale), valid)
    return dq, dk, dv


def attention_grad_rows(q, k, v, do, scale, rows, causal=False, kv_len=None, q_len=None):
    """dQ for the selected query positions only, [B, H, len(rows), D]: each dQ row depends on
    its own query row and every key, so sampled rows cost O(len(rows) * N * D)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, D = q.shape
    rows = np.asarray(rows, dtype=np.int64).reshape(-1)
    q = _drop_padding_queries(q, q_len)
    do = _drop_padding_queries(do, q_len)
    out = np.zeros((B, H, rows.size, D))
    for b in range(B):
        L = N if kv_len is None else int(np.asarray(kv_len).reshape(-1)[b])
        valid = _valid_mask(N, N, causal, L, rows=rows)
        for h in range(H):
            _, ds = _probs_and_ds(q[b, h, rows], k[b, h], v[b, h], do[b, h, rows], float(scale), valid)
            out[b, h] = scale * (ds @ k[b, h])
    return out


def tiled_backward(q, k, v, o, lse, do, scale, causal=False, kv_len=None, block_q=64, block_kv=64):
    """The recomputing backward from saved (O, LSE), block by block. Returns (dq, dk, dv).

    Delta_i = rowsum(dO_i o O_i). For every key block (outer loop) and query block (inner loop,
    skipping blocks wholly before the key block under the causal mask): rebuild
    S = scale Q_i K_j^T with masked entries removed, P = exp(S - LSE_i), then
    dV_j += P^T dO_i, dP = dO_i V_j^T, dS = P o (dP - Delta_i), dK_j += scale dS^T Q_i and
    dQ_i += scale dS K_j.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    B, H, N, D = q.shape
    if block_q < 1 or block_kv < 1:
        raise ValueError("block sizes must be positive")
    L = np.full(B, N, dtype=np.int64) if kv_len is None else np.clip(np.asarray(kv_len).reshape(-1), 0, N)
    delta = (do * o).sum(axis=-1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for k0 in range(0, N, block_kv):
        k1 = min(k0 + block_kv, N)
        cols = np.arange(k0, k1)
        for q0 in range(0, N, block_q):
            q1 = min(q0 + block_q, N)
            if causal and q1 - 1 < k0:
                continue
            rows = np.arange(q0, q1)
            s = scale * np.matmul(q[:, :, q0:q1], np.swapaxes(k[:, :, k0:k1], -1, -2))
            dead = cols[None, None, None, :] >= L[:, None, None, None]
            if causal:
                dead = dead | (cols[None, :] > rows[:, None])[None, None]
            lse_b = lse[:, :, q0:q1, None]
            live_row = lse_b > -np.inf
            p = np.where(dead | ~live_row, 0.0, np.exp(np.where(dead | ~live_row, 0.0, s - np.where(live_row, lse_b, 0.0))))
            dv[:, :, k0:k1] += np.matmul(np.swapaxes(p, -1, -2), do[:, :, q0:q1])
            dp = np.matmul(do[:, :, q0:q1], np.swapaxes(v[:, :, k0:k1], -1, -2))
            ds = p * (dp - delta[:, :, q0:q1, None])
            dk[:, :, k0:k1] += scale * np.matmul(np.swapaxes(ds, -1, -2), q[:, :, q0:q1])
            dq[:, :, q0:q1] += scale * np.matmul(ds, k[:, :, k0:k1])
    return dq, dk, dv
