"""Naive full-row softmax attention in float64: the definition of the result.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

What is computed, for every batch b, head h and query row i
("vectorized-flash-attention-kernel", Core algorithm: S = Q K^T, the causal
mask that hides key rows after the query row, softmax, weighted sum of V;
Constructor options: the softmax scale; "Paper: FlashAttention", Code:
hardened masking for padding and empty rows):

  * the valid keys of row i are J_i = { j : j < kv_len[b] and (not causal
    or j <= i) }, a prefix [0, count_i) of the key axis;
  * a query row at or past q_len[b] is padding: it is not part of the batch
    element, so it has no valid keys (J_i empty) whatever Q holds there
    (the pages' hardened masking for padding, applied to the query side);
  * if J_i is empty the row is fully masked: O = 0 and LSE = -inf
    ("js-flash-attention-tiled-online-softmax-exactness", Root causes
    addressed 2 and Verification: fully masked rows give finite zeros);
  * otherwise s_j = scale * <q_i, k_j>, m = max_j s_j, w_j = exp(s_j - m),
    l = sum_j w_j, O = sum_j w_j v_j / l and LSE = m + ln l.

Subtracting the row maximum is part of the plain definition here: without it
logits of 100*D (the pages' large-logit case) overflow even float64. Masked
keys are excluded from every sum; no -inf arithmetic is used.
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np


def key_counts(positions, n_keys, causal, kv_len_b, q_len_b=None):
    """Number of valid keys of each query position (the length of the prefix J_i); 0 for a
    padding query (position >= q_len_b)."""
    positions = np.asarray(positions, dtype=np.int64)
    counts = np.full(positions.shape, min(int(kv_len_b), int(n_keys)), dtype=np.int64)
    if causal:
        counts = np.minimum(counts, positions + 1)
    if q_len_b is not None:
        counts = np.where(positions < int(q_len_b), counts, 0)
    return np.maximum(counts, 0)


def _rows_of_one_head(q, k, v, scale, counts):
    """Attention for some query rows of one (batch, head), straight from the definition.

    q: [R, D] rows of queries, k: [N, D], v: [N, Dv], counts: [R] valid-key counts.
    Returns (o [R, Dv], lse [R]).
    """
    n_rows = q.shape[0]
    o = np.zeros((n_rows, v.shape[1]))
    lse = np.full(n_rows, -np.inf)
    kmax = int(counts.max(initial=0))
    if kmax == 0:
        return o, lse
    s = scale * (q @ k[:kmax].T)
    valid = np.arange(kmax)[None, :] < counts[:, None]
    has = counts > 0
    m = np.max(s, axis=1, where=valid, initial=-np.inf)
    m = np.where(has, m, 0.0)
    w = np.exp(np.where(valid, s - m[:, None], 0.0)) * valid
    l = w.sum(axis=1)
    o[has] = (w[has] @ v[:kmax]) / l[has, None]
    lse[has] = m[has] + np.log(l[has])
    return o, lse


def attention(q, k, v, scale, causal=False, kv_len=None, rows=None, row_chunk=512, workers=1, q_len=None):
    """Exact attention by the definition, in float64.

    Parameters
    ----------
    q, k, v : arrays [B, H, N, D] (k) and [B, H, N, Dv] (v); upcast to float64.
    scale : the softmax scale, as the exact number the caller's other path uses.
    causal : hide keys j > i from query i.
    kv_len : None (every key valid) or ints [B]; keys j >= kv_len[b] are padding.
    q_len : None (every query present) or ints [B]; query rows i >= q_len[b] are
        padding and come out as O = 0, LSE = -inf.
    rows : None for every query position, or a 1-D array of query positions;
        then only those rows are computed, for every (b, h).
    row_chunk : query rows per matrix product (bounds memory).
    workers : threads over (b, h) pairs; with more than one, each BLAS call is
        limited to one thread.

    Returns (o [B, H, R, Dv], lse [B, H, R]) with R = N or len(rows).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, D = q.shape
    if k.shape != (B, H, N, D) or v.shape[:3] != (B, H, N):
        raise ValueError("q, k, v shapes disagree")
    positions = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64).reshape(-1)
    if positions.size and (positions.min() < 0 or positions.max() >= N):
        raise ValueError("query positions out of range")
    if kv_len is not None:
        kv_len = np.asarray(kv_len).reshape(-1)
        if kv_len.shape != (B,):
            raise ValueError("kv_len must have one entry per batch")
    if q_len is not None:
        q_len = np.asarray(q_len).reshape(-1)
        if q_len.shape != (B,):
            raise ValueError("q_len must have one entry per batch")
    R = positions.size
    o = np.zeros((B, H, R, v.shape[3]))
    lse = np.empty((B, H, R))

    def one_head(bh):
        b, h = divmod(bh, H)
        L = N if kv_len is None else int(kv_len[b])
        Lq = None if q_len is None else int(q_len[b])
        for c0 in range(0, R, row_chunk):
            pos = positions[c0:c0 + row_chunk]
            counts = key_counts(pos, N, causal, L, Lq)
            o[b, h, c0:c0 + pos.size], lse[b, h, c0:c0 + pos.size] = _rows_of_one_head(
                q[b, h, pos], k[b, h], v[b, h], float(scale), counts)

    if workers > 1:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one_head, range(B * H)))
    else:
        for bh in range(B * H):
            one_head(bh)
    return o, lse
