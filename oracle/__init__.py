"""CPU oracle for exact attention: plain, slow and obviously correct, in float64.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import this package. The product path (the HIP
library and its Python binding) never imports, calls or links anything here,
and nothing here imports the product path. The two share no code.

Contents
--------
naive.attention
    Full-row softmax attention by its definition, one query-row chunk of one
    (batch, head) at a time. This is the result the tiled method must reach
    exactly, up to rounding order ("vectorized-flash-attention-kernel",
    Evidence & signatures table: exact match against standard attention;
    "js-flash-attention-tiled-online-softmax-exactness", task description:
    a naive full-softmax reference).
tiled.tiled_attention
    The pages' tiled forward with online softmax, in float64, taken step by
    step ("vectorized-flash-attention-kernel", Core algorithm and Key design
    decisions 1 and 3; "js-flash-attention-tiled-online-softmax-exactness",
    Root causes addressed 1 and 2). It pins the recurrence the GPU kernel
    runs against the naive definition at every block size.
merge.merge_states
    The associative merge of two partial softmax states, with its identity
    element ("Paper: FlashAttention", Objectives, Math & data structures).
backward.attention_grad, backward.attention_grad_rows
    Gradients dQ, dK, dV of exact attention by the chain rule through the
    definition (the softmax Jacobian written out).
backward.tiled_backward
    The pages' recomputing backward from saved (O, LSE), block by block, with
    Delta = rowsum(dO o O) ("Paper: FlashAttention", Objectives, Math & data
    structures; "vectorized-flash-attention-kernel", Key design decision 4).

Every function is pinned by tests that do not reuse its own arithmetic:
50-digit brute force on tiny inputs, closed forms, invariants and
mutation checks; the gradients by finite differences of the pinned forward,
by float64 autograd of an independent formulation, and by invariants.
"""

from .naive import attention, key_counts
from .tiled import tiled_attention
from .merge import merge_states
from .backward import attention_grad, attention_grad_rows, tiled_backward

__all__ = ["attention", "key_counts", "tiled_attention", "merge_states", "attention_grad", "attention_grad_rows",
           "tiled_backward"]
