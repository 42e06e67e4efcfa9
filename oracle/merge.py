"""Merge of two partial softmax states, in float64.

TEST INFRASTRUCTURE (see the package docstring): never imported by the
product path.

A partial state over a key set J is the pair (O_J, LSE_J): the attention
output over J alone and the log of its softmax denominator. Two states over
disjoint key sets combine into the state over their union, the operation is
associative, and (O = 0, LSE = -inf), the state of the empty set, is its
identity ("Paper: FlashAttention", Objectives, Math & data structures: partial
softmax states merge associatively and have an identity element).

    LSE = ln(exp(LSE_1) + exp(LSE_2))
    O   = exp(LSE_1 - LSE) O_1 + exp(LSE_2 - LSE) O_2
"""

import numpy as np


def merge_states(o1, lse1, o2, lse2):
    """Combine partial states (o [..., Dv], lse [...]) over disjoint key sets."""
    o1 = np.asarray(o1, dtype=np.float64)
    o2 = np.asarray(o2, dtype=np.float64)
    lse1 = np.asarray(lse1, dtype=np.float64)
    lse2 = np.asarray(lse2, dtype=np.float64)
    lse = np.logaddexp(lse1, lse2)
    empty = lse == -np.inf
    safe = np.where(empty, 0.0, lse)
    w1 = np.where(empty, 0.0, np.exp(np.where(lse1 == -np.inf, -np.inf, lse1 - safe)))
    w2 = np.where(empty, 0.0, np.exp(np.where(lse2 == -np.inf, -np.inf, lse2 - safe)))
    o = w1[..., None] * o1 + w2[..., None] * o2
    return o, lse
