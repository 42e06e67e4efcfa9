"""GPU parity on the work orders the kernels choose from the problem's shape.

Each XCD takes a contiguous run of heads. For a causal problem with no padding, B*H divisible by
8 and at most 32 units per head, it takes them rank by rank (every head's longest tile first);
otherwise head by head. Both orders must give the oracle's result; these cases sit on either
side of each condition, for the forward and for both backward kernels (whose units are query
tiles of 128 rows for dQ and key tiles of 128 keys for dK/dV).
"""

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import generate, generate_grad_output, to_f64

from test_backward_gpu import check
from test_parity_gpu import compare, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("D", [64, 96, 128])
@pytest.mark.parametrize("N", [65, 300, 1000])
def test_forward_rank_order(D, N):
    """B*H = 8, causal, short heads: rank by rank. The same shape with key padding goes head by
    head; both against the oracle."""
    for padded in (False, True):
        x = generate(2, 4, N, D, "bf16", causal=True, seed=5100 + N + D)
        kv = np.array([N, N // 2], dtype=np.int32) if padded else None
        say(f"rank order forward D={D} N={N} padded={padded}")
        o, lse = run_gpu(x, kv_len=kv)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, kv_len=kv)
        compare(o, lse, ro, rl, "bf16", f"D={D} N={N} padded={padded}")


@pytest.mark.parametrize("N", [4096, 4097])
def test_forward_rank_order_limit(N):
    """D = 64 (128-row tiles): N = 4096 gives 32 tiles per head (rank by rank), N = 4097 gives 33
    (head by head). Sampled rows of a few heads against the oracle."""
    x = generate(2, 8, N, 64, "f16", causal=True, seed=5200 + N)
    say(f"rank order limit N={N}")
    o, lse = run_gpu(x)
    ocpu, lcpu = o.float().cpu(), lse.cpu()
    rows = np.array([0, 127, 128, 2000, 4000, N - 1])
    for b, h in [(0, 0), (1, 5), (1, 7)]:
        ro, rl = oracle.attention(to_f64(x.q[b:b + 1, h:h + 1]), to_f64(x.k[b:b + 1, h:h + 1]),
                                  to_f64(x.v[b:b + 1, h:h + 1]), x.scale, causal=True, rows=rows)
        compare(ocpu[b:b + 1, h:h + 1, rows], lcpu[b:b + 1, h:h + 1, rows], ro, rl, "f16", f"N={N} b={b} h={h}")


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("bf16", 96), ("bf16", 128), ("f16", 64)])
@pytest.mark.parametrize("N", [200, 700])
def test_backward_rank_order(dtype, D, N):
    """B*H = 8, causal, short heads: both backward kernels take their units rank by rank."""
    x = generate(2, 4, N, D, dtype, causal=True, seed=5300 + N + D)
    do = generate_grad_output(2, 4, N, D, dtype, seed=5301 + N + D)
    say(f"rank order backward {dtype} D={D} N={N}")
    check(x, do, tag=f"rank order D={D} N={N}")


def test_split_rank_order():
    """The split forward with B*H = 8, causal: per head 3 query tiles x 4 parts = 12 units."""
    x = generate(2, 4, 700, 128, "bf16", causal=True, seed=5400)
    q, k, v = (t.to(torch.device("cuda:0")) for t in (x.q, x.k, x.v))
    o, lse = fa.forward(q, k, v, causal=True, scale=x.scale, n_splits=4)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True)
    compare(o, lse, ro, rl, "bf16", "split rank order")
