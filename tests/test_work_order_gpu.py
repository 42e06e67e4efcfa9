"""GPU parity on the work orders the kernels choose from the problem's shape.

Each XCD takes a contiguous run of heads. For a causal problem with no padding, B*H divisible by
8 and at most 32 units per head, it takes them rank by rank (every head's longest tile first),
over groups of as many heads as keep two [N, D] operands per head in the XCD's L2. With key
padding only (kv_len, no q_len), B*H divisible by 8 and at most 64 heads per XCD, the forward
takes its units longest first, an order each workgroup finds on the device; otherwise head by
head. Both orders must give the oracle's result; these cases sit on either
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


def test_forward_rank_groups():
    """B*H = 72 heads (9 per XCD), N = 2048, D = 64: rank by rank in groups of 8 heads (two
    [N, D] bf16 operands of 8 heads fill the 4 MB L2) plus a group of one. The same problem with
    kv_len = N everywhere takes the key-padded order (longest first, found on the device); every
    unit's arithmetic is the same, so the two
    outputs must agree bit for bit (a unit that ran twice or never shows up, the outputs being
    prefilled with NaN). Sampled rows of three heads against the oracle."""
    B, H, N = 9, 8, 2048
    x = generate(B, H, N, 64, "bf16", causal=True, seed=5500)
    say("rank groups forward")
    o, lse = run_gpu(x)
    o2, l2 = run_gpu(x, kv_len=np.full(B, N, dtype=np.int32))
    assert torch.equal(o, o2) and torch.equal(lse, l2), "rank-group order differs from head order"
    ocpu, lcpu = o.float().cpu(), lse.cpu()
    rows = np.array([0, 127, 128, 1000, 2047])
    for b, h in [(0, 0), (4, 7), (8, 3)]:
        ro, rl = oracle.attention(to_f64(x.q[b:b + 1, h:h + 1]), to_f64(x.k[b:b + 1, h:h + 1]),
                                  to_f64(x.v[b:b + 1, h:h + 1]), x.scale, causal=True, rows=rows)
        compare(ocpu[b:b + 1, h:h + 1, rows], lcpu[b:b + 1, h:h + 1, rows], ro, rl, "bf16", f"b={b} h={h}")


@pytest.mark.parametrize("dtype,D,causal", [("f16", 64, True), ("bf16", 64, False), ("bf16", 128, True),
                                             ("f16", 128, False), ("bf16", 96, True), ("f16", 32, True),
                                             ("bf16", 256, True)])
def test_forward_longest_first_order(dtype, D, causal):
    """Key padding with whole heads on every XCD (B*H = 64, 8 per XCD): the workgroups of each XCD
    find their units on the device in the order of decreasing key tiles. With kv_len = N
    everywhere the result must be bit for bit that of the same launch without kv_len (another
    order, the same arithmetic per unit; the outputs are prefilled with NaN, so a unit that
    never ran shows up). With kv_len of 0, 1, 15, 64, 129, 333, N - 1 and N, every row against
    the oracle."""
    B, H, N = 8, 8, 700
    x = generate(B, H, N, D, dtype, causal=causal, seed=5700 + D + int(causal))
    say(f"longest-first order {dtype} D={D} causal={causal}")
    o, lse = run_gpu(x)
    o2, l2 = run_gpu(x, kv_len=np.full(B, N, dtype=np.int32))
    assert torch.equal(o, o2) and torch.equal(lse, l2), "longest-first order differs from the unpadded order"
    kv = np.array([0, 1, 15, N - 1, N, 333, 64, 129], dtype=np.int32)
    o3, l3 = run_gpu(x, kv_len=kv)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal, kv_len=kv)
    compare(o3, l3, ro, rl, dtype, f"longest first D={D} causal={causal}")


@pytest.mark.parametrize("B", [64, 65])
def test_forward_longest_first_limit(B):
    """64 heads per XCD (B*H = 512) is the most the longest-first order takes, one per lane of a
    wave; 65 (B*H = 520) goes head by head. Both with random kv_len, every row against the oracle."""
    H, N, D = 8, 130, 64
    x = generate(B, H, N, D, "bf16", causal=True, seed=5800 + B, padding=True)
    say(f"longest-first limit B={B}")
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, kv_len=x.kv_len)
    compare(o, lse, ro, rl, "bf16", f"longest-first limit B={B}")


@pytest.mark.parametrize("dtype,D,causal", [("f16", 64, True), ("bf16", 64, False), ("bf16", 128, True),
                                             ("f16", 96, True), ("bf16", 32, True)])
def test_backward_longest_first_order(dtype, D, causal):
    """Key padding with whole heads on every XCD (B*H = 64): the dQ and dK/dV kernels take their
    units longest first, found on the device (key tiles past kv_len, with no work, come last).
    kv_len of 0, 1, 15, 64, 129, 200, N - 1 and N, every gradient element against the oracle."""
    B, H, N = 8, 8, 300
    x = generate(B, H, N, D, dtype, causal=causal, seed=5900 + D + int(causal))
    do = generate_grad_output(B, H, N, D, dtype, seed=5901 + D)
    kv = np.array([0, 1, 15, N - 1, N, 200, 64, 129], dtype=np.int32)
    say(f"longest-first backward {dtype} D={D} causal={causal}")
    check(x, do, kv_len=kv, tag=f"longest first D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
def test_longest_first_strided_layouts(D):
    """The key-padded longest-first order on [B, N, H, D] storage (token stride H*D), forward
    and backward (B*H = 16, two heads per XCD): bit for bit the contiguous call, which the
    oracle checks."""
    B, H, N = 2, 8, 333
    x = generate(B, H, N, D, "bf16", causal=True, seed=6100 + D)
    do = generate_grad_output(B, H, N, D, "bf16", seed=6101 + D)
    kv = torch.tensor([N - 40, 129], dtype=torch.int32)
    dev = torch.device("cuda:0")
    q, k, v, dO = (t.to(dev) for t in (x.q, x.k, x.v, do))
    say(f"longest-first strided D={D}")
    o, lse = fa.forward(q, k, v, causal=True, scale=x.scale, kv_len=kv)
    grads = fa.backward(q, k, v, o, lse, dO, causal=True, scale=x.scale, kv_len=kv)
    bnhd = lambda t: t.transpose(1, 2).contiguous().transpose(1, 2)
    qs, ks, vs, dos = (bnhd(t) for t in (q, k, v, dO))
    out = torch.full((B, N, H, D), float("nan"), dtype=q.dtype, device=dev).transpose(1, 2)
    o2, l2 = fa.forward(qs, ks, vs, causal=True, scale=x.scale, kv_len=kv, out=out)
    packed = torch.full((B, N, 3, H, D), float("nan"), dtype=q.dtype, device=dev)
    dq, dk, dv = (packed[:, :, i].transpose(1, 2) for i in range(3))
    fa.backward(qs, ks, vs, bnhd(o), lse, dos, causal=True, scale=x.scale, kv_len=kv, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2), "strided forward differs from the contiguous call"
    for a, b_, name in zip((dq, dk, dv), grads, ("dQ", "dK", "dV")):
        assert torch.equal(a, b_), f"strided {name} differs from the contiguous call"
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, kv_len=kv.numpy())
    compare(o, lse, ro, rl, "bf16", f"longest first strided D={D}")
    check(x, do, kv_len=kv.numpy(), tag=f"longest first strided D={D}")


def test_backward_rank_groups():
    """The backward kernels' units in groups of 8 heads (B*H = 72, N = 2048, D = 64, 16 units
    per head): bit for bit the result of the key-padded, longest-first order (kv_len = N)."""
    B, H, N, D = 9, 8, 2048, 64
    x = generate(B, H, N, D, "bf16", causal=True, seed=5600)
    do = generate_grad_output(B, H, N, D, "bf16", seed=5601)
    dev = torch.device("cuda:0")
    q, k, v, g = (t.to(dev) for t in (x.q, x.k, x.v, do))
    say("rank groups backward")
    o, lse = fa.forward(q, k, v, causal=True, scale=x.scale)
    a = fa.backward(q, k, v, o, lse, g, causal=True, scale=x.scale)
    kv = torch.full((B,), N, dtype=torch.int32, device=dev)
    b = fa.backward(q, k, v, o, lse, g, causal=True, scale=x.scale, kv_len=kv)
    torch.cuda.synchronize()
    for name, s, t in zip(("dQ", "dK", "dV"), a, b):
        assert not torch.isnan(s.float()).any(), f"NaN in {name}"
        assert torch.equal(s, t), f"{name}: rank-group order differs from head order"
