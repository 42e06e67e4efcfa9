"""Seeded random shapes: forward, key-split forward and backward against the oracles.

Thirty configurations drawn once from a fixed seed cover combinations that the hand-picked
cases do not name: B, H, ragged N up to 700, every head dimension, both 16-bit types (and
float32 for the forward), causal or not, key padding with random kv_len (0 included), and a
random part count for the split. Twenty more, from a second seed, add query padding (random
q_len, with NaN in the padding rows of Q and dO), forty more come from a third seed, and sixteen
more have key padding with B*H a multiple of 8, the launches whose units run longest first.
Tolerances are the ones of the dedicated tests.
"""

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import generate, generate_grad_output, to_f64

from grad_bounds import DTYPE_NAME, compare_grad, rounding_bound
from test_parity_gpu import compare, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def draw_configs(count=30, seed=2024, query_padding=False):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        dtype = ["bf16", "f16", "f32"][int(rng.integers(0, 3))]
        D = int(rng.choice([32, 64, 96, 128] + ([] if dtype == "f32" else [256])))
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        N = int(rng.integers(1, 701))
        causal = bool(rng.integers(0, 2))
        kv = None
        if rng.random() < 0.5:
            kv = rng.integers(0, N + 1, size=B).astype(np.int32)
        splits = int(rng.integers(2, 9))
        ql = rng.integers(0, N + 1, size=B).astype(np.int32) if query_padding else None
        out.append((i, B, H, N, D, dtype, causal, kv, splits, ql))
    return out


def draw_whole_head_padded(count=16, seed=4242):
    """Key padding with B*H a multiple of 8 (at most 64 heads per XCD): the launches that take
    their units longest first, in an order each workgroup finds on the device."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        while True:
            B, H = int(rng.choice([1, 2, 4, 8, 16])), int(rng.choice([1, 2, 4, 8]))
            if (B * H) % 8 == 0 and B * H <= 64:
                break
        dtype = ["bf16", "f16"][int(rng.integers(0, 2))]
        D = int(rng.choice([32, 64, 96, 128, 256]))
        N = int(rng.integers(1, 401))
        kv = rng.integers(0, N + 1, size=B).astype(np.int32)
        out.append((i, B, H, N, D, dtype, bool(rng.integers(0, 2)), kv, int(rng.integers(2, 9)), None))
    return out


CONFIGS = (draw_configs() + [(100 + c[0],) + c[1:] for c in draw_configs(20, seed=77, query_padding=True)]
           + [(200 + c[0],) + c[1:] for c in draw_configs(40, seed=31337)]
           + [(300 + c[0],) + c[1:] for c in draw_whole_head_padded()])


@pytest.mark.parametrize("cfg", CONFIGS, ids=lambda c: f"c{c[0]}")
def test_random_shape(cfg):
    i, B, H, N, D, dtype, causal, kv, splits, ql = cfg
    say(f"random c{i}: B={B} H={H} N={N} D={D} {dtype} causal={causal} kv_len={None if kv is None else kv.tolist()} "
        f"q_len={None if ql is None else ql.tolist()} splits={splits}")
    x = generate(B, H, N, D, dtype, causal=causal, seed=5000 + i)
    qin = x.q.clone()
    if ql is not None:
        for b, L in enumerate(ql):
            qin[b, :, int(L):] = float("nan")   # padding query rows are never read
    q, k, v = (t.to(DEV) for t in (qin, x.k, x.v))
    kl = None if kv is None else torch.as_tensor(kv)
    qlt = None if ql is None else torch.as_tensor(ql)
    q64, k64, v64 = to_f64(x.q), to_f64(x.k), to_f64(x.v)
    ro, rl = oracle.attention(q64, k64, v64, x.scale, causal=causal, kv_len=kv, q_len=ql)

    o, lse = fa.forward(q, k, v, causal=causal, scale=x.scale, kv_len=kl, q_len=qlt)
    torch.cuda.synchronize()
    compare(o, lse, ro, rl, dtype, f"c{i} forward")

    o2, lse2 = fa.forward(q, k, v, causal=causal, scale=x.scale, kv_len=kl, q_len=qlt, n_splits=splits)
    torch.cuda.synchronize()
    compare(o2, lse2, ro, rl, dtype, f"c{i} split {splits}")

    if dtype != "f32" and D <= 128:
        do = generate_grad_output(B, H, N, D, dtype, seed=6000 + i)
        dcopy = do.clone()
        zq, zdo = q64.copy(), to_f64(do)
        if ql is not None:
            for b, L in enumerate(ql):
                dcopy[b, :, int(L):] = float("nan")
                zq[b, :, int(L):] = 0.0
                zdo[b, :, int(L):] = 0.0
        grads = fa.backward(q, k, v, o, lse, dcopy.to(DEV), causal=causal, scale=x.scale, kv_len=kl, q_len=qlt)
        torch.cuda.synchronize()
        ref = oracle.attention_grad(q64, k64, v64, to_f64(do), x.scale, causal=causal, kv_len=kv, q_len=ql)
        T = rounding_bound(zq, k64, v64, zdo, x.scale, causal, kv, DTYPE_NAME[x.q.dtype])
        for g, r, t, name in zip(grads, ref, T, ("dQ", "dK", "dV")):
            compare_grad(g, r, t, dtype, f"c{i} {name}")
