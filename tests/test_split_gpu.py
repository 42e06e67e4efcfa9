"""GPU parity of the key-split forward (fa_fwd_split) and of the partial-state merge
(fa_merge_states) against the float64 CPU oracle.

The split forward must reach the same attention as the unsplit one, up to rounding, for
any number of parts, including parts that see no key (the merge identity). Tolerances are
those of the unsplit parity tests: float32 max |error| <= 1e-5 (LSE also 2^-22 |LSE|);
bf16/f16 |gpu - ref| <= 2e-2 + 1e-2 |ref|.
"""

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import generate, to_f64

from test_parity_gpu import compare, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def run_split(x, n_splits, kv_len=None, workspace=None):
    q, k, v = (t.to(DEV) for t in (x.q, x.k, x.v))
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=DEV)
    kl = None if kv_len is None else torch.as_tensor(np.asarray(kv_len), dtype=torch.int32)
    fa.forward(q, k, v, causal=x.causal, scale=x.scale, kv_len=kl, out=o, lse=lse, n_splits=n_splits,
               workspace=workspace)
    torch.cuda.synchronize()
    return o, lse


def nan_workspace(x, n_splits):
    B, H, N, D = x.q.shape
    nbytes = fa.fa_fwd_split_workspace_bytes(B, H, N, D, n_splits)
    ws = torch.empty(nbytes // 4 + 64, dtype=torch.float32, device=DEV).fill_(float("nan"))
    return ws


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_matches_oracle(dtype, causal):
    """Ragged N across tile edges, several part counts (more parts than key tiles included),
    a NaN-filled workspace (its contents on entry must not matter)."""
    for D in (64, 128):
        for N, S in ((1, 2), (65, 2), (300, 3), (300, 16), (1000, 7)):
            say(f"split dtype={dtype} causal={causal} D={D} N={N} S={S}")
            x = generate(2, 3, N, D, dtype, causal=causal, seed=2000 + N + S)
            o, lse = run_split(x, S, workspace=nan_workspace(x, S))
            ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
            compare(o, lse, ro, rl, dtype, f"split D={D} N={N} S={S}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("causal", [False, True])
def test_split_key_padding(dtype, causal):
    """kv_len 0 (every part empty: O = 0, LSE = -inf), 1, a tile edge, ragged, N."""
    N, D = 600, 64
    kv = np.array([0, 1, 128, 331, 600], dtype=np.int32)
    for S in (2, 5):
        say(f"split padding dtype={dtype} causal={causal} S={S}")
        x = generate(5, 2, N, D, dtype, causal=causal, seed=91 + S)
        o, lse = run_split(x, S, kv_len=kv)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal, kv_len=kv)
        compare(o, lse, ro, rl, dtype, f"split padding S={S}")
        assert (o[0] == 0).all().item() and torch.isinf(lse[0]).all().item()


@pytest.mark.parametrize("D", [32, 96, 256])
def test_split_other_head_dims(D):
    for causal in (False, True):
        say(f"split D={D} causal={causal}")
        x = generate(1, 2, 333, D, "bf16", causal=causal, seed=3000 + D)
        o, lse = run_split(x, 3)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
        compare(o, lse, ro, rl, "bf16", f"split D={D}")


def test_split_one_is_the_plain_forward():
    """n_splits = 1 through fa_fwd_split gives the plain forward's bits."""
    x = generate(2, 2, 257, 128, "bf16", causal=True, seed=5)
    say("split S=1 vs plain")
    o1, l1 = run_split(x, 1, workspace=nan_workspace(x, 2))
    q, k, v = (t.to(DEV) for t in (x.q, x.k, x.v))
    o0, l0 = fa.forward(q, k, v, causal=True, scale=x.scale)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_split_strided_layout_and_shared_kv():
    """Strided [B, N, H, D] storage and one shared K/V head, split in 4."""
    B, N, H, D = 2, 500, 4, 128
    x = generate(B, H, N, D, "bf16", causal=True, seed=6)
    q = x.q.to(DEV).transpose(1, 2).contiguous().transpose(1, 2)
    k1 = x.k[:, :1].to(DEV).expand(B, H, N, D)
    v1 = x.v[:, :1].to(DEV).expand(B, H, N, D)
    out = torch.full((B, N, H, D), float("nan"), dtype=torch.bfloat16, device=DEV).transpose(1, 2)
    say("split strided + shared kv head")
    o, lse = fa.forward(q, k1, v1, causal=True, scale=x.scale, out=out, n_splits=4)
    torch.cuda.synchronize()
    kk = np.repeat(to_f64(x.k[:, :1]), H, axis=1)
    vv = np.repeat(to_f64(x.v[:, :1]), H, axis=1)
    ro, rl = oracle.attention(to_f64(x.q), kk, vv, x.scale, causal=True)
    compare(o, lse, ro, rl, "bf16", "split strided")


def test_split_deterministic():
    x = generate(1, 4, 2048, 128, "bf16", causal=True, seed=7)
    say("split determinism")
    a = run_split(x, 4)
    b = run_split(x, 4)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_split_full_size_small_batch():
    """A long sequence with few heads (the case the split is for): B=1, H=4, N=8192, D=128,
    causal bf16 in 4 and 8 parts. Sampled rows against the oracle, and the whole output
    against the unsplit forward."""
    x = generate(1, 4, 8192, 128, "bf16", causal=True, seed=8)
    rows = np.array([0, 1, 127, 128, 2047, 4095, 4096, 6000, 8190, 8191])
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, rows=rows)
    q, k, v = (t.to(DEV) for t in (x.q, x.k, x.v))
    o0, l0 = fa.forward(q, k, v, causal=True, scale=x.scale)
    for S in (4, 8):
        say(f"split full size S={S}")
        o, lse = run_split(x, S)
        compare(o[:, :, rows], lse[:, :, rows], ro, rl, "bf16", f"full size S={S}")
        assert ((o.float() - o0.float()).abs() <= 2e-2 + 1e-2 * o0.float().abs()).all().item()
        assert (lse - l0).abs().max().item() <= 1e-4


def test_split_count_suggestions():
    """The suggested count: 1 when the query tiles already fill the device, more for a long
    sequence with few heads, 1 for a short one, never above 16; "auto" runs and matches the oracle."""
    rc, s = fa.fa_fwd_split_count(2, 32, 8192, 128, 0, fa.FA_BF16)
    assert rc == 0 and s == 1
    rc, s = fa.fa_fwd_split_count(1, 4, 8192, 128, 1, fa.FA_BF16)
    assert rc == 0 and 2 <= s <= 16
    rc, s = fa.fa_fwd_split_count(1, 1, 100, 64, 1, fa.FA_F32)
    assert rc == 0 and s == 1
    for D, dt in ((32, fa.FA_F32), (64, fa.FA_F16), (256, fa.FA_BF16)):
        rc, s = fa.fa_fwd_split_count(1, 1, 1 << 20, D, 1, dt)
        assert rc == 0 and 1 <= s <= 16
    x = generate(1, 2, 3000, 128, "bf16", causal=True, seed=12)
    q, k, v = (t.to(DEV) for t in (x.q, x.k, x.v))
    say("split auto")
    o, lse = fa.forward(q, k, v, causal=True, scale=x.scale, n_splits="auto")
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True)
    compare(o, lse, ro, rl, "bf16", "split auto")


# ---- the merge on its own, fed partial states computed by the oracle


def oracle_parts(x, bounds):
    """Partial states over the key ranges [bounds[i], bounds[i+1]) (non-causal), from the oracle:
    keys and values are rolled so the range comes first, and key padding keeps just that range
    (non-causal attention does not depend on key order). An empty range gives the identity
    (O = 0, LSE = -inf)."""
    q, k, v = to_f64(x.q), to_f64(x.k), to_f64(x.v)
    B, H, N, D = q.shape
    po, pl = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        if a == b:
            po.append(np.zeros((B, H, N, D)))
            pl.append(np.full((B, H, N), -np.inf))
            continue
        kr, vr = np.roll(k, -a, axis=2), np.roll(v, -a, axis=2)
        o, l = oracle.attention(q, kr, vr, x.scale, causal=False, kv_len=np.full(B, b - a))
        po.append(o)
        pl.append(l)
    return np.stack(po), np.stack(pl)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [32, 64, 96, 128, 256])
def test_merge_states_matches_oracle(dtype, D):
    N = 190
    x = generate(2, 2, N, D, "f32", causal=False, seed=4000 + D)
    bounds = [0, 37, 37, 120, 190]          # includes an empty part
    po, pl = oracle_parts(x, bounds)
    ref_o, ref_l = po[0], pl[0]
    for s in range(1, len(po)):
        ref_o, ref_l = oracle.merge_states(ref_o, ref_l, po[s], pl[s])
    full_o, full_l = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=False)
    assert np.abs(ref_o - full_o).max() < 1e-12 and np.abs(ref_l - full_l).max() < 1e-12
    say(f"merge dtype={dtype} D={D}")
    o, lse = fa.merge_states(torch.from_numpy(po).float().to(DEV), torch.from_numpy(pl).float().to(DEV),
                             dtype={"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[dtype])
    torch.cuda.synchronize()
    compare(o, lse, ref_o, ref_l, dtype, f"merge D={D}")


def test_merge_all_identity_rows_and_strided_out():
    """Rows whose every state is the identity give O = 0, LSE = -inf; O may be strided."""
    S, B, H, N, D = 3, 2, 3, 40, 64
    rng = np.random.default_rng(11)
    po = rng.standard_normal((S, B, H, N, D))
    pl = rng.uniform(-5, 5, (S, B, H, N))
    pl[:, 1, 2, 7] = -np.inf
    po[:, 1, 2, 7] = 0.0
    pl[0, 0, 0, :] = -np.inf
    po[0, 0, 0, :] = 0.0
    ref_o, ref_l = po[0], pl[0]
    for s in range(1, S):
        ref_o, ref_l = oracle.merge_states(ref_o, ref_l, po[s], pl[s])
    out = torch.full((B, N, H, D), float("nan"), dtype=torch.float32, device=DEV).transpose(1, 2)
    say("merge identity rows, strided out")
    o, lse = fa.merge_states(torch.from_numpy(po).float().to(DEV), torch.from_numpy(pl).float().to(DEV), out=out)
    torch.cuda.synchronize()
    assert (o[1, 2, 7] == 0).all().item() and torch.isinf(lse[1, 2, 7]).item()
    compare(o, lse, ref_o, ref_l, "f32", "merge identity")
