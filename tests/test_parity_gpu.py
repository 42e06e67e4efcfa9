"""GPU parity: the HIP kernel (through the C ABI) against the float64 CPU oracle.

Tolerances (fixed by the target, written here): float32 inputs, max |error| <= 1e-5;
bf16/f16 inputs, |gpu - ref| <= 2e-2 + 1e-2*|ref| elementwise. The same bound
applies to LSE, and -inf (fully masked rows) must match exactly. Only the tests whose
logits are deliberately large (scaled logits near 100 and beyond) let the float32 LSE
bound also allow two float32 spacings at the LSE's own magnitude (2^-22 * |LSE|): a
float32 number of magnitude 100 is resolved only to 7.6e-6, so the stored LSE cannot be
closer than that to the float64 value; each such test prints its measured error. Inputs
come from the seeded generator; the oracle sees them upcast exactly to float64.
"""

import math
import os

import numpy as np
import pytest
import torch

import oracle
import exact_tiled_attention_23_amd as fa
from exact_tiled_attention_23_amd.workloads import WORKLOADS, generate, generate_workload, to_f64

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


LSE_F32_RTOL = 2.0 ** -22


def tol(dtype):
    return (1e-5, 0.0) if dtype == "f32" else (2e-2, 1e-2)


def say(msg):
    print(msg, flush=True)


def run_gpu(x, kv_len=None, causal=None, prefill_nan=True):
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    o = torch.full_like(q, float("nan")) if prefill_nan else None
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev) if prefill_nan else None
    kl = x.kv_len if kv_len is None else kv_len
    o, lse = fa.forward(q, k, v, causal=x.causal if causal is None else causal, scale=x.scale,
                        kv_len=None if kl is None else torch.as_tensor(np.asarray(kl), dtype=torch.int32),
                        out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def compare(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what, lse_f32_spacing=False):
    """Element by element against the oracle. Returns (max |O err|, max |LSE err|, max O
    err/bound, max LSE err/bound). `lse_f32_spacing` adds 2^-22 * |LSE| to the float32 LSE
    bound (large-logit tests only)."""
    atol, rtol = tol(dtype)
    o = o_gpu.detach().float().cpu().double().numpy()
    l = lse_gpu.detach().cpu().double().numpy()
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(l).any(), f"{what}: NaN in LSE"
    inf_ref = np.isinf(lse_ref)
    assert np.array_equal(np.isinf(l), inf_ref), f"{what}: fully masked rows differ"
    assert np.array_equal(l[inf_ref], lse_ref[inf_ref]), f"{what}: LSE infinities differ"
    eo = np.abs(o - o_ref)
    bo = atol + rtol * np.abs(o_ref)
    assert (eo <= bo).all(), f"{what}: O max err {eo.max():.3e} (worst excess {(eo - bo).max():.3e})"
    fin = ~inf_ref
    el = np.abs(l[fin] - lse_ref[fin])
    lrt = max(rtol, LSE_F32_RTOL) if (dtype == "f32" and lse_f32_spacing) else rtol
    bl = atol + lrt * np.abs(lse_ref[fin])
    assert (el <= bl).all(), f"{what}: LSE max err {el.max() if el.size else 0:.3e}"
    if lse_f32_spacing and dtype == "f32" and el.size:
        say(f"  {what}: float32 LSE max err {el.max():.3e} at |LSE| up to {np.abs(lse_ref[fin]).max():.1f}")
    return (float(eo.max(initial=0.0)), float(el.max(initial=0.0)), float((eo / bo).max(initial=0.0)),
            float((el / bl).max(initial=0.0)))


SWEEP_N = [1, 2, 3, 17, 63, 64, 65, 127, 128, 129, 255, 300]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_small_sweep(dtype, D, causal):
    """Every ragged N around the 128-row and 64-key tile edges; B=2, H=3; no padding."""
    for N in SWEEP_N:
        say(f"sweep dtype={dtype} D={D} causal={causal} N={N}")
        x = generate(2, 3, N, D, dtype, causal=causal, seed=1000 + N)
        o, lse = run_gpu(x)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
        compare(o, lse, ro, rl, dtype, f"N={N}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 96])
@pytest.mark.parametrize("causal", [False, True])
def test_key_padding(dtype, D, causal):
    """Per-batch kv_len including 0, 1, a tile edge, a ragged value and N; the padding keys
    hold NaN, which must not reach O or LSE."""
    N = 200
    kv = np.array([0, 1, 64, 131, 200], dtype=np.int32)
    say(f"padding dtype={dtype} D={D} causal={causal} kv={kv.tolist()}")
    x = generate(5, 2, N, D, dtype, causal=causal, seed=77)
    k0, v0 = x.k.clone(), x.v.clone()
    for b, L in enumerate(kv):
        x.k[b, :, L:] = float("nan")
        x.v[b, :, L:] = float("nan")
    o, lse = run_gpu(x, kv_len=kv)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(k0), to_f64(v0), x.scale, causal=causal, kv_len=kv)
    compare(o, lse, ro, rl, dtype, "padding")
    assert (o[0] == 0).all().item() and torch.isinf(lse[0]).all().item() and (lse[0] < 0).all().item()


def test_kv_len_device_tensor_and_clamping():
    """A device kv_len is passed through; values outside [0, N] are clamped by the kernel."""
    N, D = 100, 128
    x = generate(4, 1, N, D, "bf16", causal=False, seed=78)
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    say("device kv_len with out-of-range values")
    o, lse = fa.forward(q, k, v, causal=False, scale=x.scale,
                        kv_len=torch.tensor([-5, 0, 50, 1000], dtype=torch.int32, device=dev))
    torch.cuda.synchronize()
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=False,
                              kv_len=np.array([0, 0, 50, 100]))
    compare(o, lse, ro, rl, "bf16", "clamped kv_len")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_and_zero_inputs(dtype):
    """N=1 attends only to itself; all-zero Q, K give the running mean of V (uniform weights)."""
    say(f"single token dtype={dtype}")
    x = generate(2, 2, 1, 64, dtype, causal=False, seed=79)
    o, lse = run_gpu(x)
    atol, _ = tol(dtype)
    assert torch.allclose(o.float().cpu(), x.v.float(), atol=atol, rtol=0)
    say(f"zero inputs dtype={dtype}")
    x = generate(1, 2, 150, 128, dtype, causal=True, seed=80)
    x.q.zero_()
    x.k.zero_()
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True)
    compare(o, lse, ro, rl, dtype, "zero Q,K")
    want = torch.log(torch.arange(1, 151, dtype=torch.float64))
    assert torch.allclose(lse.double().cpu()[0, 0], want, atol=1e-5)


def test_large_logits_no_overflow():
    """Logits up to about 100*D (rows of Q scaled up to x100 in f16): finite and matching."""
    N, D = 256, 64
    say("large logits f16")
    x = generate(1, 2, N, D, "f16", causal=True, seed=81, q_row_scale=True)
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True)
    assert np.abs(rl).max() > 100
    compare(o, lse, ro, rl, "f16", "large logits")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
def test_large_negative_logits(dtype, causal):
    """Every logit of a row shifted far below zero (a constant coordinate: Q[..., -1] = a,
    K[..., -1] = 1): nothing may underflow to an empty row, O matches, LSE shifts with it.
    float32 resolves a logit of magnitude |L| only to about |L| * 6e-8, so its shift is
    kept near -100 (scaled), where that stays inside the 1e-5 bound; the 16-bit inputs
    go to scaled logits of several thousand below zero."""
    N, D = 300, 64
    say(f"large negative logits dtype={dtype} causal={causal}")
    x = generate(2, 2, N, D, dtype, causal=causal, seed=83)
    a = {"f32": -800.0, "f16": -6000.0, "bf16": -40000.0}[dtype]
    x.q[..., -1] = a
    x.k[..., -1] = 1.0
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
    assert rl.max() < -80
    compare(o, lse, ro, rl, dtype, "large negative logits", lse_f32_spacing=True)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_rising_and_jumping_logits(dtype, D, causal):
    """Row maxima that keep rising along the keys (Q[..., -1] = 1, K[j, -1] = 2j: the scaled
    base-2 logit grows by 0.26-0.36 per key, 14-24 per 64-key tile, above the reference's
    slack of 8), so the reference maximum has to move at every key tile; and a single key
    whose logit stands 27-38 base-2 units above the rest, in the second half of a 64-key
    tile (key 100), so it moves on a key that sits late in its tile. Both against the oracle."""
    N = 300
    say(f"rising and jumping logits dtype={dtype} D={D} causal={causal}")
    x = generate(1, 2, N, D, dtype, causal=causal, seed=87)
    x.q[..., -1] = 1.0
    x.k[..., -1] = 2.0 * torch.arange(N, dtype=torch.float32).to(x.k.dtype)
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
    compare(o, lse, ro, rl, dtype, "rising logits", lse_f32_spacing=True)
    x = generate(1, 2, N, D, dtype, causal=causal, seed=88)
    x.q[..., -1] = 4.0
    x.k[..., -1] = 0.0
    x.k[:, :, 100, -1] = 60.0
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
    compare(o, lse, ro, rl, dtype, "jumping logit", lse_f32_spacing=True)


def test_deterministic():
    """No atomics: two runs are bitwise identical."""
    say("determinism bf16 N=1000")
    x = generate(2, 2, 1000, 128, "bf16", causal=True, seed=82)
    o1, l1 = run_gpu(x)
    o2, l2 = run_gpu(x)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_batch_is_noop():
    dev = torch.device("cuda:0")
    q = torch.empty(0, 2, 16, 64, dtype=torch.bfloat16, device=dev)
    o, lse = fa.forward(q, q.clone(), q.clone())
    assert o.shape == q.shape and lse.shape == (0, 2, 16)


def oracle_workers():
    return max(1, min(16, len(os.sched_getaffinity(0))))


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_full_size_workload(name):
    """Each named workload at full size, launched as the benchmark launches it: every element
    of O and LSE against the float64 oracle over the whole workload, plus properties that hold
    at any size."""
    w = WORKLOADS[name]
    say(f"full-size workload {name}: generating inputs")
    x = generate_workload(w)
    say(f"full-size workload {name}: GPU run")
    o, lse = run_gpu(x)
    assert not torch.isnan(o).any().item(), "NaN (or an unwritten element) in O"
    assert not torch.isnan(lse).any().item(), "NaN (or an unwritten element) in LSE"
    if x.kv_len is not None:
        zb = int(x.meta["zero_batch"])
        assert (o[zb] == 0).all().item(), "fully masked batch must be exactly zero"
        assert (torch.isinf(lse[zb]) & (lse[zb] < 0)).all().item(), "fully masked batch must have LSE = -inf"
    if w.causal:
        # Causal row 0 attends only to key 0 (in every batch that has a key at all).
        atol, _ = tol(w.dtype)
        live = [b for b in range(w.B) if x.kv_len is None or x.kv_len[b] > 0]
        assert torch.allclose(o.float().cpu()[live, :, 0], x.v[live, :, 0].float(), atol=atol, rtol=0)
    nw = oracle_workers()
    say(f"full-size workload {name}: float64 oracle over all {w.B * w.H} heads x {w.N} rows ({nw} threads)")
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=w.causal, kv_len=x.kv_len,
                              workers=nw)
    eo, el, ratio_o, ratio_l = compare(o, lse, ro, rl, w.dtype, name)
    del ro, rl
    say(f"full-size workload {name}: all {o.numel()} elements of O and {lse.numel()} of LSE within bounds; "
        f"max |O err| {eo:.3e} (err/bound {ratio_o:.3f}), max |LSE err| {el:.3e} (err/bound {ratio_l:.3f})")
    say(f"full-size workload {name}: determinism")
    o2, l2 = run_gpu(x)
    assert torch.equal(o, o2) and torch.equal(lse, l2)


# ---------------------------------------------------------------- workgroup shape by problem size
@pytest.mark.parametrize("D", [96, 128])
@pytest.mark.parametrize("N", [1792, 2048])
def test_causal_workgroup_shape_threshold(D, N):
    """Causal D = 96 / 128 problems run 4-wave workgroups below 2048 tiles of 256 query rows
    and 8-wave ones from there on: B=16 H=16 gives 1792 and 2048 such tiles. Sampled rows
    of a few heads against the oracle, on both sides of the threshold."""
    B, H = 16, 16
    say(f"workgroup-shape threshold D={D} N={N} ({B * H * ((N + 255) // 256)} tiles of 256 rows)")
    x = generate(B, H, N, D, "bf16", causal=True, seed=4100 + N + D)
    o, lse = run_gpu(x)
    ocpu, lcpu = o.float().cpu(), lse.cpu()
    rows = np.array([0, 1, 127, 128, 255, 256, 1000, N - 129, N - 128, N - 1])
    for b, h in [(0, 0), (7, 9), (15, 15)]:
        ro, rl = oracle.attention(to_f64(x.q[b:b + 1, h:h + 1]), to_f64(x.k[b:b + 1, h:h + 1]),
                                  to_f64(x.v[b:b + 1, h:h + 1]), x.scale, causal=True, rows=rows)
        compare(ocpu[b:b + 1, h:h + 1, rows], lcpu[b:b + 1, h:h + 1, rows], ro, rl, "bf16", f"D={D} N={N} b={b} h={h}")


# ---------------------------------------------------------------- head dimensions 32, 96 and 256
@pytest.mark.parametrize("dtype,D", [("f32", 32), ("bf16", 32), ("f16", 32), ("f32", 96), ("bf16", 96), ("f16", 96),
                                     ("bf16", 256), ("f16", 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_other_head_dims(dtype, D, causal):
    """Ragged N around the tile edges for D = 32, 96 and 256, with and without padding."""
    for N in (1, 17, 64, 129, 300):
        say(f"head dim dtype={dtype} D={D} causal={causal} N={N}")
        x = generate(3, 2, N, D, dtype, causal=causal, seed=2000 + N + D)
        kv = np.array([N, max(N - 5, 0), 0], dtype=np.int32)
        o, lse = run_gpu(x, kv_len=kv)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal, kv_len=kv)
        compare(o, lse, ro, rl, dtype, f"D={D} N={N}")


# ---------------------------------------------------------------- strided layouts
def _strided_run(x, q, k, v, out, causal, kv=None):
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    o, lse = fa.forward(q, k, v, causal=causal, scale=x.scale, out=out, lse=lse,
                        kv_len=None if kv is None else torch.as_tensor(kv, dtype=torch.int32))
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 64), ("f32", 64), ("bf16", 96), ("f32", 96), ("bf16", 256)])
@pytest.mark.parametrize("causal", [False, True])
def test_bnhd_layout(dtype, D, causal):
    """[B, N, H, D] storage seen as [B, H, N, D] (token stride H*D, head stride D), for
    Q, K, V and O alike."""
    B, H, N = 2, 3, 200
    say(f"BNHD layout dtype={dtype} D={D} causal={causal}")
    x = generate(B, H, N, D, dtype, causal=causal, seed=3000 + D)
    dev = torch.device("cuda:0")
    q, k, v = (t.transpose(1, 2).contiguous().to(dev).transpose(1, 2) for t in (x.q, x.k, x.v))
    assert q.stride() == (N * H * D, D, H * D, 1)
    out = torch.full((B, N, H, D), float("nan"), dtype=q.dtype, device=dev).transpose(1, 2)
    o, lse = _strided_run(x, q, k, v, out, causal)
    assert o.data_ptr() == out.data_ptr()
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
    compare(o, lse, ro, rl, dtype, "BNHD")


def test_padded_rows_and_offset_views():
    """Rows padded to twice their length (token stride 2D) and views that start mid-buffer."""
    B, H, N, D = 2, 2, 150, 64
    say("padded rows")
    x = generate(B, H, N, D, "bf16", causal=True, seed=3100)
    dev = torch.device("cuda:0")

    def padded(t, shift):
        buf = torch.zeros(B, H, N, 2 * D, dtype=t.dtype, device=dev)
        buf[..., shift:shift + D] = t.to(dev)
        return buf[..., shift:shift + D]

    q, k, v = padded(x.q, 0), padded(x.k, D), padded(x.v, 8)
    out = torch.full((B, H, N, 2 * D), float("nan"), dtype=q.dtype, device=dev)[..., D:]
    o, lse = _strided_run(x, q, k, v, out, True)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True)
    compare(o, lse, ro, rl, "bf16", "padded rows")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_shared_kv_head(dtype):
    """One K/V head shared by every query head (head stride 0 on K and V)."""
    B, H, N, D = 2, 4, 180, 128 if dtype == "bf16" else 64
    say(f"shared K/V head dtype={dtype}")
    x = generate(B, H, N, D, dtype, causal=True, seed=3200)
    dev = torch.device("cuda:0")
    k1, v1 = x.k[:, :1].contiguous(), x.v[:, :1].contiguous()
    k = k1.to(dev).expand(B, H, N, D)
    v = v1.to(dev).expand(B, H, N, D)
    assert k.stride(1) == 0
    q = x.q.to(dev)
    kv = np.array([N, 77], dtype=np.int32)
    o, lse = _strided_run(x, q, k, v, None, True, kv)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(k1.expand(B, H, N, D)), to_f64(v1.expand(B, H, N, D)),
                              x.scale, causal=True, kv_len=kv)
    compare(o, lse, ro, rl, dtype, "shared K/V head")


# ---------------------------------------------------------------- scale of either sign
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 32), ("bf16", 64), ("bf16", 96),
                                     ("bf16", 128), ("bf16", 256), ("f16", 64), ("f16", 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_scale_of_either_sign(dtype, D, causal):
    """The softmax scale may be negative or zero ("vectorized-flash-attention-kernel",
    Constructor options: softmaxScale carries no sign restriction). A negative scale makes the
    row maximum that of s*scale, not scale*max(s); a zero scale weighs every valid key the
    same. Padding keys hold NaN. The plain forward and the split forward (3 parts)."""
    N = 200
    kv = np.array([0, 1, 64, 131, 200], dtype=np.int32)
    x = generate(5, 2, N, D, dtype, causal=causal, seed=3300 + D)
    k0, v0 = x.k.clone(), x.v.clone()
    for b, L in enumerate(kv):
        x.k[b, :, L:] = float("nan")
        x.v[b, :, L:] = float("nan")
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (x.q, x.k, x.v))
    kl = torch.as_tensor(kv)
    for sc in (-x.scale, -3.0 * x.scale, 0.0):
        say(f"scale {sc:+.4f} dtype={dtype} D={D} causal={causal}")
        ro, rl = oracle.attention(to_f64(x.q), to_f64(k0), to_f64(v0), sc, causal=causal, kv_len=kv)
        for splits in (1, 3):
            o, lse = fa.forward(q, k, v, causal=causal, scale=sc, kv_len=kl, n_splits=splits,
                                out=torch.full_like(q, float("nan")),
                                lse=torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev))
            torch.cuda.synchronize()
            compare(o, lse, ro, rl, dtype, f"scale {sc:+.4f} splits {splits}")
        if sc == 0.0:
            counts = np.minimum(kv[:, None], np.arange(1, N + 1)[None, :]) if causal else np.repeat(kv[:, None], N, 1)
            want = np.where(counts > 0, np.log(np.maximum(counts, 1)), -np.inf)
            got = lse.cpu().double().numpy()
            assert np.allclose(got, np.broadcast_to(want[:, None, :], got.shape), atol=tol(dtype)[0], rtol=0)


# ---------------------------------------------------------------- float32: both forward paths
@pytest.mark.parametrize("D", [32, 64, 96, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_f32_wave_split_and_regular_paths(D, causal):
    """float32 problems of at most 64 query tiles of 128 rows run 32-row blocks whose key tiles
    are split over the waves of a workgroup and merged through LDS; larger ones run the regular
    kernel. Shapes on both sides of that line (64 and 65 tiles of 128 rows, ragged N, key
    padding with NaN-filled padding keys), every element against the oracle."""
    for B, H, N in ((2, 4, 1000), (5, 13, 129), (1, 1, 1), (1, 1, 33)):
        tiles = B * H * ((N + 127) // 128)
        say(f"f32 paths D={D} causal={causal} B={B} H={H} N={N} ({tiles} tiles of 128 rows)")
        x = generate(B, H, N, D, "f32", causal=causal, seed=3400 + N + D)
        kv = np.array([max(N - 17 * b, 0) for b in range(B)], dtype=np.int32)
        k0, v0 = x.k.clone(), x.v.clone()
        for b, L in enumerate(kv):
            x.k[b, :, L:] = float("nan")
            x.v[b, :, L:] = float("nan")
        o, lse = run_gpu(x, kv_len=kv)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(k0), to_f64(v0), x.scale, causal=causal, kv_len=kv)
        compare(o, lse, ro, rl, "f32", f"B={B} H={H} N={N}")


# ---------------------------------------------------------------- untested tiles: sum check and retry
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_jumps_after_quiet_tiles(dtype, D, causal):
    """After a few quiet key tiles the 16-bit kernels form a tile's probabilities without first
    taking its row maximum, and check each lane's sum of them instead. One key whose base-2 logit
    stands about 12, 40 or 200 above the rest, placed well past the tiles that test the reference
    first (key 300 of 1000, and a second one at key 700), exercises the three outcomes: a sum above
    2^8 (the next tile tests again), a sum beyond the bound (the workgroup computes its unit
    again, every tile tested), and an infinite sum. Each against the oracle."""
    N = 1000
    c = float(np.float32(1.0 / np.sqrt(D))) * 1.4426950408889634   # base-2 logit per unit of q.k
    for jump in (12.0, 40.0, 200.0):
        say(f"reference jump +{jump} dtype={dtype} D={D} causal={causal}")
        x = generate(2, 2, N, D, dtype, causal=causal, seed=3500 + D + int(jump))
        x.q[..., -1] = 1.0
        x.k[..., -1] = 0.0
        x.k[:, :, 300, -1] = jump / c
        x.k[:, 1, 700, -1] = 1.5 * jump / c
        o, lse = run_gpu(x)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
        compare(o, lse, ro, rl, dtype, f"jump +{jump}")
        o2, l2 = run_gpu(x)
        assert torch.equal(o, o2) and torch.equal(lse, l2), "not deterministic"


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_untested_probability_near_float16_limit(dtype, D, causal):
    """One key whose probability, taken against a reference fixed by earlier tiles, lands on an
    untested tile at 2^14.9 (finite in float16, below the sum bound: kept) and at 2^15.9999
    (about 65531, which rounds to infinity in float16: the sum bound must send the unit to the
    all-tested pass). Every other key after the first two tiles has a negligible probability,
    so that lane's sum is that one probability. Against the oracle."""
    N = 512
    for lg in (14.9, 15.9999):
        say(f"untested probability 2^{lg} dtype={dtype} D={D} causal={causal}")
        x = generate(1, 2, N, D, dtype, causal=causal, seed=3600 + D)
        x.scale = float(np.float32(lg / 1.4426950408889634))  # base-2 logit of q.k = 1
        x.q.zero_()
        x.q[..., 0] = 1.0
        x.k.zero_()                 # keys 0..127: logit 0, which fixes the reference at 0
        x.k[:, :, 128:, 0] = -2.0   # then probabilities of about 2^-32
        x.k[:, :, 300, 0] = 1.0     # one key at the chosen logit, in a later (untested) tile
        o, lse = run_gpu(x)
        ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=causal)
        compare(o, lse, ro, rl, dtype, f"probability 2^{lg}")


# ---------------------------------------------------------------- key groups (long causal, D = 64)
@pytest.mark.parametrize("dtype,N,H", [("bf16", 8192, 2), ("f16", 7000, 3)])
def test_key_groups_long_causal(dtype, N, H):
    """Causal D = 64 with few heads and long query tiles takes the key-group kernel: three
    groups of waves split each query tile's key tiles and merge their partial states. Every
    element against the oracle (ragged N included), with a NaN prefill and a determinism check."""
    x = generate(1, H, N, 64, dtype, causal=True, seed=3700 + N)
    say(f"key groups {dtype} N={N} H={H}")
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, workers=oracle_workers())
    compare(o, lse, ro, rl, dtype, f"key groups N={N}")
    o2, l2 = run_gpu(x)
    assert torch.equal(o, o2) and torch.equal(lse, l2), "not deterministic"


def test_key_groups_reference_jump():
    """A key whose logit stands 40 (base 2) above the rest, late in a long causal row, under the
    key-group kernel: the group that holds it overflows its untested sum and the whole workgroup
    takes the all-tested pass; the merge then weighs the groups by their references."""
    N = 8192
    c = float(np.float32(1.0 / np.sqrt(64))) * 1.4426950408889634
    x = generate(1, 2, N, 64, "bf16", causal=True, seed=3800)
    x.q[..., -1] = 1.0
    x.k[..., -1] = 0.0
    x.k[:, :, 6000, -1] = 40.0 / c
    say("key groups reference jump")
    o, lse = run_gpu(x)
    ro, rl = oracle.attention(to_f64(x.q), to_f64(x.k), to_f64(x.v), x.scale, causal=True, workers=oracle_workers())
    compare(o, lse, ro, rl, "bf16", "key groups jump")
