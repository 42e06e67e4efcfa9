"""Pins for an exact-attention implementation with the oracle's signature.

Each ``pin_*`` function takes ``attn(q, k, v, scale, causal=False, kv_len=None)
-> (o, lse)`` (float64 arrays [B,H,N,D] in, [B,H,N,Dv] and [B,H,N] out) and
raises AssertionError when the implementation breaks a fact that the pages or
the mathematics fix. None of them re-runs the implementation's own formula:
they compare against 50-digit brute force, hand-derived closed forms, library
routines on special cases, and invariants. ``test_oracle.py`` runs them on the
oracle; ``test_oracle_mutants.py`` runs them on one-line mutants of the oracle
and requires every mutant to be caught.
"""

import json
import os

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "closed_forms.json")


def _close(got, want, rtol, atol, what):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    inf_want = np.isinf(want)
    assert np.array_equal(np.isinf(got), inf_want), f"{what}: infinities differ"
    assert np.array_equal(got[inf_want], want[inf_want]), f"{what}: infinite entries differ"
    assert not np.isnan(got).any(), f"{what}: NaN"
    fin = ~inf_want
    err = np.abs(got[fin] - want[fin])
    bound = atol + rtol * np.abs(want[fin])
    assert (err <= bound).all(), f"{what}: max err {err.max() if err.size else 0:.3e}"


# --------------------------------------------------------------------------- brute force
def brute_force(q, k, v, scale, causal, kv_len):
    """Direct softmax definition at 50 digits, with no max subtraction (mpmath has no overflow)."""
    B, H, N, D = q.shape
    Dv = v.shape[3]
    o = np.zeros((B, H, N, Dv))
    lse = np.zeros((B, H, N))
    with mpmath.workdps(50):
        sc = mpmath.mpf(float(scale))
        for b in range(B):
            L = N if kv_len is None else int(kv_len[b])
            for h in range(H):
                for i in range(N):
                    J = [j for j in range(N) if j < L and (not causal or j <= i)]
                    if not J:
                        lse[b, h, i] = -np.inf
                        continue
                    e = {j: mpmath.exp(sc * mpmath.fsum(mpmath.mpf(float(q[b, h, i, d])) * mpmath.mpf(float(k[b, h, j, d]))
                                                        for d in range(D))) for j in J}
                    z = mpmath.fsum(e.values())
                    for c in range(Dv):
                        o[b, h, i, c] = float(mpmath.fsum(e[j] * mpmath.mpf(float(v[b, h, j, c])) for j in J) / z)
                    lse[b, h, i] = float(mpmath.log(z))
    return o, lse


def pin_brute_force_exhaustive(attn):
    """Every causal flag and kv_len on tiny dyadic inputs; non-square shapes so a transposed operand shows."""
    rng = np.random.default_rng(11)
    for N in (1, 2, 3, 4):
        for D in (1, 2, 3):
            q = rng.integers(-8, 9, size=(1, 1, N, D)) / 4.0
            k = rng.integers(-8, 9, size=(1, 1, N, D)) / 4.0
            v = rng.integers(-8, 9, size=(1, 1, N, D + 1)) / 4.0
            for scale in (1.0, 0.3, -0.6):
                for causal in (False, True):
                    for L in range(N + 1):
                        kv = np.array([L])
                        want = brute_force(q, k, v, scale, causal, kv)
                        got = attn(q, k, v, scale, causal=causal, kv_len=kv)
                        tag = f"brute N={N} D={D} scale={scale} causal={causal} kv_len={L}"
                        _close(got[0], want[0], 1e-13, 1e-14, tag + " O")
                        _close(got[1], want[1], 1e-13, 1e-14, tag + " LSE")


def pin_brute_force_batched(attn):
    """Several batches and heads with per-batch kv_len, random normal values."""
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, 3, 5, 4))
    k = rng.standard_normal((2, 3, 5, 4))
    v = rng.standard_normal((2, 3, 5, 6))
    kv = np.array([3, 5])
    for causal in (False, True):
        want = brute_force(q, k, v, 0.5, causal, kv)
        got = attn(q, k, v, 0.5, causal=causal, kv_len=kv)
        _close(got[0], want[0], 1e-13, 1e-14, f"batched causal={causal} O")
        _close(got[1], want[1], 1e-13, 1e-14, f"batched causal={causal} LSE")


# --------------------------------------------------------------------------- closed forms
def pin_golden(attn):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    with mpmath.workdps(50):
        env = {"e": mpmath.e, "log": mpmath.log, "exp": mpmath.exp, "inf": mpmath.inf, "__builtins__": {}}

        def ev(x):
            return float(eval(x, env, {}))   # expressions from the committed fixture only

        for c in cases:
            q = np.array([[[[ev(x) for x in row] for row in c["q"]]]])
            k = np.array([[[[ev(x) for x in row] for row in c["k"]]]])
            v = np.array([[[[ev(x) for x in row] for row in c["v"]]]])
            kv = None if c["kv_len"] is None else np.array([c["kv_len"]])
            want_o = np.array([[[[ev(x) for x in row] for row in c["o"]]]])
            want_l = np.array([[[ev(x) for x in c["lse"]]]])
            got = attn(q, k, v, ev(c["scale"]), causal=c["causal"], kv_len=kv)
            _close(got[0], want_o, 1e-14, 1e-14, c["id"] + " O")
            _close(got[1], want_l, 1e-14, 1e-14, c["id"] + " LSE")


def pin_single_token(attn):
    """N = 1 attends only to itself; causal row 0 of any length does too (bitwise)."""
    rng = np.random.default_rng(13)
    for causal in (False, True):
        q = rng.standard_normal((2, 2, 1, 16))
        k = rng.standard_normal((2, 2, 1, 16))
        v = rng.standard_normal((2, 2, 1, 16))
        o, lse = attn(q, k, v, 0.25, causal=causal)
        assert np.array_equal(o, v), "N=1 output is not V"
        want = brute_force(q, k, v, 0.25, causal, None)[1]
        _close(lse, want, 1e-14, 1e-15, "N=1 LSE")
    q = rng.standard_normal((1, 2, 9, 8))
    k = rng.standard_normal((1, 2, 9, 8))
    v = rng.standard_normal((1, 2, 9, 8))
    o, lse = attn(q, k, v, 0.35, causal=True)
    assert np.array_equal(o[:, :, 0], v[:, :, 0]), "causal row 0 is not V[0]"


def pin_zero_inputs(attn):
    """All-zero Q and K: uniform weights, O_i = mean of V over the valid prefix, LSE = ln(count)."""
    rng = np.random.default_rng(14)
    B, H, N, D = 2, 2, 7, 5
    q = np.zeros((B, H, N, D))
    k = np.zeros((B, H, N, D))
    v = rng.standard_normal((B, H, N, D))
    kv = np.array([4, 7])
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.125, causal=causal, kv_len=kv)
        for b in range(B):
            for i in range(N):
                cnt = min(int(kv[b]), i + 1) if causal else int(kv[b])
                _close(o[b, :, i], v[b, :, :cnt].mean(axis=1), 1e-14, 1e-15, f"zero-input mean b={b} i={i}")
                _close(lse[b, :, i], np.full(H, np.log(cnt)), 1e-14, 1e-15, f"zero-input LSE b={b} i={i}")
    o, lse = attn(q, k, np.zeros_like(v), 0.125, causal=False)
    assert not o.any(), "all-zero V must give zero O"


def pin_identical_keys(attn):
    """Identical key rows give uniform weights whatever Q is."""
    rng = np.random.default_rng(15)
    q = rng.standard_normal((1, 3, 6, 4))
    k = np.broadcast_to(rng.standard_normal((1, 3, 1, 4)), (1, 3, 6, 4)).copy()
    v = rng.standard_normal((1, 3, 6, 4))
    o, lse = attn(q, k, v, 0.5, causal=True)
    for i in range(6):
        _close(o[0, :, i], v[0, :, :i + 1].mean(axis=1), 1e-13, 1e-14, f"identical keys row {i}")


def pin_large_logits(attn):
    """Logits up to 100*D: the winning key takes all the weight, exactly; no overflow."""
    D = 16
    scale = 1.0 / np.sqrt(D)
    t = np.array([0.25, 1.0, -0.5, 0.4, 0.1])          # key 1 wins; runner-up gap > 745
    c = 100.0 * D / scale
    N = t.size
    q = np.zeros((1, 1, N, D))
    k = np.zeros((1, 1, N, D))
    q[..., 0] = c
    k[0, 0, :, 0] = t
    v = np.random.default_rng(16).standard_normal((1, 1, N, D))
    o, lse = attn(q, k, v, scale, causal=False)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow at large logits"
    assert np.array_equal(o[0, 0], np.broadcast_to(v[0, 0, 1], (N, D))), "winner does not take all"
    _close(lse, np.full((1, 1, N), 100.0 * D), 1e-15, 0.0, "large-logit LSE")
    # Causal: row 0 cannot see the winning key 1, whose logit dwarfs its own; it must still
    # put all its weight on key 0 (a max taken over masked keys would underflow every weight).
    o, lse = attn(q, k, v, scale, causal=True)
    assert np.isfinite(o).all() and np.isfinite(lse).all(), "overflow at large causal logits"
    assert np.array_equal(o[0, 0, 0], v[0, 0, 0]), "causal row 0 must attend to key 0 only"
    assert np.array_equal(o[0, 0, 1:], np.broadcast_to(v[0, 0, 1], (N - 1, D))), "winner does not take all"
    _close(lse[0, 0, 0], 100.0 * D * t[0], 1e-15, 0.0, "causal large-logit LSE row 0")


def pin_shift(attn):
    """A constant added to every logit of a row (large and negative) leaves O alone and shifts LSE."""
    rng = np.random.default_rng(17)
    B, H, N, D = 1, 2, 9, 8
    scale = 0.25
    q = rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    v = rng.standard_normal((B, H, N, D))
    a = -100.0 * D / scale
    q2 = np.concatenate([q, np.full((B, H, N, 1), a)], axis=-1)
    k2 = np.concatenate([k, np.ones((B, H, N, 1))], axis=-1)
    for causal in (False, True):
        o1, l1 = attn(q, k, v, scale, causal=causal)
        o2, l2 = attn(q2, k2, v, scale, causal=causal)
        _close(o2, o1, 1e-10, 1e-11, "shifted O")
        _close(l2 - scale * a, l1, 1e-10, 1e-10, "shifted LSE")


def pin_masks(attn):
    """kv_len = 0 gives zeros and -inf; causal row i equals the padding mask kv_len = i+1."""
    rng = np.random.default_rng(18)
    B, H, N, D = 3, 2, 6, 4
    q = rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    v = rng.standard_normal((B, H, N, D))
    kv = np.array([0, 6, 3])
    for causal in (False, True):
        o, lse = attn(q, k, v, 0.5, causal=causal, kv_len=kv)
        assert not np.isnan(o).any() and not np.isnan(lse).any(), "NaN in masked output"
        assert np.array_equal(o[0], np.zeros_like(o[0])), "fully masked rows must be zero"
        assert (lse[0] == -np.inf).all(), "fully masked rows must have LSE = -inf"
    oc, lc = attn(q, k, v, 0.5, causal=True)
    for i in range(N):
        op, lp = attn(q, k, v, 0.5, causal=False, kv_len=np.full(B, i + 1))
        _close(oc[:, :, i], op[:, :, i], 1e-14, 1e-15, f"causal row {i} vs padding")
        _close(lc[:, :, i], lp[:, :, i], 1e-14, 1e-15, f"causal LSE row {i} vs padding")


def pin_permutation(attn):
    """Without the causal mask, a joint permutation of key and value rows changes nothing."""
    rng = np.random.default_rng(19)
    q = rng.standard_normal((1, 2, 7, 5))
    k = rng.standard_normal((1, 2, 7, 5))
    v = rng.standard_normal((1, 2, 7, 3))
    perm = rng.permutation(7)
    o1, l1 = attn(q, k, v, 0.4, causal=False)
    o2, l2 = attn(q, k[:, :, perm], v[:, :, perm], 0.4, causal=False)
    _close(o2, o1, 1e-13, 1e-14, "permuted O")
    _close(l2, l1, 1e-13, 1e-14, "permuted LSE")


def pin_convex(attn):
    """O is a convex combination of the valid V rows: inside their per-column range."""
    rng = np.random.default_rng(20)
    B, H, N, D = 2, 2, 11, 4
    q = 3.0 * rng.standard_normal((B, H, N, D))
    k = rng.standard_normal((B, H, N, D))
    v = rng.standard_normal((B, H, N, D))
    kv = np.array([5, 11])
    o, _ = attn(q, k, v, 0.7, causal=True, kv_len=kv)
    for b in range(B):
        for i in range(N):
            cnt = min(int(kv[b]), i + 1)
            lo = v[b, :, :cnt].min(axis=1) - 1e-12
            hi = v[b, :, :cnt].max(axis=1) + 1e-12
            assert ((o[b, :, i] >= lo) & (o[b, :, i] <= hi)).all(), f"not convex b={b} i={i}"


def pin_scale_sign(attn):
    """A negative scale is the positive one applied to -Q (exactly, since negation is exact),
    and matches 50-digit brute force; a zero scale weighs every valid key the same: O is the
    mean of V over the valid prefix and LSE = ln(count), whatever Q and K hold."""
    rng = np.random.default_rng(16)
    q = rng.standard_normal((2, 2, 6, 3))
    k = rng.standard_normal((2, 2, 6, 3))
    v = rng.standard_normal((2, 2, 6, 4))
    kv = np.array([6, 4])
    for causal in (False, True):
        neg = attn(q, k, v, -0.7, causal=causal, kv_len=kv)
        flip = attn(-q, k, v, 0.7, causal=causal, kv_len=kv)
        _close(neg[0], flip[0], 0.0, 0.0, f"negative scale = negated Q causal={causal} O")
        _close(neg[1], flip[1], 0.0, 0.0, f"negative scale = negated Q causal={causal} LSE")
        want = brute_force(q, k, v, -0.7, causal, kv)
        _close(neg[0], want[0], 1e-13, 1e-14, f"negative scale brute causal={causal} O")
        _close(neg[1], want[1], 1e-13, 1e-14, f"negative scale brute causal={causal} LSE")
        o, lse = attn(q, k, v, 0.0, causal=causal, kv_len=kv)
        for b in range(2):
            for i in range(6):
                cnt = min(int(kv[b]), i + 1) if causal else int(kv[b])
                _close(o[b, :, i], v[b, :, :cnt].mean(axis=1), 1e-14, 1e-15, f"zero scale mean b={b} i={i}")
                _close(lse[b, :, i], np.full(2, np.log(cnt)), 1e-14, 1e-15, f"zero scale LSE b={b} i={i}")


ALL_PINS = [pin_brute_force_exhaustive, pin_brute_force_batched, pin_golden, pin_single_token,
            pin_zero_inputs, pin_identical_keys, pin_large_logits, pin_shift, pin_masks,
            pin_permutation, pin_convex, pin_scale_sign]


def pin_query_padding(attn):
    """Query padding (q_len): rows are independent in the definition, so a row before q_len[b]
    equals the unpadded result (to rounding: the matrix products run over fewer rows), a row at
    or past it is exactly O = 0, LSE = -inf, q_len = N changes nothing, and NaN in the padding
    rows of Q reaches nothing."""
    rng = np.random.default_rng(61)
    q, k, v = (rng.standard_normal((2, 2, 7, 3)) for _ in range(3))
    for causal in (False, True):
        for kv in (None, np.array([5, 2])):
            o0, l0 = attn(q, k, v, 0.8, causal=causal, kv_len=kv)
            o, l = attn(q, k, v, 0.8, causal=causal, kv_len=kv, q_len=np.array([7, 7]))
            assert np.array_equal(o, o0) and np.array_equal(l, l0), "q_len = N"
            for ql in (np.array([3, 0]), np.array([6, 1])):
                qn = q.copy()
                for b in range(2):
                    qn[b, :, ql[b]:] = np.nan
                for qq in (q, qn):
                    with np.errstate(invalid="ignore"):
                        o, l = attn(qq, k, v, 0.8, causal=causal, kv_len=kv, q_len=ql)
                    for b in range(2):
                        L = int(ql[b])
                        tag = f"causal={causal} kv={kv} q_len={ql} b={b}"
                        _close(o[b, :, :L], o0[b, :, :L], 1e-14, 1e-15, "rows before q_len " + tag)
                        _close(l[b, :, :L], l0[b, :, :L], 1e-14, 1e-15, "LSE before q_len " + tag)
                        assert (o[b, :, L:] == 0).all(), "padding rows O " + tag
                        assert (np.isneginf(l[b, :, L:])).all(), "padding rows LSE " + tag


def failing_pins(attn):
    """Names of the pins that ``attn`` breaks (an exception of any kind counts as broken)."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except Exception:
            bad.append(pin.__name__)
    return bad
