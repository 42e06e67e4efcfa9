"""CPU check of the longest-first unit order that key-padded launches decode on the device.

`longest_first` (csrc/fa_fwd_kernel.h) gives each workgroup its unit from closed-form counts of
a head's units with at least t units of work. This test restates those steps in Python and
checks three properties against brute-force work counts taken from each kernel's loop bounds:
- the decode is a bijection onto the XCD's units;
- the work it infers for a unit equals the work the kernel's loop bounds give it;
- each XCD's sequence of work never increases.
Models: the forward and dQ kernels (query tiles of BR rows, key tiles of BC), and the dK/dV
kernels (key tiles of 128 keys, query steps of 64 rows). The dispatch puts workgroup bid on XCD
bid % 8, and an XCD holds head slots [x*hx, (x+1)*hx), with the slots running over the batch
fastest.
"""

import random

import pytest


def cdiv(a, b):
    return -(-a // b)


def decode(bid, B, H, N, kv_len, per_head, max_work, more_work_last, at_least):
    heads = B * H
    hx = heads // 8
    x, i = bid % 8, bid // 8
    kv = [min(max(int(kv_len[(x * hx + s) % B]), 0), N) for s in range(hx)]
    count = lambda t: sum(at_least(t, k) for k in kv)
    lo, hi = 0, max_work + 1
    assert count(hi) == 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if count(mid) > i:
            lo = mid
        else:
            hi = mid
    ts = lo
    j = i - count(ts + 1)
    e = [at_least(ts, k) - at_least(ts + 1, k) for k in kv]
    pre, s = 0, hx - 1
    for idx, ev in enumerate(e):
        if pre + ev > j:
            s = idx
            break
        pre += ev
    jj = j - pre
    above = at_least(ts + 1, kv[s])
    unit = per_head - 1 - above - jj if more_work_last else above + jj
    slot = x * hx + s
    return (slot % B) * H + slot // B, unit, ts


def query_tile_model(N, causal, BR, BC):
    per_head = cdiv(N, BR)

    def at_least(t, kvl):
        if t <= 0:
            return per_head
        if kvl <= (t - 1) * BC:
            return 0
        return max(0, per_head - ((t - 1) * BC) // BR) if causal else per_head

    def work(kvl, qt):  # the forward / dQ loop: key tiles below min(kv_len, end of the query tile)
        hi = min(kvl, BR * (qt + 1)) if causal else kvl
        return cdiv(hi, BC) if hi > 0 else 0

    return per_head, cdiv(N, BC), True, at_least, work


def key_tile_model(N, causal, BKV=128, BQ=64):
    per_head, nq = cdiv(N, BKV), cdiv(N, BQ)

    def at_least(t, kvl):
        if t <= 0:
            return per_head
        live = cdiv(kvl, BKV)
        if not causal:
            return live if t <= nq else 0
        lim = nq - t + 1
        return 0 if lim <= 0 else min(live, cdiv(lim * BQ, BKV))

    def work(kvl, kt):  # the dK/dV loop: query tiles t0 .. nqt-1 of a key tile below kv_len
        k0 = kt * BKV
        if k0 >= kvl:
            return 0
        return nq - (k0 // BQ if causal else 0)

    return per_head, nq, False, at_least, work


def models(N, causal):
    yield "forward BR=128 BC=64", query_tile_model(N, causal, 128, 64)
    yield "forward BR=256 BC=64", query_tile_model(N, causal, 256, 64)
    yield "forward BR=128 BC=128", query_tile_model(N, causal, 128, 128)
    yield "dK/dV", key_tile_model(N, causal)


def check_case(B, H, N, kv_len, causal):
    for name, (per_head, max_work, more_last, at_least, work) in models(N, causal):
        seen, last = set(), {}
        for bid in range(B * H * per_head):
            bh, unit, ts = decode(bid, B, H, N, kv_len, per_head, max_work, more_last, at_least)
            assert 0 <= unit < per_head, name
            assert (bh, unit) not in seen, f"{name}: unit decoded twice"
            seen.add((bh, unit))
            kvl = min(max(int(kv_len[bh // H]), 0), N)
            assert ts == work(kvl, unit), f"{name}: decoded work {ts}, loop bounds give {work(kvl, unit)}"
            x = bid % 8
            assert last.get(x, ts) >= ts, f"{name}: XCD {x} order increases"
            last[x] = ts
        assert len(seen) == B * H * per_head, f"{name}: units missed"


@pytest.mark.parametrize("causal", [True, False])
def test_named_padded_shape(causal):
    """B8 H8 N4096 with the benchmark's kv_len draw (one batch element at 0, one at 15)."""
    check_case(8, 8, 4096, [2281, 1364, 15, 3065, 0, 2953, 2560, 1991], causal)


def test_random_shapes():
    rng = random.Random(11)
    done = 0
    while done < 150:
        B = rng.choice([1, 2, 4, 8, 16])
        H = rng.choice([1, 2, 4, 8, 16])
        if (B * H) % 8 or B * H // 8 > 64:
            continue
        N = rng.choice([1, 5, 64, 127, 128, 129, 300, 1000, 2049])
        kv = [rng.choice([0, 1, N, N - 1, rng.randint(-5, N + 5)]) for _ in range(B)]
        check_case(B, H, N, kv, rng.random() < 0.7)
        done += 1
