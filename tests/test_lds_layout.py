"""CPU model of the LDS tile layouts of the 16-bit kernels (fa_fwd_mfma16.h, fa_bwd.h).

The model restates the kernels' index arithmetic: the copy plan (1 KB per copy instruction,
lane i filling the 16-byte slot i), the XOR swizzles of 16-byte chunks, the K row-fragment
reads, the V^T transpose reads, and for D = 96 the padding of 192-byte rows to the 256-byte
row of D = 128. For every head dimension and tile shape the kernels use it checks that

  * the copies fill every (row, data chunk) of a tile exactly once and never a padding slot;
  * every fragment read finds the (row, chunk) it asks for;
  * no read pass has a bank conflict, in the model of 64 banks of 4 bytes and 16 lanes per pass
    (16-byte row reads and 8-byte transpose reads alike).

The GPU parity tests check the kernels themselves; this pins the layout arithmetic they share.
"""

import pytest

# (D, key tile BC, waves NW) of the forward kernel per head dimension
FWD_SHAPES = [(32, 128, 4), (64, 64, 4), (96, 64, 8), (128, 64, 8), (256, 64, 4), (96, 64, 4), (128, 64, 4)]
# (D, tile rows, waves) of the backward's tile plans: dQ kernel K/V tiles, dK/dV Q/dO tiles, and
# the LDS dK/dV kernel's K/V and Q/dO tiles (D = 96, 128)
BWD_PLANS = [(32, 64, 4), (64, 64, 4), (96, 64, 4), (128, 64, 4), (96, 128, 8), (96, 64, 8),
             (128, 128, 8), (128, 64, 8)]


def lds_cols(D):
    return 128 if D == 96 else D


def swz_k(DL, j):
    if DL >= 128:
        return j & 15
    if DL == 64:
        return (j >> 1) & 7
    return (j >> 2) & 3


def swz_v(DL, j):
    if DL >= 128:
        return 4 * (j & 3)
    if DL == 64:
        return 4 * ((j >> 1) & 1)
    return 0


def swz_u(DL, j):
    if DL >= 128:
        return 4 * (j & 3) + ((j >> 2) & 3)
    if DL == 64:
        return 2 * ((j >> 1) & 3) + ((j >> 3) & 1)
    return (j >> 2) & 3


def acc_key(i, g):
    return 16 * (i // 8) + 8 * g + (i % 8)


def a_row_key(r):
    return acc_key(4 * (r // 8) + (r % 4), (r // 4) % 2)


def copy_slots(D, rows, nw, swz):
    """LDS byte offset -> (row, logical chunk) filled by the copy plan."""
    DL = lds_cols(D)
    rowb, cpr, vch = 2 * DL, DL // 8, D // 8
    rpb = 1024 // rowb
    lpw = rows * rowb // 1024 // nw
    assert rows * rowb % (1024 * nw) == 0
    slot = {}
    for wave in range(nw):
        for i in range(lpw):
            for lane in range(64):
                j = (wave * lpw + i) * rpb + lane // cpr
                pc = lane % cpr
                lc = pc ^ swz(DL, j)
                off = (wave * lpw + i) * 1024 + lane * 16
                assert off == j * rowb + pc * 16
                if lc < vch:                       # padding chunks are not copied
                    assert off not in slot
                    slot[off] = (j, lc)
    assert set(slot.values()) == {(j, c) for j in range(rows) for c in range(vch)}
    return slot


def banks(addr, nbytes):
    return [((addr + b) // 4) % 64 for b in range(0, nbytes, 4)]


def conflict_free(addrs, nbytes):
    """addrs: 64 per-lane byte addresses of one instruction; 16 lanes per pass."""
    for p in range(4):
        used = [b for a in addrs[16 * p:16 * p + 16] for b in banks(a, nbytes)]
        if len(used) != len(set(used)):
            return False
    return True


def row_read(slot, rows_base, rowb, DL, swz, s, lane):
    """Row fragment: lane (r, g) reads logical chunk 2s+g of row rows_base + a_row_key(r)."""
    r, g = lane & 31, lane >> 5
    row = rows_base + a_row_key(r)
    off = row * rowb + ((2 * s + g) ^ swz(DL, row)) * 16
    assert slot[off] == (row, 2 * s + g)
    return off


def tr_reads(slot, row0, rowb, DL, swz, dt, lane):
    """Transpose fragment: two 8-byte reads of 4 consecutive rows x 4 chunks per 16 lanes."""
    g, s16 = lane >> 5, lane & 15
    s4, sm, q2 = s16 >> 2, s16 & 3, (lane >> 4) & 1
    c = 4 * dt + 2 * q2 + (sm >> 1)
    out = []
    for extra in (0, 4):
        row = row0 + 8 * g + s4 + extra
        off = row * rowb + (c ^ swz(DL, row)) * 16 + (sm & 1) * 8
        assert slot[off - off % 16] == (row, c)
        out.append(off)
    return out


@pytest.mark.parametrize("D,BC,NW", FWD_SHAPES)
def test_forward_tiles(D, BC, NW):
    DL = lds_cols(D)
    rowb = 2 * DL
    kslot = copy_slots(D, BC, NW, swz_k)
    vslot = copy_slots(D, BC, NW, swz_v)
    for u in range(BC // 32):
        for s in range(D // 16):                  # K row fragments of sub-tile u, step s
            addrs = [row_read(kslot, 32 * u, rowb, DL, swz_k, s, lane) for lane in range(64)]
            assert conflict_free(addrs, 16), (D, u, s)
        for h in range(2):                        # V^T fragments of sub-tile u, half h
            for dt in range(D // 32):
                pairs = [tr_reads(vslot, 32 * u + 16 * h, rowb, DL, swz_v, dt, lane) for lane in range(64)]
                for k in range(2):
                    assert conflict_free([p[k] for p in pairs], 8), (D, u, h, dt, k)


@pytest.mark.parametrize("D,ROWS,NW", BWD_PLANS)
def test_backward_tiles(D, ROWS, NW):
    DL = lds_cols(D)
    rowb = 2 * DL
    slot = copy_slots(D, ROWS, NW, swz_u)
    for base in range(0, ROWS, 32):
        for s in range(D // 16):
            addrs = [row_read(slot, base, rowb, DL, swz_u, s, lane) for lane in range(64)]
            assert conflict_free(addrs, 16), (D, base, s)
    # the LDS dK/dV kernel also reads K and V rows in natural order (row base + r)
    for base in range(0, ROWS, 32):
        for s in range(D // 16):
            addrs = []
            for lane in range(64):
                r, g = lane & 31, lane >> 5
                row = base + r
                off = row * rowb + ((2 * s + g) ^ swz_u(DL, row)) * 16
                assert slot[off] == (row, 2 * s + g)
                addrs.append(off)
            assert conflict_free(addrs, 16), (D, base, s, "natural")
    for row0 in range(0, ROWS, 16):
        for dt in range(D // 32):
            pairs = [tr_reads(slot, row0, rowb, DL, swz_u, dt, lane) for lane in range(64)]
            for k in range(2):
                assert conflict_free([p[k] for p in pairs], 8), (D, row0, dt, k)


def test_padded_rows_leave_padding_untouched():
    """D = 96: a quarter of the LDS row is padding, and no copy or read touches it."""
    for swz in (swz_k, swz_v, swz_u):
        slot = copy_slots(96, 64, 8, swz)
        assert len(slot) == 64 * 12
        assert all(c < 12 for _, c in slot.values())
