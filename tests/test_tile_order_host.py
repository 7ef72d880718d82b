"""Workgroup orders of the prefill kernel, on the CPU.

The prefill kernel maps each workgroup id to one (batch, query head, query
tile) by one of four orders (the `fwd_bf16_kernel` entry and `tile_at` in
csrc/fwd_bf16.hip).  These tests restate that integer arithmetic in Python,
with the same names, and check what the kernel relies on:

* every order is a bijection from the ids onto all tiles of the grid;
* the list order of ragged grids puts tiles in non-increasing work (key
  tiles a tile walks), ties by sequence, then query tile from the last,
  with the tiles that have no work at all at the end;
* the unit order keeps whole (batch, KV head) units on one XCD (ids i,
  i + 8, ... run on XCD i mod 8);
* the zig-zag order pairs a long and a short causal tile on ids id and
  id + grid/2.

The GPU tests check the device code itself (every tile written, results
against the oracle); these tests check the orders' design over many more
shapes than a GPU run can.  The masks follow "Implementing attention from
scratch", *Masks* and *KV caching* (causal alignment at the bottom right).
"""

import math
import random

import pytest

# (BM query rows, BN keys per tile) of the kernel's workgroup shapes:
# one key group (8 waves, 256 rows, 64-key tiles) and two key groups
# (4 + 4 waves, 128 rows; 64-key tiles at D = 64, 32-key tiles at D = 128)
SHAPES = [(256, 64), (128, 64), (128, 32)]
ORDER_MAX_B = 64


def tiles_above(BM, BN, causal, Lk, nq, off, w):
    if nq == 0 or Lk <= w * BN:
        return 0
    if not causal:
        return nq
    x = w * BN - off
    qmin = 0 if x < 0 else x // BM
    return max(0, nq - qmin)


def seq_info(kv_lens, B, Tq, Tk, BM):
    out = []
    for b in range(B):
        Lk = min(max(kv_lens[b], 0), Tk)
        Lq = Lk if Tq == Tk else Tq
        out.append((Lk, (Lq + BM - 1) // BM, Lk - Lq))
    return out


def tile_at(BM, BN, causal, p, kv_lens, B, Hq, Hkv, Tq, Tk, nqt):
    """Position p of the ragged list -> (b, hq, hk, qt)."""
    G = Hq // Hkv
    info = seq_info(kv_lens, B, Tq, Tk, BM)
    wmax = (Tk + BN - 1) // BN

    def above(w):
        return [tiles_above(BM, BN, causal, Lk, nq, off, w) for Lk, nq, off in info]

    above0 = above(0)
    F0 = Hq * sum(above0)
    zero = p >= F0
    if zero:
        r, cnt_hi, cnt_lo = p - F0, above0, [0] * B
    else:
        lo, hi = 1, wmax
        while lo < hi:
            mid = (lo + hi) >> 1
            if Hq * sum(above(mid)) <= p:
                hi = mid
            else:
                lo = mid + 1
        cnt_hi, cnt_lo = above(lo), above(lo - 1)
        r = p - Hq * sum(cnt_hi)
    mine = [nqt - cnt_hi[l] for l in range(B)] if zero else [cnt_lo[l] - cnt_hi[l] for l in range(B)]
    pre = 0
    for l in range(B):
        if r < Hq * (pre + mine[l]):
            break
        pre += mine[l]
    else:
        raise AssertionError(f"position {p} lies in no sequence's range")
    jj = r - Hq * pre
    t, hr = divmod(jj, Hq)
    g, hk = divmod(hr, Hkv)
    hq = hk * G + g
    nq_l, hi_l = info[l][1], cnt_hi[l]
    if zero:
        zlo = nq_l - hi_l
        qt = t if t < zlo else nq_l + (t - zlo)
    else:
        qt = nq_l - hi_l - 1 - t
    return l, hq, hk, qt


def work(BM, BN, causal, Lk, Lq, off, qt):
    """Key tiles query tile qt walks: those up to the key its last valid row
    sees (0 for padding tiles and for rows that see no key)."""
    if qt * BM >= Lq:
        return 0
    keys = Lk if not causal else min(Lk, min((qt + 1) * BM, Lq) - 1 + off + 1)
    return max(0, math.ceil(keys / BN))


def dense_order(order, id_, B, Hq, Hkv, nqt):
    """ORDER_ID_UNITS / NATURAL / ZIG of the kernel entry -> (b, hq, qt)."""
    G = Hq // Hkv
    if order == "units":
        xcd, k = id_ & 7, id_ >> 3
        ul, r = divmod(k, G * nqt)
        tq_slot = r // G
        u = xcd + 8 * ul
        b = u // Hkv
        hq = (u - b * Hkv) * G + (r - tq_slot * G)
    else:
        BH = B * Hq
        tq_slot, bh = divmod(id_, BH)
        b, hq = divmod(bh, Hq)
    half = (nqt + 1) // 2
    qt = tq_slot - half if (order == "zig" and tq_slot >= half) else nqt - 1 - tq_slot
    return b, hq, qt


def check_list(BM, BN, causal, kv_lens, Hq, Hkv, Tq, Tk):
    B = len(kv_lens)
    nqt = (Tq + BM - 1) // BM
    info = seq_info(kv_lens, B, Tq, Tk, BM)
    seen, prev = set(), None
    zero_started = False
    for p in range(B * Hq * nqt):
        b, hq, hk, qt = tile_at(BM, BN, causal, p, kv_lens, B, Hq, Hkv, Tq, Tk, nqt)
        assert 0 <= b < B and 0 <= hq < Hq and 0 <= qt < nqt and hk == hq // (Hq // Hkv)
        assert (b, hq, qt) not in seen
        seen.add((b, hq, qt))
        Lk = min(max(kv_lens[b], 0), Tk)
        Lq = Lk if Tq == Tk else Tq
        w = work(BM, BN, causal, Lk, Lq, Lk - Lq, qt)
        key = (-w, b, -qt)
        if w == 0:
            zero_started = True
        else:
            assert not zero_started, "a tile with work after the zero tiles"
            # non-increasing work; within equal work by sequence, then tile from the last
            assert prev is None or prev[0] < key[0] or (prev[0] == key[0] and prev[1:] <= key[1:]), (prev, key)
            prev = key
    assert len(seen) == B * Hq * nqt
    # the count above any level agrees with the per-tile work
    for w0 in range(0, (Tk + BN - 1) // BN + 1):
        direct = sum(1 for (Lk, nq, off), b in zip(info, range(B)) for qt in range(nqt)
                     if work(BM, BN, causal, Lk, Lk if Tq == Tk else Tq, off, qt) > w0)
        assert sum(tiles_above(BM, BN, causal, Lk, nq, off, w0) for Lk, nq, off in info) == direct


@pytest.mark.parametrize("BM,BN", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_list_order_ragged_workload_lengths(BM, BN, causal):
    """The ragged workload's seed-0 lengths (B8, 16 heads, T4096), two heads."""
    lens = [1, 2609, 2094, 1106, 1261, 168, 309, 68]
    check_list(BM, BN, causal, lens, 2, 2, 4096, 4096)


@pytest.mark.parametrize("seed", range(400))
def test_list_order_random_shapes(seed):
    rng = random.Random(seed)
    BM, BN = rng.choice(SHAPES)
    causal = rng.random() < 0.5
    B = rng.choice([1, 2, 3, 5, 8, 17, ORDER_MAX_B])
    Hkv = rng.choice([1, 2])
    Hq = Hkv * rng.choice([1, 2, 3])
    Tk = rng.randint(1, 700)
    Tq = Tk if rng.random() < 0.6 else rng.randint(1, 700)
    lens = [rng.randint(-3, Tk + 5) for _ in range(B)]
    if rng.random() < 0.2:
        lens = [0] * B                 # nothing but zero tiles
    check_list(BM, BN, causal, lens, Hq, Hkv, Tq, Tk)


def check_dense(order, B, Hq, Hkv, nqt):
    grid = B * Hq * nqt
    got = [dense_order(order, i, B, Hq, Hkv, nqt) for i in range(grid)]
    assert len(set(got)) == grid
    assert all(0 <= b < B and 0 <= hq < Hq and 0 <= qt < nqt for b, hq, qt in got)
    return got


@pytest.mark.parametrize("B,Hq,Hkv,nqt", [(1, 32, 32, 128), (2, 32, 8, 16), (4, 16, 16, 8), (8, 4, 1, 5)])
def test_unit_order_keeps_units_on_one_xcd(B, Hq, Hkv, nqt):
    assert (B * Hkv) % 8 == 0
    got = check_dense("units", B, Hq, Hkv, nqt)
    G = Hq // Hkv
    xcd_of_unit = {}
    for i, (b, hq, qt) in enumerate(got):
        u = b * Hkv + hq // G
        assert xcd_of_unit.setdefault(u, i & 7) == i & 7
    # within an XCD a unit's tiles come heaviest (last query tile) first
    for x in range(8):
        qts = {}
        for i in range(x, len(got), 8):
            b, hq, qt = got[i]
            qts.setdefault((b, hq), []).append(qt)
        assert all(v == sorted(v, reverse=True) for v in qts.values())


@pytest.mark.parametrize("B,Hq,Hkv,nqt", [(4, 16, 16, 4), (1, 3, 1, 7), (2, 2, 2, 1), (3, 5, 5, 9)])
def test_natural_and_zigzag_orders(B, Hq, Hkv, nqt):
    nat = check_dense("natural", B, Hq, Hkv, nqt)
    # heaviest causal tiles first: the query-tile index falls with the id
    assert [qt for _, _, qt in nat] == sorted((qt for _, _, qt in nat), reverse=True)
    zig = check_dense("zig", B, Hq, Hkv, nqt)
    grid = len(zig)
    if nqt % 2 == 0:
        # ids id and id + grid/2 (on one CU) hold tiles whose causal work adds up to nqt + 1 tiles
        for i in range(grid // 2):
            assert zig[i][2] + 1 + zig[i + grid // 2][2] + 1 == nqt + 1
            assert zig[i][:2] == zig[i + grid // 2][:2]


def dkdv_order(uorder, id_, B, Hkv, nkt):
    """Workgroup id -> (b, hk, kt) of the dK/dV kernel (bwd_dkdv_pair_kernel)."""
    NU = B * Hkv
    if uorder:
        k = id_ >> 3
        ul = k // nkt
        kt = k - ul * nkt
        u = (id_ & 7) + 8 * ul
        b, hk = divmod(u, Hkv)
    else:
        kt, bh = divmod(id_, NU)
        b, hk = divmod(bh, Hkv)
    return b, hk, kt


@pytest.mark.parametrize("B,Hkv,nkt", [(1, 32, 256), (2, 8, 16), (4, 2, 7), (8, 1, 3), (3, 5, 4)])
def test_gradient_key_tile_orders(B, Hkv, nkt):
    """The dK/dV kernel owns one (batch, KV head, key tile) per workgroup.
    Both orders are bijections, key tiles run from the first (under a causal
    mask the first key tiles are seen by the most queries); with a multiple
    of 8 units the unit order keeps each unit on one XCD.  The dQ kernel
    maps its ids like the prefill's natural and unit orders (checked
    above)."""
    grid = B * Hkv * nkt
    for uorder in ([0, 1] if (B * Hkv) % 8 == 0 else [0]):
        got = [dkdv_order(uorder, i, B, Hkv, nkt) for i in range(grid)]
        assert len(set(got)) == grid
        assert all(0 <= b < B and 0 <= hk < Hkv and 0 <= kt < nkt for b, hk, kt in got)
        per_unit = {}
        for i, (b, hk, kt) in enumerate(got):
            per_unit.setdefault((b, hk), []).append((i, kt))
        for v in per_unit.values():
            assert [kt for _, kt in v] == sorted(kt for _, kt in v)
            if uorder:
                assert len({i & 7 for i, _ in v}) == 1
