"""Masking in the prefill kernel, on the CPU.

The prefill kernel (`fwd_tile` in csrc/fwd_bf16.hip) never evaluates the
mask on every score.  A workgroup walks only the key tiles up to the last
key its rows may see.  A wave skips a tile none of its rows sees (kmax).  It
masks only a tile that crosses the last key its first row sees (kfull),
and then with one compare per score: the score's constant key offset
within the tile, as laid out in the MFMA accumulator, against one per-lane
bound.  This test restates those integer rules and the accumulator layout
of v_mfma_f32_32x32 (lane 32 h + r32 holds query column r32; element r of
key block kb holds key 32 kb + 8 (r >> 2) + 4 h + (r & 3)).  It checks that
the (query, key) pairs that reach the softmax are exactly the pairs the
mask allows, each once, over the three workgroup shapes and many lengths:
key padding, padded query rows and bottom-right causal alignment
("Implementing attention from scratch", *Masks* and *KV caching*).
"""

import random

import pytest

# (query rows per workgroup BM, keys per tile BN, key groups KSPLIT, waves per group NWG)
SHAPES = [(256, 64, 1, 8), (128, 64, 2, 4), (128, 32, 2, 4)]


def kernel_pairs(BM, BN, KSPLIT, NWG, causal, Lk, Lq, qt):
    """(query, key) pairs whose scores reach the softmax of query tile qt."""
    off = Lk - Lq
    q0 = qt * BM
    rows_end = min(q0 + BM, Lq)
    kend = 0
    if rows_end > q0:
        kend = min(Lk, rows_end + off) if causal else Lk
    kend = max(kend, 0)
    ntiles_all = (kend + BN - 1) // BN
    out = []
    if ntiles_all == 0:
        return out
    KB = BN // 32
    for kg in range(KSPLIT):
        ntiles = (ntiles_all - kg + KSPLIT - 1) // KSPLIT if ntiles_all > kg else 0
        for wg in range(NWG):
            wrow0 = q0 + 32 * wg
            kmax = -1
            if wrow0 < Lq:
                kmax = min(Lk - 1, min(wrow0 + 31, Lq - 1) + off) if causal else Lk - 1
            kfull = min(Lk - 1, wrow0 + off) if causal else Lk - 1
            for lt in range(ntiles):
                kbase = (lt * KSPLIT + kg) * BN
                if kbase > kmax:
                    continue                      # no row of the wave sees this tile
                need_mask = kbase + BN - 1 > kfull
                for h in range(2):
                    for r32 in range(32):
                        qrow = wrow0 + r32
                        if qrow >= Lq:
                            continue              # padding row: computed, never stored
                        lim = min(Lk - 1, qrow + off) if causal else Lk - 1
                        rel = lim - kbase - 4 * h
                        for kb in range(KB):
                            for r in range(16):
                                k_off = 32 * kb + 8 * (r >> 2) + (r & 3)
                                if need_mask and k_off > rel:
                                    continue
                                out.append((qrow, kbase + 4 * h + k_off))
    return out


def allowed_pairs(BM, causal, Lk, Lq, qt):
    off = Lk - Lq
    return [(i, j) for i in range(qt * BM, min(qt * BM + BM, Lq)) for j in range(Lk)
            if not causal or j <= i + off]


def check(shape, causal, Lk, Lq):
    BM, BN, KSPLIT, NWG = shape
    assert BM == 32 * NWG
    for qt in range(max(1, (Lq + BM - 1) // BM) + 1):
        got = kernel_pairs(BM, BN, KSPLIT, NWG, causal, Lk, Lq, qt)
        want = allowed_pairs(BM, causal, Lk, Lq, qt)
        assert len(got) == len(set(got)), "a pair reached the softmax twice"
        assert sorted(got) == want, (shape, causal, Lk, Lq, qt)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lk,Lq", [(1, 1), (64, 64), (65, 65), (300, 300), (300, 37), (37, 300), (0, 5),
                                   (130, 0), (257, 1)])
def test_masks_edges(shape, causal, Lk, Lq):
    check(shape, causal, Lk, Lq)


@pytest.mark.parametrize("seed", range(60))
def test_masks_random_lengths(seed):
    rng = random.Random(seed)
    shape = rng.choice(SHAPES)
    causal = rng.random() < 0.6
    Lk = rng.randint(0, 700)
    Lq = Lk if rng.random() < 0.5 else rng.randint(0, 700)
    check(shape, causal, Lk, Lq)
