"""Masking in the prefill and dK/dV kernels, on the CPU.

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
("Implementing attention from scratch", *Masks* and *KV caching*).  The
same is checked for the dK/dV kernel's query steps (`dkdv_pairs`).
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


def dkdv_pairs(D, causal, Lk, Lq, G, kt):
    """(query head in the group, query row, key) triples whose weights reach
    dK/dV of key tile kt in `bwd_dkdv_pair_kernel` (csrc/bwd_bf16.hip): four
    wave pairs of 32 keys each, query steps of 32 rows over the group's query
    heads, a step skipped by the pair at D = 64 when none of its keys is
    seen, masked when it crosses a boundary.  Accumulator element r of lane
    32 h + r32 is query row q0 + 8 (r >> 2) + 4 h + (r & 3) against key
    wkey0 + r32."""
    NPAIR, BMQ = 4, 32
    BNK = 32 * NPAIR
    off = Lk - Lq
    k0 = kt * BNK
    qfirst = qend = 0
    if k0 < Lk:
        qfirst = max(0, k0 - off) if causal else 0
        qend = Lq
    nsteps_h = (qend - qfirst + BMQ - 1) // BMQ if qend > qfirst else 0
    out = []
    for pr in range(NPAIR):
        wkey0 = k0 + 32 * pr
        qwave_first = wkey0 - off if causal else 0
        for sidx in range(G * nsteps_h):
            g, j = divmod(sidx, nsteps_h)
            q0 = qfirst + j * BMQ
            if D == 64 and (wkey0 >= Lk or q0 + BMQ - 1 < qwave_first):
                continue
            needs_mask = (q0 + BMQ > Lq) or (wkey0 + 31 >= Lk) or (causal and wkey0 + 31 > q0 + off)
            for h in range(2):
                for r32 in range(32):
                    key = wkey0 + r32
                    for r in range(16):
                        i = q0 + 8 * (r >> 2) + 4 * h + (r & 3)
                        if needs_mask and not (i < Lq and key < Lk and (not causal or key <= i + off)):
                            continue
                        out.append((g, i, key))
    return out


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lk,Lq,G", [(1, 1, 1), (128, 128, 2), (129, 129, 1), (300, 300, 3), (300, 37, 1),
                                     (37, 300, 2), (0, 5, 1), (5, 0, 1), (257, 1, 4)])
def test_gradient_key_tile_masks(D, causal, Lk, Lq, G):
    """Every allowed (query head, row, key) pair of a key tile reaches dK/dV
    exactly once, and nothing else does."""
    off = Lk - Lq
    for kt in range(max(1, (Lk + 127) // 128) + 1):
        got = dkdv_pairs(D, causal, Lk, Lq, G, kt)
        want = [(g, i, j) for g in range(G) for i in range(Lq) for j in range(kt * 128, min(kt * 128 + 128, Lk))
                if not causal or j <= i + off]
        assert len(got) == len(set(got))
        assert sorted(got) == sorted(want), (D, causal, Lk, Lq, G, kt)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Lk,Lq", [(1, 1), (32, 32), (33, 33), (300, 300), (300, 37), (37, 300), (0, 5), (130, 0),
                                   (257, 1), (1000, 999)])
def test_gradient_query_tile_masks(causal, Lk, Lq):
    """The dQ kernel (`bwd_dq_kernel`) and the fp32 prefill (`fwd_f32_kernel`,
    csrc/fwd_f32.hip) walk key tiles with the bf16 prefill's rules: 128
    query rows of 4 waves, 32-key tiles, one key block per tile
    (accumulator key 8 (r >> 2) + 4 h + (r & 3)), the same kmax skip, kfull
    test and per-lane bound."""
    check((128, 32, 1, 4), causal, Lk, Lq)
