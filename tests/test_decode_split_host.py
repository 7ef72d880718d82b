"""Work split of the split-K decode, on the CPU.

`decode_split_kernel` (csrc/decode.hip) enumerates work items (sequence b,
head block hbk = hkv * NHB + hb, split s of 512 keys), gives each wave one
contiguous range of C = ceil(U / waves) items, and accumulates consecutive
splits of one (sequence, head block) into one running softmax, a run,
whose partial it writes to the workspace slot of the run's first split.
`decode_merge_kernel` does not see the waves: it recomputes where the runs
of each (sequence, query head) start from the item count alone, and reads
those slots.  The two must agree exactly, or the merge reads a slot nothing
wrote (or misses a run).  The split across chunks and the merge by
log-sum-exp follow "Implementing attention from scratch", *KV caching* and
*Stable softmax*.

These tests restate both sides' integer arithmetic in Python (same names as
the kernels) and check, over many shapes and grid sizes, that the slots
written are exactly the slots read, that runs partition every sequence's
splits, and that every slot stays inside the workspace row the host sizes.
"""

import random

import pytest

SPLIT_KEYS = 512     # kDecodeSplitKeys (csrc/launch.h)


def clamp(x, lo, hi):
    return max(lo, min(hi, x))


def items(lens, S_max, HBK):
    """Work items in the kernel's order: sequence, head block, split."""
    out = []
    for b, L in enumerate(lens):
        ns = (clamp(L, 0, S_max) + SPLIT_KEYS - 1) // SPLIT_KEYS
        for hbk in range(HBK):
            for s in range(ns):
                out.append((b, hbk, s, ns))
    return out


def split_side(lens, S_max, HBK, NWAV):
    """Runs the waves accumulate: {(b, hbk): set of first splits}."""
    it = items(lens, S_max, HBK)
    U = len(it)
    C = (U + NWAV - 1) // NWAV
    written = {}
    for W in range(NWAV):
        t, tend = W * C, min(W * C + C, U)
        if t >= tend:
            continue
        b, hbk, s, ns = it[t]
        s0 = s
        while True:
            t += 1
            if t < tend and s + 1 < ns:       # the next split of the same (sequence, head block)
                s += 1
                assert it[t] == (b, hbk, s, ns)
                continue
            written.setdefault((b, hbk), []).append(s0)   # run done: slot of its first split
            if t >= tend:
                break
            b, hbk, s, ns = it[t]
            s0 = s
    return written, U


def merge_side(lens, S_max, Hq, Hkv, NHB, NWAV, U):
    """Run starts the merge reads: {(b, hq): [first splits]}."""
    G = Hq // Hkv
    HBK = Hkv * NHB
    C = (U + NWAV - 1) // NWAV
    P, acc = [], 0                    # splits of the sequences before b (ws_idx[1 + b])
    for L in lens:
        P.append(acc)
        acc += (clamp(L, 0, S_max) + SPLIT_KEYS - 1) // SPLIT_KEYS
    read = {}
    for b, L in enumerate(lens):
        ns = (clamp(L, 0, S_max) + SPLIT_KEYS - 1) // SPLIT_KEYS
        for hq in range(Hq):
            hkv = hq // G
            hb = (hq - hkv * G) // 16
            base = P[b] * HBK + (hkv * NHB + hb) * ns
            rem = base % C if C > 0 else 0
            s1 = C if rem == 0 else C - rem
            nruns = 0 if ns == 0 else 1 + ((ns - 1 - s1) // C + 1 if s1 < ns else 0)
            read[(b, hq)] = [0 if k == 0 else s1 + (k - 1) * C for k in range(nruns)]
    return read


def check(lens, S_max, Hq, Hkv, NWAV):
    G = Hq // Hkv
    NHB = (G + 15) // 16
    HBK = Hkv * NHB
    NS = (S_max + SPLIT_KEYS - 1) // SPLIT_KEYS      # the workspace's slots per (sequence, query head)
    written, U = split_side(lens, S_max, HBK, NWAV)
    read = merge_side(lens, S_max, Hq, Hkv, NHB, NWAV, U)
    for b, L in enumerate(lens):
        ns = (clamp(L, 0, S_max) + SPLIT_KEYS - 1) // SPLIT_KEYS
        for hq in range(Hq):
            hkv = hq // G
            hbk = hkv * NHB + (hq - hkv * G) // 16
            w = sorted(written.get((b, hbk), []))
            assert read[(b, hq)] == w, (b, hq, read[(b, hq)], w)
            assert all(0 <= s < ns <= NS for s in w)
            # runs start at split 0 and cover every split once
            assert (not w and ns == 0) or w[0] == 0


@pytest.mark.parametrize("NWAV", [1, 3, 4, 64, 2048, 4096, 100000])
def test_decode_workload_grid_sizes(NWAV):
    """The decode workload's shape (B64, Hq32, Hkv8, S_max 32768, lengths
    1024..32768) at several grid sizes, down to one wave and past one item
    per wave."""
    rng = random.Random(0)
    lens = [rng.randint(1024, 32768) for _ in range(64)]
    check(lens, 32768, 32, 8, NWAV)


@pytest.mark.parametrize("seed", range(300))
def test_random_shapes(seed):
    rng = random.Random(seed)
    Hkv = rng.choice([1, 2, 3, 8])
    Hq = Hkv * rng.choice([1, 2, 4, 16, 17, 40])     # head blocks of 16 with a partial last one
    S_max = rng.choice([1, 511, 512, 513, 4096, 70000])
    B = rng.choice([1, 2, 5, 63, 64, 65, 130])
    lens = [rng.choice([0, 1, rng.randint(-5, S_max + 9)]) for _ in range(B)]
    NWAV = 4 * rng.randint(1, 600)
    check(lens, S_max, Hq, Hkv, NWAV)


def test_workspace_size_covers_every_slot():
    """attn_decode_workspace_size: B * Hq * NS * (D + 2) floats of partials
    (D outputs, then max and sum, per slot) plus B + 1 ints of bookkeeping;
    the largest slot index written stays below B * Hq * NS."""
    import ctypes
    import os

    lib_path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "exact_tiled_attention_13_amd", "libmiattn.so")
    if not os.path.exists(lib_path):
        pytest.skip("libmiattn.so not built")
    lib = ctypes.CDLL(lib_path)
    lib.attn_decode_workspace_size.argtypes = [ctypes.c_int] * 5
    lib.attn_decode_workspace_size.restype = ctypes.c_size_t
    for B, Hq, Hkv, S_max, D in [(64, 32, 8, 32768, 128), (1, 1, 1, 1, 64), (3, 48, 3, 513, 128)]:
        NS = (S_max + SPLIT_KEYS - 1) // SPLIT_KEYS
        assert lib.attn_decode_workspace_size(B, Hq, Hkv, S_max, D) == 4 * (B * Hq * NS * (D + 2) + B + 1)
        lens = [S_max] * B
        written, _ = split_side(lens, S_max, Hkv * ((Hq // Hkv + 15) // 16), 4 * 512)
        top = max(((b * Hq + hq) * NS + max(v)) for (b, hbk), v in written.items() for hq in range(Hq))
        assert top < B * Hq * NS


def paged_geometry(num_pages, page_size, max_blocks, Hkv):
    """The host's checks and derived sizes for the paged calls (api.cpp):
    page shift, and S_max = max_blocks * page_size (lengths are clamped to it)."""
    if page_size < 8 or page_size > 65536 or page_size & (page_size - 1):
        return None
    sh = page_size.bit_length() - 1
    cap = max_blocks * page_size
    if cap > 0x7FFFFFFF or num_pages * Hkv * page_size > (1 << 40):
        return None
    return sh, cap


@pytest.mark.parametrize("seed", range(200))
def test_paged_rows_stay_in_the_pool(seed):
    """For every key of every item of a paged decode: the lane that holds
    its page number is one of the wave's 64, the block-table entry read is
    inside the table row (entries past it read as 0), the page is clamped
    into the pool whatever the table holds, and the row's offset is inside
    the pool.  Logical key j is row j % P of page block_table[b][j // P]."""
    rng = random.Random(seed)
    P = 1 << rng.randint(3, 11)
    Hkv = rng.choice([1, 2, 8])
    D = rng.choice([64, 128])
    max_blocks = rng.randint(1, 3 * SPLIT_KEYS // P + 3)
    num_pages = rng.randint(1, 40)
    sh, S_max = paged_geometry(num_pages, P, max_blocks, Hkv)
    B = rng.randint(1, 4)
    table = [[rng.randint(-5, num_pages + 5) for _ in range(max_blocks)] for _ in range(B)]
    lens = [rng.randint(-2, S_max + 50) for _ in range(B)]
    pool = num_pages * Hkv * P * D
    for b in range(B):
        L = clamp(lens[b], 0, S_max)
        ns = (L + SPLIT_KEYS - 1) // SPLIT_KEYS
        for s in range(ns):
            k0, k1 = s * SPLIT_KEYS, min(s * SPLIT_KEYS + SPLIT_KEYS, L)
            # tile == 0: lane i loads the page number of block (k0 >> sh) + i
            pvec = []
            for lane in range(64):
                blk = (k0 >> sh) + lane
                p = table[b][blk] if blk < max_blocks else 0
                pvec.append(clamp(p, 0, num_pages - 1))
            for key in range(k0, k1):
                src = (key >> sh) - (k0 >> sh)
                assert 0 <= src < 64
                assert (k0 >> sh) + src < max_blocks            # the entry that key's page came from
                page = pvec[src]
                for hkv in range(Hkv):
                    off = (((page * Hkv + hkv) << sh) + (key & (P - 1))) * D
                    assert 0 <= off and off + D <= pool
                # the page is the table's when the entry is valid
                e = table[b][key >> sh]
                if 0 <= e < num_pages:
                    assert page == e



@pytest.mark.parametrize("BN", [32, 64])          # keys per tile: bf16 cache, E4M3 cache
@pytest.mark.parametrize("L", [0, 1, 31, 32, 33, 511, 512, 513, 1000, 4097])
def test_decode_tiles_cover_each_key_once(BN, L):
    """Keys of a sequence reach the softmax once each: items of 512 keys
    [k0, k1), tiles of BN keys from k0, and on a tile that passes k1 the
    mask keeps key < k1.  Accumulator element r of lane 16 g + j in key
    block kb is key kt + 16 kb + 4 g + r (v_mfma_f32_16x16, head column j)."""
    got = []
    ns = (L + SPLIT_KEYS - 1) // SPLIT_KEYS
    for s in range(ns):
        k0, k1 = s * SPLIT_KEYS, min(s * SPLIT_KEYS + SPLIT_KEYS, L)
        ntiles = (k1 - k0 + BN - 1) // BN
        for tile in range(ntiles):
            kt = k0 + tile * BN
            need_mask = kt + BN > k1
            for kb in range(BN // 16):
                for g in range(4):
                    for r in range(4):
                        key = kt + 16 * kb + 4 * g + r
                        if need_mask and key >= k1:
                            continue
                        got.append(key)
    assert sorted(got) == list(range(L))
