"""Host logic of the launch-table tuner (CPU): the buckets it tunes, the
problems it times for them, its margin rule, and the coverage of the
committed table.  The table adapts the tile choice to the sequence length
and the grid size, as the NumPy build guide's *Extending It* suggests
(best tile sizes per head dimension and hardware, adapted to the lengths).
"""

import math

import pytest

from exact_tiled_attention_13_amd import tiles, tune

ALL = tune.ALL


def partitions(intervals, lo=1, hi=ALL):
    """Closed intervals [a, b], in order, cover [lo, hi] with no gap or overlap."""
    nxt = lo
    for a, b in intervals:
        if a != nxt or b < a:
            return False
        nxt = b + 1
    return nxt == hi + 1


def test_fwd_buckets_partition_lengths_and_sizes():
    assert partitions([(t_lo, t_hi) for (t_lo, t_hi, _), _ in tune.FWD_BUCKETS])
    for (t_lo, t_hi, T), sizes in tune.FWD_BUCKETS:
        assert t_lo <= T <= t_hi
        assert partitions([(lo, hi) for lo, hi, _ in sizes])
        for lo, hi, wg in sizes:
            assert lo <= wg <= hi


def test_fwd_problems_land_in_their_buckets():
    """The problem timed for a bucket (B * H heads of T rows, B a divisor of
    8, size = ceil(T / 256) * B * H) is keyed into that same bucket."""
    for (t_lo, t_hi, T), sizes in tune.FWD_BUCKETS:
        slots = math.ceil(T / 256)
        for lo, hi, wg in sizes:
            BH = max(1, wg // slots)
            B = math.gcd(BH, 8)
            H = BH // B
            assert B * H == BH and 8 % B == 0
            assert lo <= slots * B * H <= hi, (T, lo, hi, wg)


def test_decode_buckets():
    assert partitions([(lo, hi) for lo, hi, _ in tune.DEC_BUCKETS])
    B, Hq, Hkv = 64, 32, 8
    for lo, hi, S in tune.DEC_BUCKETS:
        size = B * math.ceil(S / 512) * Hkv * math.ceil(Hq // Hkv / 16)
        assert lo <= size <= hi


@pytest.mark.parametrize("times,builtin,want", [
    ({"a": 1.00, "b": 0.97}, "a", "b"),      # 3% faster: taken
    ({"a": 1.00, "b": 0.985}, "a", "a"),     # within the 2% margin: the built-in choice stays
    ({"a": 1.00, "b": 1.20}, "a", "a"),
    ({"a": 0.90, "b": 1.00}, "b", "a"),
    ({"a": 1.00, "b": 0.99}, "c", "b"),      # no timing of the built-in choice: the fastest
])
def test_margin_rule(times, builtin, want):
    assert tune.MARGIN == pytest.approx(0.02)
    assert tune._conservative(times, builtin) == want


def test_committed_table_covers_every_key():
    """For every (op, dtype, D, causal) it holds, the committed table's
    entries tile the (sequence length, size) plane without gaps or
    overlaps, so no call of those keys falls back to the built-in rule by
    accident."""
    import json

    with open(tiles.DEFAULT_PATH) as fh:
        doc = json.load(fh)
    groups = {}
    for e in doc["entries"]:
        groups.setdefault((e["op"], e["dtype"], e["D"], e["causal"]), []).append(e)
    assert {k[0] for k in groups} == {"fwd", "decode"}
    for key, es in groups.items():
        by_t = {}
        for e in es:
            by_t.setdefault((e.get("t_lo", 0), e.get("t_hi", ALL)), []).append((e["size_lo"], e["size_hi"]))
        t_lo0 = 0 if key[0] == "decode" else 1
        assert partitions(sorted(by_t), lo=t_lo0), key
        for t, sizes in by_t.items():
            assert partitions(sorted(sizes)), (key, t)
    # the rows the library receives are well formed
    assert len(tiles.entries_from_json(doc)) == len(doc["entries"])
