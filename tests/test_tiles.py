"""The launch-choice table: C ABI validation and lookup, and the JSON file
the tuner writes (host-side only; nothing is launched).

Entries are { op, dtype, D, causal, t_lo, t_hi, size_lo, size_hi, v0, v1 }
(include/miattn.h); T is the sequence length (Tk for prefill, S_max for
decode)."""

import json
import os
import threading

import pytest

import exact_tiled_attention_13_amd as ea  # noqa: F401
from exact_tiled_attention_13_amd import _lib, tiles

FWD, DEC, BF16, E4M3 = _lib.MIATTN_TILE_FWD, _lib.MIATTN_TILE_DECODE, _lib.MIATTN_BF16, _lib.MIATTN_E4M3
ALL = 2**31 - 1


@pytest.fixture
def clean_table():
    _lib.load()
    _lib.attn_set_tile_table([])
    yield
    _lib.attn_set_tile_table([])
    tiles.apply_default()


def test_builtin_rule(clean_table):
    # prefill: 128-row workgroups with two key groups below 512 256-row workgroups
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 256) == (1, -1)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 511) == (1, -1)
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 0, 32768, 512) == (0, -1)
    # decode: two workgroups per CU
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 32768, 10**6) == (2, 0)
    assert _lib.attn_tile_table_size() == 0


def test_first_matching_entry_wins(clean_table):
    _lib.attn_set_tile_table([
        [FWD, BF16, 64, 1, 0, ALL, 0, 99, 0, 1],
        [FWD, BF16, 64, 1, 0, ALL, 50, 1000, 1, 0],
        [DEC, E4M3, 128, 1, 0, ALL, 100, 200, 3, 0],
    ])
    assert _lib.attn_tile_table_size() == 3
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 60) == (0, 1)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 100) == (1, 0)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 1001) == (0, -1)   # uncovered: built-in rule
    assert _lib.attn_tile_choice(FWD, BF16, 64, 0, 1024, 60) == (1, -1)     # other key
    assert _lib.attn_tile_choice(DEC, E4M3, 128, 1, 4096, 150) == (3, 0)
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 4096, 150) == (2, 0)


def test_sequence_length_key(clean_table):
    # one size bucket, two length buckets with different choices: a short
    # sequence with many heads and a long one with few give the same size
    _lib.attn_set_tile_table([
        [FWD, E4M3, 128, 1, 1, 2047, 1024, 4095, 1, -1],
        [FWD, E4M3, 128, 1, 2048, ALL, 1024, 4095, 0, -1],
        [DEC, BF16, 128, 1, 1, 8191, 0, ALL, 1, 0],
    ])
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 1, 1024, 1536) == (1, -1)
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 1, 2047, 4095) == (1, -1)
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 1, 2048, 1024) == (0, -1)
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 1, 32768, 4096) == (0, -1)   # size past the bucket: built-in
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 8191, 10) == (1, 0)
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 8192, 10) == (2, 0)       # built-in
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 1, 0, 1536) == (0, -1)       # T below every bucket


@pytest.mark.parametrize("row", [
    [2, BF16, 64, 1, 0, ALL, 0, 9, 0, 0],          # unknown op
    [FWD, 0, 64, 1, 0, ALL, 0, 9, 0, 0],           # fp32 has no table
    [FWD, BF16, 96, 1, 0, ALL, 0, 9, 0, 0],        # D
    [FWD, BF16, 64, 2, 0, ALL, 0, 9, 0, 0],        # causal
    [FWD, BF16, 64, 1, 0, ALL, 9, 0, 0, 0],        # empty size range
    [FWD, BF16, 64, 1, 0, ALL, -1, 9, 0, 0],       # negative size
    [FWD, BF16, 64, 1, 5, 4, 0, 9, 0, 0],          # empty length range
    [FWD, BF16, 64, 1, -1, 4, 0, 9, 0, 0],         # negative length
    [FWD, BF16, 64, 1, 0, ALL, 0, 9, 2, 0],        # shape
    [FWD, BF16, 64, 1, 0, ALL, 0, 9, 0, 2],        # zig
    [DEC, BF16, 64, 1, 0, ALL, 0, 9, 0, 0],        # workgroups per CU
    [DEC, BF16, 64, 1, 0, ALL, 0, 9, 9, 0],
    [DEC, BF16, 64, 1, 0, ALL, 0, 9, 2, 1],
])
def test_invalid_entries_are_rejected_and_keep_the_old_table(clean_table, row):
    _lib.attn_set_tile_table([[FWD, BF16, 128, 0, 0, ALL, 0, 10, 1, 0]])
    assert _lib.attn_set_tile_table([row], check=False) == -3
    assert _lib.attn_tile_table_size() == 1
    assert _lib.attn_tile_choice(FWD, BF16, 128, 0, 100, 5) == (1, 0)


def test_abi_argument_checks(clean_table):
    lib = _lib.load()
    assert lib.attn_set_tile_table(None, 1) == -1
    assert lib.attn_set_tile_table(None, -1) == -2
    assert lib.attn_set_tile_table(None, 257) == -2
    assert lib.attn_tile_choice(FWD, BF16, 64, 1, 100, 5, None) == -1
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 100, -5, check=False) == -2
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, -100, 5, check=False) == -2
    assert _lib.attn_tile_choice(FWD, 7, 64, 1, 100, 5, check=False) == -3
    with pytest.raises(ValueError):
        _lib.attn_set_tile_table([[FWD, BF16, 64, 1, 0, 9, 0, 0]])   # old 8-field rows


def test_concurrent_set_and_lookup(clean_table):
    """Lookups running while other threads replace the table see either the
    old or the new table (never a mix, never a crash)."""
    a = [[FWD, BF16, 64, 1, 0, ALL, 0, ALL, 0, 1]]
    b = [[FWD, BF16, 64, 1, 0, ALL, 0, ALL, 1, 0]]
    _lib.attn_set_tile_table(a)
    stop = threading.Event()
    bad = []

    def reader():
        while not stop.is_set():
            c = _lib.attn_tile_choice(FWD, BF16, 64, 1, 1024, 77)
            if c not in ((0, 1), (1, 0)):
                bad.append(c)

    def writer():
        for i in range(300):
            _lib.attn_set_tile_table(a if i % 2 else b)

    ts = [threading.Thread(target=reader) for _ in range(3)] + [threading.Thread(target=writer) for _ in range(2)]
    for t in ts:
        t.start()
    for t in ts[3:]:
        t.join()
    stop.set()
    for t in ts[:3]:
        t.join()
    assert not bad


def test_packaged_table_loads_and_is_applied():
    if not os.path.exists(tiles.DEFAULT_PATH):
        pytest.skip("no tuned table committed")
    with open(tiles.DEFAULT_PATH) as fh:
        doc = json.load(fh)
    rows = tiles.entries_from_json(doc)
    assert rows and doc["arch"] == "gfx950"
    _lib.load()
    tiles.apply_default()
    assert _lib.attn_tile_table_size() == len(rows)
    for e, r in zip(doc["entries"], rows):
        # the recorded choice is a measured candidate within 2% of the fastest
        t = e["times_ms"]
        key = f"{r[8]},{r[9]}" if e["op"] == "fwd" else str(r[8])
        assert key in t and t[key] <= min(t.values()) / (1.0 - 0.02) + 1e-9
        assert _lib.attn_tile_choice(r[0], r[1], r[2], r[3], r[4], r[6]) == (r[8], r[9])
    # buckets of one key do not overlap: (T range, size range) boxes are disjoint
    keys = {}
    for r in rows:
        keys.setdefault(tuple(r[:4]), []).append((r[4], r[5], r[6], r[7]))
    for boxes in keys.values():
        for i, a in enumerate(boxes):
            for b in boxes[i + 1:]:
                assert a[1] < b[0] or b[1] < a[0] or a[3] < b[2] or b[3] < a[2]


def test_json_without_length_bounds_covers_every_length():
    rows = tiles.entries_from_json({"entries": [
        {"op": "decode", "dtype": "bf16", "D": 128, "causal": 1, "size_lo": 0, "size_hi": 5, "choice": [3, 0]}]})
    assert rows == [[DEC, BF16, 128, 1, 0, ALL, 0, 5, 3, 0]]


def test_bad_json_is_refused(tmp_path):
    with pytest.raises(ValueError):
        tiles.entries_from_json({"entries": [{"op": "fwd"}]})
    with pytest.raises(ValueError):
        tiles.entries_from_json([])


def test_tuner_merge_keeps_other_keys():
    """`tune --only OP,DTYPE,D` re-measures one key set and keeps the rest of
    the table: every entry of the other keys survives unchanged, the old
    entries of the re-tuned key are replaced, and the merged document loads."""
    from exact_tiled_attention_13_amd import tune

    with open(tiles.DEFAULT_PATH) as fh:
        doc = json.load(fh)
    old = doc["entries"]
    key = ("fwd", "bf16", 128)
    fresh = [dict(e, choice=[1, -1]) for e in old if (e["op"], e["dtype"], e["D"]) == key]
    assert fresh, "the packaged table has entries for the re-tuned key"
    merged = tune.merge_only(old, fresh, key)
    others = [e for e in old if (e["op"], e["dtype"], e["D"]) != key]
    assert merged[: len(others)] == others
    assert merged[len(others):] == fresh
    assert len(merged) == len(old)
    tiles.entries_from_json(dict(doc, entries=merged))
    with pytest.raises(ValueError):
        tune.merge_only(old, [dict(fresh[0], D=64)], key)
