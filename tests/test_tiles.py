"""The launch-choice table: C ABI validation and lookup, and the JSON file
the tuner writes (host-side only; nothing is launched)."""

import json
import os

import pytest

import exact_tiled_attention_13_amd as ea
from exact_tiled_attention_13_amd import _lib, tiles

FWD, DEC, BF16, E4M3 = _lib.MIATTN_TILE_FWD, _lib.MIATTN_TILE_DECODE, _lib.MIATTN_BF16, _lib.MIATTN_E4M3


@pytest.fixture
def clean_table():
    _lib.load()
    _lib.attn_set_tile_table([])
    yield
    _lib.attn_set_tile_table([])
    tiles.apply_default()


def test_builtin_rule(clean_table):
    # prefill: 128-row workgroups with two key groups below 512 256-row workgroups
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 256) == (1, -1)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 511) == (1, -1)
    assert _lib.attn_tile_choice(FWD, E4M3, 128, 0, 512) == (0, -1)
    # decode: two workgroups per CU
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 10**6) == (2, 0)
    assert _lib.attn_tile_table_size() == 0


def test_first_matching_entry_wins(clean_table):
    _lib.attn_set_tile_table([
        [FWD, BF16, 64, 1, 0, 99, 0, 1],
        [FWD, BF16, 64, 1, 50, 1000, 1, 0],
        [DEC, E4M3, 128, 1, 100, 200, 3, 0],
    ])
    assert _lib.attn_tile_table_size() == 3
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 60) == (0, 1)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 100) == (1, 0)
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, 1001) == (0, -1)       # uncovered: built-in rule
    assert _lib.attn_tile_choice(FWD, BF16, 64, 0, 60) == (1, -1)         # other key
    assert _lib.attn_tile_choice(DEC, E4M3, 128, 1, 150) == (3, 0)
    assert _lib.attn_tile_choice(DEC, BF16, 128, 1, 150) == (2, 0)


@pytest.mark.parametrize("row", [
    [2, BF16, 64, 1, 0, 9, 0, 0],          # unknown op
    [FWD, 0, 64, 1, 0, 9, 0, 0],           # fp32 has no table
    [FWD, BF16, 96, 1, 0, 9, 0, 0],        # D
    [FWD, BF16, 64, 2, 0, 9, 0, 0],        # causal
    [FWD, BF16, 64, 1, 9, 0, 0, 0],        # empty range
    [FWD, BF16, 64, 1, -1, 9, 0, 0],       # negative size
    [FWD, BF16, 64, 1, 0, 9, 2, 0],        # shape
    [FWD, BF16, 64, 1, 0, 9, 0, 2],        # zig
    [DEC, BF16, 64, 1, 0, 9, 0, 0],        # workgroups per CU
    [DEC, BF16, 64, 1, 0, 9, 9, 0],
    [DEC, BF16, 64, 1, 0, 9, 2, 1],
])
def test_invalid_entries_are_rejected_and_keep_the_old_table(clean_table, row):
    _lib.attn_set_tile_table([[FWD, BF16, 128, 0, 0, 10, 1, 0]])
    assert _lib.attn_set_tile_table([row], check=False) == -3
    assert _lib.attn_tile_table_size() == 1
    assert _lib.attn_tile_choice(FWD, BF16, 128, 0, 5) == (1, 0)


def test_abi_argument_checks(clean_table):
    lib = _lib.load()
    assert lib.attn_set_tile_table(None, 1) == -1
    assert lib.attn_set_tile_table(None, -1) == -2
    assert lib.attn_set_tile_table(None, 257) == -2
    assert lib.attn_tile_choice(FWD, BF16, 64, 1, 5, None) == -1
    assert _lib.attn_tile_choice(FWD, BF16, 64, 1, -5, check=False) == -2
    assert _lib.attn_tile_choice(FWD, 7, 64, 1, 5, check=False) == -3


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
        key = f"{r[6]},{r[7]}" if e["op"] == "fwd" else str(r[6])
        assert key in t and t[key] <= min(t.values()) / (1.0 - 0.02) + 1e-9
        assert _lib.attn_tile_choice(r[0], r[1], r[2], r[3], r[4]) == (r[6], r[7])
    # buckets of one key do not overlap
    keys = {}
    for r in rows:
        keys.setdefault(tuple(r[:4]), []).append((r[4], r[5]))
    for spans in keys.values():
        spans.sort()
        assert all(a[1] < b[0] for a, b in zip(spans, spans[1:]))


def test_bad_json_is_refused(tmp_path):
    with pytest.raises(ValueError):
        tiles.entries_from_json({"entries": [{"op": "fwd"}]})
    with pytest.raises(ValueError):
        tiles.entries_from_json([])
