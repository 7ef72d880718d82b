"""The launch-choice table as JSON.

``tiles_gfx950.json`` (written by ``python -m exact_tiled_attention_13_amd.tune``
on the GPU) records, per (operation, dtype, D, causal, sequence-length bucket,
size bucket), the launch shape that measured fastest, with the timings it
was chosen from.
``load()`` applies it to the library through ``attn_set_tile_table``; keys
it does not cover keep the library's built-in rule.  Set ``MIATTN_TILES=off``
to skip it, or ``MIATTN_TILES=<path>`` to use another file.

Format::

    {"arch": "gfx950", "fields": [...], "entries": [
        {"op": "fwd", "dtype": "bf16", "D": 64, "causal": 1, "t_lo": 1, "t_hi": 2047,
         "size_lo": 0, "size_hi": 511, "choice": [1, -1], "times_ms": {...}, "problem": {...}}, ...]}

The sequence length T is Tk for "fwd" and S_max for "decode"; an entry
without t_lo / t_hi covers every length.

``choice`` is (v0, v1) of include/miattn.h: for "fwd" the workgroup shape
(0 = 256 rows, 1 = 128 rows in two key groups) and the zig-zag flag; for
"decode" the split kernel's workgroups per CU and 0.
"""

from __future__ import annotations

import json
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
DEFAULT_PATH = os.path.join(_PKG, "tiles_gfx950.json")
OPS = {"fwd": 0, "decode": 1}
DTYPES = {"bf16": 1, "e4m3": 2}
FIELDS = ["op", "dtype", "D", "causal", "t_lo", "t_hi", "size_lo", "size_hi", "v0", "v1"]
T_ALL = (0, 2**31 - 1)


def entries_from_json(doc) -> list[list[int]]:
    """The int32 rows of a table document (raises ValueError on a bad one)."""
    if not isinstance(doc, dict) or not isinstance(doc.get("entries"), list):
        raise ValueError("tile table: expected an object with an 'entries' list")
    rows = []
    for e in doc["entries"]:
        try:
            choice = e["choice"]
            rows.append([OPS[e["op"]], DTYPES[e["dtype"]], int(e["D"]), int(e["causal"]),
                         int(e.get("t_lo", T_ALL[0])), int(e.get("t_hi", T_ALL[1])), int(e["size_lo"]),
                         int(e["size_hi"]), int(choice[0]), int(choice[1])])
        except (KeyError, TypeError, IndexError, ValueError) as ex:
            raise ValueError(f"tile table: bad entry {e!r}: {ex}") from ex
    return rows


def read(path: str) -> list[list[int]]:
    with open(path) as fh:
        return entries_from_json(json.load(fh))


def apply_default(lib=None):
    """Apply the JSON table named by MIATTN_TILES, else the packaged one if present."""
    from . import _lib

    path = os.environ.get("MIATTN_TILES") or DEFAULT_PATH
    if not os.path.exists(path):
        if os.environ.get("MIATTN_TILES"):
            raise FileNotFoundError(f"MIATTN_TILES={path} does not exist")
        return 0
    rows = read(path)
    _lib.attn_set_tile_table(rows)
    return len(rows)
