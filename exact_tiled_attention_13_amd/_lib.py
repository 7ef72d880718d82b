"""ctypes binding of libmiattn.so: the C ABI of include/miattn.h, one Python
function per exported symbol, with the same names.  Argument marshalling only.
"""

from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MIATTN_LIB") or os.path.join(_PKG, "libmiattn.so")

MIATTN_F32 = 0
MIATTN_BF16 = 1
MIATTN_E4M3 = 2
MIATTN_TILE_FWD = 0
MIATTN_TILE_DECODE = 1
MIATTN_TILE_FIELDS = 10

EXPORTED = ("attn_fwd", "attn_fwd_fp8", "attn_decode_workspace_size", "attn_decode", "attn_decode_paged", "attn_decode_fp8",
            "attn_decode_paged_fp8", "attn_bwd_workspace_size", "attn_bwd", "attn_set_tile_table",
            "attn_tile_table_size", "attn_tile_choice", "attn_strerror", "attn_abi_version",
            "attn_decode_noalloc", "attn_decode_noalloc_max_bytes")

_lib = None


class MiattnError(RuntimeError):
    """A negative return code from the library."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"miattn error {code}: {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    """Load libmiattn.so (built in-tree); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m exact_tiled_attention_13_amd.build` "
            "(the HIP library is the only compute path; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_fwd_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, f, f, i, vp, vp]
    lib.attn_fwd_fp8.restype = i
    lib.attn_decode_workspace_size.argtypes = [i, i, i, i, i]
    lib.attn_decode_workspace_size.restype = sz
    lib.attn_decode.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, vp, sz, i, vp]
    lib.attn_decode.restype = i
    lib.attn_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, i, vp]
    lib.attn_decode_noalloc.restype = i
    lib.attn_decode_noalloc_max_bytes.argtypes = []
    lib.attn_decode_noalloc_max_bytes.restype = sz
    lib.attn_decode_paged.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp, vp, sz, i, vp]
    lib.attn_decode_paged.restype = i
    lib.attn_decode_fp8.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, f, f, f, vp, vp, sz, vp]
    lib.attn_decode_fp8.restype = i
    lib.attn_decode_paged_fp8.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, f, f, f, vp, vp, sz, vp]
    lib.attn_decode_paged_fp8.restype = i
    lib.attn_bwd_workspace_size.argtypes = [i, i, i]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, i, vp, vp, sz, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_set_tile_table.argtypes = [vp, i]
    lib.attn_set_tile_table.restype = i
    lib.attn_tile_table_size.argtypes = []
    lib.attn_tile_table_size.restype = i
    lib.attn_tile_choice.argtypes = [i, i, i, i, ctypes.c_longlong, ctypes.c_longlong, vp]
    lib.attn_tile_choice.restype = i
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_abi_version.argtypes = []
    lib.attn_abi_version.restype = i
    _lib = lib
    if os.environ.get("MIATTN_TILES", "") != "off":
        from . import tiles
        tiles.apply_default(lib)
    return lib


def attn_strerror(code: int) -> str:
    return load().attn_strerror(int(code)).decode()


def attn_abi_version() -> int:
    return int(load().attn_abi_version())


def attn_decode_workspace_size(B: int, Hq: int, Hkv: int, S_max: int, D: int) -> int:
    return int(load().attn_decode_workspace_size(B, Hq, Hkv, S_max, D))


def attn_bwd_workspace_size(B: int, Hq: int, Tq: int) -> int:
    return int(load().attn_bwd_workspace_size(B, Hq, Tq))


def _check(code: int) -> int:
    if code != 0:
        raise MiattnError(code, attn_strerror(code))
    return code


def attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, D, scale, causal, kv_lens, dtype, stream, check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_fwd(q or None, k or None, v or None, o or None, lse or None, B, Hq, Hkv, Tq, Tk, D,
                           float(scale), int(causal), kv_lens or None, dtype, stream or None)
    return _check(code) if check else code


def attn_fwd_fp8(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, D, scale, q_scale, k_scale, v_scale, causal, kv_lens, stream,
                 check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_fwd_fp8(q or None, k or None, v or None, o or None, lse or None, B, Hq, Hkv, Tq, Tk, D,
                               float(scale), float(q_scale), float(k_scale), float(v_scale), int(causal),
                               kv_lens or None, stream or None)
    return _check(code) if check else code


def attn_decode(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, workspace,
                workspace_bytes, dtype, stream, check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_decode(q or None, k_cache or None, v_cache or None, o or None, lse or None, B, Hq, Hkv,
                              S_max, D, float(scale), kv_lens or None, workspace or None, workspace_bytes, dtype,
                              stream or None)
    return _check(code) if check else code


def attn_decode_noalloc(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, kv_lens, dtype, stream,
                        check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_decode_noalloc(q or None, k_cache or None, v_cache or None, o or None, lse or None, B, Hq,
                                      Hkv, S_max, D, float(scale), kv_lens or None, dtype, stream or None)
    return _check(code) if check else code


def attn_decode_noalloc_max_bytes() -> int:
    return int(load().attn_decode_noalloc_max_bytes())


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Tq, Tk, D, scale, causal, kv_lens, workspace,
             workspace_bytes, dtype, stream, check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_bwd(q or None, k or None, v or None, o or None, lse or None, dout or None, dq or None,
                           dk or None, dv or None, B, Hq, Hkv, Tq, Tk, D, float(scale), int(causal),
                           kv_lens or None, workspace or None, workspace_bytes, dtype, stream or None)
    return _check(code) if check else code


def attn_decode_paged(q, k_pages, v_pages, block_table, o, lse, B, Hq, Hkv, num_pages, page_size, max_blocks, D,
                      scale, kv_lens, workspace, workspace_bytes, dtype, stream, check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_decode_paged(q or None, k_pages or None, v_pages or None, block_table or None, o or None,
                                    lse or None, B, Hq, Hkv, num_pages, page_size, max_blocks, D, float(scale),
                                    kv_lens or None, workspace or None, workspace_bytes, dtype, stream or None)
    return _check(code) if check else code


def attn_decode_fp8(q, k_cache, v_cache, o, lse, B, Hq, Hkv, S_max, D, scale, q_scale, k_scale, v_scale, kv_lens,
                    workspace, workspace_bytes, stream, check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_decode_fp8(q or None, k_cache or None, v_cache or None, o or None, lse or None, B, Hq, Hkv,
                                  S_max, D, float(scale), float(q_scale), float(k_scale), float(v_scale),
                                  kv_lens or None, workspace or None, workspace_bytes, stream or None)
    return _check(code) if check else code


def attn_decode_paged_fp8(q, k_pages, v_pages, block_table, o, lse, B, Hq, Hkv, num_pages, page_size, max_blocks,
                          D, scale, q_scale, k_scale, v_scale, kv_lens, workspace, workspace_bytes, stream,
                          check=True):
    """Raw C-ABI call; pointers are integers (0 = NULL)."""
    code = load().attn_decode_paged_fp8(q or None, k_pages or None, v_pages or None, block_table or None,
                                        o or None, lse or None, B, Hq, Hkv, num_pages, page_size, max_blocks, D,
                                        float(scale), float(q_scale), float(k_scale), float(v_scale),
                                        kv_lens or None, workspace or None, workspace_bytes, stream or None)
    return _check(code) if check else code


def attn_set_tile_table(entries, check=True):
    """entries: a sequence of MIATTN_TILE_FIELDS-int rows (see include/miattn.h)."""
    rows = [list(map(int, e)) for e in entries]
    for r in rows:
        if len(r) != MIATTN_TILE_FIELDS:
            raise ValueError(f"a tile-table entry has {MIATTN_TILE_FIELDS} fields, got {len(r)}")
    arr = (ctypes.c_int32 * (MIATTN_TILE_FIELDS * max(1, len(rows))))(*[x for r in rows for x in r])
    code = load().attn_set_tile_table(ctypes.cast(arr, ctypes.c_void_p), len(rows))
    return _check(code) if check else code


def attn_tile_table_size() -> int:
    return int(load().attn_tile_table_size())


def attn_tile_choice(op, dtype, D, causal, T, size, check=True):
    """(v0, v1) that a launch with this key uses (see include/miattn.h)."""
    out = (ctypes.c_int32 * 2)()
    code = load().attn_tile_choice(int(op), int(dtype), int(D), int(causal), int(T), int(size),
                                   ctypes.cast(out, ctypes.c_void_p))
    if check:
        _check(code)
        return int(out[0]), int(out[1])
    return code
