"""Exact tiled attention for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libmiattn.so`` (C ABI in
``include/miattn.h``); this package is its thin binding.  PyTorch is used for
device memory and the current stream only.

    o, lse = fwd(q, k, v, causal=True)                 # prefill
    o, lse = fwd_fp8(q8, k8, v8, q_scale=.., k_scale=.., v_scale=.., causal=True)   # E4M3 prefill
    o, lse = decode(q, k_cache, v_cache, kv_lens)      # one KV-cache decode step
    o, lse = decode_paged(q, k_pages, v_pages, block_table, kv_lens)   # paged cache
    o, lse = decode_fp8(q8, k8, v8, kv_lens, q_scale=.., k_scale=.., v_scale=..)   # E4M3 cache
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=True) # gradients of the prefill

The C-ABI functions are re-exported under their C names (``attn_fwd``, ``attn_fwd_fp8``,
``attn_decode``, ``attn_decode_paged``, ``attn_decode_fp8``, ``attn_decode_paged_fp8``,
``attn_decode_workspace_size``, ``attn_bwd``,
``attn_bwd_workspace_size``, ``attn_strerror``).
"""

from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MIATTN_BF16,
    MIATTN_F32,
    MiattnError,
    attn_abi_version,
    attn_bwd,
    attn_bwd_workspace_size,
    attn_decode,
    attn_decode_fp8,
    attn_decode_noalloc,
    attn_decode_noalloc_max_bytes,
    attn_decode_paged,
    attn_decode_paged_fp8,
    attn_decode_workspace_size,
    attn_fwd,
    attn_fwd_fp8,
    attn_set_tile_table,
    attn_strerror,
    attn_tile_choice,
    attn_tile_table_size,
    load,
)

__all__ = ["fwd", "fwd_fp8", "decode", "decode_noalloc", "attn_decode_noalloc", "attn_decode_noalloc_max_bytes",
           "decode_paged", "decode_fp8", "decode_paged_fp8", "bwd", "attn_fwd", "attn_decode",
           "attn_decode_paged", "attn_decode_fp8", "attn_decode_paged_fp8", "attn_fwd_fp8",
           "attn_decode_workspace_size", "attn_bwd",
           "attn_bwd_workspace_size", "attn_set_tile_table", "attn_tile_table_size", "attn_tile_choice",
           "attn_strerror", "MiattnError", "load"]


def _torch():
    import torch

    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MIATTN_BF16
    if t.dtype == torch.float32:
        return MIATTN_F32
    raise ValueError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check_tensor(name, t, ndim, dtype, device, shape=None, align=16):
    """A tensor the library reads or writes: dims, dtype, device, contiguity,
    exact shape (when given) and the alignment of its first element (16 bytes
    for tensors the kernels move in 16-byte pieces, 4 for lse and int32
    arrays)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on the device of q ({device}), got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (call .contiguous())")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must start on a {align}-byte boundary (a view with a storage offset "
                         "may not; call .clone())")


def _on_gpu(q):
    if q.device.type != "cuda":
        raise ValueError(f"q must be on a GPU device, got {q.device}")


def _no_alias(outs, ins):
    """Outputs must not overlap any input or each other (include/miattn.h)."""
    def span(t):
        a = t.data_ptr()
        return a, a + t.numel() * t.element_size()
    for i, (on, o) in enumerate(outs):
        a0, a1 = span(o)
        for n, t in list(ins) + outs[i + 1:]:
            b0, b1 = span(t)
            if a0 < b1 and b0 < a1:
                raise ValueError(f"{on} overlaps {n}")


def _out(name, t, shape, dtype, device):
    """A caller-supplied output buffer (checked), or a new one."""
    torch = _torch()
    if t is None:
        return torch.empty(shape, dtype=dtype, device=device)
    _check_tensor(name, t, len(shape), dtype, device, shape=shape, align=4 if dtype == torch.float32 else 16)
    return t


def _workspace(t, nbytes, device):
    torch = _torch()
    if t is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    if not isinstance(t, torch.Tensor) or t.device != device or not t.is_contiguous():
        raise ValueError(f"workspace must be a contiguous tensor on {device}")
    if t.numel() * t.element_size() < nbytes:
        raise ValueError(f"workspace holds {t.numel() * t.element_size()} bytes, {nbytes} needed")
    if t.data_ptr() % 16:
        raise ValueError("workspace must start on a 16-byte boundary")
    return t


def _lens(kv_lens, B, device, required):
    """kv_lens as a contiguous int32 tensor on q's device (a list or array of
    ints is copied there), or None."""
    torch = _torch()
    if kv_lens is None:
        if required:
            raise ValueError("kv_lens is required")
        return None
    if not isinstance(kv_lens, torch.Tensor):
        kv_lens = torch.as_tensor(kv_lens, dtype=torch.int32, device=device)
    if kv_lens.dtype != torch.int32:
        raise ValueError("kv_lens must be int32")
    if tuple(kv_lens.shape) != (B,):
        raise ValueError(f"kv_lens must have shape ({B},)")
    if kv_lens.device != device:
        raise ValueError("kv_lens must live on the same GPU as q")
    kv_lens = kv_lens.contiguous()
    if kv_lens.data_ptr() % 4:
        raise ValueError("kv_lens must start on a 4-byte boundary")
    return kv_lens


def fwd(q, k, v, *, causal: bool = False, kv_lens=None, scale: float | None = None, out=None, lse=None):
    """Prefill attention.  q (B,Hq,Tq,D), k/v (B,Hkv,Tk,D), bf16 or fp32, on the GPU.

    Returns (o (B,Hq,Tq,D) of q's dtype, lse (B,Hq,Tq) float32).  ``out`` and
    ``lse`` may be given (exact shapes and dtypes, contiguous, on q's device,
    not overlapping the inputs).
    """
    torch = _torch()
    dt = _dtype_code(q)
    _on_gpu(q)
    _check_tensor("q", q, 4, q.dtype, q.device)
    B, Hq, Tq, D = q.shape
    _check_tensor("k", k, 4, q.dtype, q.device)
    _check_tensor("v", v, 4, q.dtype, q.device)
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Tk = k.shape[1], k.shape[2]
    lens = _lens(kv_lens, B, q.device, False)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = _out("out", out, (B, Hq, Tq, D), q.dtype, q.device)
    l_out = _out("lse", lse, (B, Hq, Tq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out)], [("q", q), ("k", k), ("v", v)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l_out.data_ptr(), B, Hq, Hkv, Tq, Tk, D,
             scale, 1 if causal else 0, 0 if lens is None else lens.data_ptr(), dt, stream)
    return o, l_out


def decode(q, k_cache, v_cache, kv_lens, *, scale: float | None = None, workspace=None, out=None, lse=None):
    """One decode step.  q (B,Hq,D), caches (B,Hkv,S_max,D), kv_lens int32 (B,) on the GPU.

    kv_lens[b] counts the valid cached keys including the new token.
    Returns (o (B,Hq,D), lse (B,Hq) float32).
    """
    torch = _torch()
    dt = _dtype_code(q)
    _on_gpu(q)
    _check_tensor("q", q, 3, q.dtype, q.device)
    B, Hq, D = q.shape
    _check_tensor("k_cache", k_cache, 4, q.dtype, q.device)
    _check_tensor("v_cache", v_cache, 4, q.dtype, q.device)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    lens = _lens(kv_lens, B, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = attn_decode_workspace_size(B, Hq, Hkv, S_max, D)
    if dt == MIATTN_BF16 or workspace is not None:
        workspace = _workspace(workspace, nbytes, q.device)
    o = _out("out", out, (B, Hq, D), q.dtype, q.device)
    l_out = _out("lse", lse, (B, Hq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out)] + ([] if workspace is None else [("workspace", workspace)]),
              [("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("kv_lens", lens)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws_ptr = 0 if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    attn_decode(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), l_out.data_ptr(), B, Hq, Hkv,
                S_max, D, scale, lens.data_ptr(), ws_ptr, ws_bytes, dt, stream)
    return o, l_out


def decode_noalloc(q, k_cache, v_cache, kv_lens, *, out, lse, scale: float | None = None):
    """decode() through attn_decode_noalloc: the library's fixed scratch
    replaces the workspace, and the caller passes the outputs, so the call
    allocates no device memory (usable under graph capture).  kv_lens must be
    an int32 tensor on q's device.  Returns (out, lse)."""
    torch = _torch()
    dt = _dtype_code(q)
    _on_gpu(q)
    _check_tensor("q", q, 3, q.dtype, q.device)
    B, Hq, D = q.shape
    _check_tensor("k_cache", k_cache, 4, q.dtype, q.device)
    _check_tensor("v_cache", v_cache, 4, q.dtype, q.device)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    if not isinstance(kv_lens, torch.Tensor):
        raise ValueError("kv_lens must be an int32 tensor on the GPU of q (no copy is made here)")
    lens = _lens(kv_lens, B, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check_tensor("out", out, 3, q.dtype, q.device, shape=(B, Hq, D))
    _check_tensor("lse", lse, 2, torch.float32, q.device, shape=(B, Hq), align=4)
    _no_alias([("out", out), ("lse", lse)], [("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("kv_lens", lens)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_decode_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), out.data_ptr(), lse.data_ptr(), B, Hq,
                        Hkv, S_max, D, scale, lens.data_ptr(), dt, stream)
    return out, lse


def _block_table(block_table, B, device):
    torch = _torch()
    if not isinstance(block_table, torch.Tensor) or block_table.dtype != torch.int32 or block_table.dim() != 2 \
            or block_table.shape[0] != B:
        raise ValueError("block_table must be int32 (B, max_blocks)")
    if block_table.device != device or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous tensor on the GPU of q")
    if block_table.data_ptr() % 4:
        raise ValueError("block_table must start on a 4-byte boundary")
    return block_table.shape[1]


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, *, scale: float | None = None, workspace=None, out=None,
                 lse=None):
    """One decode step against a paged cache.  q (B,Hq,D) bf16; k_pages / v_pages (num_pages,Hkv,page_size,D)
    bf16; block_table int32 (B, max_blocks); kv_lens int32 (B,); all on the GPU.

    Logical key j of sequence b is row j % page_size of page block_table[b, j // page_size].
    Returns (o (B,Hq,D), lse (B,Hq) float32).
    """
    torch = _torch()
    if q.dtype != torch.bfloat16:
        raise ValueError("decode_paged takes bfloat16 tensors")
    _on_gpu(q)
    _check_tensor("q", q, 3, q.dtype, q.device)
    B, Hq, D = q.shape
    _check_tensor("k_pages", k_pages, 4, q.dtype, q.device)
    _check_tensor("v_pages", v_pages, 4, q.dtype, q.device)
    if k_pages.shape != v_pages.shape or k_pages.shape[3] != D:
        raise ValueError("page pool shapes do not match q")
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_blocks = _block_table(block_table, B, q.device)
    lens = _lens(kv_lens, B, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = attn_decode_workspace_size(B, Hq, Hkv, max_blocks * page_size, D)
    workspace = _workspace(workspace, nbytes, q.device)
    o = _out("out", out, (B, Hq, D), q.dtype, q.device)
    l_out = _out("lse", lse, (B, Hq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out), ("workspace", workspace)],
              [("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
               ("kv_lens", lens)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_decode_paged(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(), o.data_ptr(),
                      l_out.data_ptr(), B, Hq, Hkv, num_pages, page_size, max_blocks, D, scale, lens.data_ptr(),
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(), MIATTN_BF16, stream)
    return o, l_out


def _e4m3_bytes(name, t, ndim, device):
    """Check an E4M3 tensor (torch.float8_e4m3fn or its uint8 codes)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError(f"{name} must be float8_e4m3fn or uint8 E4M3 codes, got {getattr(t, 'dtype', type(t))}")
    _check_tensor(name, t, ndim, t.dtype, device)


def fwd_fp8(q, k, v, *, q_scale: float, k_scale: float, v_scale: float, causal: bool = False, kv_lens=None,
            scale: float | None = None, out=None, lse=None):
    """Prefill on E4M3 inputs.  q (B,Hq,Tq,D), k/v (B,Hkv,Tk,D): float8_e4m3fn (or uint8 codes) on the GPU,
    each standing for its codes times its scale.

    Scores are scale * (q_scale q).(k_scale k) and O = P (v_scale V).
    Returns (o (B,Hq,Tq,D) bfloat16, lse (B,Hq,Tq) float32).
    """
    torch = _torch()
    _on_gpu(q)
    _e4m3_bytes("q", q, 4, q.device)
    B, Hq, Tq, D = q.shape
    _e4m3_bytes("k", k, 4, q.device)
    _e4m3_bytes("v", v, 4, q.device)
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    Hkv, Tk = k.shape[1], k.shape[2]
    lens = _lens(kv_lens, B, q.device, False)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = _out("out", out, (B, Hq, Tq, D), torch.bfloat16, q.device)
    l_out = _out("lse", lse, (B, Hq, Tq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out)], [("q", q), ("k", k), ("v", v)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l_out.data_ptr(), B, Hq, Hkv, Tq, Tk, D,
                 scale, q_scale, k_scale, v_scale, 1 if causal else 0, 0 if lens is None else lens.data_ptr(), stream)
    return o, l_out


def decode_fp8(q, k_cache, v_cache, kv_lens, *, q_scale: float, k_scale: float, v_scale: float,
               scale: float | None = None, workspace=None, out=None, lse=None):
    """One decode step on an E4M3 cache.  q (B,Hq,D), caches (B,Hkv,S_max,D): float8_e4m3fn (or uint8
    codes) on the GPU, each standing for its codes times its scale; kv_lens int32 (B,).

    Scores are scale * (q_scale q).(k_scale k) and O = P (v_scale V).
    Returns (o (B,Hq,D) bfloat16, lse (B,Hq) float32).
    """
    torch = _torch()
    _on_gpu(q)
    _e4m3_bytes("q", q, 3, q.device)
    B, Hq, D = q.shape
    _e4m3_bytes("k_cache", k_cache, 4, q.device)
    _e4m3_bytes("v_cache", v_cache, 4, q.device)
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != D:
        raise ValueError("cache shapes do not match q")
    Hkv, S_max = k_cache.shape[1], k_cache.shape[2]
    lens = _lens(kv_lens, B, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = attn_decode_workspace_size(B, Hq, Hkv, S_max, D)
    workspace = _workspace(workspace, nbytes, q.device)
    o = _out("out", out, (B, Hq, D), torch.bfloat16, q.device)
    l_out = _out("lse", lse, (B, Hq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out), ("workspace", workspace)],
              [("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("kv_lens", lens)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_decode_fp8(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), o.data_ptr(), l_out.data_ptr(), B, Hq,
                    Hkv, S_max, D, scale, q_scale, k_scale, v_scale, lens.data_ptr(), workspace.data_ptr(),
                    workspace.numel() * workspace.element_size(), stream)
    return o, l_out


def decode_paged_fp8(q, k_pages, v_pages, block_table, kv_lens, *, q_scale: float, k_scale: float,
                     v_scale: float, scale: float | None = None, workspace=None, out=None, lse=None):
    """decode_paged on E4M3 pools (num_pages,Hkv,page_size,D) with per-tensor scales, as decode_fp8.

    Returns (o (B,Hq,D) bfloat16, lse (B,Hq) float32).
    """
    torch = _torch()
    _on_gpu(q)
    _e4m3_bytes("q", q, 3, q.device)
    B, Hq, D = q.shape
    _e4m3_bytes("k_pages", k_pages, 4, q.device)
    _e4m3_bytes("v_pages", v_pages, 4, q.device)
    if k_pages.shape != v_pages.shape or k_pages.shape[3] != D:
        raise ValueError("page pool shapes do not match q")
    num_pages, Hkv, page_size = k_pages.shape[0], k_pages.shape[1], k_pages.shape[2]
    max_blocks = _block_table(block_table, B, q.device)
    lens = _lens(kv_lens, B, q.device, True)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = attn_decode_workspace_size(B, Hq, Hkv, max_blocks * page_size, D)
    workspace = _workspace(workspace, nbytes, q.device)
    o = _out("out", out, (B, Hq, D), torch.bfloat16, q.device)
    l_out = _out("lse", lse, (B, Hq), torch.float32, q.device)
    _no_alias([("out", o), ("lse", l_out), ("workspace", workspace)],
              [("q", q), ("k_pages", k_pages), ("v_pages", v_pages), ("block_table", block_table),
               ("kv_lens", lens)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_decode_paged_fp8(q.data_ptr(), k_pages.data_ptr(), v_pages.data_ptr(), block_table.data_ptr(),
                          o.data_ptr(), l_out.data_ptr(), B, Hq, Hkv, num_pages, page_size, max_blocks, D, scale,
                          q_scale, k_scale, v_scale, lens.data_ptr(), workspace.data_ptr(),
                          workspace.numel() * workspace.element_size(), stream)
    return o, l_out


def bwd(q, k, v, o, lse, do, *, causal: bool = False, kv_lens=None, scale: float | None = None, workspace=None,
        dq=None, dk=None, dv=None):
    """Gradients of the prefill.  q, o, do (B,Hq,Tq,D) and k, v (B,Hkv,Tk,D) bf16, lse (B,Hq,Tq) float32,
    all on the GPU; o and lse as fwd returned them with the same causal / kv_lens / scale.

    Returns (dq, dk, dv) in bf16 with the shapes of q, k, v.
    """
    torch = _torch()
    if q.dtype != torch.bfloat16:
        raise ValueError("bwd takes bfloat16 tensors")
    _on_gpu(q)
    _check_tensor("q", q, 4, torch.bfloat16, q.device)
    B, Hq, Tq, D = q.shape
    for name, t in (("o", o), ("do", do)):
        _check_tensor(name, t, 4, torch.bfloat16, q.device, shape=q.shape)
    _check_tensor("k", k, 4, torch.bfloat16, q.device)
    _check_tensor("v", v, 4, torch.bfloat16, q.device)
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)} does not match q {tuple(q.shape)}")
    _check_tensor("lse", lse, 3, torch.float32, q.device, shape=(B, Hq, Tq), align=4)
    Hkv, Tk = k.shape[1], k.shape[2]
    lens = _lens(kv_lens, B, q.device, False)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    nbytes = attn_bwd_workspace_size(B, Hq, Tq)
    workspace = _workspace(workspace, nbytes, q.device)
    dq = _out("dq", dq, tuple(q.shape), torch.bfloat16, q.device)
    dk = _out("dk", dk, tuple(k.shape), torch.bfloat16, q.device)
    dv = _out("dv", dv, tuple(v.shape), torch.bfloat16, q.device)
    _no_alias([("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)],
              [("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("do", do)])
    stream = torch.cuda.current_stream(q.device).cuda_stream
    attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
             dk.data_ptr(), dv.data_ptr(), B, Hq, Hkv, Tq, Tk, D, scale, 1 if causal else 0,
             0 if lens is None else lens.data_ptr(), workspace.data_ptr(),
             workspace.numel() * workspace.element_size(), MIATTN_BF16, stream)
    return dq, dk, dv
