"""Seeded synthetic inputs for the five attention workloads.

This module draws random tensors and lengths and nothing else: it holds none
of the attention arithmetic, so both the HIP path and the float64 oracle can
be fed from it without sharing any of the method's code.

Workloads (shapes follow "Implementing attention from scratch", *Shapes
first*: Q (B, Hq, Tq, D), K/V (B, Hkv, Tk, D); decode caches
(B, Hkv, S_max, D)):

=========  ===================================================================
name       description
=========  ===================================================================
single     1 head, non-causal, Q 256x64, K/V 512x64, fp32 N(0,1) drawn with
           the NumPy legacy generator seeded with 0 in the order Q, K, V (the
           NumPy build guide, *Step 1*).
causal     causal self-attention prefill, B=4, H=16, T=1024, D=64, bf16.
ragged     non-causal with key padding, B=8, H=16, T=4096 padded, D=128,
           bf16; lengths uniform in [1, 4096], the first forced to 1.
decode     KV-cache decode with GQA, B=64, Hq=32, Hkv=8, D=128, one query per
           sequence, cached lengths uniform in [1024, 32768], cache
           (B, Hkv, 32768, D) bf16.
long       long-context causal prefill, B=1, H=32, T=32768, D=128, bf16.
decode-fp8 the decode workload with q and the caches as E4M3 codes (FP8, one
           scale per tensor).
causal-fp8, long-fp8
           the causal and long prefill workloads with E4M3 Q, K, V.
=========  ===================================================================

bf16 tensors are drawn as float32 N(0,1) from a seeded ``torch.Generator``
and rounded to bf16 (round-to-nearest-even, torch's ``.to``); the oracle is
then given exactly those bf16 values.  Lengths come from
``numpy.random.default_rng(seed)``.

E4M3 tensors are the same N(0,1) draws divided by a per-tensor scale chosen
so that 6 standard deviations map to the largest code (6 / 448), clamped to
+-448 and rounded by torch's float8_e4m3fn cast; the tensor then stands for
codes * scale, and the oracle decodes exactly those codes.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str          # "fwd" or "decode"
    B: int
    Hq: int
    Hkv: int
    Tq: int            # 1 for decode
    Tk: int            # S_max for decode
    D: int
    dtype: str         # "f32", "bf16" or "e4m3"
    causal: bool
    lens: tuple | None = None   # (lo, hi, force_first_one) or None
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


WORKLOADS = {
    "single": Workload("single", "fwd", 1, 1, 1, 256, 512, 64, "f32", False, None,
                       "1 head, non-causal, Q 256x64, K/V 512x64, fp32, seed 0"),
    "causal": Workload("causal", "fwd", 4, 16, 16, 1024, 1024, 64, "bf16", True, None,
                       "causal prefill B=4 H=16 T=1024 D=64 bf16"),
    "ragged": Workload("ragged", "fwd", 8, 16, 16, 4096, 4096, 128, "bf16", False, (1, 4096, True),
                       "ragged non-causal B=8 H=16 T=4096 D=128 bf16, lengths U[1,4096]"),
    "decode": Workload("decode", "decode", 64, 32, 8, 1, 32768, 128, "bf16", True, (1024, 32768, False),
                       "decode GQA B=64 Hq=32 Hkv=8 D=128, lengths U[1024,32768]"),
    "long": Workload("long", "fwd", 1, 32, 32, 32768, 32768, 128, "bf16", True, None,
                     "long causal prefill B=1 H=32 T=32768 D=128 bf16"),
    "causal-fp8": Workload("causal-fp8", "fwd", 4, 16, 16, 1024, 1024, 64, "e4m3", True, None,
                           "causal prefill B=4 H=16 T=1024 D=64, E4M3 Q/K/V"),
    "long-fp8": Workload("long-fp8", "fwd", 1, 32, 32, 32768, 32768, 128, "e4m3", True, None,
                         "long causal prefill B=1 H=32 T=32768 D=128, E4M3 Q/K/V"),
    "decode-fp8": Workload("decode-fp8", "decode", 64, 32, 8, 1, 32768, 128, "e4m3", True, (1024, 32768, False),
                           "decode GQA B=64 Hq=32 Hkv=8 D=128, lengths U[1024,32768], E4M3 q/K/V"),
}

# Largest finite E4M3 magnitude, and the per-tensor scale of the synthetic
# E4M3 inputs (a standard deviation of 1 spread over the code range).
E4M3_MAX = 448.0
E4M3_SCALE = 6.0 / E4M3_MAX


def draw_lengths(B: int, lo: int, hi: int, force_first_one: bool = False, seed: int = 0) -> np.ndarray:
    """Per-sequence lengths, uniform integers in [lo, hi]."""
    lens = np.random.default_rng(seed).integers(lo, hi + 1, size=B).astype(np.int32)
    if force_first_one and B > 0:
        lens[0] = 1
    return lens


def randn_bf16(shape, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """float32 N(0,1) draws rounded to bf16."""
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(torch.bfloat16)


def randn_e4m3(shape, gen: torch.Generator, scale: float = E4M3_SCALE, device="cpu") -> torch.Tensor:
    """E4M3 codes (torch.float8_e4m3fn) of float32 N(0,1) draws divided by ``scale``."""
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) / scale
    return x.clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)


def make_fwd_inputs(B, Hq, Hkv, Tq, Tk, D, dtype="bf16", seed=0, device="cpu"):
    """Q, K, V for a prefill call, drawn in the order Q, K, V."""
    if dtype == "f32":
        g = torch.Generator(device=device).manual_seed(seed)
        mk = lambda s: torch.randn(s, generator=g, device=device, dtype=torch.float32)  # noqa: E731
    else:
        g = torch.Generator(device=device).manual_seed(seed)
        mk = lambda s: randn_bf16(s, g, device)  # noqa: E731
    q = mk((B, Hq, Tq, D))
    k = mk((B, Hkv, Tk, D))
    v = mk((B, Hkv, Tk, D))
    return q, k, v


def make_single(seed: int = 0):
    """The NumPy build guide's Step 1 inputs, as (1, 1, T, 64) float32 tensors."""
    rs = np.random.RandomState(seed)
    q = rs.randn(256, 64).astype(np.float32)
    k = rs.randn(512, 64).astype(np.float32)
    v = rs.randn(512, 64).astype(np.float32)
    t = lambda a: torch.from_numpy(a).reshape(1, 1, *a.shape)  # noqa: E731
    return t(q), t(k), t(v)


def poison_tail_(x: torch.Tensor, lens, value=float("nan")) -> torch.Tensor:
    """Fill rows >= lens[b] along the sequence axis (dim 2) of (B, H, T, D) with ``value``."""
    for b, L in enumerate(np.asarray(lens).reshape(-1).tolist()):
        L = max(0, min(int(L), x.shape[2]))
        if L < x.shape[2]:
            x[b, :, L:, :] = value
    return x


def make_decode_inputs(B, Hq, Hkv, S_max, D, lens, seed=0, device="cpu", poison=False):
    """q (B, Hq, D) and caches (B, Hkv, S_max, D), bf16; the caches are drawn one
    sequence at a time from one generator so the full float32 tensor is never held."""
    g = torch.Generator(device=device).manual_seed(seed)
    q = randn_bf16((B, Hq, D), g, device)
    k = torch.empty((B, Hkv, S_max, D), dtype=torch.bfloat16, device=device)
    v = torch.empty((B, Hkv, S_max, D), dtype=torch.bfloat16, device=device)
    for b in range(B):
        k[b] = randn_bf16((Hkv, S_max, D), g, device)
    for b in range(B):
        v[b] = randn_bf16((Hkv, S_max, D), g, device)
    if poison:
        poison_tail_(k, lens)
        poison_tail_(v, lens)
    return q, k, v


def make_fwd_inputs_fp8(B, Hq, Hkv, Tq, Tk, D, seed=0, device="cpu",
                        scales=(E4M3_SCALE, E4M3_SCALE, E4M3_SCALE)):
    """E4M3 Q, K, V for a prefill call (drawn in that order) and their scales."""
    g = torch.Generator(device=device).manual_seed(seed)
    qs, ks, vs = scales
    q = randn_e4m3((B, Hq, Tq, D), g, qs, device)
    k = randn_e4m3((B, Hkv, Tk, D), g, ks, device)
    v = randn_e4m3((B, Hkv, Tk, D), g, vs, device)
    return q, k, v, (qs, ks, vs)


def make_decode_inputs_fp8(B, Hq, Hkv, S_max, D, lens, seed=0, device="cpu", poison=False,
                           scales=(E4M3_SCALE, E4M3_SCALE, E4M3_SCALE)):
    """E4M3 q (B, Hq, D) and caches (B, Hkv, S_max, D) plus their scales
    (q_scale, k_scale, v_scale); poisoned rows hold the NaN code 0x7f."""
    g = torch.Generator(device=device).manual_seed(seed)
    qs, ks, vs = scales
    q = randn_e4m3((B, Hq, D), g, qs, device)
    k = torch.empty((B, Hkv, S_max, D), dtype=torch.float8_e4m3fn, device=device)
    v = torch.empty((B, Hkv, S_max, D), dtype=torch.float8_e4m3fn, device=device)
    for b in range(B):
        k[b] = randn_e4m3((Hkv, S_max, D), g, ks, device)
    for b in range(B):
        v[b] = randn_e4m3((Hkv, S_max, D), g, vs, device)
    if poison:
        for t in (k, v):
            poison_tail_(t.view(torch.uint8), lens, 0x7F)
    return q, k, v, (qs, ks, vs)


def make(name: str, seed: int = 0, device="cpu", poison=False):
    """Inputs for a named workload.

    Returns a dict with q, k, v, kv_lens (int32 tensor or None), scale, causal
    and the Workload record.
    """
    w = WORKLOADS[name]
    lens = None
    if w.lens is not None:
        lo, hi, force = w.lens
        lens = draw_lengths(w.B, lo, hi, force, seed)
    if name == "single":
        q, k, v = make_single(seed)
        q, k, v = q.to(device), k.to(device), v.to(device)
    elif w.kind == "decode" and w.dtype == "e4m3":
        q, k, v, fp8_scales = make_decode_inputs_fp8(w.B, w.Hq, w.Hkv, w.Tk, w.D, lens, seed, device, poison)
    elif w.kind == "decode":
        q, k, v = make_decode_inputs(w.B, w.Hq, w.Hkv, w.Tk, w.D, lens, seed, device, poison)
    elif w.dtype == "e4m3":
        q, k, v, fp8_scales = make_fwd_inputs_fp8(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.D, seed, device)
        if poison and lens is not None:
            poison_tail_(k.view(torch.uint8), lens, 0x7F)
            poison_tail_(v.view(torch.uint8), lens, 0x7F)
    else:
        q, k, v = make_fwd_inputs(w.B, w.Hq, w.Hkv, w.Tq, w.Tk, w.D, w.dtype, seed, device)
        if poison and lens is not None:
            poison_tail_(k, lens)
            poison_tail_(v, lens)
    kv = None if lens is None else torch.from_numpy(lens).to(device)
    out = dict(q=q, k=k, v=v, kv_lens=kv, lens=lens, scale=w.scale, causal=w.causal, workload=w)
    if w.dtype == "e4m3":
        out["fp8_scales"] = fp8_scales
    return out
