"""Attention on 8-bit floating-point (E4M3) inputs.  TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the HIP product path never does.

Source, by page: the self-attention interview question ("Self-Attention:
Implementation, Complexity ..."), Follow-up questions, names FP8 support as
one of FlashAttention-3's additions.  The page fixes neither the number
format nor how values are scaled, so the plainest reading is taken:

* Each of Q, K and V arrives as a tensor of E4M3 codes (the "fn" variant of
  the OCP 8-bit floating-point formats: 1 sign bit, 4 exponent bits with bias
  7, 3 mantissa bits, subnormals, no infinities, codes 0x7f / 0xff are NaN,
  largest finite magnitude 448) and one float scale per tensor.  The value
  an element stands for is scale * decode(code).
* The operation is then exactly the attention of ``oracle.attention`` on
  those values:  O = softmax(s * (q_scale Q)(k_scale K)^T + mask)(v_scale V)
  with the same causal, key-padding and grouped-query semantics, and the
  same LSE.

``e4m3_decode`` is written from the format definition above, value by value;
nothing here converts through a library's float8 type.
"""

from __future__ import annotations

import numpy as np

from .attention import attention, attention_rows, decode, decode_paged


def _e4m3_table() -> np.ndarray:
    """float64 value of each of the 256 codes (NaN for the two NaN codes)."""
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            out[code] = np.nan
        elif e == 0:
            out[code] = sign * (m / 8.0) * 2.0 ** (1 - 7)          # subnormal
        else:
            out[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)    # normal
    return out


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of an array of E4M3 codes (any integer dtype, or a
    torch uint8 / float8_e4m3fn tensor viewed as bytes)."""
    if hasattr(codes, "detach"):   # a torch tensor: take its raw bytes
        import torch
        t = codes.detach().cpu()
        if t.dtype != torch.uint8:
            t = t.view(torch.uint8)
        codes = t.numpy()
    c = np.asarray(codes)
    return E4M3_VALUES[c.astype(np.int64) & 0xFF]


class Scaled:
    """Lazily decoded view of an E4M3 code array times a per-tensor scale.

    Indexing returns the float64 values of the selected codes only, so a
    full-size cache is never decoded as a whole; ``shape`` is the codes'."""

    def __init__(self, codes, scale):
        if hasattr(codes, "detach"):
            import torch
            t = codes.detach().cpu()
            codes = (t if t.dtype == torch.uint8 else t.view(torch.uint8)).numpy()
        self.codes = np.asarray(codes)
        self.scale = float(scale)
        self.shape = self.codes.shape

    def __getitem__(self, idx):
        return e4m3_decode(self.codes[idx]) * self.scale


def attention_fp8(q8, k8, v8, q_scale, k_scale, v_scale, scale, causal=False, kv_lens=None):
    """(O, LSE) of attention on E4M3 inputs with per-tensor scales.

    q8: codes (B, Hq, Tq, D); k8, v8: codes (B, Hkv, Tk, D)."""
    q = e4m3_decode(q8) * float(q_scale)
    k = e4m3_decode(k8) * float(k_scale)
    v = e4m3_decode(v8) * float(v_scale)
    return attention(q, k, v, scale, causal=causal, kv_lens=kv_lens)


def attention_rows_fp8(q8, k8, v8, rows, q_scale, k_scale, v_scale, scale, causal=False, kv_lens=None):
    """``attention_rows`` on E4M3 inputs: only the touched heads are decoded."""
    return attention_rows(Scaled(q8, q_scale), Scaled(k8, k_scale), Scaled(v8, v_scale), rows, scale,
                          causal=causal, kv_lens=kv_lens)


def decode_fp8(q8, k8_cache, v8_cache, kv_lens, q_scale, k_scale, v_scale, scale, batches=None):
    """One decode step on an E4M3 cache.  q8 (B, Hq, D); caches (B, Hkv,
    S_max, D).  Only rows below kv_lens[b] are decoded."""
    return decode(Scaled(q8, q_scale), Scaled(k8_cache, k_scale), Scaled(v8_cache, v_scale), kv_lens, scale,
                  batches=batches)


def decode_paged_fp8(q8, k8_pages, v8_pages, block_table, kv_lens, q_scale, k_scale, v_scale, scale, batches=None):
    """One decode step on an E4M3 paged cache (pools (num_pages, Hkv, P, D))."""
    return decode_paged(Scaled(q8, q_scale), Scaled(k8_pages, k_scale), Scaled(v8_pages, v_scale), block_table,
                        kv_lens, scale, batches=batches)
