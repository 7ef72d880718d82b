"""Tile-by-tile online softmax in float64.  TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the HIP product path never does.

The algorithm, in the order the pages give it:

* NumPy build guide, *Architecture Overview* and *Step 5*: split the query rows
  into tiles of ``tile_q`` rows and the keys/values into tiles of ``tile_k``
  rows; loop over query tiles, then over key tiles, accumulating a partial
  output per query tile.
* "Implementing attention from scratch", *Stable softmax*: process keys in
  blocks while keeping a running row maximum m and a running denominator l;
  whenever the maximum grows, rescale the earlier partial results by
  exp(m_old - m_new).  (The same step is the online-softmax task and Hint 1
  of "Self-Attention: Implementation, Complexity, and Efficient Variants",
  and Figure 9.8 of Transformers in Action, section 9.4.1.)

The NumPy guide's own Step 5 normalises every tile by its own sum and adds
the tile outputs; that is not softmax over the whole row (with V = 1 it
returns the number of key tiles, not 1), so the accumulation here is the
running-max / running-sum rescale above, which is what its prose describes.

This module exists to pin that the tiled method reaches the plain definition
(``oracle.attention``) to float64 rounding; it is not a model of the GPU
kernels' tile shapes or instruction order.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, valid_lengths


def tiled_attention(q, k, v, scale: float, causal: bool = False, kv_lens=None,
                    tile_q: int = 64, tile_k: int = 64):
    """Online-softmax attention, one (query tile, key tile) pair at a time.

    Shapes and mask semantics as ``oracle.attention``.  Returns
    (o (B, Hq, Tq, D) float64, lse (B, Hq, Tq) float64).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, _ = k.shape
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    o = np.zeros((B, Hq, Tq, D), dtype=np.float64)
    lse = np.full((B, Hq, Tq), -np.inf, dtype=np.float64)
    for b in range(B):
        lk, lq = lk_all[b], lq_all[b]
        off = lk - lq
        for h in range(Hq):
            hk = h // G
            for q_start in range(0, Tq, tile_q):
                q_end = min(q_start + tile_q, Tq)
                rows = np.arange(q_start, q_end)
                qt = q[b, h, q_start:q_end]
                n = q_end - q_start
                m = np.full(n, -np.inf)       # running row maximum
                l = np.zeros(n)               # running denominator
                acc = np.zeros((n, D))        # running un-normalised output
                for k_start in range(0, Tk, tile_k):
                    k_end = min(k_start + tile_k, Tk)
                    cols = np.arange(k_start, k_end)
                    s = scale * (qt @ k[b, hk, k_start:k_end].T)   # tile scores
                    allowed = (cols[None, :] < lk) & (rows[:, None] < lq)
                    if causal:
                        allowed &= cols[None, :] <= rows[:, None] + off
                    s = np.where(allowed, s, -np.inf)
                    m_new = np.maximum(m, s.max(axis=1))
                    # a row that has seen no allowed key yet keeps m = -inf;
                    # use 0 as its reference so that no -inf - (-inf) arises
                    ref = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - ref)                        # rescale of old partials
                    p = np.where(allowed, np.exp(s - ref[:, None]), 0.0)
                    l = alpha * l + p.sum(axis=1)
                    acc = alpha[:, None] * acc + p @ np.where(allowed.any(axis=0)[:, None],
                                                              v[b, hk, k_start:k_end], 0.0)
                    m = m_new
                ok = l > 0
                o[b, h, q_start:q_end][ok] = acc[ok] / l[ok, None]
                lse[b, h, q_start:q_end][ok] = m[ok] + np.log(l[ok])
    return o, lse
