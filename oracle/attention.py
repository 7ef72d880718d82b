"""Plain float64 attention: the definition written out.  TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the HIP product path never does.

What is computed (sources, by page title and section):

* "Implementing attention from scratch", *Shapes first*: Q is (B, H, T, D),
  K and V are (B, H, S, D); scores are (B, H, T, S).
* "Implementing attention from scratch", *Why scale by sqrt(D)* and the NumPy
  build guide's *Step 2* / *Verification*: scores are scale * q . k, with
  scale = 1/sqrt(D) by default (the caller passes it).
* "Implementing attention from scratch", *Stable softmax*: subtract the row
  maximum before exponentiating (mathematically identical result).
* "Implementing attention from scratch", *Masks*: a causal row i sees keys
  j <= i; padding removes keys; a row with every key masked needs explicit
  handling (here: O = 0, LSE = -inf, never NaN).
* "Implementing attention from scratch", *KV caching*: when query and key
  lengths differ the causal mask is aligned bottom-right, i.e. row i sees
  keys j <= i + (Lk - Lq); grouped-query attention shares one KV head among
  consecutive query heads (query head h uses KV head h // (Hq // Hkv)).
* The log-sum-exp of a row is the natural log of its softmax denominator,
  LSE_i = log sum_j exp(scale * q_i . k_j) over the allowed keys.

Valid lengths (the library's key-padding semantics): with ``kv_lens`` given,
sequence b has Lk = clamp(kv_lens[b], 0, Tk) valid keys; when Tq == Tk the
first Lk query rows are valid too (self-attention with padding: rows past the
length are padding, O = 0 and LSE = -inf there).  Otherwise every query row is
valid.  The causal offset is off = Lk - Lq.
"""

from __future__ import annotations

import numpy as np


def valid_lengths(B: int, Tq: int, Tk: int, kv_lens=None):
    """Per-sequence (Lk, Lq) under the key-padding semantics described above."""
    if kv_lens is None:
        return [Tk] * B, [Tq] * B
    lens = np.asarray(kv_lens).reshape(-1).astype(np.int64)
    if lens.shape[0] != B:
        raise ValueError("kv_lens must have B entries")
    lk = [int(min(max(x, 0), Tk)) for x in lens]
    lq = list(lk) if Tq == Tk else [Tq] * B
    return lk, lq


def _as_f64(x):
    """Upcast to a float64 numpy array (exact for fp32 and bf16 inputs)."""
    try:  # torch tensors (bf16 has no numpy dtype, so go through float32: exact)
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def _rows_block(q_rows, k_all, v_all, scale, row_idx, lk, off, causal):
    """Softmax attention of a block of query rows against one KV head.

    q_rows: (n, D) float64, the query rows with absolute indices ``row_idx``.
    k_all, v_all: (Tk, D) float64.  Returns (o (n, D), lse (n,)).
    """
    n, d = q_rows.shape
    o = np.zeros((n, d), dtype=np.float64)
    lse = np.full((n,), -np.inf, dtype=np.float64)
    if lk <= 0 or n == 0:
        return o, lse
    # keys a row may see: j < lk and, if causal, j <= i + off
    hi = lk
    if causal:
        hi = min(lk, int(row_idx.max()) + off + 1)
    if hi <= 0:
        return o, lse
    s = scale * (q_rows @ k_all[:hi].T)  # (n, hi)
    j = np.arange(hi)[None, :]
    allowed = np.ones((n, hi), dtype=bool)
    if causal:
        allowed = j <= (row_idx[:, None] + off)
    s = np.where(allowed, s, -np.inf)
    any_allowed = allowed.any(axis=1)
    m = np.where(any_allowed, s.max(axis=1), 0.0)
    p = np.where(allowed, np.exp(s - m[:, None]), 0.0)
    l = p.sum(axis=1)
    ok = any_allowed & (l > 0)
    o[ok] = (p[ok] @ v_all[:hi]) / l[ok, None]
    lse[ok] = m[ok] + np.log(l[ok])
    return o, lse


def attention(q, k, v, scale: float, causal: bool = False, kv_lens=None, row_chunk: int = 256):
    """Exact attention in float64.

    q: (B, Hq, Tq, D); k, v: (B, Hkv, Tk, D), Hq a multiple of Hkv.
    Returns (o (B, Hq, Tq, D) float64, lse (B, Hq, Tq) float64).

    Query rows are processed ``row_chunk`` at a time against all keys they may
    see, so no (Tq, Tk) matrix is formed for long sequences; each chunk is the
    plain softmax over the full row, so chunking does not change the result.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    B, Hq, Tq, D = q.shape
    Bk, Hkv, Tk, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("shape mismatch")
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    o = np.zeros((B, Hq, Tq, D), dtype=np.float64)
    lse = np.full((B, Hq, Tq), -np.inf, dtype=np.float64)
    for b in range(B):
        lk, lq = lk_all[b], lq_all[b]
        off = lk - lq
        for h in range(Hq):
            hk = h // G
            for i0 in range(0, min(lq, Tq), row_chunk):
                i1 = min(i0 + row_chunk, lq, Tq)
                idx = np.arange(i0, i1)
                ob, lb = _rows_block(q[b, h, i0:i1], k[b, hk], v[b, hk], scale, idx, lk, off, causal)
                o[b, h, i0:i1] = ob
                lse[b, h, i0:i1] = lb
    return o, lse


def attention_rows(q, k, v, rows, scale: float, causal: bool = False, kv_lens=None, row_chunk: int = 256):
    """The same definition, evaluated only at the listed (b, h, i) rows.

    ``rows`` is an iterable of (b, h, i).  Rows of one (b, h) are evaluated
    together, ``row_chunk`` at a time, each against every key it may see (the
    plain softmax over the full row, as in ``attention``); only the touched
    query rows and K/V heads are upcast, so this reaches full-size inputs
    (e.g. a 32k causal prefill).
    Returns (o (n, D) float64, lse (n,) float64) in the order of ``rows``.
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    B, Hq, Tq, D = q.shape
    _, Hkv, Tk, _ = k.shape
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    o = np.zeros((len(rows), D), dtype=np.float64)
    lse = np.full((len(rows),), -np.inf, dtype=np.float64)
    groups = {}
    for n, (b, h, i) in enumerate(rows):
        if i < lq_all[b]:
            groups.setdefault((b, h), []).append((i, n))
    kv_cache = {}
    for (b, h), members in sorted(groups.items()):
        lk, lq = lk_all[b], lq_all[b]
        hk = h // G
        if (b, hk) not in kv_cache:
            kv_cache.clear()
            kv_cache[(b, hk)] = (_as_f64(k[b, hk, :lk]), _as_f64(v[b, hk, :lk]))
        kk, vv = kv_cache[(b, hk)]
        members.sort()
        for c0 in range(0, len(members), row_chunk):
            part = members[c0:c0 + row_chunk]
            idx = np.array([i for i, _ in part], dtype=np.int64)
            qi = np.stack([_as_f64(q[b, h, i]) for i in idx.tolist()])
            ob, lb = _rows_block(qi, kk, vv, scale, idx, lk, lk - lq, causal)
            for r, (_, n) in enumerate(part):
                o[n] = ob[r]
                lse[n] = lb[r]
    return o, lse


def decode(q, k_cache, v_cache, kv_lens, scale: float, batches=None):
    """One decode step: one new query per (sequence, query head).

    "Implementing attention from scratch", *KV caching* and *Cost model*: a
    decode step attends one new query over the cached positions, and reads
    the whole cache.  ``kv_lens[b]`` counts the valid cached keys *including*
    the new token, whose K/V the caller has already written at index
    kv_lens[b] - 1; the new query sits at that position and so sees keys
    0 .. kv_lens[b] - 1 (bottom-right causal alignment with one query row).

    q: (B, Hq, D); k_cache, v_cache: (B, Hkv, S_max, D); kv_lens: (B,) ints.
    ``batches`` optionally restricts the work to a subset of sequences (other
    rows of the result stay zero / -inf).
    Returns (o (B, Hq, D) float64, lse (B, Hq) float64).
    """
    B, Hq, D = q.shape
    _, Hkv, S_max, _ = k_cache.shape
    G = Hq // Hkv
    lens = np.asarray(_as_f64(kv_lens)).reshape(-1)
    o = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B) if batches is None else batches:
        L = int(min(max(lens[b], 0), S_max))
        if L == 0:
            continue
        for hk in range(Hkv):
            kk = _as_f64(k_cache[b, hk, :L])
            vv = _as_f64(v_cache[b, hk, :L])
            qg = _as_f64(q[b, hk * G : (hk + 1) * G])  # (G, D)
            s = scale * (qg @ kk.T)  # (G, L)
            m = s.max(axis=1, keepdims=True)
            p = np.exp(s - m)
            l = p.sum(axis=1, keepdims=True)
            o[b, hk * G : (hk + 1) * G] = (p @ vv) / l
            lse[b, hk * G : (hk + 1) * G] = (m + np.log(l))[:, 0]
    return o, lse


def decode_paged(q, k_pages, v_pages, block_table, kv_lens, scale: float, batches=None):
    """The decode step of ``decode`` over a paged cache.

    The per-sequence cache is held in fixed-size pages of one pool (the
    PagedAttention layout named in the introduction of "Implementing attention
    from scratch"): logical key j of sequence b and KV head hk is
    ``k_pages[block_table[b, j // P], hk, j % P]`` with P the page size, and
    the same for V.  The step itself is the decode definition above over the
    logical keys 0 .. kv_lens[b] - 1 (clamped to the table's capacity).

    q: (B, Hq, D); k_pages, v_pages: (num_pages, Hkv, P, D);
    block_table: (B, max_blocks) ints.  Returns (o, lse) as ``decode``.
    """
    B, Hq, D = q.shape
    _, Hkv, P, _ = k_pages.shape
    bt = np.asarray(_as_f64(block_table)).astype(np.int64)
    cap = bt.shape[1] * P
    lens = np.asarray(_as_f64(kv_lens)).reshape(-1).astype(np.int64)
    o = np.zeros((B, Hq, D), dtype=np.float64)
    lse = np.full((B, Hq), -np.inf, dtype=np.float64)
    for b in range(B) if batches is None else batches:
        L = int(min(max(lens[b], 0), cap))
        if L == 0:
            continue
        j = np.arange(L)
        pages, rows = bt[b, j // P], j % P
        kk = np.stack([_as_f64(k_pages[pages, hk, rows]) for hk in range(Hkv)])[None]   # (1, Hkv, L, D)
        vv = np.stack([_as_f64(v_pages[pages, hk, rows]) for hk in range(Hkv)])[None]
        ob, lb = decode(_as_f64(q[b:b + 1]), kk, vv, [L], scale)
        o[b], lse[b] = ob[0], lb[0]
    return o, lse
