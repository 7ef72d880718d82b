"""Plain float64 gradients of attention.  TEST INFRASTRUCTURE ONLY.

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module; the HIP product path never does.

What is computed (sources, by page title and section):

* The NumPy tiled-attention build guide, *Extending It*: the kernel extended
  to produce dL/dQ, dL/dK and dL/dV by the chain rule through the softmax.
* The self-attention interview question ("Self-Attention: Implementation,
  Complexity ..."), Task 2 and Hint 2: the backward pass recomputes the
  attention weights from the inputs instead of storing the N x N matrix;
  only the forward's per-row statistics are kept.
* The forward it differentiates is ``oracle.attention``: O = softmax(scale *
  Q K^T + mask) V with causal (bottom-right), key-padding and grouped-query
  semantics, rows with no allowed key giving O = 0.

For one query head and its KV head, with P the softmax weights (zero on
masked keys and on rows without keys) and dO the upstream gradient:

    dV   = P^T dO                      (summed over the heads of a KV group)
    dP   = dO V^T
    Drow = sum_j P_ij dP_ij            (= sum_d dO_id O_id)
    dS   = P * (dP - Drow)             (softmax Jacobian, row by row)
    dQ   = scale * dS K
    dK   = scale * dS^T Q              (summed over the heads of a KV group)

These are the derivatives of the scalar L = sum(dO * O); every line is the
chain rule through the definition above, evaluated in float64.
"""

from __future__ import annotations

import numpy as np

from .attention import _as_f64, valid_lengths


def _weights(q_rows, k_all, scale, row_idx, lk, off, causal):
    """Softmax weights P (n, lk) of a block of rows; zero where masked and
    on rows without any allowed key."""
    n = q_rows.shape[0]
    if lk <= 0 or n == 0:
        return np.zeros((n, max(lk, 0)), dtype=np.float64)
    s = scale * (q_rows @ k_all[:lk].T)
    j = np.arange(lk)[None, :]
    allowed = np.ones((n, lk), dtype=bool)
    if causal:
        allowed &= j <= (row_idx[:, None] + off)
    s = np.where(allowed, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    has = np.isfinite(m[:, 0])
    m = np.where(np.isfinite(m), m, 0.0)
    e = np.where(allowed, np.exp(s - m), 0.0)
    l = e.sum(axis=1, keepdims=True)
    p = np.where(has[:, None], e / np.where(l > 0, l, 1.0), 0.0)
    return p


def attention_backward(q, k, v, do, scale, causal=False, kv_lens=None, row_chunk=256):
    """dQ, dK, dV (float64 numpy arrays) of L = sum(dO * attention(q, k, v)).

    q, do: (B, Hq, Tq, D); k, v: (B, Hkv, Tk, D).  Padding query rows (and
    rows without keys) have zero weights, so they contribute nothing and get
    dQ = 0; keys past a sequence's length get dK = dV = 0.
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    do = _as_f64(do)
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        lk, lq = lk_all[b], lq_all[b]
        off = lk - lq
        if lk <= 0:
            continue
        for h in range(Hq):
            hk = h // G
            kk, vv = k[b, hk, :lk], v[b, hk, :lk]
            for r0 in range(0, lq, row_chunk):
                rows = np.arange(r0, min(lq, r0 + row_chunk))
                p = _weights(q[b, h, rows], kk, scale, rows, lk, off, causal)   # (n, lk)
                g = do[b, h, rows]                                              # (n, D)
                dv[b, hk, :lk] += p.T @ g
                dp = g @ vv.T
                drow = (p * dp).sum(axis=1, keepdims=True)
                ds = p * (dp - drow)
                dq[b, h, rows] = scale * (ds @ kk)
                dk[b, hk, :lk] += scale * (ds.T @ q[b, h, rows])
    return dq, dk, dv


def backward_rows(q, k, v, do, rows, scale, causal=False, kv_lens=None, row_chunk=256):
    """dQ of selected (b, h, i) rows only (float64, shape (len(rows), D)).

    A row's dQ needs only that row's softmax, so this reaches sizes where the
    full backward is too slow on the CPU.  Rows of one (b, h) are evaluated
    together, ``row_chunk`` at a time, each against every key it sees."""
    rows = [tuple(int(x) for x in r) for r in rows]
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    out = np.zeros((len(rows), D), dtype=np.float64)
    groups = {}
    for n, (b, h, i) in enumerate(rows):
        if i < lq_all[b] and lk_all[b] > 0:
            groups.setdefault((b, h), []).append((i, n))
    for (b, h), members in sorted(groups.items()):
        lk, lq = lk_all[b], lq_all[b]
        hk = h // G
        kk = _as_f64(k[b, hk, :lk])
        vv = _as_f64(v[b, hk, :lk])
        members.sort()
        for c0 in range(0, len(members), row_chunk):
            part = members[c0:c0 + row_chunk]
            idx = np.array([i for i, _ in part], dtype=np.int64)
            qi = np.stack([_as_f64(q[b, h, i]) for i in idx.tolist()])
            g = np.stack([_as_f64(do[b, h, i]) for i in idx.tolist()])
            p = _weights(qi, kk, scale, idx, lk, lk - lq, causal)
            dp = g @ vv.T
            ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
            dq = scale * (ds @ kk)
            for r, (_, n) in enumerate(part):
                out[n] = dq[r]
    return out


def backward_key_rows(q, k, v, do, o, lse, keys, scale, causal=False, kv_lens=None):
    """dK and dV of selected keys (b, hk, j) only (float64, each (len(keys), D)).

    The Interview question's Task 2 / Hint 2 recomputes the weights from the
    inputs and the forward's saved per-row statistics; this does the same
    for a set of keys: with the forward's output o and natural-log row
    statistic lse given, P_ij = exp(scale q_i . k_j - lse_i) and
    Drow_i = sum_d dO_id O_id for every query row i of the KV head's query
    heads that sees key j, then

        dV_j = sum_i P_ij dO_i,   dK_j = scale sum_i P_ij (dO_i . v_j - Drow_i) q_i,

    summed over the query heads sharing the KV head.  Rows that are padding
    or have lse = -inf contribute nothing; keys at or past a sequence's
    length get zeros.  A key's gradient needs only the rows that see it, so
    this reaches sizes where ``attention_backward`` is too slow.
    """
    keys = [tuple(int(x) for x in r) for r in keys]
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    lk_all, lq_all = valid_lengths(B, Tq, Tk, kv_lens)
    dk = np.zeros((len(keys), D), dtype=np.float64)
    dv = np.zeros((len(keys), D), dtype=np.float64)
    groups = {}
    for n, (b, hk, j) in enumerate(keys):
        if j < lk_all[b]:
            groups.setdefault((b, hk), []).append((j, n))
    for (b, hk), members in sorted(groups.items()):
        lk, lq = lk_all[b], lq_all[b]
        off = lk - lq
        js = np.array([j for j, _ in members], dtype=np.int64)
        kj = _as_f64(k[b, hk])[js]                     # (m, D)
        vj = _as_f64(v[b, hk])[js]
        gk = np.zeros_like(kj)
        gv = np.zeros_like(vj)
        i = np.arange(lq)
        for h in range(hk * G, (hk + 1) * G):
            qh = _as_f64(q[b, h, :lq])                 # (lq, D)
            gh = _as_f64(do[b, h, :lq])
            oh = _as_f64(o[b, h, :lq])
            lh = _as_f64(lse[b, h, :lq]).reshape(-1)
            seen = np.isfinite(lh)[:, None] & np.ones((lq, len(js)), dtype=bool)
            if causal:
                seen &= js[None, :] <= (i[:, None] + off)
            s = scale * (qh @ kj.T)                    # (lq, m)
            p = np.where(seen, np.exp(np.where(seen, s - np.where(np.isfinite(lh), lh, 0.0)[:, None], 0.0)), 0.0)
            drow = (gh * oh).sum(axis=1, keepdims=True)
            dp = gh @ vj.T
            ds = p * (dp - drow)
            gv += p.T @ gh
            gk += scale * (ds.T @ qh)
        for r, (_, n) in enumerate(members):
            dk[n] = gk[r]
            dv[n] = gv[r]
    return dk, dv
