"""Tile order of prefill grids with per-sequence lengths.

With kv_lens and at most 64 sequences the prefill launches its workgroups
in list order: tiles by work (key tiles) descending, then the tiles with
no work at all (padding rows, rows that see no key), which only write
zeros.  The order changes which workgroup computes which tile, never how a
tile is computed, so:

* every (batch, head, query tile) must be written: outputs start as NaN
  and none may remain;
* values match the float64 oracle on sampled rows, padding rows are
  O = 0 and LSE = -inf;
* with every length equal to T the list order and the dense order give
  bit-identical results.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle
from exact_tiled_attention_13_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def gen(shape, seed, dtype=torch.bfloat16):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype).cuda()


def rows_to_check(B, H, Tq, lens, n, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        L = min(max(lens[b], 0), Tq)
        for i in {0, 127, 128, 255, 256, L - 1, L, Tq - 1}:
            if 0 <= i < Tq:
                rows.add((b, int(rng.integers(H)), i))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(Tq))))
    return sorted(rows)


def run(B, Hq, Hkv, Tq, Tk, D, causal, lens, seed, n_rows=400):
    q = gen((B, Hq, Tq, D), seed)
    k = gen((B, Hkv, Tk, D), seed + 1)
    v = gen((B, Hkv, Tk, D), seed + 2)
    workloads.poison_tail_(k, lens)
    workloads.poison_tail_(v, lens)
    if Tq == Tk:
        workloads.poison_tail_(q, lens)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = 1.0 / math.sqrt(D)
    o = torch.full((B, Hq, Tq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    ea.fwd(q, k, v, causal=causal, kv_lens=kv, scale=sc, out=o, lse=lse)
    torch.cuda.synchronize()
    what = f"B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tk{Tk} D{D} causal={causal}"
    print(f"  {what}", flush=True)
    assert not torch.isnan(o).any(), f"{what}: a tile of O was not written"
    assert not torch.isnan(lse).any(), f"{what}: a tile of LSE was not written"
    if Tq == Tk:
        for b, L in enumerate(lens):
            L = min(max(L, 0), Tk)
            assert torch.all(o[b, :, L:] == 0) and torch.all(torch.isneginf(lse[b, :, L:])), f"{what}: padding of {b}"
    rows = rows_to_check(B, Hq, Tq, lens, n_rows, seed)
    o_ref, l_ref = oracle.attention_rows(q.cpu(), k.cpu(), v.cpu(), rows, sc, causal, lens)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    og = o[idx].double().cpu().numpy()
    lg = lse[idx].double().cpu().numpy()
    assert np.array_equal(np.isneginf(lg), np.isneginf(l_ref)), f"{what}: -inf pattern"
    fin = np.isfinite(l_ref)
    err_o = float(np.abs(og - o_ref).max())
    err_l = float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    print(f"    max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= 2e-2 and err_l <= 1e-3, what


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_list_order_small_grid(D, causal):
    """13 sequences (not a multiple of 8), GQA, lengths from 0 to past T:
    128-row workgroups with two key groups."""
    lens = [0, 700, 1, 333, 905, 128, 129, 699, 64, 500, 2, 256, 257]
    run(13, 4, 2, 700, 700, D, causal, lens, seed=100 + D + causal)


@pytest.mark.parametrize("causal", [False, True])
def test_list_order_large_grid(causal):
    """16 sequences x 16 heads x 4 query tiles: 256-row workgroups, several
    rounds of the chip."""
    rng = np.random.default_rng(31)
    lens = [int(x) for x in rng.integers(1, 1025, 16)]
    lens[3] = 1024
    lens[7] = 0
    run(16, 16, 16, 1024, 1024, 128, causal, lens, seed=200 + causal)


@pytest.mark.parametrize("B", [64, 65])
def test_list_order_limit(B):
    """64 sequences is the most the list order takes (one per lane); 65 take
    the dense order.  Both must cover every tile."""
    rng = np.random.default_rng(B)
    lens = [int(x) for x in rng.integers(0, 513, B)]
    run(B, 2, 1, 512, 512, 128, True, lens, seed=300 + B, n_rows=300)


def test_rows_that_see_no_key():
    """Tq > Tk with lengths: under the bottom-right causal alignment the
    first Tq - Lk rows see no key; their tiles take the zero-writing path.
    Every row is checked against the oracle."""
    B, Hq, Hkv, Tq, Tk, D = 3, 4, 2, 700, 333, 128
    lens = [333, 50, 10]
    q = gen((B, Hq, Tq, D), 71)
    k = gen((B, Hkv, Tk, D), 72)
    v = gen((B, Hkv, Tk, D), 73)
    workloads.poison_tail_(k, lens)
    workloads.poison_tail_(v, lens)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = 1.0 / math.sqrt(D)
    o = torch.full((B, Hq, Tq, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, Hq, Tq), float("nan"), dtype=torch.float32, device="cuda")
    ea.fwd(q, k, v, causal=True, kv_lens=kv, scale=sc, out=o, lse=lse)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), sc, True, lens)
    og = o.double().cpu().numpy()
    lg = lse.double().cpu().numpy()
    assert not np.isnan(og).any() and not np.isnan(lg).any()
    assert np.array_equal(np.isneginf(lg), np.isneginf(l_ref))
    fin = np.isfinite(l_ref)
    assert float(np.abs(og - o_ref).max()) <= 2e-2
    assert float(np.abs(lg[fin] - l_ref[fin]).max()) <= 1e-3
    # rows before the first key they may see: exactly zero
    for b, L in enumerate(lens):
        assert torch.all(o[b, :, : Tq - L] == 0) and torch.all(torch.isneginf(lse[b, :, : Tq - L]))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_list_order_matches_dense_order_bitwise(D, causal):
    """All lengths equal to T: list order (kv_lens given) and the dense order
    (kv_lens NULL) compute the same tiles in the same way."""
    B, Hq, Hkv, T = 8, 8, 2, 1024
    q = gen((B, Hq, T, D), 400 + D)
    k = gen((B, Hkv, T, D), 401 + D)
    v = gen((B, Hkv, T, D), 402 + D)
    kv = torch.full((B,), T, dtype=torch.int32, device="cuda")
    o1, l1 = ea.fwd(q, k, v, causal=causal, kv_lens=kv)
    o2, l2 = ea.fwd(q, k, v, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_list_order_matches_dense_order_bitwise_fp8():
    B, Hq, Hkv, T, D = 4, 8, 8, 2048, 128
    g = torch.Generator().manual_seed(5)
    q = workloads.randn_e4m3((B, Hq, T, D), g).cuda()
    k = workloads.randn_e4m3((B, Hkv, T, D), g).cuda()
    v = workloads.randn_e4m3((B, Hkv, T, D), g).cuda()
    kv = torch.full((B,), T, dtype=torch.int32, device="cuda")
    s = workloads.E4M3_SCALE
    o1, l1 = ea.fwd_fp8(q, k, v, q_scale=s, k_scale=s, v_scale=s, causal=True, kv_lens=kv)
    o2, l2 = ea.fwd_fp8(q, k, v, q_scale=s, k_scale=s, v_scale=s, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
