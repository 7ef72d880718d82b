"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances: O max-abs error <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs (the oracle gets the same bf16 values, upcast exactly); LSE within
1e-3 on finite entries; -inf entries must match by position; no NaN.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle
from exact_tiled_attention_13_amd import workloads

pytestmark = pytest.mark.gpu

TOL_O = {torch.float32: 1e-4, torch.bfloat16: 2e-2}
TOL_LSE = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def to_np(t):
    return t.detach().float().cpu().double().numpy()


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    o = to_np(o_gpu)
    l = to_np(lse_gpu)
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    assert not np.isnan(l).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(l), np.isneginf(lse_ref)), f"{what}: -inf pattern of LSE differs"
    assert np.isfinite(o).all(), f"{what}: non-finite O"
    fin = np.isfinite(lse_ref)
    err_o = float(np.abs(o - o_ref).max()) if o.size else 0.0
    err_l = float(np.abs(l[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: max|dO|={err_o:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O[dtype], f"{what}: O error {err_o}"
    assert err_l <= TOL_LSE, f"{what}: LSE error {err_l}"
    return err_o, err_l


def gen(shape, seed, dtype, device="cuda"):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype).to(device)


def run_case(B, Hq, Hkv, Tq, Tk, D, dtype, causal, lens=None, scale=None, seed=0, poison=False, poison_q=False):
    q = gen((B, Hq, Tq, D), seed, dtype)
    k = gen((B, Hkv, Tk, D), seed + 1, dtype)
    v = gen((B, Hkv, Tk, D), seed + 2, dtype)
    if poison and lens is not None:
        workloads.poison_tail_(k, lens)
        workloads.poison_tail_(v, lens)
    if poison_q and lens is not None:
        # with Tq == Tk the lengths cover the query rows too: the rest is padding
        workloads.poison_tail_(q, lens)
    kv = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    o, lse = ea.fwd(q, k, v, causal=causal, kv_lens=kv, scale=sc)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), sc, causal, lens)
    return check(o, lse, o_ref, l_ref, dtype, f"B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tk{Tk} D{D} {dtype} causal={causal}")


# ------------------------------------------------------------------ the five workloads
def test_single_head_fp32_workload():
    w = workloads.make("single", device="cuda")
    o, lse = ea.fwd(w["q"], w["k"], w["v"], causal=False, scale=w["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(w["q"].cpu(), w["k"].cpu(), w["v"].cpu(), w["scale"])
    check(o, lse, o_ref, l_ref, torch.float32, "single fp32 256x512x64")


def test_causal_prefill_workload_full():
    w = workloads.make("causal", device="cpu")
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    o, lse = ea.fwd(q, k, v, causal=True, scale=w["scale"])
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(w["q"], w["k"], w["v"], w["scale"], True)
    check(o, lse, o_ref, l_ref, torch.bfloat16, "causal B4 H16 T1024 D64")


def sample_rows(B, H, T, lens_q, n, seed):
    """Rows to check at full size: first/last valid rows, tile edges, random ones."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        lq = lens_q[b]
        for i in {0, 1, 63, 64, 127, 128, 129, lq - 1, lq, min(lq + 5, T - 1), T - 1}:
            if 0 <= i < T:
                rows.add((b, int(rng.integers(H)), i))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(H)), int(rng.integers(T))))
    return sorted(rows)


def test_ragged_workload_sampled():
    w = workloads.make("ragged", device="cpu", poison=True)
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    lens = w["lens"]
    assert lens[0] == 1
    o, lse = ea.fwd(q, k, v, causal=False, kv_lens=w["kv_lens"].cuda(), scale=w["scale"])
    torch.cuda.synchronize()
    W = w["workload"]
    rows = sample_rows(W.B, W.Hq, W.Tq, lens, 400, 1)
    o_ref, l_ref = oracle.attention_rows(w["q"], w["k"], w["v"], rows, w["scale"], False, lens)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(o[idx], lse[idx], o_ref, l_ref, torch.bfloat16, "ragged B8 H16 T4096 D128 (sampled)")
    # every padded row of every head is exactly zero with LSE -inf
    for b, L in enumerate(lens):
        assert torch.all(o[b, :, L:] == 0) and torch.all(torch.isneginf(lse[b, :, L:]))
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def test_decode_workload_sampled():
    W = workloads.WORKLOADS["decode"]
    w = workloads.make("decode", device="cuda", poison=True)
    lens = w["lens"]
    o, lse = ea.decode(w["q"], w["k"], w["v"], w["kv_lens"], scale=w["scale"])
    torch.cuda.synchronize()
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 0, 17, W.B - 1})
    o_ref, l_ref = oracle.decode(w["q"].cpu(), w["k"], w["v"], lens, w["scale"], batches=pick)
    check(o[pick], lse[pick], o_ref[pick], l_ref[pick], torch.bfloat16, f"decode B64 Hq32 Hkv8 D128 batches {pick}")
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def long_rows(W, heads, n_random, seed):
    """Every row of `heads` plus n_random distinct (h, i) rows of the other
    heads (the long workload's check: error grows with T, so whole heads
    are compared, first and last row included)."""
    rng = np.random.default_rng(seed)
    others = [h for h in range(W.Hq) if h not in heads]
    picked = set()
    while len(picked) < n_random:
        picked.add((int(rng.choice(others)), int(rng.integers(W.Tq))))
    return sorted((0, h, i) for h, i in picked)


def test_long_causal_workload_two_heads_and_random_rows():
    """The long-context causal workload (B1 H32 T32768 D128) at full size:
    all 32768 rows of heads 0 and 31 against the dense oracle, plus 4096
    random rows of the other heads against the row oracle."""
    W = workloads.WORKLOADS["long"]
    w = workloads.make("long", device="cpu")
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    o, lse = ea.fwd(q, k, v, causal=True, scale=w["scale"])
    torch.cuda.synchronize()
    heads = (0, W.Hq - 1)
    errs = []
    for h in heads:
        sl = slice(h, h + 1)
        o_ref, l_ref = oracle.attention(w["q"][:, sl], w["k"][:, sl], w["v"][:, sl], w["scale"], True)
        errs.append(check(o[:, sl], lse[:, sl], o_ref, l_ref, torch.bfloat16, f"long head {h}, all {W.Tq} rows"))
    rows = long_rows(W, heads, 4096, 5)
    o_ref, l_ref = oracle.attention_rows(w["q"], w["k"], w["v"], rows, w["scale"], True)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    errs.append(check(o[idx], lse[idx], o_ref, l_ref, torch.bfloat16, f"long, {len(rows)} random rows of other heads"))
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    print(f"  long workload max|dO| {max(e[0] for e in errs):.3e} max|dLSE| {max(e[1] for e in errs):.3e}")


# ------------------------------------------------------------------ long sequences
def test_prefill_131072_keys_sampled():
    """Four times the long workload's length (B1 H2 T131072 D128 causal,
    1024 query tiles per head), and a chunk of 4096 new queries at the end
    of 131072 keys with lengths: rows at tile edges, the first and last rows
    and random rows against the row oracle.  Offsets of a head slab reach
    2^25 elements here."""
    B, H, T, D = 1, 2, 131072, 128
    q = gen((B, H, T, D), 61, torch.bfloat16)
    k = gen((B, H, T, D), 62, torch.bfloat16)
    v = gen((B, H, T, D), 63, torch.bfloat16)
    sc = 1.0 / math.sqrt(D)
    o, lse = ea.fwd(q, k, v, causal=True, scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(8)
    rows = sorted({(0, h, i) for h in range(H) for i in (0, 1, 255, 256, 65535, 65536, T - 257, T - 256, T - 1)} |
                  {(0, int(rng.integers(H)), int(rng.integers(T))) for _ in range(240)})
    o_ref, l_ref = oracle.attention_rows(q.cpu(), k.cpu(), v.cpu(), rows, sc, True)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(o[idx], lse[idx], o_ref, l_ref, torch.bfloat16, f"prefill T{T}, {len(rows)} rows")
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()
    # chunked: 4096 new queries after the first Lk - 4096 of Lk keys
    Tq, lens = 4096, [T - 1000]
    qc = gen((B, H, Tq, D), 64, torch.bfloat16)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    workloads.poison_tail_(k, lens)
    workloads.poison_tail_(v, lens)
    oc, lc = ea.fwd(qc, k, v, causal=True, kv_lens=kv, scale=sc)
    torch.cuda.synchronize()
    rows = sorted({(0, h, i) for h in range(H) for i in (0, 255, 256, Tq - 1)} |
                  {(0, int(rng.integers(H)), int(rng.integers(Tq))) for _ in range(120)})
    o_ref, l_ref = oracle.attention_rows(qc.cpu(), k.cpu(), v.cpu(), rows, sc, True, lens)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(oc[idx], lc[idx], o_ref, l_ref, torch.bfloat16, f"chunked prefill Tq{Tq} Lk{lens[0]}, {len(rows)} rows")


def test_decode_million_key_cache():
    """One decode step over caches of 2^20 keys (B2 Hq8 Hkv1 D128, 2048
    splits per sequence), one sequence full and one ragged, NaN past the
    lengths, against the decode oracle."""
    B, Hq, Hkv, S, D = 2, 8, 1, 1 << 20, 128
    lens = [S, S - 333]
    q = gen((B, Hq, D), 71, torch.bfloat16)
    kc = gen((B, Hkv, S, D), 72, torch.bfloat16)
    vc = gen((B, Hkv, S, D), 73, torch.bfloat16)
    workloads.poison_tail_(kc, lens)
    workloads.poison_tail_(vc, lens)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.decode(q, kc, vc, kv, scale=0.09)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens, 0.09)
    check(o, lse, o_ref, l_ref, torch.bfloat16, f"decode S_max {S}")


# ------------------------------------------------------------------ edge cases
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 7, 65, 300])
def test_small_shapes(dtype, D, causal, T):
    run_case(2, 4, 2, T, T, D, dtype, causal, seed=T)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Tq,Tk", [(1, 1000), (17, 300), (130, 129), (300, 17), (64, 64), (257, 513)])
def test_bottom_right_causal(dtype, Tq, Tk):
    run_case(1, 2, 1, Tq, Tk, 64, dtype, True, seed=Tq + Tk)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_with_poison(dtype, causal):
    lens = [1, 0, 700, 129, 64, 65]
    run_case(6, 4, 2, 700, 700, 128, dtype, causal, lens=lens, seed=3, poison=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_padding_query_rows_hold_nan(D, dtype, causal):
    """Padding query rows (Tq == Tk, rows >= kv_lens[b]) filled with NaN, as
    are the padding keys and values: those rows come out O = 0, LSE = -inf,
    and the NaN reaches no valid row; lengths that end inside a wave's rows."""
    lens = [300, 17, 256, 0, 511]
    run_case(5, 4, 2, 512, 512, D, dtype, causal, lens=lens, seed=21 + D, poison=True, poison_q=True)


@pytest.mark.parametrize("causal", [False, True])
def test_kv_lens_with_unequal_lengths(causal):
    # Tq != Tk with lengths: every query row is valid, off = Lk - Tq
    run_case(3, 2, 2, 40, 333, 64, torch.bfloat16, causal, lens=[333, 50, 10], seed=4, poison=True)


@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_groups(G):
    run_case(2, 8, 8 // G, 200, 200, 128, torch.bfloat16, True, seed=10 + G)


@pytest.mark.parametrize("D,causal", [(64, False), (128, True)])
def test_unit_order_covers_every_tile(D, causal):
    """A grid of several rounds (1024 workgroups of 256 rows) whose (batch,
    KV head) unit count is a multiple of 8 takes the per-XCD unit order;
    one row of every (batch, query head, query tile), GQA with 4 query heads
    per KV head, against the row oracle."""
    B, Hq, Hkv, T = 2, 32, 8, 4096
    q = gen((B, Hq, T, D), 41, torch.bfloat16)
    k = gen((B, Hkv, T, D), 42, torch.bfloat16)
    v = gen((B, Hkv, T, D), 43, torch.bfloat16)
    sc = 1.0 / math.sqrt(D)
    o, lse = ea.fwd(q, k, v, causal=causal, scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    rows = [(b, h, t * 256 + int(rng.integers(256))) for b in range(B) for h in range(Hq) for t in range(T // 256)]
    o_ref, l_ref = oracle.attention_rows(q.cpu(), k.cpu(), v.cpu(), rows, sc, causal)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(o[idx], lse[idx], o_ref, l_ref, torch.bfloat16, f"unit order B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,Hq,Hkv", [(1, 8, 2), (2, 32, 8)])
def test_both_workgroup_shapes(D, causal, B, Hq, Hkv):
    """The launcher takes 256-row workgroups with one key group once there
    are at least 512 of them (B=2, Hq=32, T=2048: 512) and 128-row
    workgroups with two key groups below that (B=1, Hq=8: 64); both with
    ragged lengths and GQA, rows sampled at the larger size."""
    T = 2048
    lens = [T, 1337, 700][:B] if B > 1 else [1999]
    q = gen((B, Hq, T, D), 21, torch.bfloat16)
    k = gen((B, Hkv, T, D), 22, torch.bfloat16)
    v = gen((B, Hkv, T, D), 23, torch.bfloat16)
    workloads.poison_tail_(k, lens)
    workloads.poison_tail_(v, lens)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    sc = 1.0 / math.sqrt(D)
    o, lse = ea.fwd(q, k, v, causal=causal, kv_lens=kv, scale=sc)
    torch.cuda.synchronize()
    rows = sample_rows(B, Hq, T, lens, 300, 9)
    o_ref, l_ref = oracle.attention_rows(q.cpu(), k.cpu(), v.cpu(), rows, sc, causal, lens)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(o[idx], lse[idx], o_ref, l_ref, torch.bfloat16, f"B{B} Hq{Hq} Hkv{Hkv} T{T} D{D} causal={causal} lens={lens}")
    for b, L in enumerate(lens):
        assert torch.all(o[b, :, L:] == 0) and torch.all(torch.isneginf(lse[b, :, L:]))


@pytest.mark.parametrize("scale", [-0.3, 0.0, 2.0])
def test_unusual_scales(scale):
    run_case(1, 2, 2, 100, 100, 64, torch.bfloat16, True, scale=scale, seed=7)


def test_large_magnitude_scores_no_overflow():
    # scores up to ~1e3: exp overflows without the running max
    q = (gen((1, 2, 130, 64), 1, torch.float32) * 8).to(torch.bfloat16).cuda()
    k = (gen((1, 2, 130, 64), 2, torch.float32) * 8).to(torch.bfloat16).cuda()
    v = gen((1, 2, 130, 64), 3, torch.bfloat16)
    o, lse = ea.fwd(q, k, v, causal=True, scale=1.0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), 1.0, True)
    check(o, lse, o_ref, l_ref, torch.bfloat16, "large scores")


# ------------------------------------------------------------------ decode
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (32, 8), (32, 1), (6, 3)])
def test_decode_small(dtype, D, Hq, Hkv):
    B, S = 5, 1100
    lens = [1, 0, 1100, 256, 513]
    q = gen((B, Hq, D), 1, dtype)
    kc = gen((B, Hkv, S, D), 2, dtype)
    vc = gen((B, Hkv, S, D), 3, dtype)
    workloads.poison_tail_(kc, lens)
    workloads.poison_tail_(vc, lens)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.decode(q, kc, vc, kv, scale=0.1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode(q.cpu(), kc.cpu(), vc.cpu(), lens, 0.1)
    check(o, lse, o_ref, l_ref, dtype, f"decode Hq{Hq} Hkv{Hkv} D{D} {dtype}")


def test_incremental_decode_equals_full_forward():
    """Decode every position of a sequence through the cache and compare with
    the causal prefill rows (both on the GPU) and with the oracle."""
    B, Hq, Hkv, T, D = 2, 8, 2, 300, 128
    q = gen((B, Hq, T, D), 11, torch.bfloat16)
    k = gen((B, Hkv, T, D), 12, torch.bfloat16)
    v = gen((B, Hkv, T, D), 13, torch.bfloat16)
    o_full, l_full = ea.fwd(q, k, v, causal=True)
    S_max = 320
    kc = torch.full((B, Hkv, S_max, D), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, float("nan"))
    o_steps, l_steps = [], []
    for t in range(T):
        kc[:, :, t] = k[:, :, t]
        vc[:, :, t] = v[:, :, t]
        lens = torch.full((B,), t + 1, dtype=torch.int32, device="cuda")
        o_t, l_t = ea.decode(q[:, :, t].contiguous(), kc, vc, lens)
        o_steps.append(o_t)
        l_steps.append(l_t)
    torch.cuda.synchronize()
    o_inc = torch.stack(o_steps, dim=2)
    l_inc = torch.stack(l_steps, dim=2)
    # same computation, different tiling: equal within bf16 output rounding
    assert (o_inc.float() - o_full.float()).abs().max().item() <= 2e-2
    assert (l_inc - l_full).abs().max().item() <= 1e-3
    o_ref, l_ref = oracle.attention(q.cpu(), k.cpu(), v.cpu(), 1 / math.sqrt(D), True)
    check(o_inc, l_inc, o_ref, l_ref, torch.bfloat16, "incremental decode")


# ------------------------------------------------------------------ hygiene
def test_deterministic():
    q = gen((2, 4, 500, 128), 1, torch.bfloat16)
    k = gen((2, 2, 500, 128), 2, torch.bfloat16)
    v = gen((2, 2, 500, 128), 3, torch.bfloat16)
    a = ea.fwd(q, k, v, causal=True)
    b = ea.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_no_writes_outside_outputs():
    B, H, T, D = 2, 2, 77, 64
    q = gen((B, H, T, D), 1, torch.bfloat16)
    k = gen((B, H, T, D), 2, torch.bfloat16)
    v = gen((B, H, T, D), 3, torch.bfloat16)
    n, nl = B * H * T * D, B * H * T
    pad = 4096
    obuf = torch.full((n + 2 * pad,), 7.0, dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((nl + 2 * pad,), 7.0, dtype=torch.float32, device="cuda")
    o = obuf[pad:pad + n].view(B, H, T, D)
    lse = lbuf[pad:pad + nl].view(B, H, T)
    ea.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    assert torch.all(obuf[:pad] == 7) and torch.all(obuf[pad + n:] == 7)
    assert torch.all(lbuf[:pad] == 7) and torch.all(lbuf[pad + nl:] == 7)


def test_null_lse_is_allowed():
    q = gen((1, 2, 50, 64), 1, torch.bfloat16)
    o, _ = ea.fwd(q, q, q)
    o2 = torch.empty_like(q)
    ea.attn_fwd(q.data_ptr(), q.data_ptr(), q.data_ptr(), o2.data_ptr(), 0, 1, 2, 2, 50, 50, 64, 0.125, 0, 0,
                ea.MIATTN_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
