"""GPU parity of the E4M3 (FP8) entry points (attn_fwd_fp8, attn_decode_fp8,
attn_decode_paged_fp8 through the C ABI) against the float64 oracle on the
same codes and scales.

Tolerance: O <= 2e-2 x (size of the V values, ~1 for the default scales),
LSE <= 1e-3.  The kernels' scores are exact products of the codes summed in
fp32 and V is widened to bf16 exactly, so the rounding left is the bf16 path's
(P and O rounded to bf16), hence the bf16 bound.  Rows past each length hold
the NaN code 0x7f and must never reach the result.
"""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle
from exact_tiled_attention_13_amd import workloads

pytestmark = pytest.mark.gpu

S0 = workloads.E4M3_SCALE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def check(o, lse, o_ref, l_ref, what, vmag=1.0):
    a, l = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isfinite(a).all(), what
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref)), what
    fin = np.isfinite(l_ref)
    eo = float(np.abs(a - o_ref).max())
    el = float(np.abs(l[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: max|dO| {eo:.3e} max|dLSE| {el:.3e}", flush=True)
    assert eo <= 2e-2 * vmag and el <= 1e-3, what


def run(B, Hq, Hkv, S, D, lens, scale=None, scales=(S0, S0, S0), seed=0):
    q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, lens, seed=seed, poison=True, scales=scales)
    scale = 1 / np.sqrt(D) if scale is None else scale
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.decode_fp8(q.cuda(), k.cuda(), v.cuda(), kv, q_scale=sc[0], k_scale=sc[1], v_scale=sc[2],
                           scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_fp8(q, k, v, lens, *sc, scale)
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (8, 8), (16, 1), (40, 2)])
def test_fp8_decode_shapes(D, Hq, Hkv):
    lens = [1, 511, 512, 513, 1500, 0, 2048]
    o, lse, o_ref, l_ref = run(len(lens), Hq, Hkv, 2048, D, lens, seed=D + Hq)
    check(o, lse, o_ref, l_ref, f"fp8 D{D} Hq{Hq} Hkv{Hkv}")


@pytest.mark.parametrize("scales", [(0.01, 0.02, 0.03), (0.02, -0.015, S0), (S0, S0, -2 * S0)])
def test_fp8_decode_scales(scales):
    lens = [777, 64, 3000]
    o, lse, o_ref, l_ref = run(3, 16, 4, 3072, 128, lens, scales=scales, seed=11)
    check(o, lse, o_ref, l_ref, f"fp8 scales {scales}", vmag=abs(scales[2]) / S0)


def test_fp8_decode_negative_softmax_scale():
    lens = [100, 1000]
    o, lse, o_ref, l_ref = run(2, 8, 2, 1024, 64, lens, scale=-0.2, seed=12)
    check(o, lse, o_ref, l_ref, "fp8 negative scale")


def test_fp8_decode_full_size_sampled():
    """The E4M3 decode workload at full size; the oracle checks a sample of sequences."""
    w = workloads.WORKLOADS["decode-fp8"]
    inp = workloads.make("decode-fp8", seed=0, poison=True)
    sc = inp["fp8_scales"]
    o, lse = ea.decode_fp8(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), inp["kv_lens"].cuda(),
                           q_scale=sc[0], k_scale=sc[1], v_scale=sc[2])
    torch.cuda.synchronize()
    batches = [0, 17, 40, 63]
    o_ref, l_ref = oracle.decode_fp8(inp["q"], inp["k"], inp["v"], inp["lens"], *sc, w.scale, batches=batches)
    check(o[batches], lse[batches], o_ref[batches], l_ref[batches], "fp8 full-size sample")
    assert torch.isfinite(o.float()).all()


def _paginate(k, v, lens, P, max_blocks, seed):
    """Scatter contiguous E4M3 caches into a shuffled pool (NaN codes elsewhere)."""
    B, Hkv, S, D = k.shape
    rng = np.random.default_rng(seed)
    need = [-(-L // P) for L in lens]
    num_pages = sum(need) + 5
    perm = rng.permutation(num_pages)
    kp = torch.full((num_pages, Hkv, P, D), 0x7F, dtype=torch.uint8)
    vp = torch.full_like(kp, 0x7F)
    bt = rng.integers(0, num_pages, (B, max_blocks)).astype(np.int32)
    used = 0
    k8, v8 = k.view(torch.uint8), v.view(torch.uint8)
    for b, L in enumerate(lens):
        for i in range(need[b]):
            pg = int(perm[used])
            used += 1
            bt[b, i] = pg
            n = min(P, L - i * P)
            kp[pg, :, :n] = k8[b, :, i * P:i * P + n]
            vp[pg, :, :n] = v8[b, :, i * P:i * P + n]
    return kp, vp, bt


@pytest.mark.parametrize("P", [8, 16, 128])
@pytest.mark.parametrize("D", [64, 128])
def test_fp8_paged_decode(P, D):
    B, Hq, Hkv, S = 4, 16, 4, 1536
    lens = [1, 1500, P, 700]
    q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, lens, seed=P + D, poison=True,
                                                   scales=(0.012, 0.02, S0))
    kp, vp, bt = _paginate(k, v, lens, P, S // P, seed=P)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.decode_paged_fp8(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(bt).cuda(), kv,
                                 q_scale=sc[0], k_scale=sc[1], v_scale=sc[2], scale=0.1)
    o_c, lse_c = ea.decode_fp8(q.cuda(), k.cuda(), v.cuda(), kv, q_scale=sc[0], k_scale=sc[1], v_scale=sc[2],
                               scale=0.1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_paged_fp8(q, kp, vp, bt, lens, *sc, 0.1)
    check(o, lse, o_ref, l_ref, f"fp8 paged P{P} D{D}")
    # same tiles in the same order as the contiguous call: bit-identical
    assert torch.equal(o, o_c) and torch.equal(lse, lse_c)


# ------------------------------------------------------------------ prefill
def run_fwd(B, Hq, Hkv, Tq, Tk, D, causal, lens=None, scale=None, scales=(S0, S0, S0), seed=0, poison=False,
            poison_q=False):
    q, k, v, sc = workloads.make_fwd_inputs_fp8(B, Hq, Hkv, Tq, Tk, D, seed=seed, scales=scales)
    if poison and lens is not None:
        workloads.poison_tail_(k.view(torch.uint8), lens, 0x7F)
        workloads.poison_tail_(v.view(torch.uint8), lens, 0x7F)
    if poison_q and lens is not None:
        workloads.poison_tail_(q.view(torch.uint8), lens, 0x7F)
    scale = 1 / np.sqrt(D) if scale is None else scale
    kv = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = ea.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), q_scale=sc[0], k_scale=sc[1], v_scale=sc[2], causal=causal,
                        kv_lens=kv, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fp8(q, k, v, *sc, scale, causal=causal, kv_lens=lens)
    return o, lse, o_ref, l_ref


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 63, 200, 513])
def test_fp8_prefill_small(D, causal, T):
    """Small grids: the launcher takes the 128-row workgroups with two key groups."""
    o, lse, o_ref, l_ref = run_fwd(2, 4, 2, T, T, D, causal, seed=T + D)
    check(o, lse, o_ref, l_ref, f"fp8 prefill T{T} D{D} causal{causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_prefill_large_grid(D, causal):
    """512+ workgroups of 256 rows: the one-key-group shape."""
    o, lse, o_ref, l_ref = run_fwd(4, 64, 16, 520, 520, D, causal, seed=7 + D)
    check(o, lse, o_ref, l_ref, f"fp8 prefill large grid D{D} causal{causal}")


@pytest.mark.parametrize("Tq,Tk", [(37, 300), (256, 1000), (1, 777)])
def test_fp8_prefill_chunked(Tq, Tk):
    """Tq < Tk: causal aligned bottom-right (a chunk of new queries against a longer cache)."""
    o, lse, o_ref, l_ref = run_fwd(2, 8, 2, Tq, Tk, 128, True, seed=Tq)
    check(o, lse, o_ref, l_ref, f"fp8 chunked Tq{Tq} Tk{Tk}")


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_prefill_padding(causal):
    lens = [1, 0, 300, 512, 77]
    o, lse, o_ref, l_ref = run_fwd(5, 4, 4, 512, 512, 64, causal, lens=lens, seed=3, poison=True)
    check(o, lse, o_ref, l_ref, f"fp8 padding causal{causal}")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_prefill_padding_query_rows_hold_nan(D, causal):
    """The E4M3 NaN code in every padding query row as well as the padding keys
    and values: those rows come out O = 0, LSE = -inf, valid rows unaffected."""
    lens = [300, 17, 256, 0, 511]
    o, lse, o_ref, l_ref = run_fwd(5, 4, 2, 512, 512, D, causal, lens=lens, seed=5 + D, poison=True, poison_q=True)
    check(o, lse, o_ref, l_ref, f"fp8 NaN query padding D{D} causal{causal}")


@pytest.mark.parametrize("scales", [(0.01, 0.02, 0.03), (0.02, -0.015, S0), (S0, S0, -2 * S0)])
def test_fp8_prefill_scales(scales):
    o, lse, o_ref, l_ref = run_fwd(2, 4, 2, 300, 300, 128, True, scales=scales, seed=9)
    check(o, lse, o_ref, l_ref, f"fp8 prefill scales {scales}", vmag=abs(scales[2]) / S0)


def test_fp8_prefill_full_size_causal():
    """The E4M3 causal workload at full size against the full oracle."""
    w = workloads.WORKLOADS["causal-fp8"]
    inp = workloads.make("causal-fp8", seed=0)
    sc = inp["fp8_scales"]
    o, lse = ea.fwd_fp8(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), q_scale=sc[0], k_scale=sc[1],
                        v_scale=sc[2], causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention_fp8(inp["q"], inp["k"], inp["v"], *sc, w.scale, causal=True)
    check(o, lse, o_ref, l_ref, "fp8 causal full size")


def test_fp8_prefill_long_two_heads_and_random_rows():
    """The E4M3 long-context workload (B1 H32 T32768 D128) at full size: all
    rows of heads 0 and 31 against the dense oracle, plus 4096 random rows
    of the other heads against the row oracle."""
    w = workloads.WORKLOADS["long-fp8"]
    inp = workloads.make("long-fp8", seed=0)
    sc = inp["fp8_scales"]
    o, lse = ea.fwd_fp8(inp["q"].cuda(), inp["k"].cuda(), inp["v"].cuda(), q_scale=sc[0], k_scale=sc[1],
                        v_scale=sc[2], causal=True)
    torch.cuda.synchronize()
    heads = (0, w.Hq - 1)
    for h in heads:
        sl = slice(h, h + 1)
        o_ref, l_ref = oracle.attention_fp8(inp["q"][:, sl], inp["k"][:, sl], inp["v"][:, sl], *sc, w.scale,
                                            causal=True)
        check(o[:, sl], lse[:, sl], o_ref, l_ref, f"fp8 long head {h}, all {w.Tq} rows")
    rng = np.random.default_rng(1)
    others = [h for h in range(w.Hq) if h not in heads]
    picked = set()
    while len(picked) < 4096:
        picked.add((int(rng.choice(others)), int(rng.integers(w.Tq))))
    rows = sorted((0, h, i) for h, i in picked)
    o_ref, l_ref = oracle.attention_rows_fp8(inp["q"], inp["k"], inp["v"], rows, *sc, w.scale, causal=True)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    check(o[idx], lse[idx], o_ref, l_ref, f"fp8 long, {len(rows)} random rows of other heads")


def test_fp8_prefill_matches_bf16_path_on_exact_values():
    """E4M3 values are exact in bf16: with unit scales the E4M3 prefill and the
    bf16 prefill see the same numbers; both stay within the bf16 bound of the
    oracle and of each other."""
    q, k, v, _ = workloads.make_fwd_inputs_fp8(2, 8, 4, 700, 700, 128, seed=21, scales=(1.0, 1.0, 1.0))
    # N(0,1) codes at unit scale: values up to ~4 with 3-bit mantissas
    o8, l8 = ea.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), q_scale=1.0, k_scale=1.0, v_scale=1.0, causal=True,
                        scale=0.05)
    ob, lb = ea.fwd(q.to(torch.bfloat16).cuda(), k.to(torch.bfloat16).cuda(), v.to(torch.bfloat16).cuda(),
                    causal=True, scale=0.05)
    torch.cuda.synchronize()
    assert float((o8.float() - ob.float()).abs().max()) <= 2e-2
    assert float((l8 - lb).abs().max()) <= 1e-3
