"""Every launch choice the table can force gives a correct result (GPU,
through the C ABI, against the float64 oracle; same tolerances as the other
parity tests).  Zig-zag pairing only reorders workgroups, so it must not
change a single bit."""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle
from exact_tiled_attention_13_amd import _lib, tiles, workloads

pytestmark = pytest.mark.gpu
S0 = workloads.E4M3_SCALE


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()
    yield
    _lib.attn_set_tile_table([])
    tiles.apply_default()


def force(op, dtype, D, causal, v0, v1):
    _lib.attn_set_tile_table([[op, dtype, D, causal, 0, 2**31 - 1, 0, 2**31 - 1, v0, v1]])


def check(o, lse, o_ref, l_ref, what):
    a, l = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isfinite(a).all(), what
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref)), what
    fin = np.isfinite(l_ref)
    eo = float(np.abs(a - o_ref).max())
    el = float(np.abs(l[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: max|dO| {eo:.3e} max|dLSE| {el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-3, what


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_forced_prefill_shapes(dtype, D, causal):
    B, H, T = 2, 6, 700
    lens = [700, 333]
    g = torch.Generator().manual_seed(D + causal)
    if dtype == "e4m3":
        q, k, v, sc = workloads.make_fwd_inputs_fp8(B, H, H, T, T, D, seed=D + causal)
        o_ref, l_ref = oracle.attention_fp8(q, k, v, *sc, 1 / np.sqrt(D), causal=bool(causal), kv_lens=lens)
        call = lambda: ea.fwd_fp8(q.cuda(), k.cuda(), v.cuda(), q_scale=sc[0], k_scale=sc[1], v_scale=sc[2],  # noqa: E731
                                  causal=bool(causal), kv_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
        dt = _lib.MIATTN_E4M3
    else:
        q, k, v = (workloads.randn_bf16((B, H, T, D), g) for _ in range(3))
        o_ref, l_ref = oracle.attention(q, k, v, 1 / np.sqrt(D), causal=bool(causal), kv_lens=lens)
        call = lambda: ea.fwd(q.cuda(), k.cuda(), v.cuda(), causal=bool(causal),  # noqa: E731
                              kv_lens=torch.tensor(lens, dtype=torch.int32, device="cuda"))
        dt = _lib.MIATTN_BF16
    for shape in (0, 1):
        outs = []
        for zig in (0, 1):
            force(_lib.MIATTN_TILE_FWD, dt, D, causal, shape, zig)
            o, lse = call()
            torch.cuda.synchronize()
            check(o, lse, o_ref, l_ref, f"{dtype} D{D} causal{causal} shape{shape} zig{zig}")
            outs.append((o, lse))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


@pytest.mark.parametrize("dtype", ["bf16", "e4m3"])
@pytest.mark.parametrize("per_cu", [1, 2, 3, 4])
def test_forced_decode_workgroups(dtype, per_cu):
    B, Hq, Hkv, S, D = 9, 16, 4, 5000, 128
    lens = [1, 5000, 512, 513, 2048, 0, 4999, 77, 1024]
    if dtype == "e4m3":
        q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, lens, seed=per_cu, poison=True)
        o_ref, l_ref = oracle.decode_fp8(q, k, v, lens, *sc, 1 / np.sqrt(D))
        force(_lib.MIATTN_TILE_DECODE, _lib.MIATTN_E4M3, D, 1, per_cu, 0)
        o, lse = ea.decode_fp8(q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"),
                               q_scale=sc[0], k_scale=sc[1], v_scale=sc[2])
    else:
        q, k, v = workloads.make_decode_inputs(B, Hq, Hkv, S, D, lens, seed=per_cu, poison=True)
        o_ref, l_ref = oracle.decode(q, k, v, lens, 1 / np.sqrt(D))
        force(_lib.MIATTN_TILE_DECODE, _lib.MIATTN_BF16, D, 1, per_cu, 0)
        o, lse = ea.decode(q.cuda(), k.cuda(), v.cuda(), torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    check(o, lse, o_ref, l_ref, f"decode {dtype} {per_cu} workgroups per CU")
