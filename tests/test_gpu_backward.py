"""GPU parity of the attention gradients (attn_bwd through the C ABI) against
the float64 backward oracle.

Inputs of the GPU call are independent of the HIP path: q, k, v, dO are
seeded bf16 draws, and O and LSE come from the float64 forward oracle
(rounded to bf16 and fp32 as attn_fwd would store them).

Tolerance: every gradient tensor must satisfy max|g - g_ref| <= 2e-2 *
max|g_ref|.  The kernels round P and dS to bf16 (relative 2^-9) before the
matrix products and the outputs to bf16; 2% of the tensor's scale is the
forward's bf16 bar (2e-2 on outputs of unit scale) applied to the gradient's
own scale.  No NaN anywhere, padded rows/keys exactly zero.
"""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle
from exact_tiled_attention_13_amd import workloads

pytestmark = pytest.mark.gpu
TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def gen(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def run(B, Hq, Hkv, Tq, Tk, D, causal, lens=None, scale=None, seed=0, poison=False):
    q, k, v, do = gen((B, Hq, Tq, D), seed), gen((B, Hkv, Tk, D), seed + 1), gen((B, Hkv, Tk, D), seed + 2), \
        gen((B, Hq, Tq, D), seed + 3)
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    o_ref, lse_ref = oracle.attention(q, k, v, sc, causal, lens)
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).to(torch.float32)
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(q, k, v, do, sc, causal, lens)
    if poison and lens is not None:
        lk, lq = oracle.valid_lengths(B, Tq, Tk, lens)
        for b in range(B):
            k[b, :, lk[b]:] = float("nan")
            v[b, :, lk[b]:] = float("nan")
            q[b, :, lq[b]:] = float("nan")
            do[b, :, lq[b]:] = float("nan")
            o[b, :, lq[b]:] = float("nan")
    dev = [x.cuda() for x in (q, k, v, o, lse, do)]
    kv = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    dq, dk, dv = ea.bwd(*dev, causal=causal, kv_lens=kv, scale=sc)
    torch.cuda.synchronize()
    what = f"B{B} Hq{Hq} Hkv{Hkv} Tq{Tq} Tk{Tk} D{D} causal={causal} lens={lens}"
    for name, g, ref in (("dq", dq, dq_ref), ("dk", dk, dk_ref), ("dv", dv, dv_ref)):
        a = g.float().cpu().double().numpy()
        assert np.isfinite(a).all(), f"{what}: non-finite {name}"
        scale_ref = float(np.abs(ref).max()) if ref.size else 0.0
        err = float(np.abs(a - ref).max()) if ref.size else 0.0
        print(f"  {what}: {name} max err {err:.3e} (ref max {scale_ref:.3e})", flush=True)
        assert err <= TOL * scale_ref + 1e-6, f"{what}: {name} err {err} vs scale {scale_ref}"
    if lens is not None:
        lk, lq = oracle.valid_lengths(B, Tq, Tk, lens)
        for b in range(B):
            assert torch.all(dq[b, :, lq[b]:] == 0)
            assert torch.all(dk[b, :, lk[b]:] == 0) and torch.all(dv[b, :, lk[b]:] == 0)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("T", [1, 33, 130, 300])
def test_small_shapes(D, causal, T):
    run(2, 4, 2, T, T, D, causal, seed=T)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Tq,Tk", [(1, 200), (17, 300), (130, 129), (300, 17), (257, 513)])
def test_bottom_right_causal(Tq, Tk, D):
    run(1, 2, 1, Tq, Tk, D, True, seed=Tq + Tk)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_with_poison(D, causal):
    run(5, 4, 2, 300, 300, D, causal, lens=[1, 0, 300, 129, 64], seed=3, poison=True)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_gqa_groups(G, D):
    run(2, 8, 8 // G, 200, 200, D, True, seed=10 + G)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("scale", [-0.3, 0.0, 1.5])
def test_unusual_scales(scale, D):
    run(1, 2, 2, 100, 100, D, True, scale=scale, seed=7)


def elementwise(what, got, ref):
    """The per-tensor bar: max|g - g_ref| <= 2e-2 * max|g_ref|, element by element."""
    a = got.float().cpu().double().numpy() if isinstance(got, torch.Tensor) else got
    assert np.isfinite(a).all(), f"{what}: non-finite"
    err = float(np.abs(a - ref).max())
    scale_ref = float(np.abs(ref).max())
    print(f"  {what}: max err {err:.3e} (ref max {scale_ref:.3e})", flush=True)
    assert err <= TOL * scale_ref + 1e-6, f"{what}: err {err} vs scale {scale_ref}"


def test_causal_workload_full():
    """The causal prefill workload (B4 H16 T1024 D64) at full size: every
    element of dQ, dK and dV against the full float64 backward."""
    w = workloads.make("causal", device="cpu")
    q, k, v, sc = w["q"], w["k"], w["v"], w["scale"]
    do = gen(q.shape, 99)
    o_ref, lse_ref = oracle.attention(q, k, v, sc, True)
    dev = [x.cuda() for x in (q, k, v, torch.from_numpy(o_ref).to(torch.bfloat16),
                             torch.from_numpy(lse_ref).to(torch.float32), do)]
    dq, dk, dv = ea.bwd(*dev, causal=True, scale=sc)
    torch.cuda.synchronize()
    dq_ref, dk_ref, dv_ref = oracle.attention_backward(q, k, v, do, sc, True)
    elementwise("causal workload dq", dq, dq_ref)
    elementwise("causal workload dk", dk, dk_ref)
    elementwise("causal workload dv", dv, dv_ref)


def sampled_gradients(q, k, v, do, o_ref, lse_ref, dq, dk, dv, sc, causal, rows, keys, what):
    """dQ of the sampled rows and dK, dV of the sampled keys, elementwise
    against the row and key oracles (fed with the forward oracle's o, lse)."""
    ref = oracle.backward_rows(q, k, v, do, rows, sc, causal)
    idx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(rows).T)
    elementwise(f"{what} dq ({len(rows)} rows)", dq[idx], ref)
    gk, gv = oracle.backward_key_rows(q, k, v, do, o_ref, lse_ref, keys, sc, causal)
    kidx = tuple(torch.as_tensor(a, device="cuda") for a in np.array(keys).T)
    elementwise(f"{what} dk ({len(keys)} keys)", dk[kidx], gk)
    elementwise(f"{what} dv ({len(keys)} keys)", dv[kidx], gv)


def test_unit_order_grids_rows_and_keys_sampled():
    """dQ and dK/dV grids of several rounds (2048 and 1024 workgroups) with a
    multiple of 8 (batch, KV head) units take the per-XCD unit order.  One
    dQ row of every (batch, query head, 128-row query tile) against the row
    oracle; one key of every (batch, KV head, 128-key tile) against the key
    oracle, elementwise."""
    B, Hq, Hkv, T, D = 8, 32, 16, 1024, 64
    q, k, v, do = gen((B, Hq, T, D), 51), gen((B, Hkv, T, D), 52), gen((B, Hkv, T, D), 53), gen((B, Hq, T, D), 54)
    sc = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attention(q, k, v, sc, True)
    dev = [x.cuda() for x in (q, k, v, torch.from_numpy(o_ref).to(torch.bfloat16),
                             torch.from_numpy(lse_ref).to(torch.float32), do)]
    dq, dk, dv = ea.bwd(*dev, causal=True, scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(6)
    rows = [(b, h, t * 128 + int(rng.integers(128))) for b in range(B) for h in range(Hq) for t in range(T // 128)]
    keys = [(b, h, t * 128 + int(rng.integers(128))) for b in range(B) for h in range(Hkv) for t in range(T // 128)]
    sampled_gradients(q, k, v, do, o_ref, lse_ref, dq, dk, dv, sc, True, rows, keys, "unit order")


def test_long_causal_gradients_rows_and_keys_sampled():
    """Gradients at a long causal shape (B1 H32 T8192 D128; both gradient
    grids take the per-XCD unit order): dQ of two rows per (head, 512-row
    span) and dK/dV of two keys per (head, 512-key span), elementwise, tile
    edges included."""
    B, H, T, D = 1, 32, 8192, 128
    q, k, v, do = gen((B, H, T, D), 61), gen((B, H, T, D), 62), gen((B, H, T, D), 63), gen((B, H, T, D), 64)
    sc = 1.0 / math.sqrt(D)
    o_ref, lse_ref = oracle.attention(q, k, v, sc, True)
    dev = [x.cuda() for x in (q, k, v, torch.from_numpy(o_ref).to(torch.bfloat16),
                             torch.from_numpy(lse_ref).to(torch.float32), do)]
    dq, dk, dv = ea.bwd(*dev, causal=True, scale=sc)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    rows = sorted({(0, h, s * 512 + int(rng.integers(512))) for h in range(H) for s in range(T // 512)} |
                  {(0, h, i) for h in (0, H - 1) for i in (0, 127, 128, T - 1)})
    keys = sorted({(0, h, s * 512 + int(rng.integers(512))) for h in range(H) for s in range(T // 512)} |
                  {(0, h, j) for h in (0, H - 1) for j in (0, 127, 128, T - 1)})
    sampled_gradients(q, k, v, do, o_ref, lse_ref, dq, dk, dv, sc, True, rows, keys, "long causal")


def test_deterministic():
    q, k, v, do = (gen((2, 4, 300, 128), s).cuda() for s in range(4))
    o, lse = ea.fwd(q, k, v, causal=True)
    a = ea.bwd(q, k, v, o, lse, do, causal=True)
    b = ea.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
