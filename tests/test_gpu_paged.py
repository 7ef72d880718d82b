"""GPU parity of the paged-cache decode (attn_decode_paged through the C ABI)
against the float64 oracle, same tolerances as the contiguous decode (O <=
2e-2, LSE <= 1e-3).  Pages are placed at random in a pool larger than
needed; unreferenced pages and rows past each length hold NaN."""

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
import oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def gen(shape, g):
    return torch.randn(shape, generator=g, dtype=torch.float32).to(torch.bfloat16)


def make_paged(B, Hq, Hkv, D, P, lens, max_blocks, seed, spare=7):
    """Random pool: sequence b gets ceil(lens[b]/P) distinct random pages."""
    g = torch.Generator().manual_seed(seed)
    rng = np.random.default_rng(seed)
    need = [-(-L // P) for L in lens]
    num_pages = sum(need) + spare
    perm = rng.permutation(num_pages)
    kp = torch.full((num_pages, Hkv, P, D), float("nan"), dtype=torch.bfloat16)
    vp = torch.full_like(kp, float("nan"))
    bt = np.zeros((B, max_blocks), dtype=np.int32)
    used = 0
    for b, L in enumerate(lens):
        pages = perm[used:used + need[b]]
        used += need[b]
        bt[b, :need[b]] = pages
        bt[b, need[b]:] = rng.integers(0, num_pages, max_blocks - need[b])   # never read
        for i, pg in enumerate(pages):
            n = min(P, L - i * P)
            kp[pg, :, :n] = gen((Hkv, n, D), g)
            vp[pg, :, :n] = gen((Hkv, n, D), g)
    q = gen((B, Hq, D), g)
    return q, kp, vp, bt


def check(o, lse, o_ref, l_ref, what):
    a, l = o.float().cpu().double().numpy(), lse.cpu().double().numpy()
    assert np.isfinite(a).all(), what
    assert np.array_equal(np.isneginf(l), np.isneginf(l_ref)), what
    fin = np.isfinite(l_ref)
    eo = float(np.abs(a - o_ref).max())
    el = float(np.abs(l[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    print(f"  {what}: max|dO| {eo:.3e} max|dLSE| {el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 1e-3, what


@pytest.mark.parametrize("P", [8, 16, 64, 512, 1024])
@pytest.mark.parametrize("D", [64, 128])
def test_paged_decode_page_sizes(P, D):
    B, Hq, Hkv = 5, 8, 2
    lens = [1, 0, 1100, P, 513]
    max_blocks = -(-1100 // P) + 1
    q, kp, vp, bt = make_paged(B, Hq, Hkv, D, P, lens, max_blocks, seed=P + D)
    o, lse = ea.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(bt).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"), scale=0.1)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_paged(q, kp, vp, bt, lens, 0.1)
    check(o, lse, o_ref, l_ref, f"paged P{P} D{D}")


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 1), (6, 3)])
def test_paged_decode_gqa(Hq, Hkv):
    B, D, P = 3, 128, 16
    lens = [2000, 31, 4096]
    q, kp, vp, bt = make_paged(B, Hq, Hkv, D, P, lens, 4096 // P, seed=Hq * 10 + Hkv)
    o, lse = ea.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(bt).cuda(),
                             torch.tensor(lens, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.decode_paged(q, kp, vp, bt, lens, 1 / np.sqrt(D))
    check(o, lse, o_ref, l_ref, f"paged GQA Hq{Hq} Hkv{Hkv}")


def test_paged_equals_contiguous_bitwise():
    """The same logical cache through pages or contiguous: the kernels take
    the same tiles in the same order, so the results are bit-identical."""
    B, Hq, Hkv, D, P = 4, 16, 4, 128, 64
    lens = [700, 64, 1, 3000]
    S = 3008
    q, kp, vp, bt = make_paged(B, Hq, Hkv, D, P, lens, S // P, seed=5)
    kc = torch.zeros((B, Hkv, S, D), dtype=torch.bfloat16)
    vc = torch.zeros_like(kc)
    for b, L in enumerate(lens):
        j = np.arange(L)
        kc[b, :, :L] = kp[bt[b, j // P], :, j % P].permute(1, 0, 2)
        vc[b, :, :L] = vp[bt[b, j // P], :, j % P].permute(1, 0, 2)
    kv = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o1, l1 = ea.decode(q.cuda(), kc.cuda(), vc.cuda(), kv)
    o2, l2 = ea.decode_paged(q.cuda(), kp.cuda(), vp.cuda(), torch.from_numpy(bt).cuda(), kv)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
