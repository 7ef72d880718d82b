"""Pins of the float64 backward oracle against things other than itself:
central finite differences of the forward definition, PyTorch autograd
through scaled_dot_product_attention in float64, closed forms and
invariants of the softmax Jacobian."""

import math

import numpy as np
import pytest
import torch

import oracle


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("lens", [None, [4, 2]])
def test_finite_differences(causal, lens):
    """Brute force: dL/dx for L = sum(dO * O) by central differences of the
    forward oracle, every element of q, k and v (B=2, Hq=2, Hkv=1, tiny)."""
    B, Hq, Hkv, Tq, Tk, D = 2, 2, 1, 4, (4 if lens else 6), 3
    q, k, v = rnd((B, Hq, Tq, D), 1), rnd((B, Hkv, Tk, D), 2), rnd((B, Hkv, Tk, D), 3)
    do = rnd((B, Hq, Tq, D), 4)
    sc = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, sc, causal, lens)

    def loss(qq, kk, vv):
        o, _ = oracle.attention(qq, kk, vv, sc, causal, lens)
        return float((o * do).sum())

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, atol=1e-7, rtol=1e-6), name


@pytest.mark.parametrize("Tq,Tk,causal", [(37, 37, False), (37, 37, True), (20, 37, True), (37, 20, False)])
def test_against_torch_autograd_sdpa(Tq, Tk, causal):
    """Library routine: autograd of torch's float64 SDPA (bool mask, True =
    attend, bottom-right causal built explicitly), GQA expanded by
    repeat_interleave.  Shapes chosen so no row is fully masked."""
    B, Hq, Hkv, D = 2, 4, 2, 16
    G = Hq // Hkv
    q, k, v = rnd((B, Hq, Tq, D), 5), rnd((B, Hkv, Tk, D), 6), rnd((B, Hkv, Tk, D), 7)
    do = rnd((B, Hq, Tq, D), 8)
    sc = 1 / math.sqrt(D)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, sc, causal)
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    mask = None
    if causal:
        off = Tk - Tq
        mask = torch.arange(Tk)[None, :] <= (torch.arange(Tq)[:, None] + off)
        assert mask.any(dim=1).all()
    o = torch.nn.functional.scaled_dot_product_attention(
        tq, tk.repeat_interleave(G, dim=1), tv.repeat_interleave(G, dim=1), attn_mask=mask, scale=sc)
    o.backward(torch.tensor(do))
    assert np.allclose(dq, tq.grad.numpy(), atol=1e-10)
    assert np.allclose(dk, tk.grad.numpy(), atol=1e-10)
    assert np.allclose(dv, tv.grad.numpy(), atol=1e-10)


@pytest.mark.parametrize("causal", [False, True])
def test_jacobian_invariants(causal):
    """Every softmax row's dS sums to zero, so the keys' dK sum to zero;
    every valid row's weights sum to one, so the keys' dV sum to the valid
    rows' dO.  Padding rows get dQ = 0, keys past the length dK = dV = 0."""
    B, Hq, Hkv, T, D = 3, 4, 2, 29, 8
    lens = [29, 11, 1]
    q, k, v = rnd((B, Hq, T, D), 9), rnd((B, Hkv, T, D), 10), rnd((B, Hkv, T, D), 11)
    do = rnd((B, Hq, T, D), 12)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.4, causal, lens)
    G = Hq // Hkv
    for b, L in enumerate(lens):
        for hk in range(Hkv):
            assert np.allclose(dk[b, hk].sum(axis=0), 0, atol=1e-12)
            want = do[b, hk * G:(hk + 1) * G, :L].sum(axis=(0, 1))
            assert np.allclose(dv[b, hk].sum(axis=0), want, atol=1e-12)
        assert np.all(dq[b, :, L:] == 0)
        assert np.all(dk[b, :, L:] == 0) and np.all(dv[b, :, L:] == 0)


def test_single_key_closed_form():
    """One key: every weight is 1, so dQ = dK = 0 and dV_0 = sum of dO."""
    q, k, v = rnd((1, 2, 5, 4), 13), rnd((1, 1, 1, 4), 14), rnd((1, 1, 1, 4), 15)
    do = rnd((1, 2, 5, 4), 16)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.9)
    assert np.all(dq == 0) and np.allclose(dk, 0, atol=1e-15)
    assert np.allclose(dv[0, 0, 0], do[0].sum(axis=(0, 1)), atol=1e-12)


def test_gqa_is_mha_with_summed_group_gradients():
    B, Hq, Hkv, T, D = 2, 6, 2, 17, 8
    G = Hq // Hkv
    q, k, v = rnd((B, Hq, T, D), 17), rnd((B, Hkv, T, D), 18), rnd((B, Hkv, T, D), 19)
    do = rnd((B, Hq, T, D), 20)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, 0.3, True)
    ke, ve = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    dq2, dk2, dv2 = oracle.attention_backward(q, ke, ve, do, 0.3, True)
    assert np.allclose(dq, dq2, atol=1e-12)
    assert np.allclose(dk, dk2.reshape(B, Hkv, G, T, D).sum(axis=2), atol=1e-12)
    assert np.allclose(dv, dv2.reshape(B, Hkv, G, T, D).sum(axis=2), atol=1e-12)


def test_rows_helper_matches_full():
    B, Hq, Hkv, Tq, Tk, D = 2, 4, 2, 40, 50, 8
    q, k, v = rnd((B, Hq, Tq, D), 21), rnd((B, Hkv, Tk, D), 22), rnd((B, Hkv, Tk, D), 23)
    do = rnd((B, Hq, Tq, D), 24)
    lens = [50, 7]
    dq, _, _ = oracle.attention_backward(q, k, v, do, 0.25, True, lens)
    rows = [(0, 0, 0), (0, 3, 39), (1, 1, 5), (1, 2, 39), (1, 0, 0)]
    got = oracle.backward_rows(q, k, v, do, rows, 0.25, True, lens)
    for n, (b, h, i) in enumerate(rows):
        assert np.allclose(got[n], dq[b, h, i], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("shape,lens", [((2, 4, 2, 37, 37, 8), None), ((3, 4, 1, 21, 21, 5), [21, 0, 9]),
                                        ((2, 2, 2, 7, 30, 6), None), ((2, 2, 1, 30, 7, 6), [5, 7])])
def test_key_rows_equal_full_backward(causal, shape, lens):
    """dK, dV of selected keys from the saved statistics (o, lse of the
    forward oracle) equal the full backward oracle's, which finite
    differences and autograd pin above; every key of every KV head,
    including keys past a length (zeros) and Tq != Tk (bottom-right)."""
    B, Hq, Hkv, Tq, Tk, D = shape
    q, k, v, do = rnd((B, Hq, Tq, D), 11), rnd((B, Hkv, Tk, D), 12), rnd((B, Hkv, Tk, D), 13), rnd((B, Hq, Tq, D), 14)
    sc = 0.45
    o, lse = oracle.attention(q, k, v, sc, causal, lens)
    _, dk, dv = oracle.attention_backward(q, k, v, do, sc, causal, lens)
    keys = [(b, h, j) for b in range(B) for h in range(Hkv) for j in range(Tk)]
    gk, gv = oracle.backward_key_rows(q, k, v, do, o, lse, keys, sc, causal, lens)
    ref_k = np.stack([dk[b, h, j] for b, h, j in keys])
    ref_v = np.stack([dv[b, h, j] for b, h, j in keys])
    assert np.abs(gk - ref_k).max() <= 1e-10 * max(1.0, np.abs(ref_k).max())
    assert np.abs(gv - ref_v).max() <= 1e-10 * max(1.0, np.abs(ref_v).max())
    # a scrambled key order returns the same rows
    perm = np.random.default_rng(0).permutation(len(keys))
    pk, pv = oracle.backward_key_rows(q, k, v, do, o, lse, [keys[i] for i in perm], sc, causal, lens)
    assert np.array_equal(pk, gk[perm]) and np.array_equal(pv, gv[perm])


def test_key_rows_use_the_given_statistics():
    """A planted mistake in the statistics shows: shifting lse by c scales
    every weight by exp(-c), so dV (linear in P) scales by exp(-c)."""
    B, Hq, Hkv, T, D = 1, 2, 1, 9, 4
    q, k, v, do = rnd((B, Hq, T, D), 21), rnd((B, Hkv, T, D), 22), rnd((B, Hkv, T, D), 23), rnd((B, Hq, T, D), 24)
    o, lse = oracle.attention(q, k, v, 0.5, True)
    keys = [(0, 0, j) for j in range(T)]
    _, gv = oracle.backward_key_rows(q, k, v, do, o, lse, keys, 0.5, True)
    _, gv2 = oracle.backward_key_rows(q, k, v, do, o, lse + 0.3, keys, 0.5, True)
    assert np.allclose(gv2, gv * math.exp(-0.3), rtol=1e-12, atol=1e-14)
