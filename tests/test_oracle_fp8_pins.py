"""Pins for the E4M3 part of the oracle (oracle/fp8.py).

The decoder is pinned against values the format fixes (closed forms for
particular codes, the format's ordering and symmetry) and against a library
routine (torch's float8_e4m3fn conversion, which the oracle never calls).
The attention on decoded values is pinned through properties that hold
whatever the values: the per-tensor scales enter only as the products
scale * q_scale * k_scale and v_scale, and the lazy decoded views give the
same result as decoding everything up front.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8 as ofp8
from exact_tiled_attention_13_amd import workloads


# ------------------------------------------------------------ the number format
@pytest.mark.parametrize("code,value", [
    (0x00, 0.0),
    (0x38, 1.0),                      # exponent field 7 = bias, mantissa 0
    (0x3C, 1.5),
    (0x40, 2.0),
    (0x7E, 448.0),                    # largest finite: 2^8 * 1.75
    (0x08, 2.0 ** -6),                # smallest normal
    (0x01, 2.0 ** -9),                # smallest subnormal: 2^-6 * 1/8
    (0x07, 7 * 2.0 ** -9),            # largest subnormal
    (0xB8, -1.0),
    (0xFE, -448.0),
    (0x30, 0.5),
    (0x77, 240.0),                    # 2^7 * 1.875
])
def test_e4m3_closed_forms(code, value):
    assert ofp8.E4M3_VALUES[code] == value


def test_e4m3_nan_codes_and_negative_zero():
    vals = ofp8.E4M3_VALUES
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF])
    assert np.isnan(vals).sum() == 2
    assert vals[0x80] == 0.0 and math.copysign(1.0, vals[0x80]) == -1.0
    assert np.isfinite(vals).sum() == 254 and np.nanmax(np.abs(vals)) == 448.0


def test_e4m3_ordering_and_symmetry():
    vals = ofp8.E4M3_VALUES
    pos = vals[0x00:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7e must increase strictly"
    np.testing.assert_array_equal(vals[0x80:0xFF], -vals[0x00:0x7F])
    # spacing: 2^-9 in the subnormal range and the first binade, then doubling per binade
    gaps = np.diff(pos)
    np.testing.assert_array_equal(gaps[:15], np.full(15, 2.0 ** -9))
    for e in range(1, 15):
        seg = gaps[8 * e: 8 * e + 7]
        np.testing.assert_array_equal(seg, np.full(7, 2.0 ** (e - 7 - 3)))


def test_e4m3_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = ofp8.e4m3_decode(codes.numpy())
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    # every finite value survives torch's cast back to the same code
    back = torch.from_numpy(got[~nan]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(back, codes.numpy()[~nan])


def test_decode_accepts_torch_float8_and_uint8():
    g = torch.Generator().manual_seed(3)
    x = workloads.randn_e4m3((4, 5), g)
    a = ofp8.e4m3_decode(x)
    b = ofp8.e4m3_decode(x.view(torch.uint8))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(a, x.to(torch.float64).numpy())


# ---------------------------------------------------------------- attention
def _codes(shape, seed, scale=workloads.E4M3_SCALE):
    return workloads.randn_e4m3(shape, torch.Generator().manual_seed(seed), scale).view(torch.uint8).numpy()


def test_attention_fp8_is_attention_of_scaled_values():
    q8, k8, v8 = _codes((2, 4, 9, 16), 1), _codes((2, 2, 13, 16), 2), _codes((2, 2, 13, 16), 3)
    qs, ks, vs = 0.011, 0.0137, 0.02
    o, l = ofp8.attention_fp8(q8, k8, v8, qs, ks, vs, 0.25, causal=True, kv_lens=[13, 7])
    # the torch library's own decoding of the codes, times the scales
    dec = lambda c, s: torch.from_numpy(c).view(torch.float8_e4m3fn).to(torch.float64).numpy() * s  # noqa: E731
    o2, l2 = oracle.attention(dec(q8, qs), dec(k8, ks), dec(v8, vs), 0.25, causal=True, kv_lens=[13, 7])
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_scales_enter_as_products():
    q8, k8, v8 = _codes((1, 2, 6, 8), 4), _codes((1, 2, 10, 8), 5), _codes((1, 2, 10, 8), 6)
    o, l = ofp8.attention_fp8(q8, k8, v8, 0.02, 0.03, 0.05, 0.5)
    # q_scale * k_scale * scale is what matters for the scores
    o2, l2 = ofp8.attention_fp8(q8, k8, v8, 0.06, 0.01, 0.05, 0.5)
    o3, l3 = ofp8.attention_fp8(q8, k8, v8, 0.02, 0.03, 0.05 * 3, 0.5)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(l2, l, rtol=1e-12)
    np.testing.assert_allclose(o3, 3 * o, rtol=1e-12, atol=1e-15)
    np.testing.assert_array_equal(l3, l)


def test_negative_scale_flips_scores():
    q8, k8, v8 = _codes((1, 1, 5, 8), 7), _codes((1, 1, 9, 8), 8), _codes((1, 1, 9, 8), 9)
    a = ofp8.attention_fp8(q8, k8, v8, -0.02, 0.03, 0.05, 0.5)
    neg_q = (q8 ^ 0x80).astype(np.uint8)          # sign bit flipped
    b = ofp8.attention_fp8(neg_q, k8, v8, 0.02, 0.03, 0.05, 0.5)
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13)


def test_lazy_views_match_eager_decoding():
    B, Hq, Hkv, S, D = 3, 4, 2, 40, 16
    q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, [40, 17, 1], seed=2, poison=True,
                                                   scales=(0.01, 0.02, 0.03))
    lens = [40, 17, 1]
    o, l = ofp8.decode_fp8(q, k, v, lens, *sc, 0.25)
    # eager: decode only the valid rows (the poisoned tail holds NaN codes)
    qd = ofp8.e4m3_decode(q) * sc[0]
    kd = np.nan_to_num(ofp8.e4m3_decode(k)) * sc[1]
    vd = np.nan_to_num(ofp8.e4m3_decode(v)) * sc[2]
    o2, l2 = oracle.decode(qd, kd, vd, lens, 0.25)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)
    assert np.isfinite(o).all()


def test_decode_fp8_is_last_row_of_causal_prefill():
    B, Hq, Hkv, S, D = 2, 4, 2, 24, 16
    q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, [24, 11], seed=5,
                                                   scales=(0.015, 0.02, 0.01))
    lens = [24, 11]
    o, l = ofp8.decode_fp8(q, k, v, lens, *sc, 0.3)
    for b, L in enumerate(lens):
        qq = q.view(torch.uint8).numpy()[b:b + 1, :, None, :]
        kk = k.view(torch.uint8).numpy()[b:b + 1, :, :L]
        vv = v.view(torch.uint8).numpy()[b:b + 1, :, :L]
        of, lf = ofp8.attention_fp8(qq, kk, vv, *sc, 0.3, causal=True)
        np.testing.assert_allclose(o[b], of[0, :, 0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(l[b], lf[0, :, 0], rtol=1e-12)


def test_paged_fp8_matches_contiguous():
    B, Hq, Hkv, S, D, P = 2, 2, 1, 32, 8, 8
    q, k, v, sc = workloads.make_decode_inputs_fp8(B, Hq, Hkv, S, D, [32, 20], seed=6)
    lens = [32, 20]
    k8, v8 = k.view(torch.uint8).numpy(), v.view(torch.uint8).numpy()
    nb = S // P
    perm = np.random.default_rng(0).permutation(B * nb)
    kp = np.zeros((B * nb, Hkv, P, D), np.uint8)
    vp = np.zeros_like(kp)
    bt = perm.reshape(B, nb).astype(np.int32)
    for b in range(B):
        for i in range(nb):
            kp[bt[b, i]] = k8[b, :, i * P:(i + 1) * P]
            vp[bt[b, i]] = v8[b, :, i * P:(i + 1) * P]
    o, l = ofp8.decode_paged_fp8(q, kp, vp, bt, lens, *sc, 0.35)
    o2, l2 = ofp8.decode_fp8(q, k, v, lens, *sc, 0.35)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


def test_rows_fp8_matches_dense():
    q8, k8, v8 = _codes((2, 4, 12, 16), 11), _codes((2, 2, 12, 16), 12), _codes((2, 2, 12, 16), 13)
    rows = [(0, 0, 0), (1, 3, 11), (0, 2, 5), (1, 1, 4)]
    o, l = ofp8.attention_fp8(q8, k8, v8, 0.01, 0.02, 0.03, 0.4, causal=True, kv_lens=[12, 6])
    orow, lrow = ofp8.attention_rows_fp8(q8, k8, v8, rows, 0.01, 0.02, 0.03, 0.4, causal=True, kv_lens=[12, 6])
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_allclose(orow[n], o[b, h, i], rtol=1e-12, atol=1e-15)
        if np.isfinite(l[b, h, i]):
            np.testing.assert_allclose(lrow[n], l[b, h, i], rtol=1e-12)
        else:
            assert lrow[n] == l[b, h, i]
