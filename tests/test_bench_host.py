"""Host-side logic of bench.py (CPU): the algorithmic work the throughput
figures divide by, the peaks they are measured against, the counter
summaries behind roofline.traffic and roofline.mfma_busy, the rows of the
error report, and the one-GPU guard.

The work counts follow "Implementing attention from scratch", *Cost model*
(a multiply-add per element of each of the two products, counted only over
the (query, key) pairs the mask lets through) and *Masks* (causal alignment
at the bottom right when there are fewer queries than keys); the decode
bytes are the K and V rows each sequence needs (*KV caching*).
"""

import csv
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from exact_tiled_attention_13_amd import workloads as wl  # noqa: E402


def brute_pairs(B, Hq, Tq, Tk, causal, lens):
    """Unmasked pairs by enumeration: query i of a sequence with Lk keys and
    Lq valid rows sees key j when j < Lk and (not causal or j <= i + Lk - Lq)."""
    n = 0
    for b in range(B):
        lk = Tk if lens is None else min(max(lens[b], 0), Tk)
        lq = lk if (lens is not None and Tq == Tk) else Tq
        for i in range(lq):
            for j in range(lk):
                if not causal or j <= i + lk - lq:
                    n += 1
    return n * Hq


@pytest.mark.parametrize("B,Hq,Tq,Tk,causal,lens", [
    (1, 1, 5, 5, True, None),
    (1, 2, 3, 7, True, None),        # chunked prefill: 3 new queries after 4 cached keys
    (1, 1, 7, 3, True, None),        # more queries than keys: the first 4 rows see nothing
    (2, 3, 6, 6, True, [4, 0]),
    (3, 1, 6, 6, False, [1, 6, 9]),  # a length past T is clamped to T
    (2, 1, 4, 9, True, [9, 2]),      # Tq != Tk: every row is valid, the lengths set the keys
    (2, 1, 4, 9, False, [-3, 5]),
])
def test_prefill_pairs_match_enumeration(B, Hq, Tq, Tk, causal, lens):
    assert bench.prefill_pairs(B, Hq, Tq, Tk, causal, lens) == brute_pairs(B, Hq, Tq, Tk, causal, lens)


def test_prefill_work_of_the_workloads():
    """4*D flop per unmasked pair: the closed forms of the dense and causal
    workloads, and 8192 * sum(L_b^2) for the ragged one (16 heads, D = 128)."""
    def flops(name):
        W = wl.WORKLOADS[name]
        lens = None if W.lens is None else wl.draw_lengths(W.B, W.lens[0], W.lens[1], W.lens[2], 0)
        return 4 * W.D * bench.prefill_pairs(W.B, W.Hq, W.Tq, W.Tk, W.causal, lens), lens

    assert flops("single")[0] == 4 * 64 * 256 * 512 == 33_554_432
    assert flops("causal")[0] == 4 * 64 * 4 * 16 * (1024 * 1025 // 2) == 8_598_323_200
    assert flops("long")[0] == 4 * 128 * 32 * (32768 * 32769 // 2) == 8_796_361_457_664
    f, lens = flops("ragged")
    assert lens[0] == 1 and all(1 <= x <= 4096 for x in lens)
    assert f == 8192 * int(np.sum(np.asarray(lens, dtype=np.int64) ** 2))
    # E4M3 workloads count the same pairs as their bf16 counterparts
    assert flops("causal-fp8")[0] == flops("causal")[0]
    assert flops("long-fp8")[0] == flops("long")[0]


def test_decode_bytes():
    """K and V rows actually needed (2 tensors x Hkv x D x bytes per element
    per cached key), plus q, the bf16 o, the fp32 lse and the int32 lengths."""
    W = wl.WORKLOADS["decode"]
    lens = wl.draw_lengths(W.B, W.lens[0], W.lens[1], W.lens[2], 0)
    s = int(np.sum(lens))
    assert bench.decode_bytes(W, lens) == 4096 * s + 1_057_024
    assert bench.decode_bytes(W, lens, elem=1) == 2048 * s + 64 * 32 * 128 * 3 + 64 * 32 * 4 + 64 * 4
    # lengths past the cache count only the cache's rows
    assert bench.decode_bytes(W, [40000] + [0] * 63) == 4096 * 32768 + 1_057_024


def test_peaks():
    assert bench.PEAK_BF16_TFLOPS == pytest.approx(256 * 2.4e9 * 4096 / 1e12, abs=0.05)
    assert bench.PEAK_FP8_TFLOPS == pytest.approx(2 * 256 * 2.4e9 * 4096 / 1e12, abs=0.05)
    # half the E4M3 prefill's flops (Q K^T) at the fp8 rate, half (P V) at bf16
    t = 0.5 / bench.PEAK_FP8_TFLOPS + 0.5 / bench.PEAK_BF16_TFLOPS
    assert bench.PEAK_FP8_BF16_TFLOPS == pytest.approx(1 / t)
    assert bench.PEAK_FP8_BF16_TFLOPS == pytest.approx(3355.5, abs=0.1)
    assert bench.N_SIMD == 1024


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
                                           "End_Timestamp"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def _row(kernel, counter, value, t0=0, t1=1000):
    return dict(Kernel_Name=kernel, Counter_Name=counter, Counter_Value=value, Start_Timestamp=t0, End_Timestamp=t1)


def test_traffic_summary_and_source_gating(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.traffic_for("fwd_bf16_kernel", "causal") is None      # no summary yet
    kib = bench.COPY_BYTES / 1024
    copy = "void at::native::elementwise_kernel<copy_>"
    kern = "void miattn::fwd_bf16_kernel<64, 4, 2, true, false>(FwdArgs)"
    # the copy reads half its bytes in FETCH_SIZE (scale 2) and writes all of them
    _write_counters(str(tmp_path / "cf"), [_row(copy, "FETCH_SIZE", kib / 2)])
    _write_counters(str(tmp_path / "cw"), [_row(copy, "WRITE_SIZE", kib)])
    _write_counters(str(tmp_path / "kf"), [_row(kern, "FETCH_SIZE", 900), _row(kern, "FETCH_SIZE", 1100),
                                           _row("other", "FETCH_SIZE", 1e9)])
    _write_counters(str(tmp_path / "kw"), [_row(kern, "WRITE_SIZE", 500)])
    bench.summarize_pmc("fwd_bf16_kernel", "causal", str(tmp_path / "kf"), str(tmp_path / "kw"),
                        str(tmp_path / "cf"), str(tmp_path / "cw"), "cmd")
    entry = json.load(open(tmp_path / "traffic.json"))["fwd_bf16_kernel/causal"]
    assert entry["fetch_scale"] == pytest.approx(2.0) and entry["write_scale"] == pytest.approx(1.0)
    assert entry["dispatches"] == [2, 1]
    assert bench.traffic_for("fwd_bf16_kernel", "causal") == pytest.approx((1000 * 2 + 500) * 1024)
    # a summary taken on other kernel sources is not reported
    data = json.load(open(tmp_path / "traffic.json"))
    data["fwd_bf16_kernel/causal"]["sources_sha256_16"] = "0" * 16
    json.dump(data, open(tmp_path / "traffic.json", "w"))
    assert bench.traffic_for("fwd_bf16_kernel", "causal") is None


def test_mfma_summary(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    kern = "void miattn::fwd_bf16_kernel<64, 4, 2, true, false>(FwdArgs)"
    cycles = 40000.0                      # per shader engine
    busy = 0.25 * cycles * bench.N_SIMD   # a quarter of the SIMD cycles
    W = wl.WORKLOADS["causal"]
    f_alg = 4 * W.D * bench.prefill_pairs(W.B, W.Hq, W.Tq, W.Tk, W.causal, None)
    vals = {"SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_VALU_MFMA_COEXEC_CYCLES": busy / 2,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": f_alg / 512, "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0,
            "SQ_INSTS_VALU_MFMA_MOPS_F6F4": 0.0, "SQ_BUSY_CYCLES": cycles * bench.N_SE,
            "SQ_ACTIVE_INST_VALU": 1.0, "GRBM_GUI_ACTIVE": 1.0}
    _write_counters(str(tmp_path / "pm"), [_row(kern, c, v, 0, 20000) for c, v in vals.items()])
    bench.summarize_mfma("fwd_bf16_kernel", "causal", str(tmp_path / "pm"), "cmd")
    e = json.load(open(tmp_path / "mfma.json"))["fwd_bf16_kernel/causal"]
    assert e["mfma_busy"] == pytest.approx(0.25)
    assert e["coexec_of_busy"] == pytest.approx(0.5)
    assert e["mfma_flops_over_algorithmic"] == pytest.approx(1.0)
    assert e["implied_clock_ghz"] == pytest.approx(cycles / 20e-6 / 1e9)
    assert bench.mfma_busy_for("fwd_bf16_kernel", "causal") == pytest.approx(0.25)
    assert bench.mfma_busy_for("fwd_bf16_kernel", "long") is None


def test_committed_counter_summaries_are_consistent():
    """Every committed entry names a known kernel and scales FETCH_SIZE by
    2 and WRITE_SIZE by 1 (the copy calibration on gfx950)."""
    for name in ("traffic.json", "mfma.json"):
        data = json.load(open(os.path.join(ROOT, "profiles", name)))
        for key, e in data.items():
            kernel, workload = key.split("/")
            assert kernel in bench.KERNEL_SOURCES and workload in wl.WORKLOADS, key
            if name == "traffic.json":
                assert e["fetch_scale"] == pytest.approx(2.0, rel=1e-3), key
                assert e["write_scale"] == pytest.approx(1.0, rel=1e-3), key


def test_sampled_rows():
    lens = [0, 1, 300, 4096]
    rows = bench.sampled_rows(4, 16, 4096, lens, 64, 3)
    assert rows == bench.sampled_rows(4, 16, 4096, lens, 64, 3)
    assert len(rows) == len(set(rows)) and len(rows) <= 64 + 10
    for b, h, i in rows:
        assert 0 <= h < 16 and 0 <= i < 4096
        # random rows are valid; padding rows come only from the fixed set of
        # tile-edge rows (0, 127, 128) and the first row past the length
        assert i < lens[b] or i in (0, 127, 128, lens[b])
    for b in (1, 2, 3):
        assert (b, 0) in {(r[0], min(r[2], 0)) for r in rows}       # first row of each non-empty sequence
        assert any(r[0] == b and r[2] == lens[b] - 1 for r in rows)  # and its last valid row


def test_error_report():
    import torch

    o_ref = np.zeros((3, 4))
    l_ref = np.array([0.5, -np.inf, 1.0])
    good = bench._errors(torch.zeros(3, 4), torch.tensor([0.5, -np.inf, 1.0005]), o_ref, l_ref, (2e-2, 1e-3), "x")
    assert good["within_tolerance"] and good["neg_inf_lse_match"]
    assert good["max_abs_lse"] == pytest.approx(5e-4, rel=1e-3)
    lse_inf = bench._errors(torch.zeros(3, 4), torch.tensor([0.5, 0.0, 1.0]), o_ref, l_ref, (2e-2, 1e-3), "x")
    assert not lse_inf["within_tolerance"] and not lse_inf["neg_inf_lse_match"]
    o_nan = torch.zeros(3, 4)
    o_nan[1, 2] = float("nan")
    assert not bench._errors(o_nan, torch.tensor([0.5, -np.inf, 1.0]), o_ref, l_ref, (2e-2, 1e-3), "x")[
        "within_tolerance"]
    o_far = torch.full((3, 4), 0.03)
    assert not bench._errors(o_far, torch.tensor([0.5, -np.inf, 1.0]), o_ref, l_ref, (2e-2, 1e-3), "x")[
        "within_tolerance"]


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_backward_busy_share_is_time_weighted(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.backward_mfma_busy("long") is None
    h = bench.sources_hash("bwd_dq_kernel")
    data = {"bwd_dq_kernel/long": dict(sources_sha256_16=h, mfma_busy=0.6, dispatch_seconds=1.0),
            "bwd_dkdv/long": dict(sources_sha256_16=h, mfma_busy=0.3, dispatch_seconds=2.0)}
    json.dump(data, open(tmp_path / "mfma.json", "w"))
    assert bench.backward_mfma_busy("long") == pytest.approx((0.6 * 1 + 0.3 * 2) / 3, abs=1e-4)
    assert bench.backward_mfma_busy("causal") is None            # no entries for that workload
    data["bwd_dkdv/long"]["sources_sha256_16"] = "0" * 16
    json.dump(data, open(tmp_path / "mfma.json", "w"))
    assert bench.backward_mfma_busy("long") is None              # one of the two is stale
