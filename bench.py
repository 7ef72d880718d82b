#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload causal|long|ragged|decode|decode-paged|decode-fp8|causal-fp8|long-fp8|single]
                    [--backward]

A step is one pass of the hot path over one batch of synthetic, seeded input
already resident in HBM.  The headline line measures the causal prefill
workload (B=4, H=16, T=1024, D=64, bf16) in TFLOP/s of algorithmic work
(4*D flops per unmasked (query, key) pair); the same run also times one
KV-cache decode step of the GQA decode workload (B=64, Hq=32, Hkv=8, D=128,
lengths 1024..32768) in GB/s of algorithmic bytes (the K/V rows each sequence
needs plus q, o, lse and lengths), reported under "decode", the same step on
E4M3 (FP8) q and caches under "decode_fp8", the causal prefill on E4M3 Q, K,
V under "prefill_fp8", and the gradients
of the causal workload (10*D flops per unmasked pair: the five products of
the backward), reported under "backward".  Steps are
replayed from a HIP graph (a fixed number of calls per graph) so that host
launch overhead does not enter the timing; the kernels are timed with HIP
events recorded on the stream they run on.

The float64 CPU oracle is timed on a bounded sample of the same workload
(cpu_baseline).  It is a reported baseline, not the target.

roofline.traffic (HBM bytes per launch) and roofline.mfma_busy (share of the
chip's SIMD cycles with the matrix unit busy) come from rocprofv3 counter
runs summarised into profiles/traffic.json and profiles/mfma.json
(--summarize-pmc, --summarize-mfma); they are null once the kernel's sources
differ from those the counters were taken on.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_tiled_attention_13_amd", "csrc")
# kernel name (as rocprofv3 reports it, substring) -> sources it is built from
KERNEL_SOURCES = {
    "fwd_bf16_kernel": ["fwd_bf16.hip", "device_common.h", "launch.h"],
    "fwd_f32_kernel": ["fwd_f32.hip", "device_common.h"],
    "decode_split_kernel": ["decode.hip", "device_common.h", "launch.h"],
}
COPY_BYTES = 1 << 30          # size of the calibration copy

PEAK_BF16_TFLOPS = 2516.6   # 256 CU * 2.4 GHz * 4096 dense bf16 flop/clk/CU
PEAK_FP8_TFLOPS = 5033.2    # 256 CU * 2.4 GHz * 8192 dense fp8 flop/clk/CU
# The E4M3 prefill runs Q K^T (half the flops) on fp8 and P V on bf16, so its
# matrix peak is the harmonic combination of the two.
PEAK_FP8_BF16_TFLOPS = 1.0 / (0.5 / PEAK_FP8_TFLOPS + 0.5 / PEAK_BF16_TFLOPS)
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
N_SIMD = 256 * 4            # SIMDs (matrix units) on the chip
N_SE = 32                   # SQ_BUSY_CYCLES is summed over 8 XCDs x 4 shader engines
# one rocprofv3 --pmc pass (7 SQ + 1 GRBM counters, within one pass's limits)
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
                 "SQ_INSTS_VALU_MFMA_MOPS_F8", "SQ_INSTS_VALU_MFMA_MOPS_F6F4", "SQ_BUSY_CYCLES",
                 "SQ_ACTIVE_INST_VALU", "GRBM_GUI_ACTIVE")
CALLS_PER_GRAPH = 20


def prefill_pairs(B, Hq, Tq, Tk, causal, lens):
    """Number of unmasked (query, key) pairs, summed over batch and heads."""
    total = 0
    for b in range(B):
        lk = Tk if lens is None else int(min(max(lens[b], 0), Tk))
        lq = lk if (lens is not None and Tq == Tk) else Tq
        off = lk - lq
        i = np.arange(lq, dtype=np.int64)
        seen = np.clip(np.minimum(lk, i + off + 1), 0, None) if causal else np.full(lq, lk, dtype=np.int64)
        total += int(seen.sum())
    return total * Hq


def decode_bytes(W, lens, elem=2):
    """Algorithmic bytes of one decode step: the K and V rows each sequence
    needs and q (elem bytes per element), o (bf16), lse and the lengths."""
    kv = 2 * W.Hkv * W.D * elem * int(np.sum(np.clip(lens, 0, W.Tk)))
    return kv + W.B * W.Hq * W.D * (elem + 2) + W.B * W.Hq * 4 + W.B * 4


def blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        return max(n) if n else 1
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


class Graphed:
    """A HIP graph holding CALLS_PER_GRAPH calls of fn, replayed to run steps."""

    def __init__(self, torch, fn):
        self.torch = torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()  # eager call on the capture stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            for _ in range(CALLS_PER_GRAPH):
                fn()
        torch.cuda.synchronize()

    def run(self, steps):
        for _ in range(max(1, steps // CALLS_PER_GRAPH)):
            self.g.replay()


def time_steps(torch, runner, steps, warmup):
    """Warm up, then time exactly `steps` steps (rounded to whole graphs)."""
    runner.run(warmup)
    torch.cuda.synchronize()
    n = max(1, steps // CALLS_PER_GRAPH) * CALLS_PER_GRAPH
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    runner.run(n)
    ev1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    return ev0.elapsed_time(ev1) / n, wall_ms / n, n


def setup_prefill(torch, name):
    import exact_tiled_attention_13_amd as ea
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make(name, device="cpu")
    W = w["workload"]
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    kv = None if w["kv_lens"] is None else w["kv_lens"].cuda()
    lse = torch.empty((W.B, W.Hq, W.Tq), dtype=torch.float32, device="cuda")
    kvp = 0 if kv is None else kv.data_ptr()
    if W.dtype == "e4m3":
        o = torch.empty((W.B, W.Hq, W.Tq, W.D), dtype=torch.bfloat16, device="cuda")
        qs, ks, vs = w["fp8_scales"]
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), W.B, W.Hq, W.Hkv, W.Tq,
                W.Tk, W.D, W.scale, qs, ks, vs, int(W.causal), kvp)

        def step():
            ea.attn_fwd_fp8(*args, torch.cuda.current_stream().cuda_stream)
    else:
        o = torch.empty_like(q)
        dt = ea.MIATTN_BF16 if W.dtype == "bf16" else ea.MIATTN_F32
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), W.B, W.Hq, W.Hkv, W.Tq,
                W.Tk, W.D, W.scale, int(W.causal), kvp, dt)

        def step():
            ea.attn_fwd(*args, torch.cuda.current_stream().cuda_stream)

    pairs = prefill_pairs(W.B, W.Hq, W.Tq, W.Tk, W.causal, w["lens"])
    flops = 4 * W.D * pairs
    elem = {"bf16": 2, "f32": 4, "e4m3": 1}[W.dtype]
    io_bytes = (q.numel() + k.numel() + v.numel()) * elem + o.numel() * o.element_size() + lse.numel() * 4
    keep = (q, k, v, kv, o, lse)
    return dict(w=w, W=W, step=step, flops=flops, io_bytes=io_bytes, keep=keep, out=(o, lse))


def setup_backward(torch, name):
    """Gradients of a prefill workload: q, k, v of the workload, a seeded dO,
    and O, LSE from one forward call."""
    import exact_tiled_attention_13_amd as ea
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make(name, device="cpu")
    W = w["workload"]
    if W.dtype != "bf16":
        raise SystemExit("the backward pass is bf16 only")
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    g = torch.Generator().manual_seed(1)
    do = workloads.randn_bf16(tuple(q.shape), g).cuda()
    kv = None if w["kv_lens"] is None else w["kv_lens"].cuda()
    o, lse = ea.fwd(q, k, v, causal=W.causal, kv_lens=kv, scale=W.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = ea.attn_bwd_workspace_size(W.B, W.Hq, W.Tq)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(),
            dk.data_ptr(), dv.data_ptr(), W.B, W.Hq, W.Hkv, W.Tq, W.Tk, W.D, W.scale, int(W.causal),
            0 if kv is None else kv.data_ptr(), ws.data_ptr(), nbytes, ea.MIATTN_BF16)

    def step():
        ea.attn_bwd(*args, torch.cuda.current_stream().cuda_stream)

    pairs = prefill_pairs(W.B, W.Hq, W.Tq, W.Tk, W.causal, w["lens"])
    return dict(w=w, W=W, step=step, flops=10 * W.D * pairs, keep=(q, k, v, do, kv, o, lse, ws),
                out=(dq, dk, dv))


def cpu_baseline_backward(name, budget_s):
    import oracle
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make(name, device="cpu")
    W = w["workload"]
    q, k, v = w["q"], w["k"], w["v"]
    do = workloads.randn_bf16(tuple(q.shape), __import__("torch").Generator().manual_seed(1))
    G = W.Hq // W.Hkv
    done, heads = 0, 0
    t0 = time.perf_counter()
    for b in range(W.B):
        for h in range(W.Hq):
            lens = None if w["lens"] is None else w["lens"][b:b + 1]
            oracle.attention_backward(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                                      v[b:b + 1, h // G:h // G + 1], do[b:b + 1, h:h + 1], W.scale, W.causal, lens)
            done += 10 * W.D * prefill_pairs(1, 1, W.Tq, W.Tk, W.causal, lens)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=done / dt / 1e12, unit="TFLOP/s", cores=blas_threads(), kind="oracle",
                sample=f"gradients of {heads} of {W.B * W.Hq} (batch, head) pairs of the {W.name} workload, "
                       f"float64 numpy, {dt:.1f} s")


def setup_decode(torch):
    import exact_tiled_attention_13_amd as ea
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make("decode", device="cuda")
    W = w["workload"]
    q, k, v, kv = w["q"], w["k"], w["v"], w["kv_lens"]
    o = torch.empty_like(q)
    lse = torch.empty((W.B, W.Hq), dtype=torch.float32, device="cuda")
    nbytes = ea.attn_decode_workspace_size(W.B, W.Hq, W.Hkv, W.Tk, W.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), W.B, W.Hq, W.Hkv, W.Tk, W.D,
            W.scale, kv.data_ptr(), ws.data_ptr(), nbytes, ea.MIATTN_BF16)

    def step():
        ea.attn_decode(*args, torch.cuda.current_stream().cuda_stream)

    return dict(w=w, W=W, step=step, bytes=decode_bytes(W, w["lens"]), keep=(q, k, v, kv, o, lse, ws),
                out=(o, lse))


def setup_decode_fp8(torch):
    """The decode workload with q and the caches as E4M3 codes (one scale per tensor)."""
    import exact_tiled_attention_13_amd as ea
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make("decode-fp8", device="cuda")
    W = w["workload"]
    q, k, v, kv = w["q"], w["k"], w["v"], w["kv_lens"]
    qs, ks, vs = w["fp8_scales"]
    o = torch.empty((W.B, W.Hq, W.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((W.B, W.Hq), dtype=torch.float32, device="cuda")
    nbytes = ea.attn_decode_workspace_size(W.B, W.Hq, W.Hkv, W.Tk, W.D)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), W.B, W.Hq, W.Hkv, W.Tk, W.D,
            W.scale, qs, ks, vs, kv.data_ptr(), ws.data_ptr(), nbytes)

    def step():
        ea.attn_decode_fp8(*args, torch.cuda.current_stream().cuda_stream)

    return dict(w=w, W=W, step=step, bytes=decode_bytes(W, w["lens"], elem=1), keep=(q, k, v, kv, o, lse, ws),
                out=(o, lse))


def setup_decode_paged(torch, page_size):
    """The decode workload with its cache moved into a pool of pages placed at
    random (same logical contents, so the same algorithmic bytes)."""
    import exact_tiled_attention_13_amd as ea

    dec = setup_decode(torch)
    W, w = dec["W"], dec["w"]
    k, v = w["k"], w["v"]
    B, Hkv, S, D = k.shape
    if S % page_size:
        raise SystemExit("page size must divide the cache length")
    nb = S // page_size
    g = torch.Generator(device="cuda").manual_seed(2)
    perm = torch.randperm(B * nb, generator=g, device="cuda")
    kp = torch.empty((B * nb, Hkv, page_size, D), dtype=k.dtype, device="cuda")
    vp = torch.empty_like(kp)
    kp[perm] = k.reshape(B, Hkv, nb, page_size, D).transpose(1, 2).reshape(B * nb, Hkv, page_size, D)
    vp[perm] = v.reshape(B, Hkv, nb, page_size, D).transpose(1, 2).reshape(B * nb, Hkv, page_size, D)
    bt = perm.to(torch.int32).reshape(B, nb).contiguous()
    q, kv = w["q"], w["kv_lens"]
    o, lse = dec["out"]
    ws = dec["keep"][-1]
    del dec, k, v
    w["k"] = w["v"] = None
    torch.cuda.empty_cache()
    args = (q.data_ptr(), kp.data_ptr(), vp.data_ptr(), bt.data_ptr(), o.data_ptr(), lse.data_ptr(), W.B, W.Hq,
            W.Hkv, B * nb, page_size, nb, W.D, W.scale, kv.data_ptr(), ws.data_ptr(), ws.numel(), ea.MIATTN_BF16)

    def step():
        ea.attn_decode_paged(*args, torch.cuda.current_stream().cuda_stream)

    return dict(w=w, W=W, step=step, bytes=decode_bytes(W, w["lens"]), keep=(q, kp, vp, bt, kv, o, lse, ws),
                out=(o, lse))


def check_graph_replay(torch, runner, step, out):
    """Graph replays must reproduce an eager call bit for bit."""
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in out]
    for _ in range(2):
        for t in out:
            t.fill_(0)
        runner.g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            if not torch.equal(a, b):
                raise RuntimeError("graph replay differs from the eager call")


def cpu_baseline_prefill(name, budget_s):
    import oracle
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make(name, device="cpu")
    W = w["workload"]
    q, k, v = w["q"], w["k"], w["v"]
    G = W.Hq // W.Hkv
    done_flops, heads = 0, 0
    t0 = time.perf_counter()
    for b in range(W.B):
        for h in range(W.Hq):
            lens = None if w["lens"] is None else w["lens"][b:b + 1]
            qh, kh, vh = q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1], v[b:b + 1, h // G:h // G + 1]
            if W.dtype == "e4m3":
                oracle.attention_fp8(qh, kh, vh, *w["fp8_scales"], W.scale, W.causal, lens)
            else:
                oracle.attention(qh, kh, vh, W.scale, W.causal, lens)
            done_flops += 4 * W.D * prefill_pairs(1, 1, W.Tq, W.Tk, W.causal, lens)
            heads += 1
            if time.perf_counter() - t0 > budget_s:
                break
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=done_flops / dt / 1e12, unit="TFLOP/s", cores=blas_threads(), kind="oracle",
                sample=f"{heads} of {W.B * W.Hq} (batch, head) pairs of the {W.name} workload, float64 numpy, "
                       f"{dt:.1f} s")


def cpu_baseline_decode(dec, budget_s):
    import oracle

    w, W = dec["w"], dec["W"]
    lens = w["lens"]
    qc = w["q"].cpu()
    fp8 = W.dtype == "e4m3"
    elem = 1 if fp8 else 2
    done, nb = 0, 0
    t0 = time.perf_counter()
    for b in range(W.B):
        if fp8:
            # the oracle decodes only the rows it reads, from the device cache
            kb, vb = w["k"][b:b + 1].cpu(), w["v"][b:b + 1].cpu()
            oracle.decode_fp8(qc[b:b + 1], kb, vb, lens[b:b + 1], *w["fp8_scales"], W.scale)
        else:
            oracle.decode(qc, w["k"], w["v"], lens, W.scale, batches=[b])
        done += 2 * W.Hkv * W.D * elem * int(lens[b]) + W.Hq * W.D * (elem + 2) + W.Hq * 4 + 4
        nb += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return dict(value=done / dt / 1e9, unit="GB/s", cores=blas_threads(), kind="oracle",
                sample=f"{nb} of {W.B} sequences of the {W.name} workload (cache slabs upcast to float64), "
                       f"{dt:.1f} s")


def sources_hash(kernel):
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        entry = json.load(fh).get(f"{kernel}/{workload}")
    if not entry or entry.get("sources_sha256_16") != sources_hash(kernel):
        return None
    return entry["traffic_bytes_per_launch"]


def mfma_busy_for(kernel, workload):
    """Fraction of the chip's SIMD cycles whose matrix unit was busy during
    the kernel, from the committed counter summary, or None when there is
    none or the kernel's sources changed since it was taken."""
    path = os.path.join(PROFILES, "mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        entry = json.load(fh).get(f"{kernel}/{workload}")
    if not entry or entry.get("sources_sha256_16") != sources_hash(kernel):
        return None
    return round(entry["mfma_busy"], 4)


def summarize_mfma(kernel, workload, pmc_dir, command):
    """Turn one rocprofv3 --pmc run of MFMA_COUNTERS into an entry of
    profiles/mfma.json: per dispatch of `kernel` (averaged), the cycles in
    which the shader engines held waves (SQ_BUSY_CYCLES / engines), the
    matrix units' busy fraction SQ_VALU_MFMA_BUSY_CYCLES / (those cycles x
    SIMDs), the MFMA flops the instructions performed (MOPS x 512) against
    the algorithmic flops, the share of MFMA-busy cycles in which a VALU
    instruction also issued, and the clock implied by those cycles over the
    dispatch's duration (the profiled run's own clock).  GRBM_GUI_ACTIVE is
    kept for reference: on dispatches of a few microseconds it also counts
    cycles outside the kernel's timestamps."""
    rows = {}
    durs = []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if kernel not in r["Kernel_Name"]:
                    continue
                rows.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                if r["Counter_Name"] == "SQ_BUSY_CYCLES":
                    durs.append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9)
    missing = [c for c in MFMA_COUNTERS if c not in rows]
    if missing:
        raise SystemExit(f"no rows for {missing} of {kernel} under {pmc_dir}")
    mean = {c: sum(v) / len(v) for c, v in rows.items()}
    cycles = mean["SQ_BUSY_CYCLES"] / N_SE
    from exact_tiled_attention_13_amd import workloads as wl

    W = wl.WORKLOADS[workload]
    lens = None
    if W.lens is not None:
        lens = wl.draw_lengths(W.B, W.lens[0], W.lens[1], W.lens[2], 0)
    f_alg = 4 * W.D * prefill_pairs(W.B, W.Hq, W.Tq, W.Tk, W.causal, lens)
    mops = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] + mean["SQ_INSTS_VALU_MFMA_MOPS_F8"] + \
        mean["SQ_INSTS_VALU_MFMA_MOPS_F6F4"]
    dur = sum(durs) / len(durs)
    entry = dict(kernel=kernel, workload=workload, sources_sha256_16=sources_hash(kernel),
                 dispatches=len(rows["SQ_BUSY_CYCLES"]), counters_per_dispatch=mean,
                 active_cycles=cycles, mfma_busy=mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD),
                 coexec_of_busy=mean["SQ_VALU_MFMA_COEXEC_CYCLES"] / mean["SQ_VALU_MFMA_BUSY_CYCLES"],
                 mfma_flops=mops * 512, algorithmic_flops=f_alg, mfma_flops_over_algorithmic=mops * 512 / f_alg,
                 dispatch_seconds=dur, implied_clock_ghz=cycles / dur / 1e9, command=command)
    path = os.path.join(PROFILES, "mfma.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[f"{kernel}/{workload}"] = entry
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


def copy_calibration(steps):
    """A plain copy of COPY_BYTES, for scaling FETCH_SIZE / WRITE_SIZE."""
    import torch

    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").normal_()
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x {steps}")


def _pmc_rows(dirs, counter):
    out = []
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r["Counter_Name"] == counter:
                        out.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def summarize_pmc(kernel, workload, fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, command):
    """Turn four rocprofv3 --pmc runs into a traffic entry of profiles/traffic.json."""
    def mean_for(dirs, counter, sub):
        v = [x for k, x in _pmc_rows(dirs, counter) if sub in k]
        if not v:
            raise SystemExit(f"no {counter} rows for {sub} under {dirs}")
        return sum(v) / len(v), len(v)

    copy_sub = "copy"
    cf, _ = mean_for([copy_fetch_dir], "FETCH_SIZE", copy_sub)
    cw, _ = mean_for([copy_write_dir], "WRITE_SIZE", copy_sub)
    f_scale = (COPY_BYTES / 1024) / cf
    w_scale = (COPY_BYTES / 1024) / cw
    kf, nf = mean_for([fetch_dir], "FETCH_SIZE", kernel)
    kw, nw = mean_for([write_dir], "WRITE_SIZE", kernel)
    traffic = (kf * f_scale + kw * w_scale) * 1024
    entry = dict(kernel=kernel, workload=workload, sources_sha256_16=sources_hash(kernel),
                 fetch_kib_per_dispatch=kf, write_kib_per_dispatch=kw, dispatches=(nf, nw),
                 copy_fetch_kib=cf, copy_write_kib=cw, copy_bytes=COPY_BYTES,
                 fetch_scale=f_scale, write_scale=w_scale, traffic_bytes_per_launch=traffic, command=command)
    path = os.path.join(PROFILES, "traffic.json")
    data = {}
    if os.path.exists(path):
        with open(path) as fh:
            data = json.load(fh)
    data[f"{kernel}/{workload}"] = entry
    with open(path, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
    print(json.dumps(entry, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="causal",
                    choices=["causal", "long", "ragged", "decode", "decode-paged", "decode-fp8", "causal-fp8",
                             "long-fp8", "single"])
    ap.add_argument("--page-size", type=int, default=16, help="page size of --workload decode-paged")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode measurements of the default run")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradients (attn_bwd) of the prefill workload instead of its forward")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward measurement of the default run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle time per baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB copy (for scaling the FETCH_SIZE/WRITE_SIZE counters)")
    ap.add_argument("--summarize-pmc", nargs=5, metavar=("KERNEL", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                         "COPY_WRITE_DIR"),
                    help="write profiles/traffic.json from rocprofv3 --pmc output directories")
    ap.add_argument("--pmc-command", default="", help="command line recorded with --summarize-pmc")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("KERNEL", "PMC_DIR"),
                    help="write profiles/mfma.json from a rocprofv3 --pmc run of MFMA_COUNTERS")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma[0], args.workload, args.summarize_mfma[1], args.pmc_command)
        return
    if args.summarize_pmc:
        k, fd, wd, cfd, cwd = args.summarize_pmc
        summarize_pmc(k, args.workload, fd, wd, cfd, cwd, args.pmc_command)
        return
    if args.copy_calibration:
        copy_calibration(max(1, args.steps))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_tiled_attention_13_amd as ea

    ea.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    launch_table = f"{ea.attn_tile_table_size()} tuned entries" if ea.attn_tile_table_size() else "built-in rule"
    torch.cuda.set_device(0)

    line = {}
    if args.workload in ("decode", "decode-paged", "decode-fp8"):
        paged = args.workload == "decode-paged"
        fp8 = args.workload == "decode-fp8"
        dec = (setup_decode_paged(torch, args.page_size) if paged else
               setup_decode_fp8(torch) if fp8 else setup_decode(torch))
        runner = Graphed(torch, dec["step"])
        check_graph_replay(torch, runner, dec["step"], dec["out"])
        ms, wall_ms, n = time_steps(torch, runner, args.steps, args.warmup)
        gbs = dec["bytes"] / (ms * 1e-3) / 1e9
        W = dec["W"]
        note = W.note + (f", paged cache (page size {args.page_size}, pages placed at random)" if paged else "")
        line = dict(metric="decode KV GB/s (% HBM peak)", value=round(gbs, 2), unit="GB/s", n_gpus=1, steps=n,
                    warmup=args.warmup, ms_per_step=round(wall_ms, 5), higher_is_better=True, scaling="weak",
                    vs_baseline=None, dtype="e4m3" if fp8 else "bf16", data="synthetic",
                    config=dict(workload=note, B=W.B, Hq=W.Hq, Hkv=W.Hkv, S_max=W.Tk, D=W.D,
                                sum_lengths=int(np.sum(dec["w"]["lens"])), parallelism="single GPU",
                                launch_table=launch_table),
                    roofline=dict(bound="hbm", achieved=round(gbs, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                                  frac=round(gbs / PEAK_HBM_GBS, 4),
                                  traffic=None if paged else traffic_for("decode_split_kernel", args.workload),
                                  kernels="decode_split + decode_merge"))
        if not args.no_cpu_baseline and not paged:
            line["cpu_baseline"] = cpu_baseline_decode(dec, args.cpu_budget)
        print(json.dumps(line), flush=True)
        return

    if args.backward:
        bw = setup_backward(torch, args.workload)
        runner = Graphed(torch, bw["step"])
        check_graph_replay(torch, runner, bw["step"], bw["out"])
        ms, wall_ms, n = time_steps(torch, runner, args.steps, args.warmup)
        W = bw["W"]
        tflops = bw["flops"] / (ms * 1e-3) / 1e12
        line = dict(metric="prefill backward TFLOP/s (% bf16 MFMA peak)", value=round(tflops, 3), unit="TFLOP/s",
                    n_gpus=1, steps=n, warmup=args.warmup, ms_per_step=round(wall_ms, 5), higher_is_better=True,
                    scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
                    config=dict(workload=W.note + " (gradients)", B=W.B, Hq=W.Hq, Hkv=W.Hkv, Tq=W.Tq, Tk=W.Tk,
                                D=W.D, causal=W.causal, flops_per_step=bw["flops"], parallelism="single GPU"),
                    roofline=dict(bound="mfma", achieved=round(tflops, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                                  frac=round(tflops / PEAK_BF16_TFLOPS, 4), traffic=None,
                                  kernels="bwd_prep + bwd_dq + bwd_dkdv", kernel_ms=round(ms, 5)))
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_backward(args.workload, args.cpu_budget)
        print(json.dumps(line), flush=True)
        return

    pre = setup_prefill(torch, args.workload)
    runner = Graphed(torch, pre["step"])
    check_graph_replay(torch, runner, pre["step"], pre["out"])
    ms, wall_ms, n = time_steps(torch, runner, args.steps, args.warmup)
    W = pre["W"]
    kname = "fwd_f32_kernel" if W.dtype == "f32" else "fwd_bf16_kernel"
    tflops = pre["flops"] / (ms * 1e-3) / 1e12
    peak = {"bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_MFMA_TFLOPS, "e4m3": PEAK_FP8_BF16_TFLOPS}[W.dtype]
    line = dict(
        metric="prefill attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)",
        value=round(tflops, 3), unit="TFLOP/s", n_gpus=1, steps=n, warmup=args.warmup,
        ms_per_step=round(wall_ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype=W.dtype, data="synthetic",
        config=dict(workload=W.note, B=W.B, Hq=W.Hq, Hkv=W.Hkv, Tq=W.Tq, Tk=W.Tk, D=W.D, causal=W.causal,
                    flops_per_step=pre["flops"], parallelism="single GPU", launch_table=launch_table),
        roofline=dict(bound="mfma", achieved=round(tflops, 3), peak=peak, unit="TFLOP/s",
                      frac=round(tflops / peak, 4), traffic=traffic_for(kname, args.workload), kernel=kname,
                      kernel_ms=round(ms, 5), mfma_busy=mfma_busy_for(kname, args.workload)),
    )
    del pre, runner
    if args.workload == "causal" and not args.no_decode:
        torch.cuda.empty_cache()
        dec = setup_decode(torch)
        drun = Graphed(torch, dec["step"])
        check_graph_replay(torch, drun, dec["step"], dec["out"])
        dms, dwall, dn = time_steps(torch, drun, max(20, args.steps // 4), max(5, args.warmup // 4))
        gbs = dec["bytes"] / (dms * 1e-3) / 1e9
        DW = dec["W"]
        line["decode"] = dict(workload=DW.note, value=round(gbs, 2), unit="GB/s", steps=dn, ms_per_step=round(dms, 5),
                              bytes_per_step=dec["bytes"], sum_lengths=int(np.sum(dec["w"]["lens"])),
                              roofline=dict(bound="hbm", achieved=round(gbs, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                                            frac=round(gbs / PEAK_HBM_GBS, 4),
                                            traffic=traffic_for("decode_split_kernel", "decode"),
                                            kernels="decode_split + decode_merge"))
        if not args.no_cpu_baseline:
            line["decode"]["cpu_baseline"] = cpu_baseline_decode(dec, args.cpu_budget / 2)
        del dec, drun
        torch.cuda.empty_cache()
        dec = setup_decode_fp8(torch)
        drun = Graphed(torch, dec["step"])
        check_graph_replay(torch, drun, dec["step"], dec["out"])
        dms, dwall, dn = time_steps(torch, drun, max(20, args.steps // 4), max(5, args.warmup // 4))
        gbs = dec["bytes"] / (dms * 1e-3) / 1e9
        DW = dec["W"]
        line["decode_fp8"] = dict(workload=DW.note, value=round(gbs, 2), unit="GB/s", steps=dn,
                                  ms_per_step=round(dms, 5), bytes_per_step=dec["bytes"],
                                  sum_lengths=int(np.sum(dec["w"]["lens"])), dtype="e4m3",
                                  roofline=dict(bound="hbm", achieved=round(gbs, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                                                frac=round(gbs / PEAK_HBM_GBS, 4),
                                                traffic=traffic_for("decode_split_kernel", "decode-fp8"),
                                                kernels="decode_split + decode_merge"))
        del dec, drun
    if args.workload == "causal" and not args.no_decode:
        # the same causal prefill on E4M3 inputs
        torch.cuda.empty_cache()
        pf = setup_prefill(torch, "causal-fp8")
        prun = Graphed(torch, pf["step"])
        check_graph_replay(torch, prun, pf["step"], pf["out"])
        pms, pwall, pn = time_steps(torch, prun, max(20, args.steps // 4), max(5, args.warmup // 4))
        ptf = pf["flops"] / (pms * 1e-3) / 1e12
        line["prefill_fp8"] = dict(workload=pf["W"].note, value=round(ptf, 3), unit="TFLOP/s", steps=pn,
                                   ms_per_step=round(pms, 5), flops_per_step=pf["flops"], dtype="e4m3",
                                   roofline=dict(bound="mfma", achieved=round(ptf, 3),
                                                 peak=round(PEAK_FP8_BF16_TFLOPS, 1), unit="TFLOP/s",
                                                 frac=round(ptf / PEAK_FP8_BF16_TFLOPS, 4),
                                                 traffic=traffic_for("fwd_bf16_kernel", "causal-fp8"),
                                                 mfma_busy=mfma_busy_for("fwd_bf16_kernel", "causal-fp8"),
                                                 kernel="fwd_bf16_kernel (E4M3 instance)",
                                                 peak_note="Q K^T on fp8 (5033 TFLOP/s), P V on bf16 (2517)"))
        del pf, prun
    if args.workload == "causal" and not args.no_backward:
        torch.cuda.empty_cache()
        bw = setup_backward(torch, "causal")
        brun = Graphed(torch, bw["step"])
        check_graph_replay(torch, brun, bw["step"], bw["out"])
        bms, bwall, bn = time_steps(torch, brun, max(20, args.steps // 4), max(5, args.warmup // 4))
        btf = bw["flops"] / (bms * 1e-3) / 1e12
        line["backward"] = dict(workload=bw["W"].note + " (gradients dQ, dK, dV)", value=round(btf, 3),
                                unit="TFLOP/s", steps=bn, ms_per_step=round(bms, 5), flops_per_step=bw["flops"],
                                roofline=dict(bound="mfma", achieved=round(btf, 3), peak=PEAK_BF16_TFLOPS,
                                              unit="TFLOP/s", frac=round(btf / PEAK_BF16_TFLOPS, 4), traffic=None,
                                              kernels="bwd_prep + bwd_dq + bwd_dkdv"))
        del bw, brun
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline_prefill(args.workload, args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
