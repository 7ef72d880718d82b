#!/usr/bin/env python3
"""Throughput of the exact-attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload long|causal|ragged|decode|decode-paged|decode-fp8|causal-fp8|long-fp8|single]
                    [--backward] [--only]

A step is one pass of the hot path over one batch of synthetic, seeded input
already resident in HBM.  The headline line is the long-context causal
prefill (B=1, H=32, T=32768, D=128, bf16), the largest prefill configuration,
in TFLOP/s of algorithmic work (4*D flops per unmasked (query, key) pair).
The same run measures, as extra keys of the line, each with its own roofline,
CPU baseline and max-abs errors against the float64 oracle on sampled rows:

  causal        causal prefill B=4 H=16 T=1024 D=64 bf16
  ragged        ragged key-padding prefill B=8 H=16 T=4096 D=128 bf16
  decode        KV-cache decode step, GQA B=64 Hq=32 Hkv=8 D=128, lengths
                1024..32768, in GB/s of algorithmic bytes (the K/V rows each
                sequence needs plus q, o, lse and lengths)
  decode_fp8    the same step on E4M3 q and caches
  prefill_fp8   the long causal prefill on E4M3 Q, K, V
  backward      gradients of the causal prefill (10*D flops per unmasked
                pair: the five products of the backward)
  backward_long gradients of the long prefill (5 steps)
  single        the fp32 single-head workload (latency-bound; information)

Steps are replayed from HIP graphs so that host launch overhead does not
enter the timing.  `value` is the step's algorithmic work over `ms_per_step`,
the wall-clock time of exactly K steps between two device synchronisations;
`roofline.achieved` is the same work over the kernel time measured with HIP
events recorded on the stream the kernels run on (`roofline.kernel_ms`).

The float64 CPU oracle is timed on a bounded sample of each workload
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
    "bwd_dq_kernel": ["bwd_bf16.hip", "device_common.h", "launch.h"],
    "bwd_dkdv": ["bwd_bf16.hip", "device_common.h", "launch.h"],   # bwd_dkdv_pair_kernel
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


def host_cores():
    """CPU cores this process may run on (the BLAS threads are reported as `cores`)."""
    try:
        return len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


class Graphed:
    """A HIP graph holding `calls` calls of fn, replayed to run steps."""

    def __init__(self, torch, fn, calls=CALLS_PER_GRAPH):
        self.torch = torch
        self.calls = calls
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()  # eager call on the capture stream before capture
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.g):
            for _ in range(calls):
                fn()
        torch.cuda.synchronize()

    def run(self, steps):
        """Replay whole graphs covering `steps` steps (at least one graph)."""
        for _ in range(max(1, -(-steps // self.calls))):
            self.g.replay()


def quiet_host(seconds=0.5):
    """Pause after host-side math (the oracle, CPU baselines, input
    generation) and before the GPU work of a measurement.  The CPU math
    libraries' worker threads keep spinning for a while after a call, and
    while they do they compete with the thread that submits each node of a
    graph replay to the GPU (HIP launches a graph's kernels from the host):
    a full run measured a 2.9 ms stall and gaps of tens of microseconds
    between the nodes of one replay of the short gradient step, whose
    kernels themselves ran at their usual durations."""
    time.sleep(seconds)


def time_steps(torch, runner, steps, warmup, fn):
    """`warmup` untimed eager calls, then exactly the steps of whole graph
    replays (a multiple of runner.calls, at least `steps`), bracketed by
    device synchronisations.  Returns (event ms per step, wall ms per step,
    steps timed): HIP events recorded on the current stream, which the
    graphs replay on, and the host clock around the synchronised region."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    reps = max(1, -(-steps // runner.calls))
    n = reps * runner.calls
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for _ in range(reps):
        runner.g.replay()
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
    and O, LSE of the forward.  The (batch, KV head) groups the error report
    checks get O and LSE from the float64 oracle (rounded as attn_fwd stores
    them), so that no input of that check comes from the HIP path; other
    heads, whose gradients are independent of them, take one attn_fwd call."""
    import oracle

    import exact_tiled_attention_13_amd as ea
    from exact_tiled_attention_13_amd import workloads

    w = workloads.make(name, device="cpu")
    W = w["workload"]
    if W.dtype != "bf16":
        raise SystemExit("the backward pass is bf16 only")
    q, k, v = (w[x].cuda() for x in ("q", "k", "v"))
    g = torch.Generator().manual_seed(1)
    do_cpu = workloads.randn_bf16(tuple(w["q"].shape), g)
    do = do_cpu.cuda()
    kv = None if w["kv_lens"] is None else w["kv_lens"].cuda()
    o, lse = ea.fwd(q, k, v, causal=W.causal, kv_lens=kv, scale=W.scale)
    G = W.Hq // W.Hkv
    groups = [(b, hk) for b in range(W.B) for hk in range(W.Hkv)]
    if W.B * W.Hq > 64:
        groups = [(0, 0), (W.B - 1, W.Hkv - 1)]
    o_ref = {}
    for b, hk in groups:
        hs = slice(hk * G, (hk + 1) * G)
        lb = None if w["lens"] is None else w["lens"][b:b + 1]
        ob, lbse = oracle.attention(w["q"][b:b + 1, hs], w["k"][b:b + 1, hk:hk + 1], w["v"][b:b + 1, hk:hk + 1],
                                    W.scale, W.causal, lb)
        o_ref[(b, hk)] = (ob[0], lbse[0])
        o[b, hs] = torch.from_numpy(ob[0]).to(torch.bfloat16).cuda()
        lse[b, hs] = torch.from_numpy(lbse[0]).to(torch.float32).cuda()
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
                out=(dq, dk, dv), do_cpu=do_cpu, groups=groups, o_ref=o_ref)


def backward_errors(bw, n_rows):
    """dQ of sampled rows and dK, dV of sampled keys of the oracle-fed
    (batch, KV head) groups, against the row and key oracles; the bar is
    max|g - g_ref| <= 2e-2 max|g_ref| per tensor."""
    import oracle
    import torch

    w, W = bw["w"], bw["W"]
    dq, dk, dv = bw["out"]
    G = W.Hq // W.Hkv
    rng = np.random.default_rng(4)
    lk, lq = oracle.valid_lengths(W.B, W.Tq, W.Tk, w["lens"])
    rows, keys = set(), set()
    per = max(1, n_rows // len(bw["groups"]))
    for b, hk in bw["groups"]:
        for _ in range(per):
            if lq[b] > 0:
                rows.add((b, hk * G + int(rng.integers(G)), int(rng.integers(lq[b]))))
            if lk[b] > 0:
                keys.add((b, hk, int(rng.integers(lk[b]))))
    rows, keys = sorted(rows), sorted(keys)
    o = np.zeros(tuple(w["q"].shape))
    lse = np.full(tuple(w["q"].shape[:3]), -np.inf)
    for (b, hk), (ob, lb) in bw["o_ref"].items():
        o[b, hk * G:(hk + 1) * G], lse[b, hk * G:(hk + 1) * G] = ob, lb
    q, k, v, do = w["q"], w["k"], w["v"], bw["do_cpu"]
    ref_q = oracle.backward_rows(q, k, v, do, rows, W.scale, W.causal, w["lens"])
    ref_k, ref_v = oracle.backward_key_rows(q, k, v, do, o, lse, keys, W.scale, W.causal, w["lens"])
    out = dict(checked=f"{len(rows)} dQ rows, {len(keys)} dK/dV keys of (batch, KV head) groups {bw['groups'][:4]}"
                       f"{'...' if len(bw['groups']) > 4 else ''}", rel_tol=2e-2)
    ok = True
    for nm, g, idx, ref in (("dq", dq, rows, ref_q), ("dk", dk, keys, ref_k), ("dv", dv, keys, ref_v)):
        got = g[tuple(torch.as_tensor(a, device=g.device) for a in np.array(idx).T)].float().cpu().double().numpy()
        err = float(np.abs(got - ref).max())
        scale = float(np.abs(ref).max())
        out[f"max_abs_{nm}"] = err
        out[f"max_ref_{nm}"] = scale
        ok = ok and np.isfinite(got).all() and err <= 2e-2 * scale + 1e-6
    out["within_tolerance"] = bool(ok)
    return out


def backward_traffic(workload):
    """Scaled HBM bytes per step of the two gradient kernels from the
    committed counter summary, or None (see traffic_for)."""
    total = 0.0
    for kn in ("bwd_dq_kernel", "bwd_dkdv"):
        t = traffic_for(kn, workload)
        if t is None:
            return None
        total += t
    return total


def backward_mfma_busy(workload):
    """Matrix-unit busy share of the two gradient kernels together: each
    kernel's share from the committed counter summary, weighted by its
    dispatch time there; None if either is missing or stale (see
    mfma_busy_for)."""
    path = os.path.join(PROFILES, "mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    num = den = 0.0
    for kn in ("bwd_dq_kernel", "bwd_dkdv"):
        e = data.get(f"{kn}/{workload}")
        if not e or e.get("sources_sha256_16") != sources_hash(kn):
            return None
        num += e["mfma_busy"] * e["dispatch_seconds"]
        den += e["dispatch_seconds"]
    return round(num / den, 4)


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
    return dict(value=done / dt / 1e12, unit="TFLOP/s", cores=blas_threads(),
                host_cores=host_cores(), kind="oracle",
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
                out=(o, lse), pages=(kp, vp, bt))


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
    return dict(value=done_flops / dt / 1e12, unit="TFLOP/s", cores=blas_threads(),
                host_cores=host_cores(), kind="oracle",
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
    return dict(value=done / dt / 1e9, unit="GB/s", cores=blas_threads(),
                host_cores=host_cores(), kind="oracle",
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


CONTEXT = ("The pages publish no throughput for this path; FlashAttention is said to run 2x-4x faster than "
           "naive attention kernels (Transformers in Action, section 9.4.1; hardware not stated).")
TOL = {"bf16": (2e-2, 1e-3), "e4m3": (2e-2, 1e-3), "f32": (1e-4, 1e-3)}


def sampled_rows(B, H, T, lens_q, n, seed):
    """Rows for the error report: first, last and tile-edge rows of every
    sequence (one random head each), one padding row where there is one,
    and random valid rows up to n."""
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        lq = int(lens_q[b])
        for i in (0, 127, 128, lq - 1, lq):
            if 0 <= i < T:
                rows.add((b, int(rng.integers(H)), i))
    tries = 0
    while len(rows) < n and tries < 100 * n:
        b = int(rng.integers(B))
        if lens_q[b] > 0:
            rows.add((b, int(rng.integers(H)), int(rng.integers(lens_q[b]))))
        tries += 1
    return sorted(rows)


def _errors(o_gpu, l_gpu, o_ref, l_ref, tol, what):
    o = o_gpu.float().cpu().double().numpy()
    lg = l_gpu.float().cpu().double().numpy()
    fin = np.isfinite(l_ref)
    eo = float(np.abs(o - o_ref).max()) if o.size else 0.0
    el = float(np.abs(lg[fin] - l_ref[fin]).max()) if fin.any() else 0.0
    inf_ok = bool(np.array_equal(np.isneginf(lg), np.isneginf(l_ref)))
    return dict(checked=what, max_abs_o=eo, max_abs_lse=el, neg_inf_lse_match=inf_ok, tol_o=tol[0], tol_lse=tol[1],
                within_tolerance=bool(eo <= tol[0] and el <= tol[1] and inf_ok and np.isfinite(o).all()))


def prefill_errors(pre, n_rows):
    """Max-abs O and LSE errors of the last replay's outputs against the
    float64 oracle on sampled rows (the row oracle: only those rows)."""
    import oracle

    w, W = pre["w"], pre["W"]
    o, lse = pre["out"]
    lq = [W.Tq] * W.B if w["lens"] is None else [int(min(max(x, 0), W.Tq)) if W.Tq == W.Tk else W.Tq for x in w["lens"]]
    rows = sampled_rows(W.B, W.Hq, W.Tq, lq, n_rows, 3)
    if W.dtype == "e4m3":
        o_ref, l_ref = oracle.attention_rows_fp8(w["q"], w["k"], w["v"], rows, *w["fp8_scales"], W.scale, W.causal,
                                                 w["lens"])
    else:
        o_ref, l_ref = oracle.attention_rows(w["q"], w["k"], w["v"], rows, W.scale, W.causal, w["lens"])
    import torch

    idx = tuple(torch.as_tensor(a, device=o.device) for a in np.array(rows).T)
    return _errors(o[idx], lse[idx], o_ref, l_ref, TOL[W.dtype], f"{len(rows)} sampled rows")


def decode_errors(dec, n_seq=3):
    import oracle

    w, W = dec["w"], dec["W"]
    o, lse = dec["out"]
    lens = w["lens"]
    pick = sorted({int(np.argmin(lens)), int(np.argmax(lens)), W.B // 2})[:n_seq]
    if "pages" in dec:
        kp, vp, bt = dec["pages"]
        ob, lb = oracle.decode_paged(w["q"].cpu(), kp, vp, bt.cpu(), lens, W.scale, batches=pick)
        o_ref, l_ref = ob[pick], lb[pick]
    elif W.dtype == "e4m3":
        o_ref = np.zeros((len(pick), W.Hq, W.D))
        l_ref = np.zeros((len(pick), W.Hq))
        for n, b in enumerate(pick):
            ob, lb = oracle.decode_fp8(w["q"][b:b + 1].cpu(), w["k"][b:b + 1].cpu(), w["v"][b:b + 1].cpu(),
                                       lens[b:b + 1], *w["fp8_scales"], W.scale)
            o_ref[n], l_ref[n] = ob[0], lb[0]
    else:
        ob, lb = oracle.decode(w["q"].cpu(), w["k"], w["v"], lens, W.scale, batches=pick)
        o_ref, l_ref = ob[pick], lb[pick]
    return _errors(o[pick], lse[pick], o_ref, l_ref, TOL[W.dtype], f"sequences {pick} (all query heads)")


def prefill_entry(torch, name, steps, warmup, calls, args, headline=False):
    pre = setup_prefill(torch, name)
    quiet_host()
    runner = Graphed(torch, pre["step"], calls)
    check_graph_replay(torch, runner, pre["step"], pre["out"])
    ev_ms, wall_ms, n = time_steps(torch, runner, steps, warmup, pre["step"])
    W = pre["W"]
    kname = "fwd_f32_kernel" if W.dtype == "f32" else "fwd_bf16_kernel"
    peak = {"bf16": PEAK_BF16_TFLOPS, "f32": PEAK_F32_MFMA_TFLOPS, "e4m3": PEAK_FP8_BF16_TFLOPS}[W.dtype]
    flops = pre["flops"]
    achieved = flops / (ev_ms * 1e-3) / 1e12
    e = dict(workload=W.note, value=round(flops / (wall_ms * 1e-3) / 1e12, 3), unit="TFLOP/s", steps=n,
             warmup=warmup, ms_per_step=round(wall_ms, 5), dtype=W.dtype, flops_per_step=flops,
             roofline=dict(bound="mfma", achieved=round(achieved, 3), peak=round(peak, 1), unit="TFLOP/s",
                           frac=round(achieved / peak, 4), traffic=traffic_for(kname, name),
                           mfma_busy=mfma_busy_for(kname, name), kernel=kname, kernel_ms=round(ev_ms, 5)))
    if W.dtype == "e4m3":
        e["roofline"]["peak_note"] = "Q K^T on fp8 (5033 TFLOP/s), P V on bf16 (2517)"
    if W.dtype == "f32":
        e["roofline"]["peak_note"] = "fp32 matrix peak; 33.6 Mflop per step, launch-latency bound"
    e["parity"] = prefill_errors(pre, args.check_rows)
    del runner, pre
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        e["cpu_baseline"] = cpu_baseline_prefill(name, args.cpu_budget)
    return e


def decode_entry(torch, name, steps, warmup, calls, args):
    paged = name == "decode-paged"
    dec = (setup_decode_paged(torch, args.page_size) if paged else
           setup_decode_fp8(torch) if name == "decode-fp8" else setup_decode(torch))
    quiet_host()
    runner = Graphed(torch, dec["step"], calls)
    check_graph_replay(torch, runner, dec["step"], dec["out"])
    ev_ms, wall_ms, n = time_steps(torch, runner, steps, warmup, dec["step"])
    W = dec["W"]
    achieved = dec["bytes"] / (ev_ms * 1e-3) / 1e9
    note = W.note + (f", paged cache (page size {args.page_size}, pages placed at random)" if paged else "")
    e = dict(workload=note, value=round(dec["bytes"] / (wall_ms * 1e-3) / 1e9, 2), unit="GB/s", steps=n,
             warmup=warmup, ms_per_step=round(wall_ms, 5), dtype=W.dtype, bytes_per_step=dec["bytes"],
             sum_lengths=int(np.sum(dec["w"]["lens"])),
             roofline=dict(bound="hbm", achieved=round(achieved, 2), peak=PEAK_HBM_GBS, unit="GB/s",
                           frac=round(achieved / PEAK_HBM_GBS, 4),
                           traffic=None if paged else traffic_for("decode_split_kernel", name),
                           kernels="decode_split + decode_merge", kernel_ms=round(ev_ms, 5)))
    e["parity"] = decode_errors(dec)
    if not args.no_cpu_baseline and not paged:
        e["cpu_baseline"] = cpu_baseline_decode(dec, args.cpu_budget)
    del runner, dec
    torch.cuda.empty_cache()
    return e


def backward_entry(torch, name, steps, warmup, calls, args):
    bw = setup_backward(torch, name)
    quiet_host()
    runner = Graphed(torch, bw["step"], calls)
    check_graph_replay(torch, runner, bw["step"], bw["out"])
    ev_ms, wall_ms, n = time_steps(torch, runner, steps, warmup, bw["step"])
    W = bw["W"]
    achieved = bw["flops"] / (ev_ms * 1e-3) / 1e12
    e = dict(workload=W.note + " (gradients dQ, dK, dV)", value=round(bw["flops"] / (wall_ms * 1e-3) / 1e12, 3),
             unit="TFLOP/s", steps=n, warmup=warmup, ms_per_step=round(wall_ms, 5), dtype="bf16",
             flops_per_step=bw["flops"],
             roofline=dict(bound="mfma", achieved=round(achieved, 3), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                           frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                           traffic=backward_traffic(name), mfma_busy=backward_mfma_busy(name),
                           kernels="bwd_dq + bwd_dkdv",
                           kernel_ms=round(ev_ms, 5)))
    e["parity"] = backward_errors(bw, args.check_rows)
    del runner, bw
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        e["cpu_baseline"] = cpu_baseline_backward(name, args.cpu_budget)
    return e


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long",
                    choices=["causal", "long", "ragged", "decode", "decode-paged", "decode-fp8", "causal-fp8",
                             "long-fp8", "single"])
    ap.add_argument("--only", action="store_true", help="measure only --workload (no extra keys)")
    ap.add_argument("--page-size", type=int, default=16, help="page size of --workload decode-paged")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradients (attn_bwd) of the prefill workload instead of its forward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle time per baseline")
    ap.add_argument("--check-rows", type=int, default=256, help="sampled rows for the error report")
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
    # the headline: exactly K steps of the named workload, in one graph of K calls
    K, Wm = max(1, args.steps), max(0, args.warmup)
    name = args.workload
    if args.backward:
        head = backward_entry(torch, name, K, Wm, K, args)
        metric = "prefill backward TFLOP/s (% bf16 MFMA peak)"
    elif name.startswith("decode"):
        head = decode_entry(torch, name, K, Wm, K, args)
        metric = "decode KV GB/s (% HBM peak)"
    else:
        head = prefill_entry(torch, name, K, Wm, K, args)
        metric = "prefill attn TFLOP/s (% bf16 MFMA peak); decode KV GB/s (% HBM peak)"
    from exact_tiled_attention_13_amd import workloads as wl

    # the paged decode runs the decode workload through a block table
    W = wl.WORKLOADS["decode" if name == "decode-paged" else name]
    line = dict(metric=metric, value=head["value"], unit=head["unit"], n_gpus=1, steps=head["steps"],
                warmup=head["warmup"], ms_per_step=head["ms_per_step"], higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype=head["dtype"], data="synthetic",
                config=dict(workload=head["workload"], B=W.B, Hq=W.Hq, Hkv=W.Hkv, Tq=W.Tq, Tk=W.Tk, D=W.D,
                            causal=W.causal, parallelism="single GPU", launch_table=launch_table,
                            timing="value = work per step / ms_per_step (wall clock of exactly `steps` graph-replayed "
                                   "steps between device synchronisations); roofline.achieved = work / "
                                   "roofline.kernel_ms (HIP events on the kernels' stream, same steps)"),
                roofline=head["roofline"], parity=head["parity"], context=CONTEXT)
    for key in ("flops_per_step", "bytes_per_step", "sum_lengths"):
        if key in head:
            line["config"][key] = head[key]
    if "cpu_baseline" in head:
        line["cpu_baseline"] = head["cpu_baseline"]
    if not args.only and not args.backward and name == "long":
        ex = max(20, K)
        line["causal"] = prefill_entry(torch, "causal", 10 * ex, 5, 20, args)
        line["ragged"] = prefill_entry(torch, "ragged", 2 * ex, 5, 20, args)
        line["decode"] = decode_entry(torch, "decode", ex, 5, 20, args)
        line["decode_fp8"] = decode_entry(torch, "decode-fp8", ex, 5, 20, args)
        line["prefill_fp8"] = prefill_entry(torch, "long-fp8", ex, 3, 20, args)
        line["backward"] = backward_entry(torch, "causal", 2 * ex, 5, 20, args)
        line["backward_long"] = backward_entry(torch, "long", 5, 2, 5, args)
        line["single"] = prefill_entry(torch, "single", 10 * ex, 5, 20, args)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
