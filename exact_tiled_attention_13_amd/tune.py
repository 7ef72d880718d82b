"""Tuner for the launch-choice table (run on the GPU):

    python -m exact_tiled_attention_13_amd.tune [--out PATH] [--reps N]

For every (operation, dtype, D, causal, sequence-length bucket, size bucket)
it times each launch choice on a representative synthetic problem of that
bucket, with the choice forced through a one-entry table, and records the
fastest together with all timings.  The result is the JSON file ``tiles.py``
loads (by default ``tiles_gfx950.json`` next to this file).  Keys are the ones
the library computes for the call (include/miattn.h):

* prefill: T = Tk and size = ceil(Tq / 256) * B * Hq; problems with
  Tq = Tk = the bucket's representative length and Hkv = Hq;
* decode: T = S_max (every length) and size = B * ceil(S_max / 512) * Hkv *
  ceil(G / 16); problems with B = 64, Hq = 32, Hkv = 8 and every sequence at
  full length.
"""

from __future__ import annotations

import argparse
import json
import math
import statistics
import sys

import torch

from . import _lib, tiles
from . import fwd, fwd_fp8, decode, decode_fp8
from . import workloads

ALL = 2**31 - 1
# Sequence-length buckets (t_lo, t_hi, representative T), each with its size
# buckets (size_lo, size_hi, representative size).  Up to 256 the 128-row
# shape's grid (2 * size workgroups) is resident at once on 256 CUs, which
# is where zig-zag pairing can help, so that boundary is a bucket edge.
FWD_BUCKETS = [
    ((1, 2047, 1024), [(1, 63, 48), (64, 127, 96), (128, 256, 256), (257, 511, 384), (512, 1023, 768),
                       (1024, 2047, 1536), (2048, ALL, 3072)]),
    ((2048, 8191, 4096), [(1, 127, 64), (128, 256, 256), (257, 511, 384), (512, 1023, 768), (1024, 2047, 1536),
                          (2048, ALL, 3072)]),
    ((8192, ALL, 32768), [(1, 255, 128), (256, 1023, 512), (1024, 2047, 1536), (2048, ALL, 4096)]),
]
DEC_BUCKETS = [(1, 4095, 2048), (4096, 16383, 8192), (16384, ALL, 32768)]


def _time(fn, reps, calls):
    """Median over reps of the mean time (ms) of `calls` back-to-back calls."""
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(calls):
            fn()
        b.record()
        b.synchronize()
        out.append(a.elapsed_time(b) / calls)
    return statistics.median(out)


def _forced(row):
    _lib.attn_set_tile_table([row])


# a candidate replaces the built-in choice only when it is faster by more
# than this fraction (smaller differences are within run-to-run noise)
MARGIN = 0.02


def _conservative(times, builtin):
    best = min(times, key=times.get)
    if builtin in times and times[best] >= (1.0 - MARGIN) * times[builtin]:
        return builtin
    return best


def tune_fwd(dtype, D, causal, reps):
    entries = []
    for (t_lo, t_hi, T), sizes in FWD_BUCKETS:
        slots = math.ceil(T / 256)
        for lo, hi, wg in sizes:
            BH = max(1, wg // slots)
            B = math.gcd(BH, 8)
            H = BH // B
            g = torch.Generator(device="cuda").manual_seed(0)
            if dtype == "e4m3":
                q, k, v = (workloads.randn_e4m3((B, H, T, D), g, device="cuda") for _ in range(3))
                s = workloads.E4M3_SCALE
                call = lambda: fwd_fp8(q, k, v, q_scale=s, k_scale=s, v_scale=s, causal=bool(causal))  # noqa: E731
            else:
                q, k, v = (workloads.randn_bf16((B, H, T, D), g, device="cuda") for _ in range(3))
                call = lambda: fwd(q, k, v, causal=bool(causal))  # noqa: E731
            size = slots * B * H
            # zig-zag pairing is only offered where the 128-row grid is
            # resident at once (size <= 256): elsewhere it only scatters the
            # order in which K/V tiles are reused from L2 (measured: 2.3x the
            # HBM traffic of the long prefill at equal speed)
            zigs = (-1, 0, 1) if causal and size <= 256 else (-1,)
            cands = [(shape, z) for shape in (0, 1) for z in zigs]
            calls = 10 if T <= 4096 else 3
            times = {}
            for shape, zig in cands:
                _forced([tiles.OPS["fwd"], tiles.DTYPES[dtype], D, causal, 0, ALL, 0, ALL, shape, zig])
                times[f"{shape},{zig}"] = round(_time(call, reps, calls), 5)
            best = _conservative(times, f"{0 if size >= 512 else 1},-1")
            entries.append(dict(op="fwd", dtype=dtype, D=D, causal=causal, t_lo=t_lo, t_hi=t_hi, size_lo=lo,
                                size_hi=hi, choice=[int(x) for x in best.split(",")], times_ms=times,
                                problem=dict(B=B, Hq=H, Hkv=H, Tq=T, Tk=T, size=size)))
            print(f"fwd {dtype} D{D} causal{causal} T {T:5d} size {size:5d}: {times} -> {best}", flush=True)
            del q, k, v
            torch.cuda.empty_cache()
    return entries


def tune_decode(dtype, D, reps):
    entries = []
    B, Hq, Hkv = 64, 32, 8
    for lo, hi, S in DEC_BUCKETS:
        g = torch.Generator(device="cuda").manual_seed(0)
        lens = torch.full((B,), S, dtype=torch.int32, device="cuda")
        if dtype == "e4m3":
            q = workloads.randn_e4m3((B, Hq, D), g, device="cuda")
            kc = workloads.randn_e4m3((B, Hkv, S, D), g, device="cuda")
            vc = workloads.randn_e4m3((B, Hkv, S, D), g, device="cuda")
            s = workloads.E4M3_SCALE
            call = lambda: decode_fp8(q, kc, vc, lens, q_scale=s, k_scale=s, v_scale=s)  # noqa: E731
        else:
            q = workloads.randn_bf16((B, Hq, D), g, device="cuda")
            kc = workloads.randn_bf16((B, Hkv, S, D), g, device="cuda")
            vc = workloads.randn_bf16((B, Hkv, S, D), g, device="cuda")
            call = lambda: decode(q, kc, vc, lens)  # noqa: E731
        size = B * math.ceil(S / 512) * Hkv * math.ceil(Hq // Hkv / 16)
        times = {}
        for per_cu in (1, 2, 3, 4):
            _forced([tiles.OPS["decode"], tiles.DTYPES[dtype], D, 1, 0, ALL, 0, ALL, per_cu, 0])
            times[str(per_cu)] = round(_time(call, reps, 5), 5)
        best = _conservative(times, "2")
        entries.append(dict(op="decode", dtype=dtype, D=D, causal=1, t_lo=0, t_hi=ALL, size_lo=lo, size_hi=hi,
                            choice=[int(best), 0], times_ms=times,
                            problem=dict(B=B, Hq=Hq, Hkv=Hkv, S_max=S, lengths="all S_max", size=size)))
        print(f"decode {dtype} D{D} size {size:6d}: {times} -> {best}", flush=True)
        del q, kc, vc
    return entries


def merge_only(old, new, only):
    """The entries of a table re-tuned for one (op, dtype, D): `old`'s
    entries of the other keys, in their order, then `new` (whose entries
    must all carry that key).  Keys of different (op, dtype, D) never match
    the same call, so their order does not matter."""
    if any((e["op"], e["dtype"], e["D"]) != tuple(only) for e in new):
        raise ValueError(f"re-tuned entries outside {only}")
    return [e for e in old if (e["op"], e["dtype"], e["D"]) != tuple(only)] + list(new)


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", default=tiles.DEFAULT_PATH)
    ap.add_argument("--reps", type=int, default=5)
    ap.add_argument("--only", default=None, metavar="OP,DTYPE,D",
                    help="re-tune only these keys (e.g. fwd,bf16,128) and keep the other entries of --out")
    args = ap.parse_args(argv)
    if not torch.cuda.is_available():
        sys.exit("the tuner needs a GPU")
    only = None
    if args.only:
        op, dt, d = args.only.split(",")
        if op not in ("fwd", "decode") or dt not in ("bf16", "e4m3") or d not in ("64", "128"):
            sys.exit(f"--only {args.only}: expected fwd|decode,bf16|e4m3,64|128")
        only = (op, dt, int(d))
    _lib.load()
    entries = []
    try:
        for dtype in ("bf16", "e4m3"):
            for D in (64, 128):
                if only is None or only == ("fwd", dtype, D):
                    for causal in (0, 1):
                        entries += tune_fwd(dtype, D, causal, args.reps)
                if only is None or only == ("decode", dtype, D):
                    entries += tune_decode(dtype, D, args.reps)
    finally:
        _lib.attn_set_tile_table([])
    if only is not None:
        with open(args.out) as fh:
            entries = merge_only(json.load(fh)["entries"], entries, only)
    doc = dict(arch="gfx950", device=torch.cuda.get_device_name(0), fields=tiles.FIELDS,
               note="written by python -m exact_tiled_attention_13_amd.tune; times in ms per call",
               entries=entries)
    tiles.entries_from_json(doc)   # the document must load
    with open(args.out, "w") as fh:
        json.dump(doc, fh, indent=1)
    print(f"wrote {len(entries)} entries to {args.out}")


if __name__ == "__main__":
    main()
