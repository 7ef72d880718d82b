"""attn_decode_noalloc (through the C ABI) against attn_decode, the entry
point it stands in for: the same kernels on a fixed scratch array instead of
a caller workspace, so the outputs must be bit-identical.  Two calls in a
row, the second smaller, so that what the first left in the scratch cannot
leak into the second; cache rows past each length hold NaN."""

import math

import numpy as np
import pytest
import torch

import exact_tiled_attention_13_amd as ea
from exact_tiled_attention_13_amd import _lib, workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ea.load()


def inputs(B, Hq, Hkv, S, D, lens, seed):
    q, k, v = workloads.make_decode_inputs(B, Hq, Hkv, S, D, lens, seed=seed, device="cuda", poison=True)
    return q, k, v, torch.tensor(lens, dtype=torch.int32, device="cuda")


def both(q, k, v, kv, scale):
    B, Hq, D = q.shape
    Hkv, S = k.shape[1], k.shape[2]
    o_ref, l_ref = ea.decode(q, k, v, kv, scale=scale)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    _lib.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, Hq, Hkv, S,
                             D, scale, kv.data_ptr(), _lib.MIATTN_BF16, stream)
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_equals_decode_two_calls_second_smaller():
    rng = np.random.default_rng(11)
    cases = [
        (8, 32, 8, 8192, 128, [int(x) for x in rng.integers(1, 8193, 8)], 1),
        (3, 8, 2, 1000, 64, [1000, 0, 517], 2),
    ]
    for B, Hq, Hkv, S, D, lens, seed in cases:
        q, k, v, kv = inputs(B, Hq, Hkv, S, D, lens, seed)
        assert ea.attn_decode_workspace_size(B, Hq, Hkv, S, D) <= ea.attn_decode_noalloc_max_bytes()
        o, lse, o_ref, l_ref = both(q, k, v, kv, 1.0 / math.sqrt(D))
        print(f"  B{B} Hq{Hq} Hkv{Hkv} S{S} D{D} lens {lens}", flush=True)
        assert torch.equal(o, o_ref), "O differs from attn_decode"
        assert torch.equal(torch.isneginf(lse), torch.isneginf(l_ref))
        fin = torch.isfinite(l_ref)
        assert torch.equal(lse[fin], l_ref[fin]), "LSE differs from attn_decode"
        assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def test_noalloc_wrapper_and_size_limit():
    B, Hq, Hkv, S, D = 2, 4, 1, 300, 128
    q, k, v, kv = inputs(B, Hq, Hkv, S, D, [300, 7], 3)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    o2, l2 = ea.decode_noalloc(q, k, v, kv, out=out, lse=lse)
    o_ref, l_ref = ea.decode(q, k, v, kv)
    torch.cuda.synchronize()
    assert o2 is out and l2 is lse
    assert torch.equal(out, o_ref) and torch.equal(lse, l_ref)
    # a shape whose partials exceed the fixed scratch is refused before any launch
    big_S = 1 << 22
    assert ea.attn_decode_workspace_size(64, 64, 8, big_S, 128) > ea.attn_decode_noalloc_max_bytes()
    code = _lib.attn_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), 64, 64,
                                    8, big_S, 128, 0.1, kv.data_ptr(), _lib.MIATTN_BF16, 0, check=False)
    assert code == -7


def test_noalloc_under_graph_capture():
    """The callers it is for: the step captured once in a HIP graph (nothing
    allocated during capture) and replayed three times, with eager work
    between the replays (new queries and new lengths written in place, an
    eager decode with its own workspace), each replay bit-identical to that
    eager decode of the same inputs."""
    B, Hq, Hkv, S, D = 4, 16, 4, 4096, 128
    # cache rows past the longest length any replay uses hold NaN
    q, k, v, kv = inputs(B, Hq, Hkv, S, D, [4096, 4096, 4095, 4000], 5)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ea.decode_noalloc(q, k, v, kv, out=out, lse=lse)   # first call on the device: scratch address
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ea.decode_noalloc(q, k, v, kv, out=out, lse=lse)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ea.decode_noalloc(q, k, v, kv, out=out, lse=lse)
    gen = torch.Generator().manual_seed(9)
    for rep, lens in enumerate(([4096, 1, 2000, 3333], [17, 4096, 4095, 512], [2048, 2048, 1, 4000])):
        q.copy_(torch.randn(q.shape, generator=gen).to(torch.bfloat16))
        kv.copy_(torch.tensor(lens, dtype=torch.int32))
        o_ref, l_ref = ea.decode(q, k, v, kv)   # eager, own workspace
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        print(f"  replay {rep}: lens {lens}", flush=True)
        assert torch.equal(out, o_ref), f"replay {rep}: O differs from the eager decode"
        assert torch.equal(torch.isneginf(lse), torch.isneginf(l_ref))
        fin = torch.isfinite(l_ref)
        assert torch.equal(lse[fin], l_ref[fin]), f"replay {rep}: LSE differs"
