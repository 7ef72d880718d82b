"""Host-side tests of the C ABI: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the GPU.

Only calls whose arguments fail validation are made here, so nothing is ever
launched (these run without a GPU)."""

import ctypes
import os
import re

import pytest

import exact_tiled_attention_13_amd as ea
from exact_tiled_attention_13_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "miattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(attn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libmiattn.so is not built; run `python -m exact_tiled_attention_13_amd.build`")
    return _lib.load()


def test_header_declares_the_abi():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_abi_version(lib):
    assert ea.attn_abi_version() == 5


def test_strerror_covers_codes(lib):
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        assert ea.attn_strerror(code)
    assert "unknown" in ea.attn_strerror(-99)


FAKE = 0x1000  # never dereferenced: every call below fails validation first
ODD = 0x1002   # 2-byte aligned: fails the 16-byte rule (and the 4-byte one)
ODD4 = 0x1004  # 4-byte aligned: passes the 4-byte rule, fails the 16-byte one


@pytest.mark.parametrize("args,code", [
    # q, k, v, o null
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1),
    # sizes
    (dict(B=0), -2), (dict(Hq=0), -2), (dict(Hkv=0), -2), (dict(Tq=0), -2), (dict(Tk=-1), -2),
    (dict(Hq=6, Hkv=4), -2), (dict(scale=float("nan")), -2), (dict(scale=float("inf")), -2),
    (dict(D=0), -2),
    # unsupported
    (dict(D=96), -3), (dict(D=256), -3), (dict(dtype=2), -3), (dict(causal=2), -3),
    # alignment
    (dict(q=ODD4), -6), (dict(k=ODD), -6), (dict(v=ODD4), -6), (dict(o=ODD4), -6), (dict(lse=ODD), -6),
    (dict(kv_lens=ODD), -6), (dict(lse=ODD4, kv_lens=ODD4), 0),
])
def test_fwd_validation(lib, args, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=0, B=1, Hq=2, Hkv=1, Tq=8, Tk=8, D=64, scale=0.125,
             causal=0, kv_lens=0, dtype=1, stream=0)
    a.update(args)
    if code == 0:
        # 4-byte aligned lse and kv_lens pass the checks: prove it with a shape
        # error that is only reported after the alignment checks
        a.update(B=0)
        code = -2
    assert ea.attn_fwd(**a, check=False) == code
    with pytest.raises(ea.MiattnError) as e:
        ea.attn_fwd(**a)
    assert e.value.code == code



@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(k=0), -1), (dict(v=0), -1), (dict(o=0), -1),
    (dict(B=0), -2), (dict(Tq=0), -2), (dict(Hq=6, Hkv=4), -2), (dict(scale=float("nan")), -2),
    (dict(q_scale=float("nan")), -2), (dict(v_scale=float("inf")), -2),
    (dict(scale=1e30, q_scale=1e10, k_scale=1e10), -2),
    (dict(D=96), -3), (dict(causal=2), -3),
    (dict(q=ODD4), -6), (dict(v=ODD), -6), (dict(lse=ODD), -6),
])
def test_fwd_fp8_validation(lib, args, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=0, B=1, Hq=2, Hkv=1, Tq=8, Tk=8, D=64, scale=0.125,
             q_scale=0.01, k_scale=0.02, v_scale=0.03, causal=0, kv_lens=0, stream=0)
    a.update(args)
    assert ea.attn_fwd_fp8(**a, check=False) == code

@pytest.mark.parametrize("args,code", [
    (dict(kv_lens=0), -1), (dict(q=0), -1), (dict(k_cache=0), -1),
    (dict(S_max=0), -2), (dict(Hq=5, Hkv=2), -2), (dict(scale=float("nan")), -2),
    (dict(D=32), -3), (dict(dtype=7), -3),
    (dict(workspace=0), -4), (dict(workspace_bytes=10), -4),
    (dict(q=ODD4), -6), (dict(k_cache=ODD4), -6), (dict(v_cache=ODD), -6), (dict(o=ODD4), -6),
    (dict(lse=ODD), -6), (dict(kv_lens=ODD), -6), (dict(workspace=ODD4), -6),
])
def test_decode_validation(lib, args, code):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, S_max=100, D=128, scale=0.1,
             kv_lens=FAKE, workspace=FAKE, workspace_bytes=1 << 40, dtype=1, stream=0)
    a.update(args)
    assert ea.attn_decode(**a, check=False) == code


@pytest.mark.parametrize("args,code", [
    (dict(kv_lens=0), -1), (dict(q=0), -1), (dict(v_cache=0), -1), (dict(o=0), -1),
    (dict(q=ODD4), -6), (dict(lse=ODD), -6), (dict(kv_lens=ODD), -6),
    (dict(S_max=0), -2), (dict(Hq=5, Hkv=2), -2), (dict(scale=float("nan")), -2),
    (dict(D=32), -3), (dict(dtype=7), -3),
    # partials past the fixed scratch: 64 x 64 x 8192 splits x 130 floats
    (dict(B=64, Hq=64, Hkv=8, S_max=1 << 22), -7),
])
def test_decode_noalloc_validation(lib, args, code):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, S_max=100, D=128, scale=0.1,
             kv_lens=FAKE, dtype=1, stream=0)
    a.update(args)
    assert ea.attn_decode_noalloc(**a, check=False) == code


def test_decode_noalloc_scratch_size(lib):
    # 96 MiB: the GQA decode workload's partials (64 x 32 x 64 splits x 130 floats) fit
    assert ea.attn_decode_noalloc_max_bytes() == 96 << 20
    assert ea.attn_decode_workspace_size(64, 32, 8, 32768, 128) <= ea.attn_decode_noalloc_max_bytes()


def test_workspace_size(lib):
    # one split per 512 keys; per (sequence, query head, split): D floats + max + sum,
    # then B + 1 int32 of work bookkeeping
    assert ea.attn_decode_workspace_size(64, 32, 8, 32768, 128) == 64 * 32 * 64 * 130 * 4 + 65 * 4
    assert ea.attn_decode_workspace_size(1, 1, 1, 1, 64) == 66 * 4 + 2 * 4
    assert ea.attn_decode_workspace_size(1, 1, 1, 512, 64) == 66 * 4 + 2 * 4
    assert ea.attn_decode_workspace_size(1, 1, 1, 513, 64) == 2 * 66 * 4 + 2 * 4
    assert ea.attn_decode_workspace_size(0, 1, 1, 1, 64) == 0


@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(lse=0), -1), (dict(dout=0), -1), (dict(dq=0), -1), (dict(dv=0), -1), (dict(o=0), -1),
    (dict(B=0), -2), (dict(Hq=6, Hkv=4), -2), (dict(scale=float("nan")), -2), (dict(Tk=0), -2),
    (dict(B=65535, Hq=65535, Hkv=1, Tq=128), -2), (dict(B=65535, Hq=65535, Hkv=65535, Tk=128), -2),
    (dict(D=96), -3), (dict(dtype=0), -3), (dict(causal=3), -3),
    (dict(workspace=0), -4), (dict(workspace_bytes=10), -4),
    (dict(q=ODD4), -6), (dict(dout=ODD4), -6), (dict(dq=ODD4), -6), (dict(dk=ODD), -6), (dict(dv=ODD4), -6),
    (dict(lse=ODD), -6), (dict(kv_lens=ODD), -6), (dict(workspace=ODD4), -6), (dict(o=ODD4), -6),
])
def test_bwd_validation(lib, args, code):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, dout=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1, Hq=2, Hkv=1,
             Tq=8, Tk=8, D=64, scale=0.125, causal=0, kv_lens=0, workspace=FAKE, workspace_bytes=1 << 40,
             dtype=1, stream=0)
    a.update(args)
    assert ea.attn_bwd(**a, check=False) == code


@pytest.mark.parametrize("args,code", [
    (dict(block_table=0), -1), (dict(k_pages=0), -1), (dict(kv_lens=0), -1),
    (dict(num_pages=0), -2), (dict(max_blocks=0), -2), (dict(Hq=5, Hkv=2), -2),
    (dict(page_size=12), -3), (dict(page_size=4), -3), (dict(page_size=1 << 17), -3), (dict(dtype=0), -3),
    (dict(D=32), -3), (dict(workspace=0), -4), (dict(workspace_bytes=10), -4),
    (dict(k_pages=ODD4), -6), (dict(block_table=ODD), -6), (dict(workspace=ODD4), -6),
])
def test_decode_paged_validation(lib, args, code):
    a = dict(q=FAKE, k_pages=FAKE, v_pages=FAKE, block_table=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, num_pages=10,
             page_size=16, max_blocks=4, D=128, scale=0.1, kv_lens=FAKE, workspace=FAKE, workspace_bytes=1 << 40,
             dtype=1, stream=0)
    a.update(args)
    assert ea.attn_decode_paged(**a, check=False) == code



@pytest.mark.parametrize("args,code", [
    (dict(q=0), -1), (dict(k_cache=0), -1), (dict(v_cache=0), -1), (dict(o=0), -1), (dict(kv_lens=0), -1),
    (dict(B=0), -2), (dict(S_max=0), -2), (dict(Hq=5, Hkv=2), -2), (dict(scale=float("nan")), -2),
    (dict(q_scale=float("inf")), -2), (dict(k_scale=float("nan")), -2), (dict(v_scale=float("inf")), -2),
    (dict(scale=1e30, q_scale=1e10, k_scale=1e10), -2),          # the score factor overflows float32
    (dict(D=32), -3), (dict(workspace=0), -4), (dict(workspace_bytes=10), -4),
    (dict(q=ODD4), -6), (dict(v_cache=ODD4), -6),
])
def test_decode_fp8_validation(lib, args, code):
    a = dict(q=FAKE, k_cache=FAKE, v_cache=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, S_max=100, D=128, scale=0.1,
             q_scale=0.01, k_scale=0.02, v_scale=0.03, kv_lens=FAKE, workspace=FAKE, workspace_bytes=1 << 40,
             stream=0)
    a.update(args)
    assert ea.attn_decode_fp8(**a, check=False) == code


@pytest.mark.parametrize("args,code", [
    (dict(block_table=0), -1), (dict(v_pages=0), -1), (dict(kv_lens=0), -1),
    (dict(num_pages=0), -2), (dict(max_blocks=0), -2), (dict(q_scale=float("nan")), -2),
    (dict(page_size=12), -3), (dict(page_size=4), -3), (dict(D=96), -3),
    (dict(workspace=0), -4), (dict(workspace_bytes=10), -4),
    (dict(v_pages=ODD4), -6), (dict(block_table=ODD), -6),
])
def test_decode_paged_fp8_validation(lib, args, code):
    a = dict(q=FAKE, k_pages=FAKE, v_pages=FAKE, block_table=FAKE, o=FAKE, lse=0, B=2, Hq=8, Hkv=2, num_pages=10,
             page_size=16, max_blocks=4, D=128, scale=0.1, q_scale=0.01, k_scale=0.02, v_scale=0.03,
             kv_lens=FAKE, workspace=FAKE, workspace_bytes=1 << 40, stream=0)
    a.update(args)
    assert ea.attn_decode_paged_fp8(**a, check=False) == code

def test_bwd_workspace_size(lib):
    assert ea.attn_bwd_workspace_size(4, 16, 1024) == 8 * 4 * 16 * 1024
    assert ea.attn_bwd_workspace_size(0, 16, 1024) == 0


def test_python_wrappers_reject_bad_tensors():
    import torch

    q = torch.zeros(1, 2, 4, 64)
    with pytest.raises(ValueError):
        ea.fwd(q, q, q)  # CPU tensors are refused before any library call
    with pytest.raises(ValueError):
        ea.fwd(q.half(), q.half(), q.half())

    with pytest.raises(ValueError):
        ea.decode_fp8(q[:, :, 0], q, q, None, q_scale=1.0, k_scale=1.0, v_scale=1.0)   # not E4M3


# ---------------------------------------------------------------- wrapper checks (no GPU needed)
def test_check_tensor_rejections():
    import torch

    dev = torch.device("cpu")
    t = torch.zeros(2, 3, 4, 64, dtype=torch.bfloat16)
    ea._check_tensor("t", t, 4, torch.bfloat16, dev, shape=(2, 3, 4, 64))
    with pytest.raises(ValueError, match="dims"):
        ea._check_tensor("t", t[0], 4, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="shape"):
        ea._check_tensor("t", t, 4, torch.bfloat16, dev, shape=(2, 3, 4, 128))     # undersized out buffer
    with pytest.raises(ValueError, match="must be torch.float32"):
        ea._check_tensor("t", t, 4, torch.float32, dev)                             # wrong dtype
    with pytest.raises(ValueError, match="device"):
        ea._check_tensor("t", t, 4, torch.bfloat16, torch.device("meta"))           # other device
    with pytest.raises(ValueError, match="contiguous"):
        ea._check_tensor("t", t.transpose(2, 3), 4, torch.bfloat16, dev)
    flat = torch.zeros(2 * 3 * 4 * 64 + 8, dtype=torch.bfloat16)
    view = flat[1:1 + 2 * 3 * 4 * 64].view(2, 3, 4, 64)                            # 2-byte aligned view
    with pytest.raises(ValueError, match="16-byte"):
        ea._check_tensor("t", view, 4, torch.bfloat16, dev)
    ea._check_tensor("t", flat[8:8 + 2 * 3 * 4 * 64].view(2, 3, 4, 64), 4, torch.bfloat16, dev)
    with pytest.raises(ValueError, match="torch.Tensor"):
        ea._check_tensor("t", [1, 2], 1, torch.bfloat16, dev)


def test_out_buffers_and_aliasing():
    import torch

    dev = torch.device("cpu")
    q = torch.zeros(1, 2, 8, 64, dtype=torch.bfloat16)
    o = ea._out("out", None, (1, 2, 8, 64), torch.bfloat16, dev)
    assert o.shape == (1, 2, 8, 64) and o.dtype == torch.bfloat16
    with pytest.raises(ValueError):
        ea._out("out", torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16), (1, 2, 8, 64), torch.bfloat16, dev)
    with pytest.raises(ValueError):
        ea._out("lse", torch.zeros(1, 2, 8, dtype=torch.bfloat16), (1, 2, 8), torch.float32, dev)
    l4 = torch.zeros(17, dtype=torch.float32)[1:].view(1, 2, 8)      # 4-byte aligned: fine for lse
    assert ea._out("lse", l4, (1, 2, 8), torch.float32, dev) is l4
    with pytest.raises(ValueError, match="overlaps"):
        ea._no_alias([("out", q)], [("q", q)])
    big = torch.zeros(2, 1, 2, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="overlaps"):
        ea._no_alias([("out", big[0]), ("lse", big.view(-1)[100:200])], [])
    ea._no_alias([("out", big[0])], [("q", big[1])])


def test_workspace_and_lens_checks():
    import torch

    dev = torch.device("cpu")
    with pytest.raises(ValueError, match="bytes"):
        ea._workspace(torch.zeros(10, dtype=torch.uint8), 100, dev)
    with pytest.raises(ValueError, match="16-byte"):
        ea._workspace(torch.zeros(200, dtype=torch.uint8)[4:], 100, dev)
    assert ea._workspace(None, 100, dev).numel() == 100
    # a list of lengths is copied to the device of q (here the CPU), not rejected
    lens = ea._lens([3, 4], 2, dev, True)
    assert lens.dtype == torch.int32 and lens.device == dev and lens.tolist() == [3, 4]
    with pytest.raises(ValueError):
        ea._lens([3, 4, 5], 2, dev, True)
    with pytest.raises(ValueError):
        ea._lens(torch.tensor([3, 4], dtype=torch.int64), 2, dev, True)
    with pytest.raises(ValueError):
        ea._lens(None, 2, dev, True)
    assert ea._lens(None, 2, dev, False) is None
