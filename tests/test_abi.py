"""The C-ABI library loads, exports what include/sdpa.h declares, and rejects
bad arguments on the host before any HIP call (no GPU needed)."""

import ctypes
import os
import re

import pytest

import exact_scaled_dot_amd as sd
from exact_scaled_dot_amd import sdpa as binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sdpa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libsdpa.so not built")

FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
FAKE_K = ctypes.c_void_p(0x20000000)
FAKE_V = ctypes.c_void_p(0x40000000)
FAKE_O = ctypes.c_void_p(0x60000000)
FAKE_W = ctypes.c_void_p(0x70000000)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sdpa_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(binding.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = sd.load_library()
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    assert sd.status_string(sd.SDPA_OK) == "ok"
    assert "invalid" in sd.status_string(sd.SDPA_ERR_INVALID_ARGUMENT)
    assert sd.status_string(99) == "unknown status"


def fwd(q=FAKE, k=FAKE_K, v=FAKE_V, B=2, Hq=4, Hkv=2, Sq=128, Sk=128, D=128, scale=0.125,
        mask=0, key_lens=None, out=FAKE_O, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    return lib.sdpa_forward(q, k, v, B, Hq, Hkv, Sq, Sk, D, scale, mask, key_lens, out, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(out=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(B=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Sk=-5), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(scale=0.0), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(scale=float("nan")), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(scale=float("inf")), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(dtype=7), sd.SDPA_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(mask=4), sd.SDPA_ERR_INVALID_ARGUMENT, "mask"),
    (dict(mask=1, Sq=64), sd.SDPA_ERR_INVALID_ARGUMENT, "Sq == Sk"),
    (dict(mask=2), sd.SDPA_ERR_INVALID_ARGUMENT, "key_lens"),
    (dict(mask=0, key_lens=ctypes.c_void_p(0x50000000)), sd.SDPA_ERR_INVALID_ARGUMENT, "key_lens"),
    (dict(out=ctypes.c_void_p(0x10000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(out=ctypes.c_void_p(0x40000000 - 2)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(B=1 << 40, Hq=1 << 20), sd.SDPA_ERR_INVALID_ARGUMENT, "overflow"),
    (dict(D=1025), sd.SDPA_ERR_UNSUPPORTED, "any width up to 1024"),
    (dict(D=1032), sd.SDPA_ERR_UNSUPPORTED, "head dim"),    # past the widest (1024) kernel
    (dict(D=1040), sd.SDPA_ERR_UNSUPPORTED, "up to 1024"),
    (dict(D=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(D=98, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),   # fp32: multiples of 4
    (dict(D=132, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),  # fp32: up to 128
    (dict(D=256, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(Sq=1 << 33, Sk=1 << 33, B=1, Hq=1, Hkv=1, D=64, out=ctypes.c_void_p(1 << 46)),
     sd.SDPA_ERR_UNSUPPORTED, "32-bit"),
    (dict(Sq=1, Sk=1 << 24, B=1, Hq=1, Hkv=1, D=64, out=ctypes.c_void_p(1 << 46)),
     sd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
])
def test_forward_rejects(kw, status, needle):
    assert fwd(**kw) == status
    assert needle in sd.last_error()


def test_key_lens_must_not_alias_out():
    st = fwd(mask=2, key_lens=ctypes.c_void_p(0x60000000 + 8))
    assert st == sd.SDPA_ERR_INVALID_ARGUMENT and "key_lens" in sd.last_error()


def dec(q=FAKE, k=FAKE_K, v=FAKE_V, B=2, Hq=8, Hkv=2, Sk=1000, D=128, scale=0.1, key_lens=None,
        splits=8, ws=FAKE_W, ws_bytes=None, out=FAKE_O, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    if ws_bytes is None:
        ws_bytes = lib.sdpa_decode_workspace_size(B, Hq, D, splits)
    return lib.sdpa_decode(q, k, v, B, Hq, Hkv, Sk, D, scale, key_lens, splits, ws, ws_bytes, out,
                           dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(v=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(splits=0), sd.SDPA_ERR_INVALID_ARGUMENT, "num_splits"),
    (dict(splits=33, ws_bytes=1 << 30), sd.SDPA_ERR_INVALID_ARGUMENT, "num_splits"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(scale=-1.0), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(ws=None), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=100), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws=ctypes.c_void_p(0x60000000 - 256)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(D=1027), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=1032), sd.SDPA_ERR_UNSUPPORTED, "up to 1024"),   # the widest decode is 1024
    (dict(D=132, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),  # fp32: up to 128
    (dict(D=66, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),   # fp32: multiples of 4
])
def test_decode_rejects(kw, status, needle):
    assert dec(**kw) == status
    assert needle in sd.last_error()


def dec_noalloc(q=FAKE, k=FAKE_K, v=FAKE_V, B=2, Hq=8, Hkv=2, Sk=1000, D=128, scale=0.125,
                key_lens=None, splits=8, out=FAKE_O, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    return lib.sdpa_decode_noalloc(q, k, v, B, Hq, Hkv, Sk, D, scale, key_lens, splits, out,
                                   dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(q=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(splits=0), sd.SDPA_ERR_INVALID_ARGUMENT, "num_splits"),
    (dict(splits=33), sd.SDPA_ERR_INVALID_ARGUMENT, "num_splits"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(out=ctypes.c_void_p(0x10000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(D=1027), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=132, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    # partials of 128 x 32 heads x 32 splits x 128 dims = 64 MiB + the lse section: one byte
    # section past the scratch, so nothing is launched
    (dict(B=128, Hq=32, Hkv=8, splits=32), sd.SDPA_ERR_WORKSPACE, "scratch"),
    (dict(B=16, Hq=32, Hkv=8, D=1024, splits=32), sd.SDPA_ERR_WORKSPACE, "scratch"),
])
def test_decode_noalloc_rejects(kw, status, needle):
    assert dec_noalloc(**kw) == status
    assert needle in sd.last_error()


def test_decode_noalloc_scratch_limit():
    lib = sd.load_library()
    assert sd.NOALLOC_SCRATCH_BYTES == 64 << 20
    # the 64-sequence, 32-head, 32-split decode of 128-dim heads fits the scratch
    assert lib.sdpa_decode_workspace_size(64, 32, 128, 32) <= sd.NOALLOC_SCRATCH_BYTES
    assert lib.sdpa_decode_workspace_size(128, 32, 128, 32) > sd.NOALLOC_SCRATCH_BYTES


def test_decode_workspace_size():
    lib = sd.load_library()

    def up(x):
        return (x + 255) // 256 * 256

    for B, Hq, D, n in [(64, 32, 128, 32), (1, 1, 64, 1), (3, 5, 64, 7)]:
        assert lib.sdpa_decode_workspace_size(B, Hq, D, n) == up(B * Hq * n * D * 4) + up(B * Hq * n * 4)
    # a partial row is D floats rounded up to 4
    for D, Dp in [(1, 4), (3, 4), (17, 20), (100, 100), (255, 256), (517, 520), (1023, 1024)]:
        assert lib.sdpa_decode_workspace_size(3, 5, D, 7) == up(3 * 5 * 7 * Dp * 4) + up(3 * 5 * 7 * 4)
    # 64 x 32 heads x 32 splits x 128 dims stays inside the 64 MiB split-workspace budget
    assert lib.sdpa_decode_workspace_size(64, 32, 128, 32) <= 64 << 20
    for bad in [(0, 1, 64, 1), (1, 1, 64, 0), (1, 1, 64, 33), (1, 0, 64, 2)]:
        assert lib.sdpa_decode_workspace_size(*bad) == 0


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sd.sdpa_forward(q, q, q, 0.125)


FAKE_T = ctypes.c_void_p(0x7a000000)
FAKE_L = ctypes.c_void_p(0x7b000000)
FAKE_S = ctypes.c_void_p(0x7c000000)
FAKE_P = ctypes.c_void_p(0x7d000000)


def paged(q=FAKE, k=FAKE_K, v=FAKE_V, nq=3, Hq=8, Hkv=2, D=128, Dv=None, pages=100, page_size=16,
          tables=FAKE_T, num_seqs=2, max_pages=50, seq_lens=FAKE_L, qseq=FAKE_S, qpos=FAKE_P,
          max_seq_len=800, scale=0.1, causal=0, splits=4, ws=FAKE_W, ws_bytes=None, out=FAKE_O,
          dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    Dv = D if Dv is None else Dv
    if ws_bytes is None:
        ws_bytes = lib.sdpa_decode_workspace_size(nq, Hq, Dv, splits)
    return lib.sdpa_paged_attention(q, k, v, nq, Hq, Hkv, D, Dv, pages, page_size, tables, num_seqs,
                                    max_pages, seq_lens, qseq, qpos, max_seq_len, scale, causal,
                                    splits, ws, ws_bytes, out, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(tables=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(qpos=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(pages=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(max_seq_len=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(scale=float("nan")), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(causal=2), sd.SDPA_ERR_INVALID_ARGUMENT, "causal"),
    (dict(splits=33, ws_bytes=1 << 30), sd.SDPA_ERR_INVALID_ARGUMENT, "num_splits"),
    (dict(max_seq_len=801), sd.SDPA_ERR_INVALID_ARGUMENT, "capacity"),
    (dict(ws=None), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=64), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(out=ctypes.c_void_p(0x7a000000 - 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(D=1100), sd.SDPA_ERR_UNSUPPORTED, "any width up to 1024"),
    (dict(D=1032), sd.SDPA_ERR_UNSUPPORTED, "up to 1024"),
    (dict(D=98, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=256, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "up to 128"),
    (dict(D=64, Dv=128, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    (dict(page_size=8, max_pages=100), sd.SDPA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(Dv=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Dv=1030), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    (dict(D=102, Dv=102, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=1032, Dv=128), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=64, Dv=1025), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    # the workspace holds Dv-wide partials: one sized for D = 128 is too small at Dv = 256
    (dict(D=128, Dv=256, ws_bytes=(3 * 8 * 4 * 128 * 4 + 255) // 256 * 256 + 256),
     sd.SDPA_ERR_WORKSPACE, "workspace"),
])
def test_paged_rejects(kw, status, needle):
    assert paged(**kw) == status
    assert needle in sd.last_error()


FAKE_C = ctypes.c_void_p(0x7e000000)


def prefill(q=FAKE, k=FAKE_K, v=FAKE_V, nq=300, Hq=8, Hkv=2, D=128, Dv=None, pages=100,
            page_size=16, tables=FAKE_T, num_seqs=3, max_pages=50, seq_lens=FAKE_L, cu=FAKE_C,
            max_q=200, max_seq_len=800, scale=0.1, causal=1, out=FAKE_O, lse=None,
            dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    Dv = D if Dv is None else Dv
    return lib.sdpa_paged_prefill(q, k, v, nq, Hq, Hkv, D, Dv, pages, page_size, tables, num_seqs,
                                  max_pages, seq_lens, cu, max_q, max_seq_len, scale, causal, out,
                                  lse, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(cu=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(seq_lens=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(max_q=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(nq=-1), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(scale=float("inf")), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(causal=-1), sd.SDPA_ERR_INVALID_ARGUMENT, "causal"),
    (dict(max_seq_len=801), sd.SDPA_ERR_INVALID_ARGUMENT, "capacity"),
    (dict(out=ctypes.c_void_p(0x7e000000 - 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(D=1032), sd.SDPA_ERR_UNSUPPORTED, "up to 1024"),
    (dict(D=136, dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "up to 128"),
    (dict(page_size=24, max_pages=40), sd.SDPA_ERR_UNSUPPORTED, "multiple of 16"),
    (dict(Dv=-3), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Dv=1100), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    (dict(D=300, Dv=1028), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    (dict(D=1030), sd.SDPA_ERR_UNSUPPORTED, "any width up to 1024"),
    (dict(D=64, Dv=2048), sd.SDPA_ERR_UNSUPPORTED, "value head dim"),
    # v_cache spans 100 * 16 * 2 * Dv * 2 bytes: 1 MB in lies inside it only at Dv = 256
    (dict(Dv=256, out=ctypes.c_void_p(0x40000000 + (1 << 20))), sd.SDPA_ERR_INVALID_ARGUMENT,
     "overlaps"),
    (dict(lse=ctypes.c_void_p(0x60000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "lse overlaps"),
])
def test_paged_prefill_rejects(kw, status, needle):
    assert prefill(**kw) == status
    assert needle in sd.last_error()


def test_dtype_codes():
    # F16 is accepted everywhere (no rejection on dtype); an unknown code is invalid
    assert fwd(dtype=3) == sd.SDPA_ERR_INVALID_ARGUMENT and "dtype" in sd.last_error()
    assert dec(dtype=3) == sd.SDPA_ERR_INVALID_ARGUMENT and "dtype" in sd.last_error()
    assert paged(dtype=3) == sd.SDPA_ERR_INVALID_ARGUMENT and "dtype" in sd.last_error()
    assert prefill(dtype=3) == sd.SDPA_ERR_INVALID_ARGUMENT and "dtype" in sd.last_error()
    assert fwd(dtype=sd.SDPA_F16, D=1025) == sd.SDPA_ERR_UNSUPPORTED  # reaches the head-dim check
    assert dec(dtype=sd.SDPA_F16, D=1025) == sd.SDPA_ERR_UNSUPPORTED


def fwd_lse(lse=ctypes.c_void_p(0x78000000), dtype=sd.SDPA_BF16, q=FAKE, out=FAKE_O, Sq=128):
    lib = sd.load_library()
    return lib.sdpa_forward_lse(q, FAKE_K, FAKE_V, 2, 4, 2, Sq, 128, 128, 0.125, 0, None, out, lse,
                                dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lse=None), sd.SDPA_ERR_INVALID_ARGUMENT, "lse"),
    (dict(q=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(lse=ctypes.c_void_p(0x60000000 + 4096)), sd.SDPA_ERR_INVALID_ARGUMENT, "lse overlaps"),
    (dict(lse=ctypes.c_void_p(0x20000000 + 16)), sd.SDPA_ERR_INVALID_ARGUMENT, "lse overlaps"),
])
def test_forward_lse_rejects(kw, status, needle):
    assert fwd_lse(**kw) == status
    assert needle in sd.last_error()


FAKE_DO = ctypes.c_void_p(0x68000000)
FAKE_L = ctypes.c_void_p(0x6c000000)
FAKE_DQ = ctypes.c_void_p(0x80000000)
FAKE_DK = ctypes.c_void_p(0x90000000)
FAKE_DV = ctypes.c_void_p(0xa0000000)
FAKE_BW = ctypes.c_void_p(0xb0000000)


def bwd(q=FAKE, out=FAKE_O, dout=FAKE_DO, lse=FAKE_L, B=2, Hq=4, Hkv=2, Sq=128, Sk=128, D=128,
        scale=0.125, mask=0, key_lens=None, dq=FAKE_DQ, dk=FAKE_DK, dv=FAKE_DV, ws=FAKE_BW,
        ws_bytes=None, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    if ws_bytes is None:
        ws_bytes = lib.sdpa_backward_workspace_size(B, Hq, Sq)
    return lib.sdpa_backward(q, FAKE_K, FAKE_V, out, dout, lse, B, Hq, Hkv, Sq, Sk, D, scale, mask,
                             key_lens, dq, dk, dv, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(dout=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(lse=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(dq=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(dtype=sd.SDPA_F32, D=132), sd.SDPA_ERR_UNSUPPORTED, "fp32: a multiple of 4 up to 128"),
    (dict(dtype=sd.SDPA_F32, D=66), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(D=520), sd.SDPA_ERR_UNSUPPORTED, "up to 512"),     # the ordered backward stops at 512
    (dict(D=516), sd.SDPA_ERR_UNSUPPORTED, "head dim"),
    (dict(mask=1, Sq=64), sd.SDPA_ERR_INVALID_ARGUMENT, "Sq == Sk"),
    (dict(mask=2), sd.SDPA_ERR_INVALID_ARGUMENT, "key_lens"),
    (dict(mask=8), sd.SDPA_ERR_INVALID_ARGUMENT, "mask"),
    (dict(ws=None), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=100), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(dk=ctypes.c_void_p(0x68000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(dv=ctypes.c_void_p(0x90000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(ws=ctypes.c_void_p(0x6c000000)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(dq=ctypes.c_void_p(0x10000 + 2)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
])
def test_backward_rejects(kw, status, needle):
    assert bwd(**kw) == status
    assert needle in sd.last_error()


def test_backward_workspace_size():
    lib = sd.load_library()
    for B, Hq, Sq in [(4, 16, 4096), (1, 1, 1), (3, 5, 333)]:
        rows = B * Hq * (Sq + (Sq & 1))
        assert lib.sdpa_backward_workspace_size(B, Hq, Sq) == (rows * 8 + 255) // 256 * 256
    for bad in [(0, 1, 1), (1, 0, 1), (1, 1, 0)]:
        assert lib.sdpa_backward_workspace_size(*bad) == 0


FAKE_B = ctypes.c_void_p(0x30000000)


def fwd_bias(bias=FAKE_B, sb=0, sh=128 * 128, Sq=128, Sk=128, dtype=sd.SDPA_BF16, out=FAKE_O,
             lse=None, mask=0, D=128):
    lib = sd.load_library()
    return lib.sdpa_forward_bias(FAKE, FAKE_K, FAKE_V, 2, 4, 2, Sq, Sk, D, 0.125, mask, None, bias,
                                 sb, sh, out, lse, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(bias=None), sd.SDPA_ERR_INVALID_ARGUMENT, "bias"),
    (dict(dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "16-bit"),
    (dict(sb=-8), sd.SDPA_ERR_INVALID_ARGUMENT, "stride"),
    (dict(Sk=100, Sq=100, sh=100 * 100), sd.SDPA_ERR_UNSUPPORTED, "aligned"),
    (dict(sh=12), sd.SDPA_ERR_UNSUPPORTED, "aligned"),
    (dict(bias=ctypes.c_void_p(0x30000000 + 8)), sd.SDPA_ERR_UNSUPPORTED, "aligned"),
    (dict(Sq=1 << 15, Sk=1 << 15, sh=0), sd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
    (dict(out=ctypes.c_void_p(0x30000000 + 4096)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(lse=ctypes.c_void_p(0x30000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps"),
    (dict(mask=1, Sq=64, sh=64 * 128), sd.SDPA_ERR_INVALID_ARGUMENT, "Sq == Sk"),
    (dict(D=100), sd.SDPA_ERR_UNSUPPORTED, "a multiple of 8"),  # the bias kernels need 8 | D
])
def test_forward_bias_rejects(kw, status, needle):
    assert fwd_bias(**kw) == status
    assert needle in sd.last_error()


def test_backward_atomic_workspace_and_rejects():
    lib = sd.load_library()
    for B, Hq, Sq, D in [(4, 16, 4096, 128), (1, 1, 1, 8), (3, 5, 333, 96)]:
        st = lib.sdpa_backward_workspace_size(B, Hq, Sq)
        assert lib.sdpa_backward_atomic_workspace_size(B, Hq, Sq, D) == \
            st + (B * Hq * Sq * D * 4 + 255) // 256 * 256
    assert lib.sdpa_backward_atomic_workspace_size(1, 1, 1, 0) == 0
    ws_small = lib.sdpa_backward_workspace_size(2, 4, 128)  # enough for the ordered one only
    st = lib.sdpa_backward_atomic(FAKE, FAKE_K, FAKE_V, FAKE_O, FAKE_DO, FAKE_L, 2, 4, 2, 128, 128,
                                  128, 0.125, 0, None, FAKE_DQ, FAKE_DK, FAKE_DV, FAKE_BW, ws_small,
                                  sd.SDPA_BF16, None)
    assert st == sd.SDPA_ERR_WORKSPACE and "workspace" in sd.last_error()
    st = lib.sdpa_backward_atomic(FAKE, FAKE_K, FAKE_V, FAKE_O, FAKE_DO, FAKE_L, 1, 1, 1, 1 << 23,
                                  128, 128, 0.125, 0, None, ctypes.c_void_p(1 << 44),
                                  ctypes.c_void_p(1 << 45), ctypes.c_void_p(1 << 46),
                                  ctypes.c_void_p(1 << 47), 1 << 40, sd.SDPA_BF16, None)
    assert st == sd.SDPA_ERR_UNSUPPORTED
    # the atomic variant keeps the 128-wide kernels
    st = lib.sdpa_backward_atomic(FAKE, FAKE_K, FAKE_V, FAKE_O, FAKE_DO, FAKE_L, 2, 4, 2, 128, 128,
                                  136, 0.125, 0, None, FAKE_DQ, FAKE_DK, FAKE_DV, FAKE_BW, 1 << 30,
                                  sd.SDPA_BF16, None)
    assert st == sd.SDPA_ERR_UNSUPPORTED and "up to 128" in sd.last_error()
    # 16-bit only
    st = lib.sdpa_backward_atomic(FAKE, FAKE_K, FAKE_V, FAKE_O, FAKE_DO, FAKE_L, 2, 4, 2, 128, 128,
                                  64, 0.125, 0, None, FAKE_DQ, FAKE_DK, FAKE_DV, FAKE_BW, 1 << 30,
                                  sd.SDPA_F32, None)
    assert st == sd.SDPA_ERR_UNSUPPORTED and "16-bit" in sd.last_error()
    # and multiples of 8 only
    st = lib.sdpa_backward_atomic(FAKE, FAKE_K, FAKE_V, FAKE_O, FAKE_DO, FAKE_L, 2, 4, 2, 128, 128,
                                  100, 0.125, 0, None, FAKE_DQ, FAKE_DK, FAKE_DV, FAKE_BW, 1 << 30,
                                  sd.SDPA_BF16, None)
    assert st == sd.SDPA_ERR_UNSUPPORTED and "a multiple of 8" in sd.last_error()


def block(x=FAKE, wq=FAKE_K, wk=FAKE_V, wv=FAKE_O, wo=FAKE_W, B=2, S=128, model=512, heads=8,
          scale=0.125, mask=0, key_lens=None, y=ctypes.c_void_p(0x78000000),
          ws=ctypes.c_void_p(0x7c000000), ws_bytes=1 << 20, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    return lib.sdpa_block_forward(x, wq, wk, wv, wo, B, S, model, heads, scale, mask, key_lens, y,
                                  ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(x=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(wo=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(B=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(heads=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "16-bit"),
    (dict(dtype=9), sd.SDPA_ERR_INVALID_ARGUMENT, "dtype"),
    (dict(model=500), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(model=8256), sd.SDPA_ERR_UNSUPPORTED, "up to 1024"),   # 1032 wide
    (dict(model=168, heads=2), sd.SDPA_ERR_UNSUPPORTED, "head dim"),   # 84 wide
    (dict(scale=float("nan")), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(mask=4), sd.SDPA_ERR_INVALID_ARGUMENT, "mask"),
    (dict(mask=sd.MASK_KEY_PADDING), sd.SDPA_ERR_INVALID_ARGUMENT, "key_lens"),
    (dict(S=1 << 20, model=2048, heads=16), sd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
    (dict(ws_bytes=(1 << 20) - 1), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws=None), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(y=ctypes.c_void_p(0x10000 + 4096)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(ws=ctypes.c_void_p(0x6ff80000)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),   # reaches wo
    (dict(y=ctypes.c_void_p(0x7c000000 + 512)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),
])
def test_block_rejects(kw, status, needle):
    assert block(**kw) == status
    assert needle in sd.last_error()


def test_block_workspace_size():
    lib = sd.load_library()
    # q, k, v and the attention output, each B*S*model 16-bit values
    assert lib.sdpa_block_workspace_size(2, 128, 512) == 4 * 2 * 128 * 512 * 2 == 1 << 20
    assert lib.sdpa_block_workspace_size(1, 3, 8) == 4 * 256
    assert lib.sdpa_block_workspace_size(0, 3, 8) == 0
    assert lib.sdpa_block_workspace_size(1, 3, -8) == 0


def bwdb(q=FAKE, out=FAKE_O, dout=FAKE_DO, lse=FAKE_L, B=2, Hq=4, Hkv=2, Sq=128, Sk=128, D=128,
         scale=0.125, mask=0, key_lens=None, bias=ctypes.c_void_p(0x7a000000), sb=0, sh=128 * 128,
         dq=ctypes.c_void_p(0x50000000), dk=ctypes.c_void_p(0x52000000),
         dv=ctypes.c_void_p(0x54000000), dbias=None, ws=ctypes.c_void_p(0x56000000),
         ws_bytes=1 << 20, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    return lib.sdpa_backward_bias(q, FAKE_K, FAKE_V, out, dout, lse, B, Hq, Hkv, Sq, Sk, D, scale,
                                  mask, key_lens, bias, sb, sh, dq, dk, dv, dbias, ws, ws_bytes,
                                  dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(bias=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null bias"),
    (dict(dout=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(dtype=sd.SDPA_F32), sd.SDPA_ERR_UNSUPPORTED, "16-bit"),
    (dict(D=136), sd.SDPA_ERR_UNSUPPORTED, "up to 128"),
    (dict(D=100), sd.SDPA_ERR_UNSUPPORTED, "a multiple of 8"),
    (dict(sb=-8), sd.SDPA_ERR_INVALID_ARGUMENT, "strides"),
    (dict(sh=12), sd.SDPA_ERR_UNSUPPORTED, "16-byte aligned"),
    (dict(Sq=120, Sk=124), sd.SDPA_ERR_UNSUPPORTED, "16-byte aligned"),
    (dict(bias=ctypes.c_void_p(0x7a000008)), sd.SDPA_ERR_UNSUPPORTED, "16-byte aligned"),
    (dict(dbias=ctypes.c_void_p(0x5a000004)), sd.SDPA_ERR_UNSUPPORTED, "dbias must be 16-byte"),
    (dict(Sq=46341, Sk=46344, ws_bytes=1 << 30), sd.SDPA_ERR_UNSUPPORTED, "2 GiB"),
    (dict(ws_bytes=16), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(dbias=ctypes.c_void_p(0x7a000000 + 4096)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),
    (dict(dq=ctypes.c_void_p(0x7a000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap"),
])
def test_backward_bias_rejects(kw, status, needle):
    assert bwdb(**kw) == status
    assert needle in sd.last_error()


FAKE_DO = ctypes.c_void_p(0x80000000)
FAKE_OUT = ctypes.c_void_p(0x90000000)
FAKE_LSE = ctypes.c_void_p(0xa0000000)
FAKE_DQ = ctypes.c_void_p(0xb0000000)
FAKE_DK = ctypes.c_void_p(0xc0000000)
FAKE_DV = ctypes.c_void_p(0xd0000000)
FAKE_PW = ctypes.c_void_p(0x100000000)


def paged_bwd(q=FAKE, k=FAKE_K, v=FAKE_V, out=FAKE_OUT, dout=FAKE_DO, lse=FAKE_LSE, nq=300, Hq=8,
              Hkv=2, D=128, Dv=None, pages=100, page_size=16, tables=FAKE_T, num_seqs=3, max_pages=50,
              seq_lens=FAKE_L, cu=FAKE_C, max_seq_len=800, scale=0.1, causal=1, dq=FAKE_DQ,
              dk=FAKE_DK, dv=FAKE_DV, ws=FAKE_PW, ws_bytes=None, dtype=sd.SDPA_BF16):
    lib = sd.load_library()
    Dv = D if Dv is None else Dv
    if ws_bytes is None:
        ws_bytes = lib.sdpa_paged_backward_workspace_size(num_seqs, Hq, Hkv, max_seq_len, D, Dv, dtype)
    return lib.sdpa_paged_backward(q, k, v, out, dout, lse, nq, Hq, Hkv, D, Dv, pages, page_size, tables,
                                   num_seqs, max_pages, seq_lens, cu, max_seq_len, scale, causal,
                                   dq, dk, dv, ws, ws_bytes, dtype, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(lse=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(dk=None), sd.SDPA_ERR_INVALID_ARGUMENT, "null"),
    (dict(num_seqs=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(Hq=6, Hkv=4), sd.SDPA_ERR_INVALID_ARGUMENT, "multiple"),
    (dict(scale=0.0), sd.SDPA_ERR_INVALID_ARGUMENT, "scale"),
    (dict(causal=3), sd.SDPA_ERR_INVALID_ARGUMENT, "causal"),
    (dict(max_seq_len=801), sd.SDPA_ERR_INVALID_ARGUMENT, "capacity"),
    (dict(ws=None), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(ws_bytes=4096), sd.SDPA_ERR_WORKSPACE, "workspace"),
    (dict(dq=ctypes.c_void_p(0x10000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlaps an input"),
    (dict(dv=ctypes.c_void_p(0xc0000000 + 64)), sd.SDPA_ERR_INVALID_ARGUMENT, "overlap each other"),
    (dict(dtype=sd.SDPA_F32, D=64, Dv=32), sd.SDPA_ERR_UNSUPPORTED, "fp32 paged backward"),
    (dict(dtype=sd.SDPA_F32, D=132, nq=30, pages=10), sd.SDPA_ERR_UNSUPPORTED, "fp32 paged backward"),
    (dict(D=520, nq=30, pages=10), sd.SDPA_ERR_UNSUPPORTED, "up to 512"),
    (dict(Dv=513, nq=30, pages=10), sd.SDPA_ERR_UNSUPPORTED, "up to 512"),
    (dict(Dv=0), sd.SDPA_ERR_INVALID_ARGUMENT, ">= 1"),
    (dict(page_size=24, max_pages=40), sd.SDPA_ERR_UNSUPPORTED, "multiple of 16"),
])
def test_paged_backward_rejects(kw, status, needle):
    assert paged_bwd(**kw) == status
    assert needle in sd.last_error()


def test_paged_backward_workspace_size():
    lib = sd.load_library()

    def up(x):
        return (x + 255) // 256 * 256

    S, Hq, Hkv, L = 3, 8, 2, 800
    stats = lib.sdpa_backward_workspace_size(S, Hq, L)
    # rows W = max(D, Dv) rounded up to 8 wide
    for D, Dv, W in [(128, 128, 128), (100, 100, 104), (64, 200, 200), (3, 1, 8), (257, 13, 264)]:
        want = 4 * up(S * Hq * L * W * 2) + 4 * up(S * Hkv * L * W * 2) + up(S * Hq * L * 4) + stats
        for dt in (sd.SDPA_BF16, sd.SDPA_F16):
            assert lib.sdpa_paged_backward_workspace_size(S, Hq, Hkv, L, D, Dv, dt) == want
    # fp32: rows D floats wide
    want = 4 * up(S * Hq * L * 100 * 4) + 4 * up(S * Hkv * L * 100 * 4) + up(S * Hq * L * 4) + stats
    assert lib.sdpa_paged_backward_workspace_size(S, Hq, Hkv, L, 100, 100, sd.SDPA_F32) == want
    assert lib.sdpa_paged_backward_workspace_size(0, Hq, Hkv, L, 128, 128, sd.SDPA_BF16) == 0
    assert lib.sdpa_paged_backward_workspace_size(S, Hq, Hkv, L, 128, 0, sd.SDPA_BF16) == 0
    assert lib.sdpa_paged_backward_workspace_size(S, Hq, Hkv, L, 128, 128, 7) == 0
