"""GPU parity at head dims other than 64 and 128 (any multiple of 8 up to
1024 on the forward entry points, up to 512 on the ordered backward; 16-bit
inputs), against the fp64 oracle.

Up to 128 the 64- and 128-wide kernels serve these widths: rows are D wide in
memory, the chunks past D are read as zeros on chip and never stored.  Above
that, the paired-wave and 256-wide kernels (two 128-dim output slices) and the
head-dim-split kernels (waves of 128 dims whose partial scores are summed on
chip).  Bars: tests/parity.py."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_bias, draw_grad, draw_paged, draw_qkv
from parity import (backward_whole_check, compare, compare_grad, oracle_decode_whole,
                    oracle_forward_whole, to64)

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


@pytest.mark.parametrize("D", [8, 16, 24, 40, 56, 72, 80, 96, 104, 120])
@pytest.mark.parametrize("mask", [0, 1, 2], ids=["none", "causal", "padding"])
def test_forward_head_dims(D, mask):
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 700 + D + mask, DEV)
    lens = torch.tensor([200, 77], dtype=torch.int32, device=DEV) if mask == 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    compare(to64(out), ref, BF16, "forward D=%d mask=%d" % (D, mask))
    assert np.abs(to64(lse) - rlse).max() < 1e-2


def test_forward_head_dim_fp16_and_bias():
    B, Hq, Hkv, S, D = 2, 4, 4, 136, 96
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, F16, 720, DEV)
    out = sd.sdpa_forward(q, k, v, 0.1, sd.MASK_CAUSAL)
    bias = draw_bias((1, Hq, S, S), F16, 721, DEV)
    outb = sd.sdpa_forward_bias(q, k, v, bias, 0.1, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL), F16,
            "fp16 D=96")
    compare(to64(outb), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL,
                                       bias=to64(bias)), F16, "fp16 D=96 bias")


@pytest.mark.parametrize("D", [40, 80, 112])
@pytest.mark.parametrize("splits", [1, 5])
def test_decode_head_dims(D, splits):
    B, Hq, Hkv, Sk = 3, 16, 4, 1000
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 730 + D, DEV)
    lens = torch.tensor([1000, 333, 17], dtype=torch.int32, device=DEV)
    out = sd.sdpa_decode(q, k, v, 0.1, lens, splits)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 0.1, lens.cpu().numpy())
    compare(to64(out), ref, BF16, "decode D=%d splits=%d" % (D, splits))


@pytest.mark.parametrize("D", [48, 96])
def test_paged_head_dims(D):
    lens = [300, 129]
    inp = draw_paged(lens, [0, 1, 1], [299, 128, 64], 8, 2, D, 16, BF16, 740 + D, DEV)
    scale = 1 / math.sqrt(D)
    msl = inp["block_tables"].shape[1] * 16
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                  msl, 4)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.array(lens),
                            inp["query_seq"].cpu().numpy(), inp["query_pos"].cpu().numpy(), scale, True)
    compare(to64(out), ref, BF16, "paged decode D=%d" % D)
    # prefill chunks: the last 150 and 129 tokens
    chunks = [150, 129]
    cu = torch.tensor([0, 150, 279], dtype=torch.int32, device=DEV)
    qc = draw_qkv(1, 1, 1, sum(chunks), 1, 8 * D, BF16, 742 + D, DEV)[0].reshape(sum(chunks), 8, D)
    outp = sd.sdpa_paged_prefill(qc.contiguous(), inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                 inp["seq_lens"], cu, scale, True, max(chunks), msl)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
    refp = O.paged_attention(to64(qc), to64(inp["k_cache"]), to64(inp["v_cache"]),
                             inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale, True)
    compare(to64(outp), refp, BF16, "paged prefill D=%d" % D)


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [40, 96])
def test_backward_head_dims(dtype, D):
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 750 + D, DEV)
    dout = draw_grad((B, Hq, S, D), dtype, 751 + D, DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, sd.MASK_CAUSAL)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, O.MASK_CAUSAL)
    compare_grad(to64(dq), rq, dtype, "D=%d dq" % D)
    compare_grad(to64(dk), rk, dtype, "D=%d dk" % D)
    compare_grad(to64(dv), rv, dtype, "D=%d dv" % D)


def test_outputs_past_head_dim_untouched():
    # a D=72 output lives in a larger buffer: the elements after it keep their values
    B, Hq, S, D = 1, 2, 70, 72
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, BF16, 760, DEV)
    big = torch.full((B * Hq * S * D + 64,), 7.0, dtype=BF16, device=DEV)
    out = big[: B * Hq * S * D].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.12, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (big[B * Hq * S * D:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.12, O.MASK_CAUSAL), BF16, "D=72")


# ------------------------------------------------------------- wide head dims
# Above 128 the dense prefill pairs waves that split the head dim (partial
# scores summed on chip); with a bias or over pages it computes the output in
# two 128-dim slices (two workgroups per query block, each with the
# full-width scores).

@pytest.mark.parametrize("D", [136, 200, 256])
@pytest.mark.parametrize("mask", [0, 1, 3], ids=["none", "causal", "causal+padding"])
def test_forward_wide_head_dims(D, mask):
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 780 + D + mask, DEV)
    lens = torch.tensor([200, 77], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    compare(to64(out), ref, BF16, "wide forward D=%d mask=%d" % (D, mask))
    assert np.abs(to64(lse) - rlse).max() < 1e-2


def test_forward_wide_fp16_bias_and_gqa():
    B, Hq, Hkv, S, D = 2, 8, 2, 150, 256
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, F16, 790, DEV)
    out = sd.sdpa_forward(q, k, v, 0.07, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.07, O.MASK_CAUSAL), F16,
            "fp16 D=256")
    # Sk = 150 is not a multiple of 8: the bias path needs 16-byte rows, so use 152 keys
    S2 = 152
    q2, k2, v2 = draw_qkv(B, Hq, Hkv, S2, S2, D, F16, 792, DEV)
    bias = draw_bias((B, 1, S2, S2), F16, 793, DEV)
    outb = sd.sdpa_forward_bias(q2, k2, v2, bias, 0.07, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    compare(to64(outb), O.sdpa_forward(to64(q2), to64(k2), to64(v2), 0.07, O.MASK_CAUSAL,
                                       bias=to64(bias)), F16, "fp16 D=256 bias")


# Dense 16-bit forward from 129 to 256 dims (no bias) runs on paired waves:
# two waves share 32 query rows and split the head dim, adding each other's
# partial scores through LDS.

@pytest.mark.parametrize("D", [144, 168, 232, 248])
def test_forward_paired_wave_widths(D):
    B, Hq, Hkv, S = 2, 4, 1, 333
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 805 + D, DEV)
    lens = torch.tensor([333, 130], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, sd.MASK_CAUSAL | sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, O.MASK_CAUSAL | O.MASK_KEY_PADDING,
                               lens.cpu().numpy(), return_lse=True)
    compare(to64(out), ref, BF16, "paired D=%d" % D)
    assert np.abs(to64(lse) - rlse).max() < 1e-2


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("mask", [0, 2], ids=["none", "padding"])
def test_forward_paired_wave_cross_lengths(dtype, mask):
    # Sq != Sk, both ragged against the 128-row and 32-key tiles
    B, Hq, Hkv, Sq, Sk, D = 3, 4, 2, 77, 301, 256
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, 810 + mask, DEV)
    lens = torch.tensor([301, 33, 1], dtype=torch.int32, device=DEV) if mask else None
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.05, mask, lens)
    torch.cuda.synchronize()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), 0.05, mask,
                               None if lens is None else lens.cpu().numpy(), return_lse=True)
    compare(to64(out), ref, dtype, "paired cross mask=%d" % mask)
    assert np.abs(to64(lse) - rlse).max() < 1e-2


@pytest.mark.parametrize("D", [256, 200])
def test_forward_paired_wave_empty_batch(D):
    # key_lens = 0: no tile at all for that batch (no barrier either); its rows
    # are 0/0 = NaN with lse -inf, the other batches are unaffected
    B, Hq, Hkv, S = 3, 4, 2, 150
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 818 + D, DEV)
    lens = torch.tensor([150, 0, 64], dtype=torch.int32, device=DEV)
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.06, sd.MASK_CAUSAL | sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    o, l = to64(out), to64(lse)
    assert np.isnan(o[1]).all() and np.isneginf(l[1]).all()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), 0.06, O.MASK_CAUSAL | O.MASK_KEY_PADDING,
                               lens.cpu().numpy(), return_lse=True)
    compare(o[[0, 2]], ref[[0, 2]], BF16, "paired D=%d empty batch" % D)
    assert np.abs(l[[0, 2]] - rlse[[0, 2]]).max() < 1e-2


def test_forward_paired_wave_swept_grid():
    # more workgroups than the chip holds at once: the non-causal sweep order
    # over query blocks sharing one K/V head
    B, Hq, Hkv, S, D = 1, 80, 8, 512, 256
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 815, DEV)
    out = sd.sdpa_forward(q, k, v, 1 / 16, sd.MASK_NONE)
    torch.cuda.synchronize()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 1 / 16, O.MASK_NONE), BF16,
            "paired swept grid")


def test_wide_outputs_past_head_dim_untouched():
    # D=200: the second slice covers dims 128..199 only
    B, Hq, S, D = 1, 2, 70, 200
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, BF16, 794, DEV)
    big = torch.full((B * Hq * S * D + 64,), 7.0, dtype=BF16, device=DEV)
    out = big[: B * Hq * S * D].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.1, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (big[B * Hq * S * D:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL), BF16, "D=200")


def test_paged_prefill_wide_head_dim():
    D = 256
    lens = [300, 129]
    inp = draw_paged(lens, [0, 1, 1], [299, 128, 64], 8, 2, D, 16, BF16, 795, DEV)
    scale = 1 / math.sqrt(D)
    msl = inp["block_tables"].shape[1] * 16
    chunks = [150, 129]
    cu = torch.tensor([0, 150, 279], dtype=torch.int32, device=DEV)
    qc = draw_qkv(1, 1, 1, sum(chunks), 1, 8 * D, BF16, 796, DEV)[0].reshape(sum(chunks), 8, D)
    outp = sd.sdpa_paged_prefill(qc.contiguous(), inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                 inp["seq_lens"], cu, scale, True, max(chunks), msl)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
    refp = O.paged_attention(to64(qc), to64(inp["k_cache"]), to64(inp["v_cache"]),
                             inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale, True)
    compare(to64(outp), refp, BF16, "paged prefill D=256")


def test_forward_wide_full_size_whole_output():
    # the 256-wide causal prefill leg at its full size (B4 H8 S4096), every row
    B, H, S, D = 4, 8, 4096, 256
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 797, DEV)
    scale = 1 / math.sqrt(D)
    out = sd.sdpa_forward(q, k, v, scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, scale, O.MASK_CAUSAL)
    compare(to64(out), ref, BF16, "wide full size")


def test_block_wide_heads():
    # model 512 in 2 heads of 256
    from exact_scaled_dot_amd.workloads import draw_block
    from parity import compare_block
    x, wq, wk, wv, wo = draw_block(2, 100, 512, BF16, 799, DEV)
    y = sd.sdpa_block_forward(x, wq, wk, wv, wo, 2, None, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref = O.block_forward(to64(x), to64(wq), to64(wk), to64(wv), to64(wo), 2, None, O.MASK_CAUSAL)
    compare_block(to64(y), ref, BF16, "block hd=256")


@pytest.mark.parametrize("D", [200, 256])
@pytest.mark.parametrize("splits", [1, 7])
def test_decode_wide_head_dims(D, splits):
    B, Hq, Hkv, Sk = 3, 16, 4, 1000
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 802 + D, DEV)
    lens = torch.tensor([1000, 333, 17], dtype=torch.int32, device=DEV)
    out = sd.sdpa_decode(q, k, v, 0.07, lens, splits)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 0.07, lens.cpu().numpy())
    compare(to64(out), ref, BF16, "decode D=%d splits=%d" % (D, splits))


def test_paged_decode_wide_head_dim():
    D = 256
    lens = [300, 129]
    inp = draw_paged(lens, [0, 1, 1], [299, 128, 64], 8, 2, D, 16, BF16, 804, DEV)
    msl = inp["block_tables"].shape[1] * 16
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], 0.06, True,
                                  msl, 3)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.array(lens),
                            inp["query_seq"].cpu().numpy(), inp["query_pos"].cpu().numpy(), 0.06, True)
    compare(to64(out), ref, BF16, "paged decode D=256")


def test_backward_rejects_head_dims_past_its_kernels():
    # the ordered backward stops at 512, the atomic one and the one with a bias at 128
    q, k, v = draw_qkv(1, 2, 1, 64, 64, 520, BF16, 801, DEV)
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.1, 0)
    with pytest.raises(sd.SdpaError, match="up to 512"):
        sd.sdpa_backward(q, k, v, out, out, lse, 0.1, 0)
    q, k, v = draw_qkv(1, 2, 1, 64, 64, 256, BF16, 802, DEV)
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.1, 0)
    with pytest.raises(sd.SdpaError, match="up to 128"):
        sd.sdpa_backward(q, k, v, out, out, lse, 0.1, 0, atomic=True)


# ------------------------------------------------------------- fp32 head dims
F32 = torch.float32


@pytest.mark.parametrize("D", [4, 36, 96, 124])
@pytest.mark.parametrize("mask", [0, 1, 2], ids=["none", "causal", "padding"])
def test_forward_fp32_head_dims(D, mask):
    # any multiple of 4 up to 128 on the 64- and 128-wide fp32 kernel
    B, Hq, Hkv, S = 2, 4, 2, 150
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, F32, 810 + D + mask, DEV)
    lens = torch.tensor([150, 61], dtype=torch.int32, device=DEV) if mask == 2 else None
    scale = 1 / math.sqrt(D)
    out = sd.sdpa_forward(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln)
    compare(to64(out), ref, F32, "fp32 D=%d mask=%d" % (D, mask))


def test_fp32_outputs_past_head_dim_untouched():
    B, Hq, S, D = 1, 2, 70, 52
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, F32, 830, DEV)
    big = torch.full((B * Hq * S * D + 64,), 7.0, dtype=F32, device=DEV)
    out = big[: B * Hq * S * D].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.1, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (big[B * Hq * S * D:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL), F32, "fp32 D=52")


# ------------------------------------------------- head dims above 256 (to 1024)
# Above 256 the dense forward splits the head dim across the waves of a
# workgroup (4, 6 or 8 waves of 128 dims): partial scores per wave, summed in
# LDS; each wave keeps its own slice of the output.

@pytest.mark.parametrize("D", [264, 384, 520, 768, 1024])
@pytest.mark.parametrize("mask", [0, 1, 3], ids=["none", "causal", "causal+padding"])
def test_forward_headdim_split(D, mask):
    # 200 rows = 6 blocks of 32 + 8; 200 keys = 12 tiles of 16 + 8
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 900 + D + mask, DEV)
    lens = torch.tensor([200, 77], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    compare(to64(out), ref, BF16, "split forward D=%d mask=%d" % (D, mask))
    assert np.abs(to64(lse) - rlse).max() < 1e-2


def test_forward_headdim_split_fp16_bias_gqa():
    # 6 waves (D = 640), grouped K/V 8/2, a per-batch bias with -inf entries
    B, Hq, Hkv, S, D = 2, 8, 2, 152, 640
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, F16, 910, DEV)
    bias = draw_bias((B, 1, S, S), F16, 911, DEV)
    bias[0, 0, 5, 3:90] = float("-inf")
    out, lse = sd.sdpa_forward_bias(q, k, v, bias, 0.05, sd.MASK_CAUSAL, lse=True)
    torch.cuda.synchronize()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), 0.05, O.MASK_CAUSAL, bias=to64(bias),
                               return_lse=True)
    compare(to64(out), ref, F16, "fp16 D=640 bias")
    assert np.abs(to64(lse) - rlse).max() < 1e-2


def test_forward_headdim_split_rectangular_and_single_query():
    # Sq != Sk without a mask, and one query row per head (a decode-like call)
    for Sq, Sk, D in ((70, 333, 512), (1, 1000, 1024)):
        q, k, v = draw_qkv(3, 4, 1, Sq, Sk, D, BF16, 920 + Sq, DEV)
        out = sd.sdpa_forward(q, k, v, 1 / math.sqrt(D), sd.MASK_NONE)
        torch.cuda.synchronize()
        ref = O.sdpa_forward(to64(q), to64(k), to64(v), 1 / math.sqrt(D), O.MASK_NONE)
        compare(to64(out), ref, BF16, "split forward Sq=%d Sk=%d D=%d" % (Sq, Sk, D))


def test_forward_headdim_split_dead_rows():
    # a batch with no valid key: its rows are NaN with lse -inf, like the
    # narrow kernels; the other batch is unaffected
    B, Hq, S, D = 2, 2, 96, 512
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, BF16, 930, DEV)
    lens = torch.tensor([0, 50], dtype=torch.int32, device=DEV)
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.05, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), 0.05, O.MASK_KEY_PADDING,
                               lens.cpu().numpy(), return_lse=True)
    compare(to64(out), ref, BF16, "dead rows D=512")
    assert torch.isnan(out[0]).all() and torch.isneginf(lse[0]).all()
    assert np.abs(to64(lse[1]) - rlse[1]).max() < 1e-2


def test_headdim_split_outputs_past_head_dim_untouched():
    # D = 520: the fifth wave owns dims 512..639 and stores only 512..519
    B, Hq, S, D = 1, 2, 70, 520
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, BF16, 940, DEV)
    big = torch.full((B * Hq * S * D + 64,), 7.0, dtype=BF16, device=DEV)
    out = big[: B * Hq * S * D].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.1, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (big[B * Hq * S * D:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL), BF16, "D=520")


def test_forward_headdim_split_full_size_whole_output():
    # a 4096-token causal prefill with 1024-wide heads (the headline prefill's
    # token count and B*H*D); every row and its lse against the oracle
    B, H, S, D = 1, 8, 4096, 1024
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 950, DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref, rlse = oracle_forward_whole(O, q, k, v, scale, O.MASK_CAUSAL, row_block=512,
                                     return_lse=True)
    compare(to64(out), ref, BF16, "D=1024 full size")
    assert np.abs(to64(lse) - rlse).max() < 1e-2


@pytest.mark.parametrize("D", [264, 512, 1024])
@pytest.mark.parametrize("splits", [1, 5, 32])
def test_decode_headdim_split(D, splits):
    # grouped heads 16/4; key limits with an empty batch (every split empty:
    # NaN) and short ones (several empty splits)
    B, Hq, Hkv, Sk = 4, 16, 4, 1000
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 960 + D + splits, DEV)
    lens = torch.tensor([1000, 0, 333, 17], dtype=torch.int32, device=DEV)
    out = sd.sdpa_decode(q, k, v, 1 / math.sqrt(D), lens, splits)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 1 / math.sqrt(D), lens.cpu().numpy())
    compare(to64(out), ref, BF16, "split decode D=%d splits=%d" % (D, splits))
    assert torch.isnan(out[1]).all()


def test_decode_headdim_split_large_group_fp16():
    # 40 query heads per K/V head: two 32-head row blocks; fp16; no key_lens
    B, Hq, Hkv, Sk, D = 2, 80, 2, 777, 640
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, F16, 970, DEV)
    out = sd.sdpa_decode(q, k, v, 0.04, None, 7)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 0.04, None)
    compare(to64(out), ref, F16, "split decode fp16 G=40 D=640")


def test_decode_headdim_split_full_size_whole_output():
    # the 1024-wide decode leg at full size (B8, 32/8 heads, 32768 cached
    # keys, 32 splits; batch 5 padded to 20001 keys); every query head
    B, Hq, Hkv, Sk, D, splits = 8, 32, 8, 32768, 1024, 32
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 980, DEV)
    lens = torch.full((B,), Sk, dtype=torch.int32, device=DEV)
    lens[5] = 20001
    out = sd.sdpa_decode(q, k, v, 1 / math.sqrt(D), lens, splits)
    torch.cuda.synchronize()
    ref = oracle_decode_whole(O, q, k, v, 1 / math.sqrt(D), lens.cpu().numpy())
    compare(to64(out), ref, BF16, "D=1024 decode whole output")


@pytest.mark.parametrize("model,heads", [(1024, 2), (2048, 2), (1536, 3)])
def test_block_headdim_split(model, heads):
    # attention blocks whose heads are 512, 1024 and 512 wide: the projections
    # address the wide head layout, the attention runs on the head-dim-split
    # kernel
    from exact_scaled_dot_amd.workloads import draw_block
    from parity import compare_block
    x, wq, wk, wv, wo = draw_block(2, 100, model, BF16, 1000 + model + heads, DEV)
    y = sd.sdpa_block_forward(x, wq, wk, wv, wo, heads, None, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref = O.block_forward(to64(x), to64(wq), to64(wk), to64(wv), to64(wo), heads, None, O.MASK_CAUSAL)
    compare_block(to64(y), ref, BF16, "block model=%d heads=%d" % (model, heads))


def test_decode_wide_full_size_whole_output():
    # the 256-wide decode leg at its full size (B32, 32/8 heads, 32768 cached
    # keys, 32 splits; batch 17 padded to 9999 keys); every query head
    B, Hq, Hkv, Sk, D, splits = 32, 32, 8, 32768, 256, 32
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 1030, DEV)
    lens = torch.full((B,), Sk, dtype=torch.int32, device=DEV)
    lens[17] = 9999
    out = sd.sdpa_decode(q, k, v, 1 / math.sqrt(D), lens, splits)
    torch.cuda.synchronize()
    ref = oracle_decode_whole(O, q, k, v, 1 / math.sqrt(D), lens.cpu().numpy())
    compare(to64(out), ref, BF16, "D=256 decode whole output")


# ------------------------------------------------ backward above 128 (to 512)
# The head-dim-split backward: 2 or 4 waves of 128 dims per workgroup.

@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [136, 256, 384, 512])
@pytest.mark.parametrize("mask", [0, 1, 3], ids=["none", "causal", "causal+padding"])
def test_backward_headdim_split(dtype, D, mask):
    # grouped K/V 4/2; 200 rows and keys = 6 blocks of 32 + 8 (12 tiles of 16 + 8)
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 1200 + D + mask, DEV)
    dout = draw_grad((B, Hq, S, D), dtype, 1201 + D + mask, DEV)
    lens = torch.tensor([200, 77], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, mask, ln)
    what = "%s D=%d mask=%d" % (dtype, D, mask)
    compare_grad(to64(dq), rq, dtype, what + " dq")
    compare_grad(to64(dk), rk, dtype, what + " dk")
    compare_grad(to64(dv), rv, dtype, what + " dv")


def test_backward_headdim_split_rectangular_dead_rows_and_repeatable():
    # Sq != Sk, a batch with no valid key (its dQ rows are 0), keys past the
    # limit get dK = dV = 0, and a second call gives the same bits
    B, Hq, Hkv, Sq, Sk, D = 2, 2, 1, 70, 150, 320
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, BF16, 1210, DEV)
    dout = draw_grad((B, Hq, Sq, D), BF16, 1211, DEV)
    lens = torch.tensor([0, 99], dtype=torch.int32, device=DEV)
    out, lse = sd.sdpa_forward_lse(q, k, v, 0.05, sd.MASK_KEY_PADDING, lens)
    g1 = sd.sdpa_backward(q, k, v, out, dout, lse, 0.05, sd.MASK_KEY_PADDING, lens)
    g2 = sd.sdpa_backward(q, k, v, out, dout, lse, 0.05, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)
    dq, dk, dv = g1
    assert not dq[0].any() and not dk[0].any() and not dv[0].any()
    assert not dk[1, :, 99:].any() and not dv[1, :, 99:].any()
    rq, rk, rv = O.sdpa_backward(to64(q[1:]), to64(k[1:]), to64(v[1:]), to64(dout[1:]), 0.05,
                                 O.MASK_KEY_PADDING, np.array([99]))
    compare_grad(to64(dq[1:]), rq, BF16, "rect dq")
    compare_grad(to64(dk[1:]), rk, BF16, "rect dk")
    compare_grad(to64(dv[1:]), rv, BF16, "rect dv")


def test_backward_headdim_split_full_size_whole_output():
    # the 256-wide-head causal backward at its benchmarked size (B4 H8 S4096
    # D256, the same launch); every head against the oracle
    B, H, S, D = 4, 8, 4096, 256
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 1220, DEV)
    dout = draw_grad((B, H, S, D), BF16, 1221, DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, sd.MASK_CAUSAL)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    backward_whole_check(O, q, k, v, dout, scale, O.MASK_CAUSAL, (dq, dk, dv), BF16,
                         "D=256 full size")
