"""GPU parity of the fp16 paths (every entry point) against the fp64 oracle.

Inputs are drawn as for bf16 and rounded to fp16 (round to nearest even);
the oracle reads the same fp16 values exactly.  Bars: the 16-bit ones (the
softmax weights are rounded to fp16 before P.V, finer than bf16)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import WORKLOADS, draw_paged, draw_qkv
from parity import compare, oracle_forward_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F16 = torch.float16


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [sd.MASK_NONE, sd.MASK_CAUSAL])
def test_fp16_forward(D, mask):
    B, Hq, Hkv, S = 2, 8, 2, 333
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, F16, 41 + D + mask, DEV)
    out = sd.sdpa_forward(q, k, v, 1 / math.sqrt(D), mask)
    torch.cuda.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), 1 / math.sqrt(D), mask)
    compare(to64(out), ref, F16, "fp16 forward D=%d mask=%d" % (D, mask))


def test_fp16_forward_padded_rectangular():
    B, Hq, Hkv, Sq, Sk, D = 3, 4, 4, 200, 517, 128
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, F16, 44, DEV)
    lens = torch.tensor([517, 129, 1], dtype=torch.int32, device=DEV)
    out = sd.sdpa_forward(q, k, v, 0.1, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_KEY_PADDING, lens.cpu().numpy())
    compare(to64(out), ref, F16, "fp16 padded")


def test_fp16_constant_v_is_exact():
    # the weights are normalised by the sum of the same rounded weights, so a
    # constant V row comes back exactly (rounded to fp16)
    q, k, _ = draw_qkv(1, 2, 2, 130, 130, 64, F16, 45, DEV)
    v = torch.full_like(k, 0.7109375)  # exactly representable
    out = sd.sdpa_forward(q, k, v, 0.125, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full_like(out, 0.7109375))


@pytest.mark.parametrize("splits", [1, 7, 32])
def test_fp16_decode(splits):
    B, Hq, Hkv, Sk, D = 3, 16, 4, 2000, 128
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, F16, 46 + splits, DEV)
    lens = torch.tensor([2000, 77, 1], dtype=torch.int32, device=DEV)
    out = sd.sdpa_decode(q, k, v, 0.09, lens, splits)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 0.09, lens.cpu().numpy())
    compare(to64(out), ref, F16, "fp16 decode splits=%d" % splits)


def test_fp16_paged_attention_and_prefill():
    lens = [300, 1000, 64]
    inp = draw_paged(lens, [0, 1, 2, 1], [299, 999, 63, 500], 8, 2, 128, 16, F16, 47, DEV)
    scale = 1 / math.sqrt(128)
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                  inp["block_tables"].shape[1] * 16, 8)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.array(lens),
                            inp["query_seq"].cpu().numpy(), inp["query_pos"].cpu().numpy(), scale, True)
    compare(to64(out), ref, F16, "fp16 paged attention")
    # prefill chunks: the last 150, 130 and 64 tokens of the three sequences
    chunks = [150, 130, 64]
    nq = sum(chunks)
    inp = draw_paged(lens, [0] * nq, [0] * nq, 8, 2, 128, 32, F16, 48, DEV)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], torch.tensor(cu, device=DEV), scale, True, 150,
                                inp["block_tables"].shape[1] * 32)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu, lens)
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale, True)
    compare(to64(out), ref, F16, "fp16 paged prefill")


@pytest.mark.slow
def test_fp16_full_size_causal_prefill_whole_output():
    # the long causal prefill workload's shape and seed, in fp16, every row
    w = WORKLOADS["bf16_causal_b4_h16_s4096_d128"]
    q, k, v = draw_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, F16, w.seed, DEV)
    out = sd.sdpa_forward(q, k, v, w.scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, w.scale, O.MASK_CAUSAL)
    compare(to64(out), ref, F16, "fp16 full-size causal prefill")
