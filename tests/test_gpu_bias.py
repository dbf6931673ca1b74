"""GPU parity of the forward with a general additive mask (sdpa_forward_bias)
against the fp64 oracle (tensai guide, 'Attention の組み立て': the scaled
scores plus an arbitrary mask tensor, broadcast over size-1 axes).

The bias is drawn N(0, 4) in the input dtype, with -inf entries where a
test hides keys; the oracle reads the same 16-bit values exactly.  Bars:
tests/parity.py (the 16-bit forward bars)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_bias, draw_qkv
from parity import compare, oracle_forward_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", ["bhss", "1hss", "b1ss", "11ss"])
@pytest.mark.parametrize("mask", [0, 1, 2], ids=["none", "causal", "padding"])
def test_bias_parity(dtype, D, shape, mask):
    # grouped K/V, S = 328: five 64-key tiles plus a ragged one
    B, Hq, Hkv, S = 2, 4, 2, 328
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 600 + D + mask, DEV)
    bshape = (B if shape[0] == "b" else 1, Hq if shape[1] == "h" else 1, S, S)
    bias = draw_bias(bshape, dtype, 601 + D, DEV)
    lens = None
    if mask & sd.MASK_KEY_PADDING:
        lens = torch.tensor([328, 100], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_bias(q, k, v, bias, scale, mask, lens, lse=True)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True,
                               bias=to64(bias))
    compare(to64(out), ref, dtype, "bias %s D=%d %s mask=%d" % (dtype, D, shape, mask))
    assert np.abs(to64(lse) - rlse).max() < 1e-2


def test_minus_inf_bias_equals_the_causal_kernel():
    B, Hq, Hkv, S, D = 2, 4, 1, 256, 128
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 610, DEV)
    tri = torch.full((S, S), float("-inf"), device=DEV).triu(1).to(BF16)[None, None].contiguous()
    got = sd.sdpa_forward_bias(q, k, v, tri, 0.088)
    ref = sd.sdpa_forward(q, k, v, 0.088, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_bias_hides_keys_and_empty_rows_are_nan():
    B, Hq, Hkv, S, D = 1, 2, 2, 136, 64
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 620, DEV)
    bias = draw_bias((1, Hq, S, S), BF16, 621, DEV)
    bias[0, 0, :, 70:] = float("-inf")   # keys 70.. hidden for head 0
    bias[0, 1, 5, :] = float("-inf")     # row 5 of head 1 sees nothing
    out, lse = sd.sdpa_forward_bias(q, k, v, bias, 0.125, lse=True)
    torch.cuda.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), 0.125, bias=to64(bias))
    compare(to64(out), ref, BF16, "bias hiding")
    assert torch.isnan(out[0, 1, 5]).all() and torch.isneginf(lse[0, 1, 5])
    assert not torch.isnan(out[0, 1, :5]).any() and not torch.isnan(out[0, 1, 6:]).any()


def test_bias_full_size_whole_output():
    # the causal prefill workload (B4 H16 S4096 D128) with a per-head bias,
    # every row against the oracle
    B, H, S, D = 4, 16, 4096, 128
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 630, DEV)
    bias = draw_bias((1, H, S, S), BF16, 631, DEV)
    scale = 1 / math.sqrt(D)
    out = sd.sdpa_forward_bias(q, k, v, bias, scale, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, scale, O.MASK_CAUSAL, bias=bias)
    compare(to64(out), ref, BF16, "bias full size")
