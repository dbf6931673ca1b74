"""GPU parity of the backward with an additive bias (sdpa_forward_bias +
sdpa_backward_bias) against the fp64 oracle's dQ, dK, dV and bias gradient
(dS per batch and query head).  Bars: tests/parity.py, GRAD_* (the bias
gradient is dS, rounded to the input type like the other gradients)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_bias, draw_grad, draw_qkv
from parity import backward_whole_check, compare_grad, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


def run(q, k, v, dout, bias, scale, mask, lens, want_dbias=True):
    out, lse = sd.sdpa_forward_bias(q, k, v, bias, scale, mask, lens, lse=True)
    dq, dk, dv, db = sd.sdpa_backward_bias(q, k, v, out, dout, lse, bias, scale, mask, lens,
                                           dbias=True if want_dbias else None)
    torch.cuda.synchronize()
    return dq, dk, dv, db


def check(q, k, v, dout, bias, scale, mask, lens, what):
    dq, dk, dv, db = run(q, k, v, dout, bias, scale, mask, lens)
    ln = None if lens is None else lens.cpu().numpy()
    rq, rk, rv, rb = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, mask, ln,
                                     bias=to64(bias), return_dbias=True)
    dt = q.dtype
    compare_grad(to64(dq), rq, dt, what + " dq")
    compare_grad(to64(dk), rk, dt, what + " dk")
    compare_grad(to64(dv), rv, dt, what + " dv")
    compare_grad(to64(db), rb, dt, what + " dbias")
    return dq, dk, dv, db, rb


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [0, 1, 3], ids=["none", "causal", "causal+padding"])
def test_backward_bias_parity(dtype, D, mask):
    # grouped K/V, 200 = 3 tiles of 64 + 8, a per-(batch, head) bias
    B, Hq, Hkv, S = 2, 4, 2, 200
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 1100 + D + mask, DEV)
    dout = draw_grad((B, Hq, S, D), dtype, 1101 + D + mask, DEV)
    bias = draw_bias((B, Hq, S, S), dtype, 1102 + D + mask, DEV)
    lens = torch.tensor([200, 89], dtype=torch.int32, device=DEV) if mask & 2 else None
    check(q, k, v, dout, bias, 1 / math.sqrt(D), mask, lens, "%s D=%d mask=%d" % (dtype, D, mask))


@pytest.mark.parametrize("shape", [(1, 4), (2, 1)], ids=["per-head", "per-batch"])
def test_backward_bias_broadcast(shape):
    # a broadcast bias; dbias is dS per (batch, query head), unreduced
    B, Hq, Hkv, S, D = 2, 4, 1, 136, 128
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 1110, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 1111, DEV)
    bias = draw_bias(shape + (S, S), BF16, 1112, DEV)
    check(q, k, v, dout, bias, 0.1, sd.MASK_CAUSAL, None, "broadcast %s" % (shape,))


def test_backward_bias_minus_inf_entries_and_dead_row():
    B, Hq, Hkv, S, D = 1, 2, 1, 96, 64
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 1120, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 1121, DEV)
    bias = draw_bias((B, Hq, S, S), BF16, 1122, DEV)
    bias[0, 0, 10, :40] = float("-inf")
    bias[0, 1, 50, :] = float("-inf")      # row 50 of head 1 sees nothing
    dq, dk, dv, db, rb = check(q, k, v, dout, bias, 0.125, sd.MASK_NONE, None, "-inf bias")
    assert not dq[0, 1, 50].any() and not db[0, 1, 50].any()
    assert not db[0, 0, 10, :40].any()


def test_backward_zero_bias_is_the_plain_backward():
    B, Hq, Hkv, S, D = 2, 4, 2, 200, 128
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 1130, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 1131, DEV)
    zero = torch.zeros((1, 1, S, S), dtype=BF16, device=DEV)
    for mask, lens in ((sd.MASK_CAUSAL, None),
                       (sd.MASK_KEY_PADDING, torch.tensor([200, 57], dtype=torch.int32, device=DEV))):
        out, lse = sd.sdpa_forward_lse(q, k, v, 0.09, mask, lens)
        plain = sd.sdpa_backward(q, k, v, out, dout, lse, 0.09, mask, lens)
        biased = sd.sdpa_backward_bias(q, k, v, out, dout, lse, zero, 0.09, mask, lens)[:3]
        torch.cuda.synchronize()
        for a, b in zip(plain, biased):
            assert torch.equal(a, b)


def test_dbias_hidden_keys_are_zero():
    # causal + key padding: dbias is exactly 0 above the diagonal and past the
    # key limit (written, not left as it was)
    B, Hq, Hkv, S, D = 2, 2, 2, 264, 64
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 1140, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 1141, DEV)
    bias = draw_bias((B, Hq, S, S), BF16, 1142, DEV)
    lens = torch.tensor([264, 100], dtype=torch.int32, device=DEV)
    out, lse = sd.sdpa_forward_bias(q, k, v, bias, 0.1, 3, lens, lse=True)
    db = torch.full((B, Hq, S, S), 7.0, dtype=BF16, device=DEV)
    sd.sdpa_backward_bias(q, k, v, out, dout, lse, bias, 0.1, 3, lens, dbias=db)
    torch.cuda.synchronize()
    hidden = torch.triu(torch.ones(S, S, dtype=torch.bool, device=DEV), diagonal=1)
    assert not db[:, :, hidden].any()
    assert not db[1, :, :, 100:].any()
    assert db[0, :, ~hidden].abs().sum() > 0


def test_backward_bias_full_size_whole_output():
    # the causal prefill workload with a per-head bias [1, 16, 4096, 4096];
    # every head's dq, dk, dv and bias gradient against the oracle
    B, H, S, D = 4, 16, 4096, 128
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 1150, DEV)
    dout = draw_grad((B, H, S, D), BF16, 1151, DEV)
    bias = draw_bias((1, H, S, S), BF16, 1152, DEV)
    scale = 1 / math.sqrt(D)
    dq, dk, dv, db = run(q, k, v, dout, bias, scale, sd.MASK_CAUSAL, None)
    backward_whole_check(O, q, k, v, dout, scale, O.MASK_CAUSAL, (dq, dk, dv), BF16,
                         "bias full size", bias=bias, dbias=db)
