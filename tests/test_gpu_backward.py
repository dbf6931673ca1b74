"""GPU parity of the attention backward (sdpa_forward_lse + sdpa_backward)
against the fp64 oracle's dQ, dK, dV by the definition.

The HIP path takes the forward's own output and log-sum-exp (as a training
step would); the oracle recomputes everything in fp64 from the same 16-bit
q, k, v and dO.  Bars: tests/parity.py, GRAD_*."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_grad, draw_qkv
from parity import backward_whole_check, compare, compare_grad, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


def run_backward(q, k, v, dout, scale, mask, lens):
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, mask, lens)
    torch.cuda.synchronize()
    return out, lse, dq, dk, dv


def check_against_oracle(q, k, v, dout, scale, mask, lens, what):
    out, lse, dq, dk, dv = run_backward(q, k, v, dout, scale, mask, lens)
    ln = None if lens is None else lens.cpu().numpy()
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, mask, ln)
    dt = q.dtype
    compare_grad(to64(dq), rq, dt, what + " dq")
    compare_grad(to64(dk), rk, dt, what + " dk")
    compare_grad(to64(dv), rv, dt, what + " dv")
    return out, lse, dq, dk, dv


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_backward_parity(dtype, D, mask):
    # grouped K/V (4 query heads over 2), ragged lengths: 300 = 4 tiles of 64 + 44
    B, Hq, Hkv, S = 2, 4, 2, 300
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 500 + D + mask, DEV)
    dout = draw_grad((B, Hq, S, D), dtype, 501 + D + mask, DEV)
    lens = None
    if mask & sd.MASK_KEY_PADDING:
        lens = torch.tensor([300, 97], dtype=torch.int32, device=DEV)
    check_against_oracle(q, k, v, dout, 1 / math.sqrt(D), mask, lens,
                         "%s D=%d mask=%d" % (dtype, D, mask))


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
def test_backward_rectangular_padded(dtype):
    # Sq != Sk (no causal mask), 3 query heads per K/V head, one batch whose
    # keys end inside a 32-key block
    B, Hq, Hkv, Sq, Sk, D = 3, 6, 2, 200, 333, 128
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, 510, DEV)
    dout = draw_grad((B, Hq, Sq, D), dtype, 511, DEV)
    lens = torch.tensor([333, 129, 45], dtype=torch.int32, device=DEV)
    check_against_oracle(q, k, v, dout, 0.1, sd.MASK_KEY_PADDING, lens, "rect padded")


def test_backward_tiny_and_single_row():
    # fewer rows than one 32-row block, and Sq = 1 against many keys
    for Sq, Sk, mask in ((5, 5, sd.MASK_CAUSAL), (1, 700, 0), (70, 3, 0)):
        q, k, v = draw_qkv(1, 2, 1, Sq, Sk, 64, BF16, 520 + Sq, DEV)
        dout = draw_grad((1, 2, Sq, 64), BF16, 521 + Sq, DEV)
        check_against_oracle(q, k, v, dout, 0.125, mask, None, "Sq=%d Sk=%d" % (Sq, Sk))


def test_backward_dead_rows_contribute_nothing():
    # key_lens = 0 leaves every row of batch 1 without a visible key: its dq
    # rows and its dk, dv are 0, and the other batch is unaffected
    B, Hq, Hkv, S, D = 2, 2, 2, 130, 64
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 530, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 531, DEV)
    lens = torch.tensor([130, 0], dtype=torch.int32, device=DEV)
    out, lse, dq, dk, dv = check_against_oracle(q, k, v, dout, 0.125, sd.MASK_KEY_PADDING, lens,
                                                "dead rows")
    assert torch.isneginf(lse[1]).all()
    assert not dq[1].any() and not dk[1].any() and not dv[1].any()


def test_forward_lse_matches_oracle_and_plain_forward():
    B, Hq, Hkv, S, D = 2, 4, 1, 333, 128
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 540, DEV)
    scale = 1 / math.sqrt(D)
    for mask in (0, sd.MASK_CAUSAL):
        out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask)
        plain = sd.sdpa_forward(q, k, v, scale, mask)
        torch.cuda.synchronize()
        assert torch.equal(out, plain)  # the lse store changes nothing else
        ref_o, ref_lse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, return_lse=True)
        compare(to64(out), ref_o, BF16, "forward_lse out")
        # the denominator sums bf16-rounded weights: lse within a few 2^-9
        assert np.abs(to64(lse) - ref_lse).max() < 8e-3


def test_backward_is_deterministic():
    B, Hq, Hkv, S, D = 1, 8, 2, 520, 128
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 550, DEV)
    dout = draw_grad((B, Hq, S, D), BF16, 551, DEV)
    first = run_backward(q, k, v, dout, 0.09, sd.MASK_CAUSAL, None)[2:]
    second = run_backward(q, k, v, dout, 0.09, sd.MASK_CAUSAL, None)[2:]
    for a, b in zip(first, second):
        assert torch.equal(a, b)


def test_backward_full_size_whole_output():
    # the causal prefill workload (B4 H16 S4096 D128, bf16) end to end; every
    # dq, dk, dv row of all 64 heads against the oracle (one head per thread),
    # the bars over each whole gradient tensor
    B, H, S, D = 4, 16, 4096, 128
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 560, DEV)
    dout = draw_grad((B, H, S, D), BF16, 561, DEV)
    scale = 1 / math.sqrt(D)
    _, _, dq, dk, dv = run_backward(q, k, v, dout, scale, sd.MASK_CAUSAL, None)
    backward_whole_check(O, q, k, v, dout, scale, O.MASK_CAUSAL, (dq, dk, dv), BF16, "full size")


# ------------------------------------------------------------------ atomic dQ

def run_backward_atomic(q, k, v, dout, scale, mask, lens):
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, mask, lens, atomic=True)
    torch.cuda.synchronize()
    return dq, dk, dv


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("D", [64, 128, 96])
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_backward_atomic_parity(dtype, D, mask):
    B, Hq, Hkv, S = 2, 4, 2, 300
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, dtype, 800 + D + mask, DEV)
    dout = draw_grad((B, Hq, S, D), dtype, 801 + D + mask, DEV)
    lens = torch.tensor([300, 97], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    dq, dk, dv = run_backward_atomic(q, k, v, dout, scale, mask, lens)
    ln = None if lens is None else lens.cpu().numpy()
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, mask, ln)
    what = "atomic %s D=%d mask=%d" % (dtype, D, mask)
    compare_grad(to64(dq), rq, dtype, what + " dq")
    compare_grad(to64(dk), rk, dtype, what + " dk")
    compare_grad(to64(dv), rv, dtype, what + " dv")


def test_backward_atomic_dead_rows_and_rectangular():
    B, Hq, Hkv, Sq, Sk, D = 3, 6, 2, 200, 333, 128
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, BF16, 810, DEV)
    dout = draw_grad((B, Hq, Sq, D), BF16, 811, DEV)
    lens = torch.tensor([333, 0, 45], dtype=torch.int32, device=DEV)
    dq, dk, dv = run_backward_atomic(q, k, v, dout, 0.1, sd.MASK_KEY_PADDING, lens)
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), 0.1, O.MASK_KEY_PADDING,
                                 lens.cpu().numpy())
    compare_grad(to64(dq), rq, BF16, "atomic rect dq")
    compare_grad(to64(dk), rk, BF16, "atomic rect dk")
    compare_grad(to64(dv), rv, BF16, "atomic rect dv")
    assert not dq[1].any() and not dk[1].any() and not dv[1].any()


def test_backward_atomic_agrees_with_ordered_full_size():
    # the causal prefill workload: the two reductions agree to the bars, and
    # dK, dV of the atomic variant are reproducible call to call
    B, H, S, D = 4, 16, 4096, 128
    q, k, v = draw_qkv(B, H, H, S, S, D, BF16, 820, DEV)
    dout = draw_grad((B, H, S, D), BF16, 821, DEV)
    scale = 1 / math.sqrt(D)
    o_dq, o_dk, o_dv = run_backward(q, k, v, dout, scale, sd.MASK_CAUSAL, None)[2:]
    a_dq, a_dk, a_dv = run_backward_atomic(q, k, v, dout, scale, sd.MASK_CAUSAL, None)
    _, a_dk2, a_dv2 = run_backward_atomic(q, k, v, dout, scale, sd.MASK_CAUSAL, None)
    assert torch.equal(a_dk, a_dk2) and torch.equal(a_dv, a_dv2)
    for x, y, name in ((a_dq, o_dq, "dq"), (a_dk, o_dk, "dk"), (a_dv, o_dv, "dv")):
        d = (x.float() - y.float())
        rel = (d.norm() / y.float().norm()).item()
        print("atomic vs ordered %s: rel-L2 %.3e" % (name, rel))
        assert rel < 5e-3
    sl = (slice(1, 2), slice(7, 8))
    rq, rk, rv = O.sdpa_backward(to64(q[sl]), to64(k[sl]), to64(v[sl]), to64(dout[sl]), scale,
                                 O.MASK_CAUSAL)
    compare_grad(to64(a_dq[sl]), rq, BF16, "atomic full dq")
    compare_grad(to64(a_dk[sl]), rk, BF16, "atomic full dk")
    compare_grad(to64(a_dv[sl]), rv, BF16, "atomic full dv")
