"""GPU parity of sdpa_decode (split pass + merge) against the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import WORKLOADS, draw_qkv, make_inputs
from parity import compare, oracle_decode_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_decode(B, Hq, Hkv, Sk, D, splits, lens=None, seed=0, check_partials=True):
    scale = 1.0 / math.sqrt(D)
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, torch.bfloat16, seed, DEV)
    key_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, splits), dtype=torch.uint8, device=DEV)
    out = sd.sdpa_decode(q, k, v, scale, key_lens, splits, workspace=ws)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    nl = None if lens is None else np.array(lens)
    ref = O.sdpa_decode(q64, k64, v64, scale, nl)
    what = "B%d Hq%d Hkv%d Sk%d D%d splits%d lens=%s" % (B, Hq, Hkv, Sk, D, splits, lens)
    res = compare(to64(out), ref, torch.bfloat16, what)
    if check_partials:
        # The workspace holds fp32 partials: compare them with the oracle's split
        # partials at the fp32 bar (they are not rounded to bf16).
        op, lp = sd.decode_workspace_views(ws, B, Hq, D, splits)
        rop, rlp = O.decode_split_partials(q64, k64, v64, scale, nl, splits)
        op, lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
        empty = np.isneginf(rlp)
        assert np.array_equal(np.isneginf(lp), empty), what + ": empty-split pattern differs"
        assert (op[empty] == 0).all()
        # l is the fp32 sum of the bf16-rounded weights (the weights multiplied
        # into V); rounding each weight to nearest bf16 moves it by at most
        # 2^-9 of itself, so |ln l - ln l_exact| <= 2^-9 ~ 1.95e-3 (+ fp32 noise).
        assert np.abs(lp[~empty] - rlp[~empty]).max() <= 2.5e-3, what + ": lse"
        # P is rounded to bf16 before P.V, so partial outputs meet the bf16 bars.
        compare(op[~empty], rop[~empty], torch.bfloat16, what + ": partial outputs")
    return res


@pytest.mark.parametrize("splits", [1, 2, 7, 32])
def test_decode_splits(splits):
    run_decode(3, 8, 2, 1000, 128, splits, seed=splits)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_decode_group_sizes(D, G):
    run_decode(2, 2 * G, 2, 777, D, 5, seed=G + D)


@pytest.mark.parametrize("Sk", [1, 2, 15, 16, 17, 31, 33, 100, 4097])
def test_decode_ragged_lengths(Sk):
    run_decode(2, 4, 1, Sk, 128, min(32, max(1, Sk // 3)), seed=Sk)


def test_decode_key_lens_with_empty_splits():
    # lengths 1, a split boundary +-1, full; with 8 splits of 125 keys many are empty
    run_decode(5, 8, 2, 1000, 128, 8, lens=[1, 124, 125, 126, 1000], seed=3)
    run_decode(3, 4, 4, 64, 64, 32, lens=[1, 2, 64], seed=4)


def test_decode_more_splits_than_keys():
    run_decode(2, 4, 2, 5, 128, 32, seed=8)


def test_decode_single_key_returns_v():
    q, k, v = draw_qkv(2, 8, 2, 1, 1, 128, torch.bfloat16, 2, DEV)
    out = sd.sdpa_decode(q, k, v, 0.1, None, 4)
    torch.cuda.synchronize()
    assert torch.equal(out, v.repeat_interleave(4, dim=1))


def test_decode_equals_forward_with_one_query():
    q, k, v = draw_qkv(2, 8, 2, 1, 3000, 128, torch.bfloat16, 5, DEV)
    lens = torch.tensor([3000, 1234], dtype=torch.int32, device=DEV)
    a = sd.sdpa_decode(q, k, v, 0.088, lens, 32)
    b = sd.sdpa_forward(q, k, v, 0.088, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    compare(to64(a), to64(b).astype(np.float64), torch.bfloat16, "decode vs forward")


def test_decode_deterministic():
    q, k, v = draw_qkv(4, 32, 8, 1, 5000, 128, torch.bfloat16, 6, DEV)
    a = sd.sdpa_decode(q, k, v, 0.088, None, 32)
    b = sd.sdpa_decode(q, k, v, 0.088, None, 32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size_decode_workload_whole_output():
    # every query head of all 64 sequences against the oracle, one (sequence,
    # K/V head) group per thread (its K/V slice widened to fp64 on the host),
    # bars over the whole output tensor
    w = WORKLOADS["bf16_gqa32x8_decode_b64_sk32768_d128"]
    inp = make_inputs(w, DEV)
    out = torch.full_like(inp["q"], float("nan"))
    sd.sdpa_decode(inp["q"], inp["k"], inp["v"], w.scale, None, w.num_splits, out=out)
    torch.cuda.synchronize()
    ref = oracle_decode_whole(O, inp["q"], inp["k"], inp["v"], w.scale)
    max_abs, rel = compare(to64(out), ref, torch.bfloat16, w.name + " whole output")
    print("%s whole output: max-abs %.3e rel-L2 %.3e" % (w.name, max_abs, rel))
