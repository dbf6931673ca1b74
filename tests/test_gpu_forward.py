"""GPU parity of sdpa_forward against the fp64 oracle (through the C ABI)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import (WORKLOADS, draw_bias, draw_key_lens, draw_qkv,
                                             make_inputs)
from parity import compare, oracle_forward_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def kinds(causal, padded):
    k_lib = (sd.MASK_CAUSAL if causal else 0) | (sd.MASK_KEY_PADDING if padded else 0)
    k_orc = (O.MASK_CAUSAL if causal else 0) | (O.MASK_KEY_PADDING if padded else 0)
    return k_lib, k_orc


def run_case(B, Hq, Hkv, Sq, Sk, D, dtype, causal=False, lens=None, seed=0, scale=None):
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, seed, DEV)
    key_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    k_lib, k_orc = kinds(causal, lens is not None)
    out = sd.sdpa_forward(q, k, v, scale, k_lib, key_lens)
    torch.cuda.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), scale, k_orc,
                         None if lens is None else np.array(lens))
    return compare(to64(out), ref, dtype, "B%d Hq%d Hkv%d Sq%d Sk%d D%d causal=%s lens=%s" %
                   (B, Hq, Hkv, Sq, Sk, D, causal, lens))


# ------------------------------------------------------------ headline small workloads

@pytest.mark.parametrize("seed_off", [0, 1000, 2000])
def test_fp32_single_head_workload(seed_off):
    w = WORKLOADS["fp32_single_head_s128_d64"]
    run_case(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.dtype, seed=w.seed + seed_off)


@pytest.mark.parametrize("seed_off", [0, 1000, 2000])
def test_bf16_small_causal_workload(seed_off):
    w = WORKLOADS["bf16_causal_b8_h4_s128_d64"]
    run_case(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.dtype, causal=True, seed=w.seed + seed_off)


# fp32 when the grid of 32-row blocks fits the CUs: a workgroup owns 32 rows
# and its 4 waves take every fourth 32-key block, merging their running
# (max, sum, O) at the end.

@pytest.mark.parametrize("D", [64, 128, 36, 100])
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_fp32_key_split_waves(D, mask):
    # 6, 10 and 3 blocks of 32 keys: waves with two, three, one or no block
    B, Hq, Hkv = 3, 2, 1
    for Sq, Sk in ((190, 190), (70, 300), (129, 65)):
        if mask & 1 and Sq != Sk:
            continue
        q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, torch.float32, 830 + D + mask + Sk, DEV)
        lens = torch.tensor([Sk, 0, max(1, Sk // 3)], dtype=torch.int32, device=DEV) if mask & 2 else None
        scale = 1 / math.sqrt(D)
        out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
        torch.cuda.synchronize()
        ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask,
                                   None if lens is None else lens.cpu().numpy(), return_lse=True)
        o, l = to64(out), to64(lse)
        if mask & 2:  # batch 1 has no visible key: NaN rows, lse -inf
            assert np.isnan(o[1]).all() and np.isneginf(l[1]).all()
            o, ref, l, rlse = o[[0, 2]], ref[[0, 2]], l[[0, 2]], rlse[[0, 2]]
        compare(o, ref, torch.float32, "fp32 split D=%d mask=%d Sq=%d Sk=%d" % (D, mask, Sq, Sk))
        assert np.abs(l - rlse).max() < 1e-5


@pytest.mark.parametrize("Hq", [64, 65])
def test_fp32_key_split_grid_boundary(Hq):
    # 256 blocks of 32 rows take the key-split form, 260 the plain one
    run_case(1, Hq, 1, 100, 333, 64, torch.float32, causal=False, seed=840 + Hq)
    run_case(1, Hq, 1, 100, 100, 128, torch.float32, causal=True, seed=850 + Hq)


# ------------------------------------------------------------ ragged sweeps

SIZES = [1, 2, 17, 63, 64, 65, 127, 129, 200]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S", SIZES)
def test_ragged_causal(dtype, D, S):
    run_case(2, 2, 1, S, S, D, dtype, causal=True, seed=S * 7 + D)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 300), (5, 77), (130, 1), (64, 129), (257, 190),
                                   (300, 1000)])
def test_ragged_rectangular(dtype, Sq, Sk):
    run_case(1, 4, 2, Sq, Sk, 128, dtype, seed=Sq * 31 + Sk)
    run_case(2, 2, 2, Sq, Sk, 64, dtype, seed=Sq * 37 + Sk)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_gqa_group_sizes(dtype, G):
    run_case(2, 2 * G, 2, 150, 150, 128, dtype, causal=(G % 2 == 0), seed=G)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("causal", [False, True])
def test_key_padding(dtype, causal):
    # lengths: 1, a tile boundary +-1, full, and one past Sk (acts as Sk)
    lens = [1, 63, 64, 65, 300, 301]
    run_case(len(lens), 4, 2, 300, 300, 128, dtype, causal=causal, lens=lens, seed=11)
    run_case(len(lens), 2, 1, 300, 300, 64, dtype, causal=causal, lens=lens, seed=12)


def test_scales():
    for scale in (1e-3, 0.5, 2.0):
        run_case(1, 2, 2, 100, 100, 64, torch.bfloat16, causal=True, seed=5, scale=scale)
        run_case(1, 2, 2, 100, 100, 64, torch.float32, causal=True, seed=5, scale=scale)


def test_zero_length_rows_are_nan():
    # key_lens[b] = 0 hides every key of that batch: its rows are 0/0 = NaN.
    q, k, v = draw_qkv(2, 2, 2, 70, 70, 64, torch.bfloat16, 3, DEV)
    lens = torch.tensor([0, 70], dtype=torch.int32, device=DEV)
    out = sd.sdpa_forward(q, k, v, 0.125, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    o = to64(out)
    assert np.isnan(o[0]).all() and np.isfinite(o[1]).all()


# ------------------------------------------------------------ exact special cases

@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_single_key_returns_v_exactly(dtype):
    q, k, v = draw_qkv(2, 4, 2, 77, 1, 128, dtype, 9, DEV)
    out = sd.sdpa_forward(q, k, v, 0.1)
    torch.cuda.synchronize()
    want = v.repeat_interleave(2, dim=1).expand(-1, -1, 77, -1)
    assert torch.equal(out, want)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_causal_first_row_is_v0_exactly(dtype):
    q, k, v = draw_qkv(2, 4, 4, 190, 190, 64, dtype, 4, DEV)
    out = sd.sdpa_forward(q, k, v, 0.125, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(out[:, :, 0], v[:, :, 0])


def test_deterministic():
    q, k, v = draw_qkv(2, 8, 2, 333, 333, 128, torch.bfloat16, 21, DEV)
    a = sd.sdpa_forward(q, k, v, 0.09, sd.MASK_CAUSAL)
    b = sd.sdpa_forward(q, k, v, 0.09, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    q, k, v = draw_qkv(1, 4, 4, 256, 256, 128, torch.bfloat16, 8, DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = sd.sdpa_forward(q, k, v, 0.088, sd.MASK_CAUSAL)
    s.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), 0.088, O.MASK_CAUSAL)
    compare(to64(out), ref, torch.bfloat16, "side stream")


def test_zero_query_gives_prefix_means():
    # Q = 0: uniform weights over visible keys, i.e. prefix means of V (causal).
    _, k, v = draw_qkv(1, 2, 2, 700, 700, 128, torch.bfloat16, 6, DEV)
    q = torch.zeros(1, 2, 700, 128, dtype=torch.bfloat16, device=DEV)
    out = sd.sdpa_forward(q, k, v, 0.088, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    v64 = to64(v)
    want = np.cumsum(v64, axis=2) / np.arange(1, 701)[None, None, :, None]
    compare(to64(out), want, torch.bfloat16, "Q=0 prefix means")


# ------------------------------------------------------------ full-size workloads (whole output)

@pytest.mark.slow
@pytest.mark.parametrize("name", ["bf16_causal_b4_h16_s4096_d128", "bf16_gqa32x8_padded_b2_s8192_d128"])
def test_full_size_workload_whole_output(name):
    # every output row of the workload against the oracle: max-abs and rel-L2
    # over the whole tensor (a tile the launch skipped or wrote twice fails)
    w = WORKLOADS[name]
    inp = make_inputs(w, DEV)
    k_lib, k_orc = kinds(w.causal, w.padded)
    out = torch.full_like(inp["q"], float("nan"))
    sd.sdpa_forward(inp["q"], inp["k"], inp["v"], w.scale, k_lib, inp["key_lens"], out=out)
    torch.cuda.synchronize()
    lens = None if inp["key_lens"] is None else inp["key_lens"].cpu().numpy()
    ref = oracle_forward_whole(O, inp["q"], inp["k"], inp["v"], w.scale, k_orc, lens)
    max_abs, rel = compare(to64(out), ref, w.dtype, name)
    print("%s whole output: max-abs %.3e rel-L2 %.3e" % (name, max_abs, rel))


# ------------------------------------------------------------ many workgroups, no causal mask
# Without a causal mask each XCD sweeps the keys backwards in every other
# group of the workgroups it holds at once (64 per XCD at D=128, so launches
# of more than 512 workgroups), and Q and O are streamed.  These launches run
# 1056 workgroups (33 query blocks x 32 heads): every XCD runs forward and
# backward groups, over a ragged last query block and ragged key limits.

@pytest.mark.parametrize("D,dtype", [(64, torch.bfloat16), (128, torch.bfloat16),
                                     (128, torch.float16), (200, torch.bfloat16),
                                     (256, torch.bfloat16)])
@pytest.mark.parametrize("padded", [False, True])
def test_many_workgroups_non_causal(D, dtype, padded):
    B, Hq, Hkv, Sq, Sk = 2, 16, 4, 4100, 777
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, 700 + D + padded, DEV)
    lens = torch.tensor([777, 300], dtype=torch.int32, device=DEV) if padded else None
    kind = sd.MASK_KEY_PADDING if padded else sd.MASK_NONE
    scale = 1 / math.sqrt(D)
    out = torch.full_like(q, float("nan"))
    sd.sdpa_forward(q, k, v, scale, kind, lens, out=out)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, scale, kind, None if lens is None else lens.cpu().numpy())
    compare(to64(out), ref, dtype, "non-causal D=%d %s padded=%d" % (D, dtype, padded))


def test_many_workgroups_non_causal_bias():
    B, Hq, Hkv, Sq, Sk, D = 2, 16, 16, 4100, 336, 128
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, torch.bfloat16, 777, DEV)
    bias = draw_bias((B, 1, Sq, Sk), torch.bfloat16, 778, DEV)
    lens = torch.tensor([336, 129], dtype=torch.int32, device=DEV)
    out = sd.sdpa_forward_bias(q, k, v, bias, 0.09, sd.MASK_KEY_PADDING, lens)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, 0.09, O.MASK_KEY_PADDING, lens.cpu().numpy(), bias=bias)
    compare(to64(out), ref, torch.bfloat16, "non-causal bias")


def test_many_workgroups_non_causal_deterministic():
    q, k, v = draw_qkv(2, 16, 4, 4100, 777, 128, torch.bfloat16, 779, DEV)
    a = sd.sdpa_forward(q, k, v, 0.1)
    b = sd.sdpa_forward(q, k, v, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _hot_key_inputs(B, Hq, Sq, Sk, D, dtype, seed):
    # batch b: one key (position 3*b) scores 100 above every other key of
    # every query; without the hot key's score in the row max the weights
    # would overflow exp2, so every tile position of the hot key is tried
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    q = torch.zeros(B, Hq, Sq, D)
    q[..., 0] = 10.0
    k = torch.zeros(B, 1, Sk, D)
    for b in range(B):
        k[b, 0, 3 * b, 0] = 10.0
    v = torch.randn(B, 1, Sk, D, generator=gen)
    return [t.to(dtype).to(DEV) for t in (q, k, v)]


@pytest.mark.parametrize("D", [64, 128])
def test_row_max_covers_every_key(D):
    B, Hq, Sq, Sk = 64, 2, 40, 192
    q, k, v = _hot_key_inputs(B, Hq, Sq, Sk, D, torch.bfloat16, 77)
    out = sd.sdpa_forward(q, k, v, 1.0)
    torch.cuda.synchronize()
    ref = O.sdpa_forward(to64(q), to64(k), to64(v), 1.0)
    compare(to64(out), ref, torch.bfloat16, "hot key forward D=%d" % D)


@pytest.mark.parametrize("splits", [1, 3])
def test_decode_row_max_covers_every_key(splits):
    B, Hq, Sk, D = 64, 16, 192, 128
    q, k, v = _hot_key_inputs(B, Hq, 1, Sk, D, torch.bfloat16, 78)
    out = sd.sdpa_decode(q, k, v, 1.0, None, splits)
    torch.cuda.synchronize()
    ref = O.sdpa_decode(to64(q), to64(k), to64(v), 1.0)
    compare(to64(out), ref, torch.bfloat16, "hot key decode splits=%d" % splits)
