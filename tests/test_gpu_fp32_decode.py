"""GPU parity of fp32 inputs on the split-KV decode, the paged attention and
the paged prefill (ruDNN user guide section 9 allows F32 Q/K/V) against the
fp64 oracle, at the fp32 bar (max-abs <= 1e-4)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_paged, draw_qkv
from parity import compare, oracle_decode_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = torch.float32


def decode_case(B, Hq, Hkv, Sk, D, splits, lens, seed):
    scale = 1.0 / math.sqrt(D)
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, F32, seed, DEV)
    key_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    ws = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, splits), dtype=torch.uint8, device=DEV)
    out = sd.sdpa_decode(q, k, v, scale, key_lens, splits, workspace=ws)
    torch.cuda.synchronize()
    q64, k64, v64 = to64(q), to64(k), to64(v)
    nl = None if lens is None else np.array(lens)
    what = "fp32 decode B%d Hq%d Hkv%d Sk%d D%d splits%d" % (B, Hq, Hkv, Sk, D, splits)
    compare(to64(out), O.sdpa_decode(q64, k64, v64, scale, nl), F32, what)
    # the fp32 partials themselves against the oracle's split partials
    op, lp = sd.decode_workspace_views(ws, B, Hq, D, splits)
    rop, rlp = O.decode_split_partials(q64, k64, v64, scale, nl, splits)
    op, lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
    empty = np.isneginf(rlp)
    assert np.array_equal(np.isneginf(lp), empty), what + ": empty-split pattern"
    assert (op[empty] == 0).all()
    assert np.abs(lp[~empty] - rlp[~empty]).max() <= 1e-4, what + ": lse"
    compare(op[~empty], rop[~empty], F32, what + ": partials")
    return out


@pytest.mark.parametrize("D", [64, 128, 4, 36, 100])
@pytest.mark.parametrize("splits", [1, 7, 32])
def test_fp32_decode(D, splits):
    decode_case(3, 8, 2, 1000, D, splits, [1000, 1, 333], seed=3000 + D + splits)


@pytest.mark.parametrize("G", [1, 4, 16, 20])
def test_fp32_decode_group_sizes(G):
    decode_case(2, 2 * G, 2, 777, 128, 5, None, seed=3100 + G)


def test_fp32_decode_empty_batch_is_nan_and_short_keys():
    out = decode_case(4, 4, 4, 65, 64, 32, [0, 1, 15, 65], seed=3200)
    assert torch.isnan(out[0]).all() and not torch.isnan(out[1:]).any()


@pytest.mark.slow
def test_fp32_decode_long_history_whole_output():
    # 32768 cached keys, grouped heads 32/8, 32 splits; every query head
    B, Hq, Hkv, Sk, D = 8, 32, 8, 32768, 128
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, F32, 3300, DEV)
    lens = torch.tensor([Sk, 20001, 1, 4096, Sk, 777, 16, 30000], dtype=torch.int32, device=DEV)
    out = sd.sdpa_decode(q, k, v, 1 / math.sqrt(D), lens, 32)
    torch.cuda.synchronize()
    ref = oracle_decode_whole(O, q, k, v, 1 / math.sqrt(D), lens.cpu().numpy())
    compare(to64(out), ref, F32, "fp32 decode 32768 keys")


def test_fp32_decode_noalloc_matches_decode():
    q, k, v = draw_qkv(4, 16, 4, 1, 3000, 128, F32, 3400, DEV)
    ref = sd.sdpa_decode(q, k, v, 0.1, None, 9)
    got = torch.empty_like(q)
    sd.sdpa_decode_noalloc(q, k, v, 0.1, got, None, 9)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def paged_oracle(inp, scale, causal, qs=None, qp=None):
    return O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                             inp["block_tables"].cpu().numpy(), inp["seq_lens"].cpu().numpy(),
                             inp["query_seq"].cpu().numpy() if qs is None else qs,
                             inp["query_pos"].cpu().numpy() if qp is None else qp, scale, causal)


@pytest.mark.parametrize("D", [64, 128, 44])
@pytest.mark.parametrize("page_size,splits", [(16, 1), (32, 5), (64, 32)])
def test_fp32_paged_attention(D, page_size, splits):
    lens, qs, qp = [300, 129, 1, 1000], [0, 1, 2, 3, 3, 0], [299, 128, 0, 999, 500, 7]
    for causal in (False, True):
        inp = draw_paged(lens, qs, qp, 8, 2, D, page_size, F32, 3500 + D + page_size + causal, DEV)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                      inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                      causal, inp["block_tables"].shape[1] * page_size, splits)
        torch.cuda.synchronize()
        compare(to64(out), paged_oracle(inp, scale, causal), F32,
                "fp32 paged D=%d ps=%d splits=%d causal=%d" % (D, page_size, splits, causal))


def test_fp32_paged_invalid_pages_hidden():
    inp = draw_paged([64], [0, 0], [63, 63], 4, 2, 64, 16, F32, 3600, DEV)
    inp["block_tables"] = torch.tensor([[0, -1, 2, 99999]], dtype=torch.int32, device=DEV)
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], 0.1, False,
                                  64, 4)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            np.array([[0, 2]]), np.array([32]), np.array([0, 0]), np.array([31, 31]),
                            0.1, False)
    compare(to64(out), ref, F32, "fp32 paged: invalid pages hidden")


@pytest.mark.parametrize("D", [64, 128, 20])
@pytest.mark.parametrize("page_size", [16, 64])
def test_fp32_paged_prefill(D, page_size):
    lens, chunks = [300, 129, 1000, 70], [300, 40, 257, 1]
    nq = sum(chunks)
    for causal in (False, True):
        inp = draw_paged(lens, [0] * nq, [0] * nq, 8, 4, D, page_size, F32, 3700 + D + causal, DEV)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                    inp["seq_lens"], cu, scale, causal, max(chunks),
                                    inp["block_tables"].shape[1] * page_size)
        torch.cuda.synchronize()
        qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
        compare(to64(out), paged_oracle(inp, scale, causal, qs, qp), F32,
                "fp32 paged prefill D=%d ps=%d causal=%d" % (D, page_size, causal))


def test_fp32_paged_prefill_invalid_pages_hidden():
    inp = draw_paged([64], [0] * 10, [0] * 10, 4, 2, 128, 16, F32, 3800, DEV)
    inp["block_tables"] = torch.tensor([[0, -1, 2, 99999]], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 10], dtype=torch.int32, device=DEV)
    out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], cu, 0.1, False, 10, 64)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            np.array([[0, 2]]), np.array([32]), np.zeros(10, dtype=np.int64),
                            np.full(10, 31), 0.1, False)
    compare(to64(out), ref, F32, "fp32 paged prefill: invalid pages hidden")
