"""GPU parity at 16-bit head dims that are not multiples of 8 (1 to 1023; the
ruDNN user guide section 9 sets no alignment on the head dim), against the
fp64 oracle, on every entry point that takes them: the dense forward (and its
log-sum-exp), the split-KV decode (its partials included), the alloc-free
decode, the paged attention and the paged prefill, with value head dims of
their own.

Rows of such a width are not 16-byte aligned, so the kernels read Q, K and V
element by element into the same on-chip layout as the aligned widths and
store the output element by element; the dims past D are zeros on chip.
Above 256 the head-dim-split kernel (4, 6 or 8 waves of 128 dims) does the
same.
Sizes span several key tiles with a ragged tail.  Bars: tests/parity.py."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_paged, draw_qkv
from parity import compare, oracle_forward_whole, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16

WIDTHS = [1, 3, 17, 36, 100, 130, 200, 255]


@pytest.mark.parametrize("D", WIDTHS)
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_forward_any_width(D, mask):
    B, Hq, Hkv, S = 2, 4, 2, 333
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 5000 + D + 7 * mask, DEV)
    lens = torch.tensor([333, 70], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    what = "forward D=%d mask=%d" % (D, mask)
    assert out.shape == (B, Hq, S, D)
    compare(to64(out), ref, BF16, what)
    assert np.abs(to64(lse) - rlse).max() < 1e-2, what + ": lse"


@pytest.mark.parametrize("D", [17, 130])
def test_forward_any_width_fp16(D):
    q, k, v = draw_qkv(2, 8, 2, 200, 200, D, F16, 5100 + D, DEV)
    out = sd.sdpa_forward(q, k, v, 0.1, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.1, O.MASK_CAUSAL), F16,
            "fp16 forward D=%d" % D)


@pytest.mark.parametrize("D", [100, 200])
def test_forward_any_width_many_workgroups(D):
    # no mask, 512 workgroups (1024 at D = 200, two output slices): the
    # XCD-resident key sweep; every output row against the oracle
    B, Hq, Hkv, S = 2, 16, 4, 2048
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 5200 + D, DEV)
    scale = 1 / math.sqrt(D)
    out = sd.sdpa_forward(q, k, v, scale, 0)
    torch.cuda.synchronize()
    ref = oracle_forward_whole(O, q, k, v, scale, O.MASK_NONE)
    compare(to64(out), ref, BF16, "forward D=%d many workgroups" % D)


def test_forward_any_width_output_untouched_past_rows():
    # the element-wise stores write exactly B*Hq*S*D elements: a guard band
    # after the output keeps its sentinel
    B, Hq, S, D = 1, 2, 130, 37
    q, k, v = draw_qkv(B, Hq, Hq, S, S, D, BF16, 5300, DEV)
    buf = torch.full((B * Hq * S * D + 64,), 7.0, dtype=BF16, device=DEV)
    out = buf[: B * Hq * S * D].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.2, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (buf[B * Hq * S * D:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.2, O.MASK_CAUSAL), BF16,
            "forward D=37 into a guarded buffer")


@pytest.mark.parametrize("D", [1, 17, 100, 130, 255])
@pytest.mark.parametrize("splits", [1, 7, 32])
def test_decode_any_width(D, splits):
    B, Hq, Hkv, Sk = 3, 16, 4, 1000
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 5400 + D + splits, DEV)
    lens = torch.tensor([1000, 333, 17], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    ws = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, splits), dtype=torch.uint8, device=DEV)
    out = sd.sdpa_decode(q, k, v, scale, lens, splits, workspace=ws)
    torch.cuda.synchronize()
    q64, k64, v64, ln = to64(q), to64(k), to64(v), lens.cpu().numpy()
    what = "decode D=%d splits=%d" % (D, splits)
    compare(to64(out), O.sdpa_decode(q64, k64, v64, scale, ln), BF16, what)
    # the fp32 partials at their padded pitch against the oracle's split partials
    op, lp = sd.decode_workspace_views(ws, B, Hq, D, splits)
    rop, rlp = O.decode_split_partials(q64, k64, v64, scale, ln, splits)
    op, lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
    empty = np.isneginf(rlp)
    assert np.array_equal(np.isneginf(lp), empty), what + ": empty-split pattern"
    assert (op[empty] == 0).all(), what + ": empty partials"
    assert np.abs(lp[~empty] - rlp[~empty]).max() <= 2e-2, what + ": partial lse"
    compare(op[~empty], rop[~empty], BF16, what + ": partials")


def test_decode_noalloc_any_width_matches_decode():
    q, k, v = draw_qkv(4, 16, 4, 1, 3000, 77, BF16, 5500, DEV)
    ref = sd.sdpa_decode(q, k, v, 0.1, None, 9)
    got = torch.empty_like(q)
    sd.sdpa_decode_noalloc(q, k, v, 0.1, got, None, 9)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def value_width(inp, Dv, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 7919)
    pages, ps, Hkv, _ = inp["k_cache"].shape
    inp["v_cache"] = torch.randn(pages, ps, Hkv, Dv, generator=g, device=DEV).to(dtype)
    return inp


PAIRS = [(17, 17), (100, 100), (200, 200), (255, 255), (128, 36), (36, 130), (255, 1), (3, 250)]


@pytest.mark.parametrize("D,Dv", PAIRS)
@pytest.mark.parametrize("page_size,splits", [(16, 1), (64, 5)])
def test_paged_attention_any_width(D, Dv, page_size, splits):
    lens, qs, qp = [300, 129, 1, 50], [0, 1, 2, 0, 3, 1], [299, 128, 0, 17, 49, 3]
    for causal in (False, True):
        seed = 5600 + D + Dv + page_size + causal
        inp = value_width(draw_paged(lens, qs, qp, 8, 2, D, page_size, BF16, seed, DEV), Dv, BF16,
                          seed)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                      inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                      causal, inp["block_tables"].shape[1] * page_size, splits)
        torch.cuda.synchronize()
        assert out.shape == (len(qs), 8, Dv)
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), np.array(qs),
                                np.array(qp), scale, causal)
        compare(to64(out), ref, BF16,
                "paged D=%d Dv=%d ps=%d splits=%d causal=%d" % (D, Dv, page_size, splits, causal))


@pytest.mark.parametrize("D,Dv", PAIRS)
def test_paged_prefill_any_width(D, Dv):
    lens, chunks = [300, 129, 1000], [300, 40, 257]
    nq = sum(chunks)
    for causal in (False, True):
        seed = 5700 + D + Dv + causal
        inp = value_width(draw_paged(lens, [0] * nq, [0] * nq, 8, 2, D, 16, BF16, seed, DEV), Dv,
                          BF16, seed)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(D)
        out, lse = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"],
                                         inp["block_tables"], inp["seq_lens"], cu, scale, causal,
                                         max(chunks), inp["block_tables"].shape[1] * 16, lse=True)
        torch.cuda.synchronize()
        assert out.shape == (nq, 8, Dv)
        qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale,
                                causal)
        what = "prefill D=%d Dv=%d causal=%d" % (D, Dv, causal)
        compare(to64(out), ref, BF16, what)
        # the log-sum-exp rows against the oracle's attend
        kc, vc, q64 = to64(inp["k_cache"]), to64(inp["v_cache"]), to64(inp["q"])
        tables = inp["block_tables"].cpu().numpy()
        want = np.empty((nq, 8))
        for t in range(nq):
            n = lens[qs[t]]
            ks = O.paged_gather(kc, tables[qs[t]], n, 16)
            vs = O.paged_gather(vc, tables[qs[t]], n, 16)
            vis = np.ones((1, n), dtype=bool)
            if causal:
                vis &= (np.arange(n) <= qp[t])[None, :]
            for h in range(8):  # K/V head h // 4 (8 query heads over 2)
                want[t, h] = O.attend(q64[t, h:h + 1], ks[:, h // 4], vs[:, h // 4], scale, vis)[1][0]
        assert np.abs(to64(lse) - want).max() < 2e-3, what + ": lse"


WIDE = [257, 300, 517, 700, 1023]


@pytest.mark.parametrize("D", WIDE)
@pytest.mark.parametrize("mask", [0, 1, 3], ids=["none", "causal", "causal+padding"])
def test_forward_wide_any_width(D, mask):
    B, Hq, Hkv, S = 2, 4, 2, 150
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, 5800 + D + 7 * mask, DEV)
    lens = torch.tensor([150, 33], dtype=torch.int32, device=DEV) if mask & 2 else None
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    what = "wide forward D=%d mask=%d" % (D, mask)
    compare(to64(out), ref, BF16, what)
    assert np.abs(to64(lse) - rlse).max() < 1e-2, what + ": lse"


def test_forward_wide_any_width_fp16_guarded():
    B, Hq, S, D = 1, 4, 70, 389
    q, k, v = draw_qkv(B, Hq, 2, S, S, D, F16, 5900, DEV)
    n = B * Hq * S * D
    buf = torch.full((n + 64,), 7.0, dtype=F16, device=DEV)
    out = buf[:n].view(B, Hq, S, D)
    sd.sdpa_forward(q, k, v, 0.05, sd.MASK_CAUSAL, out=out)
    torch.cuda.synchronize()
    assert (buf[n:] == 7.0).all()
    compare(to64(out), O.sdpa_forward(to64(q), to64(k), to64(v), 0.05, O.MASK_CAUSAL), F16,
            "fp16 wide forward D=389")


@pytest.mark.parametrize("D", [300, 517, 1023])
@pytest.mark.parametrize("splits", [1, 7])
def test_decode_wide_any_width(D, splits):
    B, Hq, Hkv, Sk = 3, 8, 2, 700
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, BF16, 6000 + D + splits, DEV)
    lens = torch.tensor([700, 123, 1], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    ws = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, splits), dtype=torch.uint8, device=DEV)
    out = sd.sdpa_decode(q, k, v, scale, lens, splits, workspace=ws)
    torch.cuda.synchronize()
    q64, k64, v64, ln = to64(q), to64(k), to64(v), lens.cpu().numpy()
    what = "wide decode D=%d splits=%d" % (D, splits)
    compare(to64(out), O.sdpa_decode(q64, k64, v64, scale, ln), BF16, what)
    op, lp = sd.decode_workspace_views(ws, B, Hq, D, splits)
    rop, rlp = O.decode_split_partials(q64, k64, v64, scale, ln, splits)
    op, lp = op.cpu().double().numpy(), lp.cpu().double().numpy()
    empty = np.isneginf(rlp)
    assert np.array_equal(np.isneginf(lp), empty), what + ": empty-split pattern"
    assert (op[empty] == 0).all(), what + ": empty partials"
    compare(op[~empty], rop[~empty], BF16, what + ": partials")


@pytest.mark.parametrize("D", [300, 1023])
def test_paged_wide_any_width(D):
    lens, qs, qp = [300, 129, 1], [0, 1, 2, 0], [299, 128, 0, 17]
    for causal in (False, True):
        seed = 6100 + D + causal
        inp = draw_paged(lens, qs, qp, 4, 2, D, 16, BF16, seed, DEV)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                      inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                      causal, inp["block_tables"].shape[1] * 16, 3)
        torch.cuda.synchronize()
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), np.array(qs),
                                np.array(qp), scale, causal)
        compare(to64(out), ref, BF16, "wide paged D=%d causal=%d" % (D, causal))


@pytest.mark.parametrize("D", [300, 1023])
def test_paged_prefill_wide_any_width(D):
    lens, chunks = [300, 129, 70], [100, 40, 1]
    nq = sum(chunks)
    for causal in (False, True):
        seed = 6200 + D + causal
        inp = draw_paged(lens, [0] * nq, [0] * nq, 4, 2, D, 16, BF16, seed, DEV)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                    inp["seq_lens"], cu, scale, causal, max(chunks),
                                    inp["block_tables"].shape[1] * 16)
        torch.cuda.synchronize()
        qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale,
                                causal)
        compare(to64(out), ref, BF16, "wide prefill D=%d causal=%d" % (D, causal))


# ------------------------------------------------ the dense ordered backward


def backward_case(B, Hq, Hkv, Sq, Sk, D, mask, lens, dtype, seed):
    from exact_scaled_dot_amd.workloads import draw_grad
    from parity import compare_grad
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, seed, DEV)
    dout = draw_grad((B, Hq, Sq, D), dtype, seed + 1, DEV)
    kl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, kl)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, mask, kl)
    torch.cuda.synchronize()
    rq, rk, rv = O.sdpa_backward(to64(q), to64(k), to64(v), to64(dout), scale, mask,
                                 None if lens is None else np.array(lens))
    what = "backward D=%d mask=%d" % (D, mask)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare_grad(to64(g), r, dtype, what + " " + name)


@pytest.mark.parametrize("D", [3, 36, 100, 130, 257, 300, 511])
@pytest.mark.parametrize("mask", [1, 2], ids=["causal", "padding"])
def test_backward_any_width(D, mask):
    # ragged lengths (300 = 4 tiles of 64 + 44), grouped K/V heads
    lens = [300, 97] if mask & 2 else None
    backward_case(2, 4, 2, 300, 300, D, mask, lens, BF16, 6300 + D + mask)


def test_backward_any_width_fp16_rectangular():
    backward_case(2, 6, 3, 130, 333, 77, 2, [333, 45], F16, 6400)


# ------------------------------------- value head dims above 256 (Dv != D)

WIDE_PAIRS = [(128, 512), (512, 128), (300, 1023), (1024, 64), (257, 513), (64, 300)]


@pytest.mark.parametrize("D,Dv", WIDE_PAIRS)
@pytest.mark.parametrize("splits", [1, 5])
def test_paged_attention_wide_value_width(D, Dv, splits):
    lens, qs, qp = [300, 129, 1, 50], [0, 1, 2, 0, 3, 1], [299, 128, 0, 17, 49, 3]
    for causal in (False, True):
        seed = 6500 + D + Dv + splits + causal
        inp = value_width(draw_paged(lens, qs, qp, 4, 2, D, 16, BF16, seed, DEV), Dv, BF16, seed)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                      inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                      causal, inp["block_tables"].shape[1] * 16, splits)
        torch.cuda.synchronize()
        assert out.shape == (len(qs), 4, Dv)
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), np.array(qs),
                                np.array(qp), scale, causal)
        compare(to64(out), ref, BF16, "wide paged D=%d Dv=%d splits=%d causal=%d"
                % (D, Dv, splits, causal))


@pytest.mark.parametrize("D,Dv", WIDE_PAIRS)
def test_paged_prefill_wide_value_width(D, Dv):
    lens, chunks = [300, 129, 70], [100, 40, 1]
    nq = sum(chunks)
    for causal in (False, True):
        seed = 6600 + D + Dv + causal
        inp = value_width(draw_paged(lens, [0] * nq, [0] * nq, 4, 2, D, 16, BF16, seed, DEV), Dv,
                          BF16, seed)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(D)
        out, lse = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"],
                                         inp["block_tables"], inp["seq_lens"], cu, scale, causal,
                                         max(chunks), inp["block_tables"].shape[1] * 16, lse=True)
        torch.cuda.synchronize()
        assert out.shape == (nq, 4, Dv)
        qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale,
                                causal)
        what = "wide prefill D=%d Dv=%d causal=%d" % (D, Dv, causal)
        compare(to64(out), ref, BF16, what)
        assert np.isfinite(to64(lse)).all(), what + ": lse"


# --------------------------------------------- invalid pages, random shapes


@pytest.mark.parametrize("D,Dv", [(100, 100), (36, 130), (300, 300), (77, 513)])
def test_paged_any_width_invalid_table_entries_hide_their_keys(D, Dv):
    # logical pages 1 and 3 of a 64-key sequence point outside the cache: on
    # the element-wise paths too they are never read and their keys hidden
    inp = value_width(draw_paged([64], [0, 0], [63, 63], 4, 2, D, 16, BF16, 6700 + D + Dv, DEV), Dv,
                      BF16, 6700 + D + Dv)
    inp["block_tables"] = torch.tensor([[0, -1, 2, 99999]], dtype=torch.int32, device=DEV)
    cu = torch.tensor([0, 2], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, False,
                                  64, 3)
    pre = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], cu, scale, False, 2, 64)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            np.array([[0, 2]]), np.array([32]), np.array([0, 0]), np.array([31, 31]),
                            scale, False)
    compare(to64(out), ref, BF16, "invalid pages hidden D=%d Dv=%d (attention)" % (D, Dv))
    compare(to64(pre), ref, BF16, "invalid pages hidden D=%d Dv=%d (prefill)" % (D, Dv))


def random_cases(n, seed):
    rng = np.random.default_rng(seed)
    for i in range(n):
        G = int(rng.choice([1, 2, 3, 8]))
        Hkv = int(rng.integers(1, 3))
        D = int(rng.choice([int(rng.integers(1, 256)), int(rng.integers(257, 1024))], p=[0.75, 0.25]))
        S = int(rng.integers(1, 260))
        mask = int(rng.integers(0, 4))
        yield i, G * Hkv, Hkv, S, D, mask, int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("case", list(random_cases(24, 6800)), ids=lambda c: "r%d" % c[0])
def test_forward_and_decode_random_shapes(case):
    # seeded random shapes: head dims of any width (a quarter above 256),
    # grouped heads, short and ragged lengths, every mask; the forward with
    # its lse and the decode of the last row, against the oracle
    _, Hq, Hkv, S, D, mask, seed = case
    B = 2
    q, k, v = draw_qkv(B, Hq, Hkv, S, S, D, BF16, seed % 100000, DEV)
    lens = None
    if mask & 2:
        lens = torch.tensor([S, max(1, S // 3)], dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, lens)
    splits = 1 + seed % 9
    qd = q[:, :, -1:].contiguous()
    dec = sd.sdpa_decode(qd, k, v, scale, lens, splits)
    torch.cuda.synchronize()
    ln = None if lens is None else lens.cpu().numpy()
    what = "random Hq=%d Hkv=%d S=%d D=%d mask=%d" % (Hq, Hkv, S, D, mask)
    ref, rlse = O.sdpa_forward(to64(q), to64(k), to64(v), scale, mask, ln, return_lse=True)
    compare(to64(out), ref, BF16, what)
    assert np.abs(to64(lse) - rlse).max() < 1e-2, what + ": lse"
    compare(to64(dec), O.sdpa_decode(to64(qd), to64(k), to64(v), scale, ln), BF16,
            what + " decode splits=%d" % splits)
