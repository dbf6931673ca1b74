"""GPU parity of the paged backward (sdpa_paged_backward, with the lse output of
sdpa_paged_prefill) against the oracle's paged_attention_backward: dq and the
gradients of every cache slot, at the backward bars.  Head dims of any width
up to 512 and a value head dim of its own (ruDNN user guide section 9: D and
Dv in 1..=1024, forward and first-order backward)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_grad, draw_paged
from parity import compare_grad, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


def run(lens, chunks, Hq, Hkv, D, page_size, causal, dtype, seed, extra_pages=3, Dv=None):
    nq = int(sum(chunks))
    inp = draw_paged(lens, [0] * nq, [0] * nq, Hq, Hkv, D, page_size, dtype, seed, DEV,
                     extra_pages=extra_pages)
    if Dv is not None and Dv != D:  # V of its own width
        g = torch.Generator(device=DEV)
        g.manual_seed(seed + 7919)
        pages, ps, hk, _ = inp["k_cache"].shape
        inp["v_cache"] = torch.randn(pages, ps, hk, Dv, generator=g, device=DEV).to(dtype)
    Dv = inp["v_cache"].shape[3]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
    L = inp["block_tables"].shape[1] * page_size
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                     inp["seq_lens"], cu, scale, causal, max(chunks), L, lse=True)
    dout = draw_grad((nq, Hq, Dv), dtype, seed + 1, DEV)
    dq, dk, dv = sd.sdpa_paged_backward(inp["q"], inp["k_cache"], inp["v_cache"], out, dout, lse,
                                        inp["block_tables"], inp["seq_lens"], cu, scale, causal, L)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
    tables = inp["block_tables"].cpu().numpy()
    return inp, out, lse, dout, (dq, dk, dv), qs, qp, tables, scale


def check(lens, chunks, Hq, Hkv, D, page_size, causal, dtype=BF16, seed=0, Dv=None):
    inp, out, lse, dout, grads, qs, qp, tables, scale = run(lens, chunks, Hq, Hkv, D, page_size,
                                                            causal, dtype, seed, Dv=Dv)
    refs = O.paged_attention_backward(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                      to64(dout), tables, np.array(lens), qs, qp, scale, causal)
    what = "paged bwd lens=%s chunks=%s Hq=%d Hkv=%d D=%d Dv=%d ps=%d causal=%d" % (
        lens, chunks, Hq, Hkv, D, inp["v_cache"].shape[3], page_size, causal)
    for name, g, r in zip(("dq", "dk", "dv"), grads, refs):
        compare_grad(to64(g), r, dtype, what + " " + name)
    # slots no key of any sequence reaches: exactly zero
    reached = np.zeros(inp["k_cache"].shape[:2], dtype=bool)
    ps = inp["k_cache"].shape[1]
    for s, n in enumerate(lens):
        for j in range(n):
            reached[tables[s, j // ps], j % ps] = True
    for g in grads[1:]:
        assert not g[torch.as_tensor(~reached, device=DEV)].any(), what + ": unreached slots"
    # the forward's log-sum-exp against the oracle's, row by row
    kc, vc = to64(inp["k_cache"]), to64(inp["v_cache"])
    q64 = to64(inp["q"])
    G = Hq // Hkv
    want = np.empty((len(qs), Hq))
    for t in range(len(qs)):
        n = lens[qs[t]]
        ks = O.paged_gather(kc, tables[qs[t]], n, ps)
        vs = O.paged_gather(vc, tables[qs[t]], n, ps)
        vis = np.ones((1, n), dtype=bool)
        if causal:
            vis &= (np.arange(n) <= qp[t])[None, :]
        for h in range(Hq):
            want[t, h] = O.attend(q64[t, h:h + 1], ks[:, h // G], vs[:, h // G], scale, vis)[1][0]
    assert np.abs(to64(lse) - want).max() < 2e-3, what + ": lse"


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_backward_whole_sequences(D, page_size):
    lens = [300, 129, 1000]
    check(lens, lens, 8, 2, D, page_size, True, seed=4000 + D + page_size)


@pytest.mark.parametrize("causal", [True, False])
def test_paged_backward_chunks_after_history(causal):
    # chunks appended after cached history, one a single token, one whole
    check([500, 2000, 64, 777], [37, 256, 64, 1], 4, 4, 128, 16, causal, seed=4100 + causal)


@pytest.mark.parametrize("D", [96, 200, 256])
def test_paged_backward_general_widths(D):
    check([333, 70], [333, 17], 8, 4, D, 32, True, seed=4200 + D)


def test_paged_backward_fp16_grouped():
    check([700, 250], [200, 250], 16, 2, 128, 16, True, dtype=F16, seed=4300)


def test_paged_backward_deterministic():
    a = run([640, 100], [640, 3], 8, 2, 128, 16, True, BF16, 4400)[4]
    b = run([640, 100], [640, 3], 8, 2, 128, 16, True, BF16, 4400)[4]
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("D", [3, 100, 130, 255])
def test_paged_backward_any_width(D):
    # widths that are not multiples of 8: the copies pad to W on the fly
    check([333, 70], [333, 17], 8, 4, D, 32, True, seed=4500 + D)


@pytest.mark.parametrize("D,Dv", [(64, 128), (128, 36), (17, 250), (256, 8)])
def test_paged_backward_value_width(D, Dv):
    check([300, 129, 64], [300, 40, 1], 8, 2, D, 16, True, seed=4600 + D + Dv, Dv=Dv)


@pytest.mark.parametrize("D", [264, 300, 512])
def test_paged_backward_wide(D):
    # above 256: the head-dim-split prefill writes the lse, the head-dim-split
    # backward runs the dense pass
    check([200, 90], [200, 31], 4, 2, D, 16, True, seed=4700 + D)


def test_paged_backward_value_width_non_causal_fp16():
    check([500, 64], [77, 64], 8, 8, 96, 16, False, dtype=F16, seed=4800, Dv=40)


@pytest.mark.parametrize("D,Dv", [(128, 400), (300, 64), (512, 264)])
def test_paged_backward_wide_value_width(D, Dv):
    # the head-dim-split prefill writes the lse with a value width of its own
    check([200, 90], [200, 31], 4, 2, D, 16, True, seed=4900 + D + Dv, Dv=Dv)
