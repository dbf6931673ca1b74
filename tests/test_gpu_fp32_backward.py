"""GPU parity of the fp32 backward (ruDNN user guide section 9: F32 inputs
with the first-order backward; section 11: dq, dk, dv from the forward's
log-sum-exp, ordered reductions) against the fp64 oracle: the fp32 forward's
log-sum-exp (dense and paged prefill), sdpa_backward and sdpa_paged_backward
on fp32 tensors.  Bars: tests/parity.py (fp32 rows of GRAD_*)."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_grad, draw_paged, draw_qkv
from parity import compare, compare_grad, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = torch.float32


def dense_case(B, Hq, Hkv, Sq, Sk, D, mask, lens, seed):
    q, k, v = draw_qkv(B, Hq, Hkv, Sq, Sk, D, F32, seed, DEV)
    dout = draw_grad((B, Hq, Sq, D), F32, seed + 1, DEV)
    kl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_forward_lse(q, k, v, scale, mask, kl)
    dq, dk, dv = sd.sdpa_backward(q, k, v, out, dout, lse, scale, mask, kl)
    torch.cuda.synchronize()
    ln = None if lens is None else np.array(lens)
    q64, k64, v64 = to64(q), to64(k), to64(v)
    what = "fp32 D=%d mask=%d" % (D, mask)
    ref, rlse = O.sdpa_forward(q64, k64, v64, scale, mask, ln, return_lse=True)
    compare(to64(out), ref, F32, what + " out")
    fin = np.isfinite(rlse)
    assert np.array_equal(np.isfinite(to64(lse)), fin), what + ": lse pattern"
    assert np.abs(to64(lse)[fin] - rlse[fin]).max() <= 2e-5, what + ": lse"
    rq, rk, rv = O.sdpa_backward(q64, k64, v64, to64(dout), scale, mask, ln)
    for name, g, r in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        compare_grad(to64(g), r, F32, what + " " + name)
    return dq, dk, dv


@pytest.mark.parametrize("D", [64, 128, 4, 36, 100])
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_fp32_backward(D, mask):
    # grouped K/V heads, 300 rows = 4 tiles of 64 + 44, one short batch
    lens = [300, 97] if mask & 2 else None
    dense_case(2, 4, 2, 300, 300, D, mask, lens, 7000 + D + mask)


def test_fp32_backward_rectangular_grouped():
    # Sq != Sk, 3 query heads per K/V head, a batch with a single key
    dense_case(3, 6, 2, 130, 333, 64, 2, [333, 1, 200], 7100)


def test_fp32_backward_empty_rows_and_deterministic():
    # a batch with no visible key: its rows contribute nothing, dK = dV = 0
    a = dense_case(2, 2, 2, 70, 70, 32, 2, [0, 70], 7200)
    b = dense_case(2, 2, 2, 70, 70, 32, 2, [0, 70], 7200)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    assert not a[0][0].any() and not a[1][0].any() and not a[2][0].any()


@pytest.mark.slow
def test_fp32_backward_long_causal():
    # 2048 causal rows: many key and query tiles
    dense_case(1, 4, 2, 2048, 2048, 128, 1, None, 7300)


def paged_case(lens, chunks, Hq, Hkv, D, page_size, causal, seed):
    nq = int(sum(chunks))
    inp = draw_paged(lens, [0] * nq, [0] * nq, Hq, Hkv, D, page_size, F32, seed, DEV, extra_pages=3)
    cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
    L = inp["block_tables"].shape[1] * page_size
    scale = 1 / math.sqrt(D)
    out, lse = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                     inp["seq_lens"], cu, scale, causal, max(chunks), L, lse=True)
    dout = draw_grad((nq, Hq, D), F32, seed + 1, DEV)
    dq, dk, dv = sd.sdpa_paged_backward(inp["q"], inp["k_cache"], inp["v_cache"], out, dout, lse,
                                        inp["block_tables"], inp["seq_lens"], cu, scale, causal, L)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
    tables = inp["block_tables"].cpu().numpy()
    refs = O.paged_attention_backward(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                      to64(dout), tables, np.array(lens), qs, qp, scale, causal)
    what = "fp32 paged bwd D=%d ps=%d causal=%d" % (D, page_size, causal)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        compare_grad(to64(g), r, F32, what + " " + name)
    # the prefill's lse row by row
    kc, vc, q64 = to64(inp["k_cache"]), to64(inp["v_cache"]), to64(inp["q"])
    G = Hq // Hkv
    want = np.empty((nq, Hq))
    for t in range(nq):
        n = lens[qs[t]]
        ks = O.paged_gather(kc, tables[qs[t]], n, page_size)
        vs = O.paged_gather(vc, tables[qs[t]], n, page_size)
        vis = np.ones((1, n), dtype=bool)
        if causal:
            vis &= (np.arange(n) <= qp[t])[None, :]
        for h in range(Hq):
            want[t, h] = O.attend(q64[t, h:h + 1], ks[:, h // G], vs[:, h // G], scale, vis)[1][0]
    assert np.abs(to64(lse) - want).max() <= 2e-5, what + ": lse"


@pytest.mark.parametrize("D", [64, 36])
@pytest.mark.parametrize("causal", [True, False])
def test_fp32_paged_backward(D, causal):
    paged_case([300, 129, 77], [300, 40, 1], 8, 2, D, 16, causal, 7400 + D + causal)


def test_fp32_paged_backward_wide_pages():
    paged_case([500, 64], [200, 64], 4, 4, 128, 64, True, 7500)
