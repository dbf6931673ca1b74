"""The whole-output parity helpers (threaded per head, row blocks, streamed
gradient statistics) agree with direct oracle calls and with compare_rel on
small host inputs, so a full-size GPU test that uses them checks what it
claims."""

import numpy as np
import pytest
import torch

import oracle as O
from exact_scaled_dot_amd.workloads import draw_qkv
from parity import (backward_whole_check, check_rel_stats, compare_rel, oracle_decode_whole,
                    oracle_forward_whole, rel_stats)


@pytest.mark.parametrize("kind", [O.MASK_NONE, O.MASK_CAUSAL, O.MASK_KEY_PADDING,
                                  O.MASK_CAUSAL | O.MASK_KEY_PADDING])
def test_forward_whole_equals_oracle_forward(kind):
    q, k, v = draw_qkv(2, 4, 2, 70, 70, 16, torch.float32, 3)
    lens = np.array([70, 23]) if kind & O.MASK_KEY_PADDING else None
    got, lse = oracle_forward_whole(O, q, k, v, 0.3, kind, lens, row_block=32, return_lse=True)
    ref, rlse = O.sdpa_forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.3,
                               kind, lens, return_lse=True)
    np.testing.assert_array_equal(got, ref)
    np.testing.assert_array_equal(lse, rlse)


def test_forward_whole_with_bias():
    q, k, v = draw_qkv(2, 3, 3, 40, 40, 8, torch.float32, 4)
    bias = torch.randn(1, 3, 40, 40, generator=torch.Generator().manual_seed(5))
    got = oracle_forward_whole(O, q, k, v, 0.5, O.MASK_CAUSAL, row_block=16, bias=bias)
    ref = O.sdpa_forward(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.5,
                         O.MASK_CAUSAL, bias=bias.double().numpy())
    np.testing.assert_array_equal(got, ref)


def test_decode_whole_equals_oracle_decode():
    q, k, v = draw_qkv(3, 8, 2, 1, 50, 16, torch.float32, 6)
    lens = np.array([50, 1, 17])
    got = oracle_decode_whole(O, q, k, v, 0.25, lens)
    ref = O.sdpa_decode(q.double().numpy(), k.double().numpy(), v.double().numpy(), 0.25, lens)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-15)


def test_streamed_stats_match_compare_rel():
    rng = np.random.default_rng(7)
    ref = rng.standard_normal((4, 3, 20, 8))
    got = ref + 1e-3 * rng.standard_normal(ref.shape)
    mr, rel = compare_rel(got, ref, 1.0, 1.0, "whole")
    stats = [rel_stats(got[b], ref[b]) for b in range(4)]
    smr, srel = check_rel_stats(stats, 1.0, 1.0, "streamed")
    assert abs(smr - mr) <= 1e-12 * mr and abs(srel - rel) <= 1e-12 * rel
    with pytest.raises(AssertionError):
        check_rel_stats(stats, rel / 2, 1.0, "too tight")


def _grads(q, k, v, dout, scale, kind, bias=None):
    out = O.sdpa_backward(q.double().numpy(), k.double().numpy(), v.double().numpy(),
                          dout.double().numpy(), scale, kind,
                          bias=None if bias is None else bias.double().numpy(),
                          return_dbias=bias is not None)
    return [torch.from_numpy(g) for g in out]


def test_backward_whole_check_accepts_oracle_and_rejects_a_slip():
    q, k, v = draw_qkv(2, 3, 3, 30, 30, 8, torch.float32, 8)
    dout = torch.randn(2, 3, 30, 8, generator=torch.Generator().manual_seed(9))
    grads = _grads(q, k, v, dout, 0.4, O.MASK_CAUSAL)
    backward_whole_check(O, q, k, v, dout, 0.4, O.MASK_CAUSAL, grads, torch.bfloat16, "exact")
    bad = [g.clone() for g in grads]
    bad[1][1, 2] *= 1.5            # one head of dk off by half
    with pytest.raises(AssertionError):
        backward_whole_check(O, q, k, v, dout, 0.4, O.MASK_CAUSAL, bad, torch.bfloat16, "slip")


def test_backward_whole_check_with_bias_gradient():
    q, k, v = draw_qkv(2, 2, 2, 20, 20, 8, torch.float32, 10)
    dout = torch.randn(2, 2, 20, 8, generator=torch.Generator().manual_seed(11))
    bias = torch.randn(1, 2, 20, 20, generator=torch.Generator().manual_seed(12))
    # the per-batch bias gradient [B, H, Sq, Sk]: dS of each (b, h)
    g = [_grads(q[b:b + 1], k[b:b + 1], v[b:b + 1], dout[b:b + 1], 0.3, O.MASK_NONE, bias)
         for b in range(2)]
    dq, dk, dv, db = (torch.cat([x[i] for x in g]) for i in range(4))
    backward_whole_check(O, q, k, v, dout, 0.3, O.MASK_NONE, (dq, dk, dv), torch.bfloat16,
                         "bias", bias=bias, dbias=db)
    db2 = db.clone()
    db2[1, 0] = 0
    with pytest.raises(AssertionError):
        backward_whole_check(O, q, k, v, dout, 0.3, O.MASK_NONE, (dq, dk, dv), torch.bfloat16,
                             "bias slip", bias=bias, dbias=db2)
