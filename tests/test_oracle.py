"""Pins of the fp64 CPU oracle against things other than itself.

Each pin is a closed form, an invariant the mathematics fixes, a special case
that reduces to something elementary, or brute force on tiny inputs, chosen so
that a plausible slip in the oracle (a dropped scale, a wrong sign, a transposed
operand, the wrong softmax axis, an off-by-one mask, a wrong head map, a
missing merge weight) fails at least one of them.
"""

import itertools
import os
import math

import numpy as np
import pytest

import oracle as O

RNG = np.random.default_rng(12345)


def rand(*shape, scale=1.0):
    return RNG.standard_normal(shape) * scale


# ---------------------------------------------------------------- closed forms

def test_hand_example_square():
    # D = 1, scale = 1, q = k = [[1],[0]], v = [[1],[0]]:
    # S = [[1, 0], [0, 0]] so row 0 weights (e, 1)/(1+e), row 1 weights (1/2, 1/2).
    q = np.array([[[[1.0], [0.0]]]])
    k = q.copy()
    v = np.array([[[[1.0], [0.0]]]])
    o, lse = O.sdpa_forward(q, k, v, 1.0, return_lse=True)
    assert o[0, 0, 0, 0] == pytest.approx(math.e / (1 + math.e), abs=1e-15)
    assert o[0, 0, 1, 0] == pytest.approx(0.5, abs=1e-15)
    assert lse[0, 0, 0] == pytest.approx(math.log(math.e + 1), abs=1e-15)
    assert lse[0, 0, 1] == pytest.approx(math.log(2.0), abs=1e-15)


def test_hand_example_rectangular_asymmetric():
    # Sq = 2, Sk = 3, D = 2, scale = 1/2.  Non-square and asymmetric, so a
    # transposed product, a dropped scale or a wrong exponent sign all change it.
    q = np.array([[1.0, 0.0], [0.0, 2.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 3.0]])
    # row 0 scores (0.5, 0, 0.5); row 1 scores (0, 1, 1)
    e0 = [math.exp(0.5), 1.0, math.exp(0.5)]
    e1 = [1.0, math.e, math.e]
    want0 = [sum(e * v[j, d] for j, e in enumerate(e0)) / sum(e0) for d in range(2)]
    want1 = [sum(e * v[j, d] for j, e in enumerate(e1)) / sum(e1) for d in range(2)]
    o, lse = O.sdpa_forward(q[None, None], k[None, None], v[None, None], 0.5, return_lse=True)
    np.testing.assert_allclose(o[0, 0, 0], want0, rtol=0, atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 1], want1, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0, 0], [math.log(sum(e0)), math.log(sum(e1))], atol=1e-15)


def test_hand_example_causal_and_padding():
    # Same rectangular data made square (Sq = Sk = 3) with a causal mask:
    # row 0 sees key 0 only; row 1 sees keys 0,1; row 2 sees all three.
    q = np.array([[1.0, 0.0], [0.0, 2.0], [1.0, 1.0]])
    k = np.array([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    v = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, 3.0]])
    o = O.sdpa_forward(q[None, None], k[None, None], v[None, None], 0.5, O.MASK_CAUSAL)
    w1 = [1.0, math.e]                                  # row 1 scores (0, 1)
    w2 = [math.exp(0.5), math.exp(0.5), math.e]         # row 2 scores (.5, .5, 1)
    np.testing.assert_allclose(o[0, 0, 0], v[0], atol=0)
    np.testing.assert_allclose(o[0, 0, 1], (w1[0] * v[0] + w1[1] * v[1]) / sum(w1), atol=1e-15)
    np.testing.assert_allclose(o[0, 0, 2], (w2[0] * v[0] + w2[1] * v[1] + w2[2] * v[2]) / sum(w2),
                               atol=1e-15)
    # key padding with length 2 on the non-causal problem: row 2 sees keys 0,1
    o = O.sdpa_forward(q[None, None], k[None, None], v[None, None], 0.5, O.MASK_KEY_PADDING,
                       key_lens=np.array([2]))
    w2p = [math.exp(0.5), math.exp(0.5)]
    np.testing.assert_allclose(o[0, 0, 2], (w2p[0] * v[0] + w2p[1] * v[1]) / sum(w2p), atol=1e-15)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("mask", [O.MASK_NONE, O.MASK_CAUSAL, O.MASK_KEY_PADDING,
                                  O.MASK_CAUSAL | O.MASK_KEY_PADDING])
def test_rows_stochastic_and_masked_zero(mask):
    B, H, S, D = 2, 3, 9, 5
    q, k, v = rand(B, H, S, D), rand(B, H, S, D), rand(B, H, S, D)
    lens = np.array([4, 9]) if mask & O.MASK_KEY_PADDING else None
    o, probs = O.sdpa_forward(q, k, v, 0.7, mask, lens, return_probs=True)
    np.testing.assert_allclose(probs.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (probs >= 0).all()
    for b in range(B):
        i = np.arange(S)[:, None]
        j = np.arange(S)[None, :]
        hidden = np.zeros((S, S), bool)
        if mask & O.MASK_CAUSAL:
            hidden |= j > i
        if mask & O.MASK_KEY_PADDING:
            hidden |= j >= lens[b]
        assert (probs[b][:, hidden] == 0.0).all()
        assert (probs[b][:, ~hidden] > 0.0).all()
    # o is the weight matrix applied to V
    np.testing.assert_allclose(o, probs @ v, atol=1e-13)


def test_single_key_gives_v():
    q, k, v = rand(2, 4, 7, 8), rand(2, 2, 1, 8), rand(2, 2, 1, 8)
    o = O.sdpa_forward(q, k, v, 0.3)
    for h in range(4):
        np.testing.assert_array_equal(o[:, h], np.broadcast_to(v[:, h // 2], o[:, h].shape))


def test_identical_v_rows():
    q, k = rand(1, 2, 6, 4), rand(1, 2, 10, 4, scale=3.0)
    r = rand(4)
    v = np.broadcast_to(r, (1, 2, 10, 4)).copy()
    for mask, lens in [(O.MASK_NONE, None), (O.MASK_CAUSAL | O.MASK_KEY_PADDING, np.array([3]))]:
        if mask & O.MASK_CAUSAL:
            qq, kk, vv = q, k[:, :, :6], v[:, :, :6]
        else:
            qq, kk, vv = q, k, v
        o = O.sdpa_forward(qq, kk, vv, 1.0, mask, lens)
        np.testing.assert_allclose(o, np.broadcast_to(r, o.shape), rtol=1e-14, atol=1e-15)


def test_zero_query_gives_visible_means():
    # Q = 0 makes every visible score 0, so the weights are uniform over the
    # visible keys: plain mean, causal prefix means, or mean of the first len keys.
    B, H, S, D = 2, 2, 11, 3
    q = np.zeros((B, H, S, D))
    k, v = rand(B, H, S, D), rand(B, H, S, D)
    o, lse = O.sdpa_forward(q, k, v, 0.9, return_lse=True)
    np.testing.assert_allclose(o, np.broadcast_to(v.mean(2, keepdims=True), o.shape), atol=1e-14)
    np.testing.assert_allclose(lse, math.log(S), atol=1e-14)
    o, lse = O.sdpa_forward(q, k, v, 0.9, O.MASK_CAUSAL, return_lse=True)
    prefix = np.cumsum(v, axis=2) / np.arange(1, S + 1)[None, None, :, None]
    np.testing.assert_allclose(o, prefix, atol=1e-14)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(np.arange(1, S + 1)), lse.shape),
                               atol=1e-14)
    lens = np.array([5, 1])
    o = O.sdpa_forward(q, k, v, 0.9, O.MASK_KEY_PADDING, lens)
    for b in range(B):
        np.testing.assert_allclose(o[b], np.broadcast_to(v[b, :, :lens[b]].mean(1, keepdims=True),
                                                         o[b].shape), atol=1e-14)
    o = O.sdpa_forward(q, k, v, 0.9, O.MASK_CAUSAL | O.MASK_KEY_PADDING, lens)
    for b in range(B):
        for i in range(S):
            n = min(i + 1, lens[b])
            np.testing.assert_allclose(o[b, :, i], v[b, :, :n].mean(1), atol=1e-14)


def test_causal_first_row_is_v0():
    q, k, v = rand(3, 2, 8, 6), rand(3, 2, 8, 6), rand(3, 2, 8, 6)
    o = O.sdpa_forward(q, k, v, 0.4, O.MASK_CAUSAL)
    np.testing.assert_array_equal(o[:, :, 0], v[:, :, 0])


def test_shift_invariance_of_keys():
    # Adding the same vector u to every key adds scale*q_i.u to all of row i.
    q, k, v = rand(1, 2, 7, 5), rand(1, 2, 9, 5), rand(1, 2, 9, 5)
    u = rand(5) * 2
    for mask, lens in [(O.MASK_NONE, None), (O.MASK_KEY_PADDING, np.array([6]))]:
        o1 = O.sdpa_forward(q, k, v, 0.6, mask, lens)
        o2 = O.sdpa_forward(q, k + u, v, 0.6, mask, lens)
        np.testing.assert_allclose(o1, o2, atol=1e-12)


def test_permutation_equivariance():
    q, k, v = rand(1, 1, 6, 4), rand(1, 1, 8, 4), rand(1, 1, 8, 4)
    o = O.sdpa_forward(q, k, v, 0.8)
    pk = RNG.permutation(8)
    np.testing.assert_allclose(O.sdpa_forward(q, k[:, :, pk], v[:, :, pk], 0.8), o, atol=1e-13)
    pq = RNG.permutation(6)
    np.testing.assert_allclose(O.sdpa_forward(q[:, :, pq], k, v, 0.8), o[:, :, pq], atol=1e-13)


def test_scale_acts_on_scores_only():
    # softmax((2q) k^T * s/2) == softmax(q k^T * s): the scale multiplies scores.
    q, k, v = rand(1, 2, 5, 3), rand(1, 2, 5, 3), rand(1, 2, 5, 3)
    o1 = O.sdpa_forward(q, k, v, 0.5, O.MASK_CAUSAL)
    o2 = O.sdpa_forward(2 * q, k, v, 0.25, O.MASK_CAUSAL)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    # scale -> 0 gives uniform weights over visible keys
    o3 = O.sdpa_forward(q, k, v, 1e-300, O.MASK_CAUSAL)
    np.testing.assert_allclose(o3[0, :, 4], v[0].mean(1), atol=1e-13)


# ---------------------------------------------------------------- reductions

def test_gqa_equals_repeated_mha():
    q, k, v = rand(2, 8, 5, 4), rand(2, 2, 7, 4), rand(2, 2, 7, 4)
    o = O.sdpa_forward(q, k, v, 0.5)
    o_mha = O.sdpa_forward(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), 0.5)
    np.testing.assert_array_equal(o, o_mha)


def test_gqa_contiguous_head_groups():
    # Each K/V head's V is a distinct constant, so the output names the head read:
    # query head h must read K/V head h // (Hq / Hkv).
    Hq, Hkv = 12, 3
    q, k = rand(1, Hq, 4, 2), rand(1, Hkv, 6, 2)
    v = np.ones((1, Hkv, 6, 2)) * (np.arange(Hkv) + 1.0)[None, :, None, None]
    o = O.sdpa_forward(q, k, v, 1.0)
    for h in range(Hq):
        np.testing.assert_allclose(o[0, h], h // (Hq // Hkv) + 1.0, rtol=1e-14)


def test_causal_row_equals_prefix_problem():
    q, k, v = rand(1, 2, 10, 4), rand(1, 2, 10, 4), rand(1, 2, 10, 4)
    o = O.sdpa_forward(q, k, v, 0.7, O.MASK_CAUSAL)
    for i in range(10):
        oi = O.sdpa_forward(q[:, :, i:i + 1], k[:, :, :i + 1], v[:, :, :i + 1], 0.7)
        np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], atol=1e-14)


def test_padding_equals_truncation():
    q, k, v = rand(3, 2, 5, 4), rand(3, 2, 12, 4), rand(3, 2, 12, 4)
    lens = np.array([1, 7, 12])
    o = O.sdpa_forward(q, k, v, 0.7, O.MASK_KEY_PADDING, lens)
    for b in range(3):
        ob = O.sdpa_forward(q[b:b + 1], k[b:b + 1, :, :lens[b]], v[b:b + 1, :, :lens[b]], 0.7)
        np.testing.assert_allclose(o[b], ob[0], atol=1e-14)


def test_rows_match_full():
    q, k, v = rand(2, 4, 16, 8), rand(2, 2, 16, 8), rand(2, 2, 16, 8)
    lens = np.array([9, 16])
    for mask in (O.MASK_NONE, O.MASK_CAUSAL, O.MASK_CAUSAL | O.MASK_KEY_PADDING):
        kl = lens if mask & O.MASK_KEY_PADDING else None
        o, lse = O.sdpa_forward(q, k, v, 0.3, mask, kl, return_lse=True)
        idx = np.array([[0, 0, 0], [1, 3, 15], [0, 2, 7], [1, 1, 8], [0, 0, 5]])
        orow, lrow = O.sdpa_forward_rows(q, k, v, 0.3, mask, kl, idx)
        for n, (b, h, i) in enumerate(idx):
            np.testing.assert_allclose(orow[n], o[b, h, i], atol=1e-14)
            assert lrow[n] == pytest.approx(lse[b, h, i], abs=1e-14)


def test_decode_is_single_query_forward():
    q, k, v = rand(3, 4, 1, 8), rand(3, 2, 20, 8), rand(3, 2, 20, 8)
    lens = np.array([20, 1, 13])
    o = O.sdpa_decode(q, k, v, 0.35, lens)
    for b in range(3):
        for h in range(4):
            ob = O.sdpa_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h // 2:h // 2 + 1, :lens[b]],
                                v[b:b + 1, h // 2:h // 2 + 1, :lens[b]], 0.35)
            np.testing.assert_allclose(o[b, h, 0], ob[0, 0, 0], atol=1e-14)


# ---------------------------------------------------------------- split / merge

def test_split_ranges_partition_keys():
    for Sk, n in [(1, 1), (7, 2), (32768, 32), (5, 8), (100, 7), (1024, 32)]:
        r = O.split_ranges(Sk, n)
        assert len(r) == n and r[0][0] == 0 and r[-1][1] == Sk
        for (a, b), (c, d) in zip(r, r[1:]):
            assert b == c and a <= b
        assert all(hi - lo <= -(-Sk // n) for lo, hi in r)


@pytest.mark.parametrize("n", [1, 2, 3, 7, 32])
def test_split_merge_identity(n):
    # Merging the partials of any partition of the keys reproduces the unsplit result.
    q, k, v = rand(2, 4, 1, 8), rand(2, 2, 19, 8, scale=2.0), rand(2, 2, 19, 8)
    for lens in (None, np.array([19, 3])):
        o_full, lse_full = O.sdpa_forward(q, k, v, 0.5,
                                          O.MASK_KEY_PADDING if lens is not None else O.MASK_NONE,
                                          lens, return_lse=True)
        op, lp = O.decode_split_partials(q, k, v, 0.5, lens, n)
        o, lse = O.merge_partials(op, lp)
        np.testing.assert_allclose(o, o_full[:, :, 0], atol=1e-14)
        np.testing.assert_allclose(lse, lse_full[:, :, 0], atol=1e-13)
        # each partial is itself the attention over its own key range
        for s, (lo, hi) in enumerate(O.split_ranges(19, n)):
            top = hi if lens is None else None
            for b in range(2):
                hib = min(hi, lens[b]) if lens is not None else top
                if hib <= lo:
                    assert lp[b, :, s].tolist() == [-np.inf] * 4
                    assert (op[b, :, s] == 0).all()
                    continue
                ob, lb = O.sdpa_forward(q[b:b + 1], k[b:b + 1, :, lo:hib], v[b:b + 1, :, lo:hib],
                                        0.5, return_lse=True)
                np.testing.assert_allclose(op[b, :, s], ob[0, :, 0], atol=1e-14)
                np.testing.assert_allclose(lp[b, :, s], lb[0, :, 0], atol=1e-14)


def test_merge_closed_form():
    # Two partials with lse (0, ln 3): weights 1/4 and 3/4.
    op = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    lp = np.array([[0.0, math.log(3.0)]])
    o, lse = O.merge_partials(op, lp)
    np.testing.assert_allclose(o, [[0.25, 0.75]], atol=1e-15)
    assert lse[0] == pytest.approx(math.log(4.0), abs=1e-15)
    # an empty partial (lse = -inf) carries zero weight
    o, _ = O.merge_partials(np.array([[[5.0], [7.0]]]), np.array([[-np.inf, 2.0]]))
    assert o[0, 0] == 7.0


# ---------------------------------------------------------------- brute force

def brute_force(q, k, v, scale, mask, lens):
    """Scalar loops with exactly rounded sums (math.fsum), tiny shapes only."""
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    out = np.zeros((B, Hq, Sq, Dv))
    for b, h, i in itertools.product(range(B), range(Hq), range(Sq)):
        g = h * Hkv // Hq
        keys = [j for j in range(Sk)
                if (not mask & O.MASK_CAUSAL or j <= i)
                and (not mask & O.MASK_KEY_PADDING or j < lens[b])]
        s = {j: scale * math.fsum(q[b, h, i, d] * k[b, g, j, d] for d in range(D)) for j in keys}
        mx = max(s.values())
        e = {j: math.exp(s[j] - mx) for j in keys}
        den = math.fsum(e.values())
        for d in range(Dv):
            out[b, h, i, d] = math.fsum(e[j] * v[b, g, j, d] for j in keys) / den
    return out


@pytest.mark.parametrize("mask", [O.MASK_NONE, O.MASK_CAUSAL, O.MASK_KEY_PADDING,
                                  O.MASK_CAUSAL | O.MASK_KEY_PADDING])
def test_brute_force_tiny(mask):
    for S, D, Hq, Hkv in [(1, 1, 1, 1), (3, 2, 2, 1), (5, 4, 4, 2), (8, 3, 3, 3)]:
        q, k, v = rand(2, Hq, S, D, scale=2), rand(2, Hkv, S, D, scale=2), rand(2, Hkv, S, D)
        lens = np.array([max(1, S // 2), S]) if mask & O.MASK_KEY_PADDING else None
        o = O.sdpa_forward(q, k, v, 0.75, mask, lens)
        np.testing.assert_allclose(o, brute_force(q, k, v, 0.75, mask, lens), rtol=0, atol=1e-13)


# ------------------------------------------- value width Dv different from D

@pytest.mark.parametrize("mask", [O.MASK_NONE, O.MASK_CAUSAL, O.MASK_KEY_PADDING,
                                  O.MASK_CAUSAL | O.MASK_KEY_PADDING])
def test_brute_force_value_width(mask):
    # V of its own width: scores over D, output over Dv, by scalar loops
    for S, D, Dv, Hq, Hkv in [(4, 3, 5, 2, 1), (6, 4, 1, 4, 2), (5, 2, 7, 3, 3), (3, 6, 2, 2, 2)]:
        q, k, v = rand(2, Hq, S, D, scale=2), rand(2, Hkv, S, D, scale=2), rand(2, Hkv, S, Dv)
        lens = np.array([max(1, S // 2), S]) if mask & O.MASK_KEY_PADDING else None
        o = O.sdpa_forward(q, k, v, 0.6, mask, lens)
        assert o.shape == (2, Hq, S, Dv)
        np.testing.assert_allclose(o, brute_force(q, k, v, 0.6, mask, lens), rtol=0, atol=1e-13)


def test_value_identity_gives_the_weights():
    # V = the identity over keys (Dv = Sk): each output row is the row of
    # softmax weights itself, written out here from the definition
    B, H, S, D = 1, 2, 6, 3
    q, k = rand(B, H, S, D, scale=1.5), rand(B, H, S, D, scale=1.5)
    v = np.broadcast_to(np.eye(S), (B, H, S, S)).copy()
    o = O.sdpa_forward(q, k, v, 0.8, O.MASK_CAUSAL)
    for h, i in itertools.product(range(H), range(S)):
        s = [0.8 * float(np.dot(q[0, h, i], k[0, h, j])) for j in range(i + 1)]
        e = [math.exp(x - max(s)) for x in s]
        want = [x / math.fsum(e) for x in e] + [0.0] * (S - i - 1)
        np.testing.assert_allclose(o[0, h, i], want, rtol=0, atol=1e-14)


def test_value_width_rows_decode_and_split_merge():
    rng = np.random.default_rng(17)
    B, Hq, Hkv, S, D, Dv = 2, 4, 2, 9, 5, 3
    q, k, v = (rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)),
               rng.standard_normal((B, Hkv, S, Dv)))
    full = O.sdpa_forward(q, k, v, 0.5, O.MASK_CAUSAL)
    idx = np.array([(0, 1, 0), (1, 3, 8), (1, 0, 4)])
    rows, _ = O.sdpa_forward_rows(q, k, v, 0.5, O.MASK_CAUSAL, None, idx)
    np.testing.assert_allclose(rows, full[idx[:, 0], idx[:, 1], idx[:, 2]], rtol=0, atol=1e-13)
    q1 = q[:, :, :1]
    lens = np.array([9, 4])
    dec = O.sdpa_decode(q1, k, v, 0.5, lens)
    assert dec.shape == (B, Hq, 1, Dv)
    np.testing.assert_allclose(dec, brute_force(q1, k, v, 0.5, O.MASK_KEY_PADDING, lens), rtol=0,
                               atol=1e-13)
    op, lp = O.decode_split_partials(q1, k, v, 0.5, lens, 4)
    assert op.shape == (B, Hq, 4, Dv)
    merged, _ = O.merge_partials(op, lp)
    np.testing.assert_allclose(merged, dec[:, :, 0], rtol=0, atol=1e-13)


def test_paged_value_width():
    rng = np.random.default_rng(23)
    lens = [7, 3]
    nseq, Hq, Hkv, D, Dv, S = 2, 4, 2, 3, 6, 7
    q = rng.standard_normal((nseq, Hq, S, D))
    k = rng.standard_normal((nseq, Hkv, S, D))
    v = rng.standard_normal((nseq, Hkv, S, Dv))
    kc, vc, tables = make_paged(k, v, lens, 2, 1, rng)
    qs = np.array([s for s in range(nseq) for _ in range(lens[s])])
    qp = np.array([i for s in range(nseq) for i in range(lens[s])])
    qq = np.stack([q[s, :, i] for s, i in zip(qs, qp)])
    got = O.paged_attention(qq, kc, vc, tables, lens, qs, qp, 0.9, True)
    assert got.shape == (len(qs), Hq, Dv)
    for s in range(nseq):
        n = lens[s]
        ref = brute_force(q[s:s + 1, :, :n], k[s:s + 1, :, :n], v[s:s + 1, :, :n], 0.9,
                          O.MASK_CAUSAL, None)[0]
        np.testing.assert_allclose(got[qs == s], ref.transpose(1, 0, 2), rtol=0, atol=1e-13)


def test_backward_value_width_matches_finite_differences():
    rng = np.random.default_rng(29)
    B, Hq, Hkv, S, D, Dv = 1, 2, 1, 4, 3, 5
    q, k, v = (rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)),
               rng.standard_normal((B, Hkv, S, Dv)))
    g = rng.standard_normal((B, Hq, S, Dv))
    dq, dk, dv = O.sdpa_backward(q, k, v, g, 0.8, O.MASK_CAUSAL)
    assert dq.shape == q.shape and dk.shape == k.shape and dv.shape == v.shape
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, 0.8, O.MASK_CAUSAL, None)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], g, 0.8, O.MASK_CAUSAL, None)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)
    with pytest.raises(ValueError):
        O.sdpa_backward(q, k, v, rng.standard_normal((B, Hq, S, D)), 0.8)


def test_printed_kernel_without_max_subtraction():
    # The essay's printed kernel exponentiates raw scores and divides by the row
    # sums; on small scores (no overflow) it must agree with the max-shifted form.
    x = rand(6, 4, scale=0.5)
    wq, wk, wv = rand(4, 4), rand(4, 4), rand(4, 4)
    q, k, v = x @ wq, x @ wk, x @ wv
    scale = 1.0 / math.sqrt(x.shape[1])
    ex = [[math.exp(scale * sum(q[i, d] * k[j, d] for d in range(4))) for j in range(6)]
          for i in range(6)]
    want = np.array([[sum(ex[i][j] / sum(ex[i]) * v[j, d] for j in range(6)) for d in range(4)]
                     for i in range(6)])
    o = O.sdpa_forward(q[None, None], k[None, None], v[None, None], scale)
    np.testing.assert_allclose(o[0, 0], want, atol=1e-13)


def test_large_scores_do_not_overflow():
    # Scores far beyond exp's range: the max-shifted definition stays finite and
    # puts all weight on the largest score.
    q = np.array([[[[1000.0], [-1000.0]]]])
    k = np.array([[[[1.0], [2.0]]]])
    v = np.array([[[[3.0], [5.0]]]])
    o = O.sdpa_forward(q, k, v, 1.0)
    assert o[0, 0, 0, 0] == 5.0 and o[0, 0, 1, 0] == 3.0


def test_fully_masked_row_is_nan():
    q, k, v = rand(1, 1, 3, 2), rand(1, 1, 3, 2), rand(1, 1, 3, 2)
    o = O.sdpa_forward(q, k, v, 1.0, O.MASK_KEY_PADDING, np.array([0]))
    assert np.isnan(o).all()


def test_argument_checks():
    q, k, v = rand(1, 3, 2, 2), rand(1, 2, 2, 2), rand(1, 2, 2, 2)
    with pytest.raises(ValueError):
        O.sdpa_forward(q, k, v, 1.0)
    with pytest.raises(ValueError):
        O.sdpa_forward(rand(1, 1, 2, 2), rand(1, 1, 3, 2), rand(1, 1, 3, 2), 1.0, O.MASK_CAUSAL)
    with pytest.raises(ValueError):
        O.sdpa_forward(rand(1, 1, 2, 2), rand(1, 1, 3, 2), rand(1, 1, 3, 2), 1.0,
                       O.MASK_KEY_PADDING)


# ------------------------------------------------------------------ paged cache

def make_paged(k, v, lens, page_size, extra_pages, rng):
    """Scatter dense K/V [nseq, Hkv, S, D] into a shuffled page pool.

    Returns (k_cache, v_cache, block_tables); every unused slot and page is
    filled with large garbage so that reading one by mistake shows.
    """
    nseq, Hkv, S, D = k.shape
    Dv = v.shape[3]
    need = [-(-int(n) // page_size) for n in lens]
    max_pages = max(need)
    pages = sum(need) + extra_pages
    perm = rng.permutation(pages)
    k_cache = rng.standard_normal((pages, page_size, Hkv, D)) * 50.0
    v_cache = rng.standard_normal((pages, page_size, Hkv, Dv)) * 50.0
    tables = np.full((nseq, max_pages), -1, dtype=np.int64)
    nxt = 0
    for s in range(nseq):
        for lp in range(need[s]):
            tables[s, lp] = perm[nxt]
            nxt += 1
        for j in range(int(lens[s])):
            pg, sl = tables[s, j // page_size], j % page_size
            k_cache[pg, sl] = k[s, :, j]
            v_cache[pg, sl] = v[s, :, j]
    return k_cache, v_cache, tables


@pytest.mark.parametrize("page_size", [1, 4, 16])
def test_paged_prefill_equals_dense_causal(page_size):
    # Every position of every sequence as a packed query, causal by absolute
    # position: the rows of the dense causal forward of each sequence.
    rng = np.random.default_rng(7 + page_size)
    lens = [37, 5, 20]
    nseq, Hq, Hkv, D, S = len(lens), 4, 2, 8, max(lens)
    q = rng.standard_normal((nseq, Hq, S, D))
    k = rng.standard_normal((nseq, Hkv, S, D))
    v = rng.standard_normal((nseq, Hkv, S, D))
    kc, vc, tables = make_paged(k, v, lens, page_size, 3, rng)
    qs = np.array([s for s in range(nseq) for _ in range(lens[s])])
    qp = np.array([i for s in range(nseq) for i in range(lens[s])])
    qq = np.stack([q[s, :, i] for s, i in zip(qs, qp)])
    got = O.paged_attention(qq, kc, vc, tables, lens, qs, qp, 0.3, True)
    for s in range(nseq):
        n = lens[s]
        ref = O.sdpa_forward(q[s:s + 1, :, :n], k[s:s + 1, :, :n], v[s:s + 1, :, :n], 0.3,
                             O.MASK_CAUSAL)[0]
        rows = got[qs == s]
        np.testing.assert_allclose(rows, ref.transpose(1, 0, 2), rtol=0, atol=1e-13)


def test_paged_decode_equals_padded_decode():
    # One query per sequence: non-causal, or causal at the last position, is
    # the padded dense decode with key_lens = seq_lens.
    rng = np.random.default_rng(11)
    lens = np.array([1, 17, 64, 33])
    nseq, Hq, Hkv, D, S = len(lens), 8, 2, 16, 64
    q = rng.standard_normal((nseq, Hq, 1, D))
    k = rng.standard_normal((nseq, Hkv, S, D))
    v = rng.standard_normal((nseq, Hkv, S, D))
    kc, vc, tables = make_paged(k, v, lens, 16, 2, rng)
    ref = O.sdpa_decode(q, k, v, 0.25, lens)[:, :, 0]
    seqs = np.arange(nseq)
    for causal, pos in ((False, np.zeros(nseq, dtype=np.int64)), (True, lens - 1)):
        got = O.paged_attention(q[:, :, 0], kc, vc, tables, lens, seqs, pos, 0.25, causal)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_paged_bottom_right_chunk():
    # A chunk of 5 new queries at the end of a 29-key sequence sees exactly
    # keys 0..pos: the last 5 rows of the dense causal forward.
    rng = np.random.default_rng(3)
    L, n, Hq, Hkv, D = 29, 5, 2, 1, 8
    q = rng.standard_normal((1, Hq, L, D))
    k = rng.standard_normal((1, Hkv, L, D))
    v = rng.standard_normal((1, Hkv, L, D))
    kc, vc, tables = make_paged(k, v, [L], 8, 1, rng)
    pos = np.arange(L - n, L)
    got = O.paged_attention(q[0, :, L - n:].transpose(1, 0, 2), kc, vc, tables, [L],
                            np.zeros(n, dtype=np.int64), pos, 0.5, True)
    ref = O.sdpa_forward(q, k, v, 0.5, O.MASK_CAUSAL)[0][:, L - n:]
    np.testing.assert_allclose(got, ref.transpose(1, 0, 2), rtol=0, atol=1e-13)
    # without the causal flag every cached key is visible to every query
    got_nc = O.paged_attention(q[0, :, L - n:].transpose(1, 0, 2), kc, vc, tables, [L],
                               np.zeros(n, dtype=np.int64), pos, 0.5, False)
    ref_nc = O.sdpa_forward(q[:, :, L - n:], k, v, 0.5)[0]
    np.testing.assert_allclose(got_nc, ref_nc.transpose(1, 0, 2), rtol=0, atol=1e-13)


def test_paged_invariances():
    rng = np.random.default_rng(5)
    lens = [13, 30]
    nseq, Hq, Hkv, D, S = 2, 4, 4, 8, 30
    q = rng.standard_normal((nseq, Hq, S, D))
    k = rng.standard_normal((nseq, Hkv, S, D))
    v = rng.standard_normal((nseq, Hkv, S, D))
    kc, vc, tables = make_paged(k, v, lens, 4, 4, rng)
    qs = np.array([0] * 13 + [1] * 30)
    qp = np.array(list(range(13)) + list(range(30)))
    qq = np.stack([q[s, :, i] for s, i in zip(qs, qp)])
    base = O.paged_attention(qq, kc, vc, tables, lens, qs, qp, 0.4, True)
    # relabelling the physical pages changes nothing
    perm = rng.permutation(kc.shape[0])
    inv = np.argsort(perm)
    t2 = np.where(tables >= 0, inv[np.maximum(tables, 0)], -1)
    got = O.paged_attention(qq, kc[perm], vc[perm], t2, lens, qs, qp, 0.4, True)
    assert np.array_equal(got, base)
    # rewriting slots past a sequence's length and unreferenced pages changes nothing
    kc2, vc2 = kc.copy(), vc.copy()
    used = set()
    for s in range(nseq):
        for j in range(lens[s]):
            used.add((int(tables[s, j // 4]), j % 4))
    for pg in range(kc.shape[0]):
        for sl in range(4):
            if (pg, sl) not in used:
                kc2[pg, sl] = 1e6
                vc2[pg, sl] = -1e6
    got = O.paged_attention(qq, kc2, vc2, tables, lens, qs, qp, 0.4, True)
    assert np.array_equal(got, base)
    # query order is irrelevant: each query is answered on its own
    order = rng.permutation(len(qs))
    got = O.paged_attention(qq[order], kc, vc, tables, lens, qs[order], qp[order], 0.4, True)
    assert np.array_equal(got, base[order])


@pytest.mark.parametrize("causal", [False, True])
def test_paged_brute_force_tiny(causal):
    # Scalar loops with math.exp straight from the definition; page size 2,
    # two sequences sharing one pool, pages out of order.
    rng = np.random.default_rng(21 + causal)
    ps, Hq, Hkv, D = 2, 2, 1, 3
    kc = rng.standard_normal((5, ps, Hkv, D))
    vc = rng.standard_normal((5, ps, Hkv, D))
    tables = np.array([[3, 0, 4], [1, 2, -1]])
    lens = [5, 3]
    qs = np.array([0, 0, 1, 1])
    qp = np.array([4, 1, 2, 0])
    qq = rng.standard_normal((4, Hq, D))
    scale = 0.7
    got = O.paged_attention(qq, kc, vc, tables, lens, qs, qp, scale, causal)
    for t in range(4):
        s, p = qs[t], qp[t]
        keys = [j for j in range(lens[s]) if not causal or j <= p]
        for h in range(Hq):
            sc = []
            for j in keys:
                row = kc[tables[s][j // ps], j % ps, 0]
                sc.append(scale * sum(qq[t, h, d] * row[d] for d in range(D)))
            mx = max(sc)
            w = [math.exp(x - mx) for x in sc]
            tot = math.fsum(w)
            for d in range(D):
                ref = math.fsum(w[i] * vc[tables[s][j // ps], j % ps, 0, d]
                                for i, j in enumerate(keys)) / tot
                assert got[t, h, d] == pytest.approx(ref, abs=1e-13)


def test_chunk_positions_closed_form():
    # full prefills (chunk = whole sequence) are positions 0..n-1; a chunk of n
    # new tokens after c cached ones is c..c+n-1; an empty chunk contributes
    # nothing
    qs, qp = O.chunk_positions([0, 3, 3, 8, 9], [3, 10, 5, 40])
    assert qs.tolist() == [0, 0, 0, 2, 2, 2, 2, 2, 3]
    assert qp.tolist() == [0, 1, 2, 0, 1, 2, 3, 4, 39]
    qs, qp = O.chunk_positions([0, 4], [100])
    assert qp.tolist() == [96, 97, 98, 99]


# ------------------------------------------------------------------ backward

def _loss(q, k, v, g, scale, mask, lens):
    return float((O.sdpa_forward(q, k, v, scale, mask, lens) * g).sum())


@pytest.mark.parametrize("mask,lens", [(O.MASK_NONE, None), (O.MASK_CAUSAL, None),
                                       (O.MASK_KEY_PADDING, [3, 5])])
def test_backward_matches_finite_differences(mask, lens):
    # central differences of L = sum(O * G) through the (pinned) forward
    rng = np.random.default_rng(61 + mask)
    B, Hq, Hkv, S, D = 2, 4, 2, 5, 3
    q, k, v = (rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)),
               rng.standard_normal((B, Hkv, S, D)))
    g = rng.standard_normal((B, Hq, S, D))
    lens = None if lens is None else np.array(lens)
    dq, dk, dv = O.sdpa_backward(q, k, v, g, 0.7, mask, lens)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_loss(args_p["q"], args_p["k"], args_p["v"], g, 0.7, mask, lens)
                        - _loss(args_m["q"], args_m["k"], args_m["v"], g, 0.7, mask, lens)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)


def _paged_loss(q, kc, vc, g, tables, lens, qs, qp, scale, causal):
    return float((O.paged_attention(q, kc, vc, tables, lens, qs, qp, scale, causal) * g).sum())


@pytest.mark.parametrize("causal", [False, True])
def test_paged_backward_matches_finite_differences(causal):
    # two sequences over 7 physical pages of 2 slots; physical page 3 is in
    # both tables (its slots get both sequences' contributions), pages 5 and
    # 6 are unreached (zero gradient); Dv != D
    rng = np.random.default_rng(71 + causal)
    Hq, Hkv, D, Dv, ps = 2, 1, 3, 2, 2
    kc, vc = rng.standard_normal((7, ps, Hkv, D)), rng.standard_normal((7, ps, Hkv, Dv))
    tables = np.array([[0, 3, 1], [2, 3, 4]])
    lens = np.array([5, 6])
    qs, qp = np.array([0, 0, 1, 1, 1]), np.array([4, 2, 5, 0, 3])
    q = rng.standard_normal((5, Hq, D))
    g = rng.standard_normal((5, Hq, Dv))
    dq, dk, dv = O.paged_attention_backward(q, kc, vc, g, tables, lens, qs, qp, 0.9, causal)
    h = 1e-6
    for name, x, grad in (("q", q, dq), ("k", kc, dk), ("v", vc, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args_p = {"q": q, "k": kc, "v": vc}
            args_m = dict(args_p)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[name], args_m[name] = xp, xm
            num[idx] = (_paged_loss(args_p["q"], args_p["k"], args_p["v"], g, tables, lens, qs, qp,
                                    0.9, causal)
                        - _paged_loss(args_m["q"], args_m["k"], args_m["v"], g, tables, lens, qs, qp,
                                      0.9, causal)) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)
    assert not dk[5:].any() and not dv[5:].any()
    assert np.abs(dk[3]).sum() > 0


def test_paged_backward_equals_dense_backward_of_each_sequence():
    # whole-sequence causal chunks over shuffled pages: dq rows and the cache
    # slots' gradients are the dense causal backward of each sequence
    rng = np.random.default_rng(73)
    lens = [9, 4, 7]
    nseq, Hq, Hkv, D, S, ps = len(lens), 4, 2, 3, max(lens), 2
    q = rng.standard_normal((nseq, Hq, S, D))
    k = rng.standard_normal((nseq, Hkv, S, D))
    v = rng.standard_normal((nseq, Hkv, S, D))
    g = rng.standard_normal((nseq, Hq, S, D))
    kc, vc, tables = make_paged(k, v, lens, ps, 2, rng)
    qs = np.array([s for s in range(nseq) for _ in range(lens[s])])
    qp = np.array([i for s in range(nseq) for i in range(lens[s])])
    qq = np.stack([q[s, :, i] for s, i in zip(qs, qp)])
    gg = np.stack([g[s, :, i] for s, i in zip(qs, qp)])
    dq, dk, dv = O.paged_attention_backward(qq, kc, vc, gg, tables, lens, qs, qp, 0.6, True)
    reached = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(nseq):
        n = lens[s]
        rq, rk, rv = O.sdpa_backward(q[s:s + 1, :, :n], k[s:s + 1, :, :n], v[s:s + 1, :, :n],
                                     g[s:s + 1, :, :n], 0.6, O.MASK_CAUSAL)
        np.testing.assert_allclose(dq[qs == s], rq[0].transpose(1, 0, 2), rtol=0, atol=1e-12)
        for j in range(n):
            pg, sl = tables[s, j // ps], j % ps
            reached[pg, sl] = True
            np.testing.assert_allclose(dk[pg, sl], rk[0][:, j], rtol=0, atol=1e-12)
            np.testing.assert_allclose(dv[pg, sl], rv[0][:, j], rtol=0, atol=1e-12)
    assert not dk[~reached].any() and not dv[~reached].any()


def test_backward_key_gradients_sum_to_zero():
    # each row of dS sums to 0 (softmax is shift invariant), so the dK rows of
    # a K/V head sum to the zero vector
    rng = np.random.default_rng(62)
    q, k, v = rng.standard_normal((2, 6, 40, 8)), rng.standard_normal((2, 3, 40, 8)), \
        rng.standard_normal((2, 3, 40, 8))
    g = rng.standard_normal((2, 6, 40, 8))
    for mask in (O.MASK_NONE, O.MASK_CAUSAL):
        _, dk, _ = O.sdpa_backward(q, k, v, g, 0.3, mask)
        assert np.abs(dk.sum(axis=2)).max() < 1e-12


def test_backward_zero_query_closed_form():
    # Q = 0: every visible key gets weight 1/n_i, so dV_j = sum over the rows
    # that see key j of dO_i / n_i (causal: n_i = i + 1), and dK = 0
    rng = np.random.default_rng(63)
    S, D = 7, 4
    q = np.zeros((1, 1, S, D))
    k, v = rng.standard_normal((1, 1, S, D)), rng.standard_normal((1, 1, S, D))
    g = rng.standard_normal((1, 1, S, D))
    _, dk, dv = O.sdpa_backward(q, k, v, g, 1.0, O.MASK_CAUSAL)
    for j in range(S):
        ref = sum(g[0, 0, i] / (i + 1) for i in range(j, S))
        np.testing.assert_allclose(dv[0, 0, j], ref, rtol=0, atol=1e-14)
    assert np.abs(dk).max() < 1e-14


def test_backward_gqa_equals_summed_mha():
    rng = np.random.default_rng(64)
    B, Hq, Hkv, S, D = 1, 6, 2, 9, 5
    q, k, v = rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)), \
        rng.standard_normal((B, Hkv, S, D))
    g = rng.standard_normal((B, Hq, S, D))
    dq, dk, dv = O.sdpa_backward(q, k, v, g, 0.4, O.MASK_CAUSAL)
    kr, vr = np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1)
    dq2, dk2, dv2 = O.sdpa_backward(q, kr, vr, g, 0.4, O.MASK_CAUSAL)
    np.testing.assert_allclose(dq, dq2, atol=1e-13)
    np.testing.assert_allclose(dk, dk2.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv, dv2.reshape(B, Hkv, Hq // Hkv, S, D).sum(axis=2), atol=1e-13)


def test_backward_hidden_keys_and_dead_rows():
    rng = np.random.default_rng(65)
    q, k, v = rng.standard_normal((2, 2, 6, 4)), rng.standard_normal((2, 2, 6, 4)), \
        rng.standard_normal((2, 2, 6, 4))
    g = rng.standard_normal((2, 2, 6, 4))
    dq, dk, dv = O.sdpa_backward(q, k, v, g, 0.5, O.MASK_KEY_PADDING, np.array([4, 0]))
    assert (dk[0, :, 4:] == 0).all() and (dv[0, :, 4:] == 0).all()     # padded keys
    assert (dq[1] == 0).all() and (dk[1] == 0).all() and (dv[1] == 0).all()  # no visible key


# ------------------------------------------------------------------ additive bias

def _bias_inputs(seed, B=2, Hq=4, Hkv=2, Sq=6, Sk=6, D=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Hq, Sq, D)), rng.standard_normal((B, Hkv, Sk, D)),
            rng.standard_normal((B, Hkv, Sk, D)), rng)


def test_bias_zero_is_no_bias():
    q, k, v, _ = _bias_inputs(70)
    ref = O.sdpa_forward(q, k, v, 0.6, O.MASK_CAUSAL)
    got = O.sdpa_forward(q, k, v, 0.6, O.MASK_CAUSAL, bias=np.zeros((1, 1, 6, 6)))
    assert np.array_equal(ref, got)


def test_bias_of_zeros_and_minus_inf_is_the_causal_and_padding_masks():
    q, k, v, _ = _bias_inputs(71)
    tri = np.where(np.arange(6)[None, :] <= np.arange(6)[:, None], 0.0, -np.inf)
    assert np.array_equal(O.sdpa_forward(q, k, v, 0.6, O.MASK_CAUSAL),
                          O.sdpa_forward(q, k, v, 0.6, bias=tri[None, None]))
    lens = np.array([4, 2])
    pad = np.zeros((2, 1, 6, 6))
    pad[0, :, :, 4:] = -np.inf
    pad[1, :, :, 2:] = -np.inf
    assert np.array_equal(O.sdpa_forward(q, k, v, 0.6, O.MASK_KEY_PADDING, lens),
                          O.sdpa_forward(q, k, v, 0.6, bias=pad))


def test_row_constant_bias_changes_nothing():
    # softmax is shift invariant along a row
    q, k, v, rng = _bias_inputs(72)
    c = rng.standard_normal((2, 4, 6, 1)) * 5
    np.testing.assert_allclose(O.sdpa_forward(q, k, v, 0.6, bias=np.broadcast_to(c, (2, 4, 6, 6))),
                               O.sdpa_forward(q, k, v, 0.6), rtol=0, atol=1e-12)


def test_bias_zero_query_closed_form():
    # Q = 0: the weights of row i are softmax(bias[i]) exactly, independent of scale
    _, k, v, rng = _bias_inputs(73)
    q = np.zeros((2, 4, 6, 5))
    bias = rng.standard_normal((2, 4, 6, 6)) * 2
    got = O.sdpa_forward(q, k, v, 3.0, bias=bias)
    for b in range(2):
        for h in range(4):
            for i in range(6):
                w = [math.exp(x) for x in bias[b, h, i]]
                tot = math.fsum(w)
                ref = [math.fsum(w[j] / tot * v[b, h // 2, j, d] for j in range(6)) for d in range(5)]
                np.testing.assert_allclose(got[b, h, i], ref, rtol=0, atol=1e-13)


def test_bias_brute_force_is_added_after_the_scale():
    # exp(scale * q.k + bias) by scalar loops; scale != 1 separates the
    # bias from the scaled scores
    q, k, v, rng = _bias_inputs(74, B=1, Hq=2, Hkv=1, Sq=3, Sk=4, D=2)
    bias = rng.standard_normal((1, 2, 3, 4))
    got = O.sdpa_forward(q, k, v, 0.35, O.MASK_NONE, bias=bias)
    for h in range(2):
        for i in range(3):
            z = [0.35 * math.fsum(q[0, h, i, d] * k[0, 0, j, d] for d in range(2)) + bias[0, h, i, j]
                 for j in range(4)]
            w = [math.exp(x) for x in z]
            tot = math.fsum(w)
            ref = [math.fsum(w[j] / tot * v[0, 0, j, d] for j in range(4)) for d in range(2)]
            np.testing.assert_allclose(got[0, h, i], ref, rtol=0, atol=1e-13)


def test_bias_broadcasts_over_size_one_axes():
    q, k, v, rng = _bias_inputs(75)
    per_head = rng.standard_normal((1, 4, 6, 6))
    per_batch = rng.standard_normal((2, 1, 6, 6))
    np.testing.assert_array_equal(O.sdpa_forward(q, k, v, 0.6, bias=per_head),
                                  O.sdpa_forward(q, k, v, 0.6, bias=np.repeat(per_head, 2, axis=0)))
    np.testing.assert_array_equal(O.sdpa_forward(q, k, v, 0.6, bias=per_batch),
                                  O.sdpa_forward(q, k, v, 0.6, bias=np.repeat(per_batch, 4, axis=1)))
    # a query head's bias is its own, not its K/V head's
    h_only = np.zeros((1, 4, 6, 6))
    h_only[0, 1] = rng.standard_normal((6, 6)) * 3
    got = O.sdpa_forward(q, k, v, 0.6, bias=h_only)
    base = O.sdpa_forward(q, k, v, 0.6)
    assert np.array_equal(got[:, [0, 2, 3]], base[:, [0, 2, 3]])
    assert not np.allclose(got[:, 1], base[:, 1])


def test_bias_rows_equal_full_and_minus_inf_row_is_nan():
    q, k, v, rng = _bias_inputs(76)
    bias = rng.standard_normal((1, 4, 6, 6))
    bias[0, 2, 3, :] = -np.inf
    full, lse = O.sdpa_forward(q, k, v, 0.6, O.MASK_CAUSAL, bias=bias, return_lse=True)
    idx = np.array([[0, 0, 0], [1, 3, 5], [0, 2, 3], [1, 1, 2]])
    o, l = O.sdpa_forward_rows(q, k, v, 0.6, O.MASK_CAUSAL, None, idx, bias=bias)
    for n, (b, h, i) in enumerate(idx):
        np.testing.assert_allclose(o[n], full[b, h, i], rtol=0, atol=1e-14)
    assert np.isnan(full[:, 2, 3]).all() and np.isneginf(lse[:, 2, 3]).all()


# ------------------------------------------------------------------ attention block

def _block_inputs(seed, B=2, S=5, M=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, S, M))
    ws = [rng.standard_normal((M, M)) / np.sqrt(M) for _ in range(4)]
    return x, ws, rng


def test_block_single_head_is_the_essays_kernel():
    # one head, no mask, wo = I, scale 1/sqrt(model): the HOF essay's
    # compute_attention (section 4): q, k, v = x.w, exp(q k^T / sqrt(d)),
    # row sums, row-stochastic weights, weights . v -- by scalar loops
    x, (wq, wk, wv, _), _ = _block_inputs(90, B=1, S=4, M=3)
    y = O.block_forward(x, wq, wk, wv, np.eye(3), 1)
    xs = x[0]
    q = [[math.fsum(xs[i, a] * wq[a, j] for a in range(3)) for j in range(3)] for i in range(4)]
    k = [[math.fsum(xs[i, a] * wk[a, j] for a in range(3)) for j in range(3)] for i in range(4)]
    v = [[math.fsum(xs[i, a] * wv[a, j] for a in range(3)) for j in range(3)] for i in range(4)]
    for i in range(4):
        e = [math.exp(math.fsum(q[i][d] * k[j][d] for d in range(3)) / math.sqrt(3)) for j in range(4)]
        tot = math.fsum(e)
        ref = [math.fsum(e[j] / tot * v[j][d] for j in range(4)) for d in range(3)]
        np.testing.assert_allclose(y[0, i], ref, rtol=0, atol=1e-13)


def test_block_single_token_closed_form():
    # one token sees only itself: y = x . wv . wo, whatever wq, wk, the scale
    x, (wq, wk, wv, wo), _ = _block_inputs(91, S=1)
    for mask in (O.MASK_NONE, O.MASK_CAUSAL):
        y = O.block_forward(x, wq, wk, wv, wo, 2, scale=0.37, mask_kind=mask)
        np.testing.assert_allclose(y, x @ wv @ wo, rtol=0, atol=1e-13)


def test_block_causal_first_token_and_identity_projections():
    x, (wq, wk, wv, wo), _ = _block_inputs(92)
    y = O.block_forward(x, wq, wk, wv, wo, 2, mask_kind=O.MASK_CAUSAL)
    np.testing.assert_allclose(y[:, 0], x[:, 0] @ wv @ wo, rtol=0, atol=1e-13)
    # identity projections: head h attends with columns 4h..4h+3 of x
    I = np.eye(8)
    yi = O.block_forward(x, I, I, I, I, 2, mask_kind=O.MASK_CAUSAL)
    for h in range(2):
        xh = x[:, :, 4 * h:4 * h + 4]
        ref = O.sdpa_forward(xh[:, None], xh[:, None], xh[:, None], 0.5, O.MASK_CAUSAL)[:, 0]
        np.testing.assert_allclose(yi[:, :, 4 * h:4 * h + 4], ref, rtol=0, atol=1e-13)


def test_block_head_permutation_invariance():
    # permuting the heads (column blocks of wq, wk, wv and the matching row
    # blocks of wo) leaves y unchanged
    x, (wq, wk, wv, wo), _ = _block_inputs(93, M=12)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(4 * p, 4 * p + 4) for p in perm])
    y = O.block_forward(x, wq, wk, wv, wo, 3, mask_kind=O.MASK_CAUSAL)
    yp = O.block_forward(x, wq[:, cols], wk[:, cols], wv[:, cols], wo[cols], 3,
                         mask_kind=O.MASK_CAUSAL)
    np.testing.assert_allclose(y, yp, rtol=0, atol=1e-12)


def test_block_split_merge_heads_roundtrip():
    t = np.arange(2 * 3 * 12, dtype=np.float64).reshape(2, 3, 12)
    h = O.split_heads(t, 4)
    assert h.shape == (2, 4, 3, 3)
    assert h[1, 2, 0, 1] == t[1, 0, 2 * 3 + 1]      # (b, head, seq, d) <- (b, seq, head*hd + d)
    np.testing.assert_array_equal(O.merge_heads(h), t)


def test_block_rows_equal_full():
    # the row-sampled block is the full block at the listed (b, s), under
    # every mask, including a batch whose keys are all padded away (NaN rows)
    x, (wq, wk, wv, wo), _ = _block_inputs(94, B=3, S=7, M=12)
    lens = np.array([7, 3, 0])
    rows = np.array([[0, 0], [2, 6], [1, 2], [1, 5], [0, 6], [2, 0]])
    for mask in (O.MASK_NONE, O.MASK_CAUSAL, O.MASK_KEY_PADDING, 3):
        kl = lens if mask & O.MASK_KEY_PADDING else None
        full = O.block_forward(x, wq, wk, wv, wo, 3, 0.4, mask, kl)
        got = O.block_forward_rows(x, wq, wk, wv, wo, 3, rows, 0.4, mask, kl)
        np.testing.assert_allclose(got, full[rows[:, 0], rows[:, 1]], rtol=0, atol=1e-13)
        if kl is not None:
            assert np.isnan(got[rows[:, 0] == 2]).all()


# ------------------------------------------------------------------ page fixtures

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split() for l in f if l.strip() and not l.startswith("#")]


def test_golden_essay_single_row():
    rows = dict((l[0], np.array([float(x) for x in l[1:]])) for l in _golden_lines("essay_single_row.txt"))
    x = rows["input"].reshape(1, 1, 4)
    rng = np.random.default_rng(95)
    I = np.eye(4)
    for wq, wk in ((I, I), (rng.standard_normal((4, 4)), rng.standard_normal((4, 4)))):
        # the essay's scale 1 / sqrt(d) and another one: the single weight is 1 either way
        for scale in (0.5, 3.0):
            y = O.block_forward(x, wq, wk, I, I, 1, scale)
            np.testing.assert_allclose(y.reshape(4), rows["output"], rtol=0, atol=1e-15)


def test_golden_tensai_causal_mask():
    m = np.array([[float(x) for x in l] for l in _golden_lines("tensai_causal_mask_seq4.txt")])
    assert m.shape == (4, 4)
    # the causal flag hides exactly the -inf entries ...
    vis = O.visible_rows(O.MASK_CAUSAL, np.arange(4), 4, 0)
    np.testing.assert_array_equal(vis, m == 0)
    # ... and adding the page's mask as a bias gives the flag's result
    rng = np.random.default_rng(96)
    q, k, v = (rng.standard_normal((2, 3, 4, 8)) for _ in range(3))
    via_flag = O.sdpa_forward(q, k, v, 0.3, O.MASK_CAUSAL)
    via_bias = O.sdpa_forward(q, k, v, 0.3, O.MASK_NONE, bias=m[None, None])
    np.testing.assert_array_equal(via_bias, via_flag)


# ------------------------------------------------------------------ backward with a bias

def _loss_bias(q, k, v, g, scale, mask, lens, bias):
    return float((O.sdpa_forward(q, k, v, scale, mask, lens, bias=bias) * g).sum())


@pytest.mark.parametrize("mask,lens", [(O.MASK_NONE, None), (O.MASK_CAUSAL, None),
                                       (O.MASK_KEY_PADDING, [4, 6])])
def test_backward_bias_matches_finite_differences(mask, lens):
    # central differences of L = sum(O * G) through the (pinned) biased
    # forward, for q, k, v and every finite bias entry; some entries are -inf
    rng = np.random.default_rng(66 + mask)
    B, Hq, Hkv, S, D = 2, 4, 2, 6, 3
    q, k, v = (rng.standard_normal((B, Hq, S, D)), rng.standard_normal((B, Hkv, S, D)),
               rng.standard_normal((B, Hkv, S, D)))
    g = rng.standard_normal((B, Hq, S, D))
    bias = 1.5 * rng.standard_normal((B, Hq, S, S))
    bias[0, 1, 2, [0, 3]] = -np.inf
    bias[1, 3, 4, 1] = -np.inf
    lens = None if lens is None else np.array(lens)
    dq, dk, dv, db = O.sdpa_backward(q, k, v, g, 0.7, mask, lens, bias=bias, return_dbias=True)
    h = 1e-6
    args = {"q": q, "k": k, "v": v, "bias": bias}
    for name, grad in (("q", dq), ("k", dk), ("v", dv), ("bias", db)):
        x = args[name]
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            if not np.isfinite(x[idx]):
                continue
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            ap, am = dict(args), dict(args)
            ap[name], am[name] = xp, xm
            num[idx] = (_loss_bias(ap["q"], ap["k"], ap["v"], g, 0.7, mask, lens, ap["bias"])
                        - _loss_bias(am["q"], am["k"], am["v"], g, 0.7, mask, lens, am["bias"])) / (2 * h)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-7, err_msg=name)
    # entries hidden by the -inf bias or the mask get no gradient
    assert db[0, 1, 2, 0] == 0 and db[0, 1, 2, 3] == 0 and db[1, 3, 4, 1] == 0


def test_backward_bias_rows_sum_to_zero_and_zero_bias():
    rng = np.random.default_rng(69)
    q, k, v = rng.standard_normal((2, 4, 30, 8)), rng.standard_normal((2, 2, 30, 8)), \
        rng.standard_normal((2, 2, 30, 8))
    g = rng.standard_normal((2, 4, 30, 8))
    bias = rng.standard_normal((2, 4, 30, 30))
    _, _, _, db = O.sdpa_backward(q, k, v, g, 0.3, O.MASK_CAUSAL, bias=bias, return_dbias=True)
    # the softmax gradient of every row sums to zero (shift invariance)
    assert np.abs(db.sum(axis=3)).max() < 1e-12
    # a zero bias changes nothing, bit for bit
    base = O.sdpa_backward(q, k, v, g, 0.3, O.MASK_CAUSAL)
    zero = O.sdpa_backward(q, k, v, g, 0.3, O.MASK_CAUSAL, bias=np.zeros((1, 1, 30, 30)))
    for a, b in zip(base, zero):
        np.testing.assert_array_equal(a, b)


def test_backward_bias_dead_row_from_the_bias():
    # a row whose visible keys all carry -inf bias has no output and no gradient
    rng = np.random.default_rng(70)
    q, k, v = rng.standard_normal((1, 2, 5, 4)), rng.standard_normal((1, 1, 5, 4)), \
        rng.standard_normal((1, 1, 5, 4))
    g = rng.standard_normal((1, 2, 5, 4))
    bias = np.zeros((1, 2, 5, 5))
    bias[0, 1, 3, :] = -np.inf
    dq, dk, dv, db = O.sdpa_backward(q, k, v, g, 0.5, O.MASK_NONE, bias=bias, return_dbias=True)
    assert (dq[0, 1, 3] == 0).all() and (db[0, 1, 3] == 0).all() and np.isfinite(dk).all()
