"""Tolerance checks shared by the GPU parity tests.

Bars: fp32 inputs, max |O_gpu - O_ref| <= 1e-4; bf16 inputs, max-abs <= 2e-2
and ||O_gpu - O_ref||_2 / ||O_ref||_2 <= 5e-3 over the compared elements; no
NaN or Inf anywhere (unless the reference row itself is NaN: a row with no
visible key).  O_ref is the fp64 oracle output, never rounded first.
"""

import numpy as np
import torch

F32_MAX_ABS = 1e-4
BF16_MAX_ABS = 2e-2
BF16_REL_L2 = 5e-3

# Backward (dQ, dK, dV): P and dS are rounded to the input type before their
# products, and each gradient to the input type at the end.  Bars per gradient
# tensor, relative to its own scale: ||g - r||_2 / ||r||_2 and
# max|g - r| / max|r|.
GRAD_REL_L2 = {torch.bfloat16: 1e-2, torch.float16: 2e-3}
GRAD_MAX_REL = {torch.bfloat16: 4e-2, torch.float16: 8e-3}
# fp32 inputs: nothing is rounded to 16 bits; every product is exact in fp32
# and each sum carries a relative error of order sqrt(n) * 2^-24 (about 1e-6
# over a few hundred keys), the recomputed exponentials about 2^-22.  Bars at
# about 10x and 100x that.
GRAD_REL_L2[torch.float32] = 1e-5
GRAD_MAX_REL[torch.float32] = 1e-4

# Attention block y (projections, attention, output projection): q, k, v, the
# attention output and y are each rounded to the input type (unit roundoff u
# = 2^-9 bf16, 2^-12 fp16), and P inside the attention; each rounding adds a
# relative error of RMS about u/sqrt(3) that the following sums carry through
# unchanged in relative terms, so five of them give rel-L2 about 2.5e-3 (bf16)
# or 3e-4 (fp16).  Bars at 4x and 6x that, relative to y's own scale.
BLOCK_REL_L2 = {torch.bfloat16: 1e-2, torch.float16: 2e-3}
BLOCK_MAX_REL = {torch.bfloat16: 4e-2, torch.float16: 8e-3}


def to64(t):
    return t.detach().to("cpu", torch.float64).numpy()


def host_workers():
    """Oracle threads: the cores this process may use, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_threaded(fn, items, workers=None):
    """fn over items on a thread pool (NumPy releases the GIL in its array
    loops), BLAS held to one thread per call so the pool does not oversubscribe
    the cores.  Returns the results in order."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1, user_api="blas"):
        with ThreadPoolExecutor(min(workers or 16, host_workers())) as ex:
            return list(ex.map(fn, items))


def oracle_forward_whole(oracle, q, k, v, scale, mask_kind, key_lens=None, row_block=1024,
                         return_lse=False, workers=None, bias=None):
    """The oracle's forward over every (b, h, i) of q [B,Hq,Sq,D], k / v
    [B,Hkv,Sk,D] (device or host tensors; bias None or [B or 1, Hq or 1, Sq,
    Sk]): one head per thread, query rows in blocks of row_block (so an
    8192 x 8192 fp64 score block never exists whole).  Inputs are copied to the
    host in their own dtype and widened to fp64 one head at a time.  Returns
    o [B,Hq,Sq,D] fp64 (and lse [B,Hq,Sq])."""
    qh, kh, vh = (t.detach().cpu() for t in (q, k, v))
    bh_all = None if bias is None else bias.detach().cpu()
    B, Hq, Sq, D = qh.shape
    G = Hq // kh.shape[1]
    lens = None if key_lens is None else np.asarray(key_lens)
    ref = np.empty((B, Hq, Sq, D), dtype=np.float64)
    lse = np.empty((B, Hq, Sq), dtype=np.float64)

    def head(bh):
        b, h = bh
        q1 = qh[b, h].double().numpy()[None, None]
        k1 = kh[b, h // G].double().numpy()[None, None]
        v1 = vh[b, h // G].double().numpy()[None, None]
        b1 = None
        if bh_all is not None:
            b1 = bh_all[b if bh_all.shape[0] > 1 else 0, h if bh_all.shape[1] > 1 else 0]
            b1 = b1.double().numpy()[None, None]
        for r0 in range(0, Sq, row_block):
            rows = np.arange(r0, min(Sq, r0 + row_block))
            idx = np.stack([np.zeros_like(rows), np.zeros_like(rows), rows], axis=1)
            o, l = oracle.sdpa_forward_rows(q1, k1, v1, scale, mask_kind,
                                            None if lens is None else lens[b:b + 1], idx,
                                            bias=b1)
            ref[b, h, r0:r0 + len(rows)] = o
            lse[b, h, r0:r0 + len(rows)] = l

    run_threaded(head, [(b, h) for b in range(B) for h in range(Hq)], workers)
    return (ref, lse) if return_lse else ref


def oracle_decode_whole(oracle, q, k, v, scale, key_lens=None):
    """The oracle's decode over every (b, h) of q [B,Hq,1,D], k / v
    [B,Hkv,Sk,D] (device or host tensors): one (batch, K/V head) group per
    thread, its query heads together.  Returns o [B,Hq,1,D] fp64."""
    qh, kh, vh = (t.detach().cpu() for t in (q, k, v))
    B, Hq, _, D = qh.shape
    Hkv = kh.shape[1]
    G = Hq // Hkv
    lens = None if key_lens is None else np.asarray(key_lens)
    ref = np.empty((B, Hq, 1, D), dtype=np.float64)

    def group(bg):
        b, g = bg
        hs = slice(g * G, (g + 1) * G)
        ref[b:b + 1, hs] = oracle.sdpa_decode(
            qh[b:b + 1, hs].double().numpy(), kh[b:b + 1, g:g + 1].double().numpy(),
            vh[b:b + 1, g:g + 1].double().numpy(), scale, None if lens is None else lens[b:b + 1])

    run_threaded(group, [(b, g) for b in range(B) for g in range(Hkv)])
    return ref


def compare(got, ref, dtype, what=""):
    """Assert the bars; returns (max_abs, rel_l2) for reporting."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs" % what
    g, r = got[~nan_ref], ref[~nan_ref]
    assert np.isfinite(g).all(), "%s: non-finite output" % what
    if g.size == 0:
        return 0.0, 0.0
    max_abs = float(np.abs(g - r).max())
    den = float(np.linalg.norm(r))
    rel = float(np.linalg.norm(g - r) / den) if den > 0 else float(np.linalg.norm(g - r))
    if dtype == torch.float32:
        assert max_abs <= F32_MAX_ABS, "%s: max-abs %.3e > %.0e" % (what, max_abs, F32_MAX_ABS)
    else:
        assert max_abs <= BF16_MAX_ABS, "%s: max-abs %.3e > %.0e" % (what, max_abs, BF16_MAX_ABS)
        assert rel <= BF16_REL_L2, "%s: rel-L2 %.3e > %.0e" % (what, rel, BF16_REL_L2)
    return max_abs, rel


def sample_rows(B, Hq, Sq, n, seed, must=()):
    """n distinct (b, h, i) rows: the listed ones, tile edges, and random ones."""
    rng = np.random.default_rng(seed)
    rows = set(tuple(int(x) for x in m) for m in must)
    edges = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, Sq // 2, Sq - 2, Sq - 1]
    for i in edges:
        if 0 <= i < Sq:
            rows.add((int(rng.integers(B)), int(rng.integers(Hq)), i))
    while len(rows) < n:
        rows.add((int(rng.integers(B)), int(rng.integers(Hq)), int(rng.integers(Sq))))
    return np.array(sorted(rows), dtype=np.int64)


def compare_rel(got, ref, rel_l2, max_rel, what=""):
    """Assert ||got - ref||_2 / ||ref||_2 <= rel_l2 and max|got - ref| / max|ref|
    <= max_rel over the elements where ref is not NaN (the NaN patterns must
    agree); returns (max_rel, rel_l2) measured."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs" % what
    got, ref = got[~nan_ref], ref[~nan_ref]
    assert np.isfinite(got).all(), "%s: non-finite value" % what
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    if scale == 0.0:
        assert not got.any(), "%s: reference is 0, got nonzero" % what
        return 0.0, 0.0
    mr = float(np.abs(got - ref).max()) / scale
    rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
    print("%s: max-rel %.3e rel-L2 %.3e" % (what, mr, rel))
    assert rel <= rel_l2, "%s: rel-L2 %.3e > %.0e" % (what, rel, rel_l2)
    assert mr <= max_rel, "%s: max-rel %.3e > %.0e" % (what, mr, max_rel)
    return mr, rel


def rel_stats(got, ref, what=""):
    """Pieces of compare_rel's measures for one slice of a tensor:
    (sum (g-r)^2, sum r^2, max|g-r|, max|r|) over the non-NaN reference
    elements, after the same NaN-pattern and finiteness checks."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    nan_ref = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan_ref), "%s: NaN pattern differs" % what
    got, ref = got[~nan_ref], ref[~nan_ref]
    assert np.isfinite(got).all(), "%s: non-finite value" % what
    if ref.size == 0:
        return 0.0, 0.0, 0.0, 0.0
    d = got - ref
    return float(d @ d), float(ref @ ref), float(np.abs(d).max()), float(np.abs(ref).max())


def check_rel_stats(stats, rel_l2, max_rel, what=""):
    """compare_rel's bars over a whole tensor from the rel_stats of its slices."""
    d2 = sum(x[0] for x in stats)
    r2 = sum(x[1] for x in stats)
    dmax = max(x[2] for x in stats)
    rmax = max(x[3] for x in stats)
    if rmax == 0.0:
        assert dmax == 0.0, "%s: reference is 0, got nonzero" % what
        return 0.0, 0.0
    mr, rel = dmax / rmax, float(np.sqrt(d2 / r2))
    print("%s: max-rel %.3e rel-L2 %.3e" % (what, mr, rel))
    assert rel <= rel_l2, "%s: rel-L2 %.3e > %.0e" % (what, rel, rel_l2)
    assert mr <= max_rel, "%s: max-rel %.3e > %.0e" % (what, mr, max_rel)
    return mr, rel


def backward_whole_check(oracle, q, k, v, dout, scale, mask_kind, grads, dtype, what,
                         key_lens=None, bias=None, dbias=None):
    """Every (b, h) head of the gradients against the oracle's backward, one
    head per thread, the backward bars taken over each whole gradient tensor
    (dq, dk, dv and, with a bias, dbias [B, Hq, Sq, Sk]) without building the
    whole fp64 reference.  Needs Hq == Hkv (each head's dk, dv is its own)."""
    hosts = [t.detach().cpu() for t in (q, k, v, dout)]
    gh = [t.detach().cpu() for t in grads] + ([dbias.detach().cpu()] if dbias is not None else [])
    bh = None if bias is None else bias.detach().cpu()
    B, Hq = q.shape[:2]
    assert k.shape[1] == Hq, "one K/V head per query head"
    lens = None if key_lens is None else np.asarray(key_lens)

    def head(bh_):
        b, h = bh_
        sl = (slice(b, b + 1), slice(h, h + 1))
        kw = {}
        if bh is not None:
            kw = dict(bias=bh[:, h:h + 1].double().numpy(), return_dbias=True)
        refs = oracle.sdpa_backward(*(t[sl].double().numpy() for t in hosts), scale, mask_kind,
                                    None if lens is None else lens[b:b + 1], **kw)
        out = []
        for g, r in zip(gh, refs):
            out.append(rel_stats(g[sl].double().numpy(), r, "%s b=%d h=%d" % (what, b, h)))
        return out

    res = run_threaded(head, [(b, h) for b in range(B) for h in range(Hq)])
    names = ["dq", "dk", "dv", "dbias"]
    for i in range(len(gh)):
        check_rel_stats([r[i] for r in res], GRAD_REL_L2[dtype], GRAD_MAX_REL[dtype],
                        "%s %s" % (what, names[i]))


def compare_grad(got, ref, dtype, what=""):
    """Assert the backward bars on one gradient tensor; returns (max_rel, rel_l2)."""
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), "%s: non-finite gradient" % what
    return compare_rel(got, ref, GRAD_REL_L2[dtype], GRAD_MAX_REL[dtype], what)


def compare_block(got, ref, dtype, what=""):
    """Assert the attention-block bars on y; returns (max_rel, rel_l2)."""
    return compare_rel(got, ref, BLOCK_REL_L2[dtype], BLOCK_MAX_REL[dtype], what)
