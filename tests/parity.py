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


def compare_grad(got, ref, dtype, what=""):
    """Assert the backward bars on one gradient tensor; returns (max_rel, rel_l2)."""
    assert np.isfinite(np.asarray(got, dtype=np.float64)).all(), "%s: non-finite gradient" % what
    return compare_rel(got, ref, GRAD_REL_L2[dtype], GRAD_MAX_REL[dtype], what)


def compare_block(got, ref, dtype, what=""):
    """Assert the attention-block bars on y; returns (max_rel, rel_l2)."""
    return compare_rel(got, ref, BLOCK_REL_L2[dtype], BLOCK_MAX_REL[dtype], what)
