"""sdpa_decode_noalloc (partials in the library's static device scratch) gives
the same output as sdpa_decode (caller's workspace) through the C ABI, on
calls in a row whose later inputs are smaller than the first, so stale
partials of a larger call sit in the scratch."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_qkv
from parity import compare, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def both(B, Hq, Hkv, Sk, D, splits, lens, dtype, seed):
    scale = 1.0 / math.sqrt(D)
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, dtype, seed, DEV)
    key_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    print("noalloc decode B%d Hq%d Hkv%d Sk%d D%d splits%d %s" % (B, Hq, Hkv, Sk, D, splits, dtype),
          flush=True)
    got = torch.full_like(q, float("nan"))
    sd.sdpa_decode_noalloc(q, k, v, scale, got, key_lens, splits)
    ws = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, splits), dtype=torch.uint8, device=DEV)
    ref = sd.sdpa_decode(q, k, v, scale, key_lens, splits, workspace=ws)
    torch.cuda.synchronize()
    return q, k, v, scale, got, ref


def test_noalloc_matches_decode_on_shrinking_calls():
    rng = np.random.default_rng(5)
    cases = [
        # the 64-sequence, 32-head grouped decode at 32 splits (33.8 MB of partials)
        (64, 32, 8, 4096, 128, 32, [int(x) for x in rng.integers(1, 4097, 64)], torch.bfloat16),
        # then smaller: fewer sequences, splits and keys, a ragged key count
        (3, 8, 2, 1000, 128, 7, None, torch.bfloat16),
        (2, 4, 4, 333, 64, 5, [333, 17], torch.float16),
    ]
    for i, (B, Hq, Hkv, Sk, D, splits, lens, dtype) in enumerate(cases):
        q, k, v, scale, got, ref = both(B, Hq, Hkv, Sk, D, splits, lens, dtype, 100 + i)
        # the same kernels on the same partition: bit-identical to sdpa_decode
        assert torch.equal(got, ref), "call %d differs from sdpa_decode" % i
        if i > 0:
            nl = None if lens is None else np.array(lens)
            compare(to64(got), O.sdpa_decode(to64(q), to64(k), to64(v), scale, nl), dtype,
                    "noalloc call %d" % i)


def test_noalloc_wide_heads_then_narrow():
    # above 256 dims the split pass runs on the head-dim-split kernel: it writes
    # the same partials, here into the scratch
    for i, (B, Hq, Hkv, Sk, D, splits) in enumerate([(4, 16, 4, 2048, 512, 16),
                                                    (1, 2, 1, 100, 128, 3)]):
        q, k, v, scale, got, ref = both(B, Hq, Hkv, Sk, D, splits, None, torch.bfloat16, 200 + i)
        assert torch.equal(got, ref), "call %d differs from sdpa_decode" % i


def test_noalloc_rejects_oversize_without_launching():
    q, k, v = draw_qkv(128, 32, 8, 1, 16, 128, torch.bfloat16, 7, DEV)
    out = torch.full_like(q, 3.0)
    with pytest.raises(sd.SdpaError) as e:
        sd.sdpa_decode_noalloc(q, k, v, 0.1, out, None, 32)
    assert e.value.status == sd.SDPA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
