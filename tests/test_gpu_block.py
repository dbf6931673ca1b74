"""GPU parity of the multi-head attention block (sdpa_block_forward: the q, k,
v projections, the attention, the output projection) against the fp64
oracle's block_forward on the same 16-bit x and weights.  Bars:
tests/parity.py, BLOCK_*."""

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_block
from parity import compare_block, run_threaded, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16, F16 = torch.bfloat16, torch.float16


def run_block(B, S, model, heads, dtype, seed, mask=0, lens=None, scale=None):
    x, wq, wk, wv, wo = draw_block(B, S, model, dtype, seed, DEV)
    y = sd.sdpa_block_forward(x, wq, wk, wv, wo, heads, scale, mask, lens)
    torch.cuda.synchronize()
    return (x, wq, wk, wv, wo), y


def oracle_block(ins, heads, mask=0, lens=None, scale=None):
    ln = None if lens is None else lens.cpu().numpy()
    return O.block_forward(*(to64(t) for t in ins), heads, scale, mask, ln)


def test_block_tensai_shape():
    # the small causal block of the tensai guide: batch 8, 4 heads of 64, 128 tokens
    ins, y = run_block(8, 128, 256, 4, BF16, 900, sd.MASK_CAUSAL)
    compare_block(to64(y), oracle_block(ins, 4, O.MASK_CAUSAL), BF16, "tensai block")


@pytest.mark.parametrize("dtype", [BF16, F16], ids=["bf16", "f16"])
@pytest.mark.parametrize("mask", [0, 1, 2, 3], ids=["none", "causal", "padding", "causal+padding"])
def test_block_parity(dtype, mask):
    # 600 rows = 2 full 256-row tiles + a ragged one; 512 columns = 4 column tiles
    B, S, M, H = 2, 300, 512, 8
    lens = torch.tensor([300, 97], dtype=torch.int32, device=DEV) if mask & 2 else None
    ins, y = run_block(B, S, M, H, dtype, 910 + mask, mask, lens)
    compare_block(to64(y), oracle_block(ins, H, mask, lens), dtype, "block %s mask=%d" % (dtype, mask))


@pytest.mark.parametrize("M,H", [(1024, 8), (136, 17), (200, 5), (96, 1), (48, 6)],
                         ids=["hd128", "hd8", "hd40", "hd96", "hd8x6"])
def test_block_widths(M, H):
    # model widths that are not multiples of the 128-column tile or the
    # 32-deep contraction step, and every head-dim path of the attention
    ins, y = run_block(2, 77, M, H, BF16, 920 + M, sd.MASK_CAUSAL, scale=0.2)
    compare_block(to64(y), oracle_block(ins, H, O.MASK_CAUSAL, scale=0.2), BF16, "block M=%d H=%d" % (M, H))


def test_block_dead_batch_and_single_token():
    # key_lens 0: every row of batch 1 attends to nothing, its y rows are NaN
    # like the oracle's; S = 1 reduces the attention to the value row
    lens = torch.tensor([5, 0], dtype=torch.int32, device=DEV)
    ins, y = run_block(2, 9, 128, 2, BF16, 930, sd.MASK_KEY_PADDING, lens)
    ref = oracle_block(ins, 2, O.MASK_KEY_PADDING, lens)
    assert np.isnan(ref[1]).all()
    compare_block(to64(y), ref, BF16, "dead batch")
    ins, y = run_block(3, 1, 256, 4, F16, 931, sd.MASK_CAUSAL)
    compare_block(to64(y), oracle_block(ins, 4, O.MASK_CAUSAL), F16, "single token")


def test_block_deterministic_and_caller_buffers():
    x, wq, wk, wv, wo = draw_block(2, 200, 384, BF16, 940, DEV)
    ws = torch.empty(sd.sdpa_block_workspace_size(2, 200, 384), dtype=torch.uint8, device=DEV)
    y = torch.empty_like(x)
    a = sd.sdpa_block_forward(x, wq, wk, wv, wo, 6, None, sd.MASK_CAUSAL, y=y, workspace=ws).clone()
    ws.fill_(0xFF)  # NaN patterns in the workspace do not leak into the next call
    b = sd.sdpa_block_forward(x, wq, wk, wv, wo, 6, None, sd.MASK_CAUSAL, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_block_full_size_whole_output():
    # the causal prefill workload as a block: batch 4, 4096 tokens, 16 heads
    # of 128 (model 2048); every row of y against the oracle, one batch per
    # thread (its projections and attention computed whole)
    B, S, M, H = 4, 4096, 2048, 16
    ins, y = run_block(B, S, M, H, BF16, 950, sd.MASK_CAUSAL)
    x = ins[0].cpu()
    w64 = [to64(t) for t in ins[1:]]
    ref = np.empty((B, S, M))

    def one(b):
        xb = x[b:b + 1].double().numpy()
        rows = np.stack([np.zeros(S, dtype=np.int64), np.arange(S)], axis=1)
        ref[b] = O.block_forward_rows(xb, *w64, H, rows, None, O.MASK_CAUSAL)

    run_threaded(one, range(B))
    compare_block(to64(y), ref, BF16, "full-size block")


def test_block_tile_sizes():
    # the projections pick 256-, 128- or 64-wide tiles by grid size: batch 4,
    # 512 tokens, model 1024 runs the q/k/v projections on 128 x 128 tiles
    # (384 workgroups) and the output projection on 64 x 64 ones; the small
    # and full-size tests above cover 64 and 256
    ins, y = run_block(4, 512, 1024, 8, BF16, 960, sd.MASK_CAUSAL)
    compare_block(to64(y), oracle_block(ins, 8, O.MASK_CAUSAL), BF16, "block 128-wide tiles")
