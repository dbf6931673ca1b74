"""The entry points under HIP graph capture: the library allocates nothing and
enqueues no memset, so a captured call replays the same kernels.  Each replay
is checked bit for bit against the eager result, with eager work and
synchronizations between the replays."""

import math

import pytest
import torch

import exact_scaled_dot_amd as sd
from exact_scaled_dot_amd.workloads import draw_block, draw_qkv

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def test_graph_replays_match_eager():
    BF16 = torch.bfloat16
    q, k, v = draw_qkv(2, 8, 2, 300, 300, 128, BF16, 1040, DEV)
    qd, kd, vd = draw_qkv(4, 16, 4, 1, 3000, 128, BF16, 1041, DEV)
    lens = torch.tensor([3000, 17, 1500, 2999], dtype=torch.int32, device=DEV)
    x, wq, wk, wv, wo = draw_block(8, 128, 256, BF16, 1042, DEV)
    ws = torch.empty(sd.sdpa_decode_workspace_size(4, 16, 128, 8), dtype=torch.uint8, device=DEV)
    bws = torch.empty(sd.sdpa_block_workspace_size(8, 128, 256), dtype=torch.uint8, device=DEV)
    out_p, out_d, y = torch.empty_like(q), torch.empty_like(qd), torch.empty_like(x)

    def calls():
        sd.sdpa_forward(q, k, v, 1 / math.sqrt(128), sd.MASK_CAUSAL, None, out_p)
        sd.sdpa_decode(qd, kd, vd, 1 / math.sqrt(128), lens, 8, ws, out_d)
        sd.sdpa_block_forward(x, wq, wk, wv, wo, 4, None, sd.MASK_CAUSAL, None, y, bws)

    calls()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (out_p, out_d, y)]

    stream = torch.cuda.Stream()  # default priority
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        calls()  # warm the capture stream
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    for rep in range(3):
        for t in (out_p, out_d, y):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, ref in zip((out_p, out_d, y), eager):
            assert torch.equal(got, ref), "replay %d differs from the eager result" % rep
        # eager work between replays
        calls()
        torch.cuda.synchronize()
