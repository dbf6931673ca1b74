"""GPU parity of sdpa_paged_attention (paged K/V cache, packed queries) against
the fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import exact_scaled_dot_amd as sd
import oracle as O
from exact_scaled_dot_amd.workloads import draw_paged, draw_qkv
from parity import compare, oracle_forward_whole, run_threaded, to64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def run_paged(seq_lens, query_seq, query_pos, Hq, Hkv, D, page_size, causal, splits, seed,
              max_seq_len=None, scale=None, tables=None):
    inp = draw_paged(seq_lens, query_seq, query_pos, Hq, Hkv, D, page_size, torch.bfloat16, seed, DEV)
    if tables is not None:
        inp["block_tables"] = torch.tensor(tables, dtype=torch.int32, device=DEV)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    if max_seq_len is None:
        max_seq_len = inp["block_tables"].shape[1] * page_size
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                  causal, max_seq_len, splits)
    torch.cuda.synchronize()
    return inp, out, scale


def oracle_of(inp, scale, causal):
    return O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                             inp["block_tables"].cpu().numpy(), inp["seq_lens"].cpu().numpy(),
                             inp["query_seq"].cpu().numpy(), inp["query_pos"].cpu().numpy(),
                             scale, causal)


def check(seq_lens, query_seq, query_pos, Hq, Hkv, D, page_size, causal, splits, seed, **kw):
    inp, out, scale = run_paged(seq_lens, query_seq, query_pos, Hq, Hkv, D, page_size, causal,
                                splits, seed, **kw)
    ref = oracle_of(inp, scale, causal)
    what = "lens=%s ps=%d Hq=%d Hkv=%d D=%d causal=%d splits=%d" % (
        seq_lens, page_size, Hq, Hkv, D, causal, splits)
    return compare(to64(out), ref, torch.bfloat16, what)


@pytest.mark.parametrize("page_size", [16, 32, 64])
@pytest.mark.parametrize("splits", [1, 4, 32])
def test_paged_decode(page_size, splits):
    # one query per sequence at its last position; ragged lengths around the
    # 16-key step and page boundaries
    lens = [1, 15, 16, 17, 100, 1000]
    n = len(lens)
    for causal in (False, True):
        check(lens, range(n), [x - 1 for x in lens], 8, 2, 128, page_size, causal, splits,
              seed=page_size + splits + causal)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_paged_decode_group_sizes(D, G):
    lens = [300, 77]
    check(lens, [0, 1], [299, 76], 2 * G, 2, D, 16, True, 5, seed=G + D)


def test_paged_packed_prefill():
    # every position of three sequences as packed queries, causal by position
    lens = [37, 5, 100]
    qs = [s for s, n in enumerate(lens) for _ in range(n)]
    qp = [i for n in lens for i in range(n)]
    check(lens, qs, qp, 4, 2, 128, 16, True, 3, seed=11)
    check(lens, qs, qp, 4, 4, 64, 32, False, 1, seed=12)


def test_paged_chunked_prefill_bottom_right():
    # 20 new queries at the end of a 300-key sequence and 7 at the end of a
    # 1000-key one, interleaved in the packed order
    qs = [0, 1] * 7 + [0] * 13
    qp = [280 + i // 2 if i % 2 == 0 else 993 + i // 2 for i in range(14)] + list(range(287, 300))
    check([300, 1000], qs, qp, 8, 2, 128, 16, True, 8, seed=13)


def test_paged_random_positions_and_order():
    rng = np.random.default_rng(14)
    lens = [64, 513, 2000, 16]
    qs = rng.integers(0, 4, size=40)
    qp = [int(rng.integers(0, lens[s])) for s in qs]
    for causal in (False, True):
        check(lens, qs.tolist(), qp, 8, 1, 128, 16, causal, 7, seed=15 + causal)


def test_paged_empty_and_out_of_range():
    # seq_len 0, a query of an unknown sequence, and a causal query at a
    # negative position see no key: NaN rows, the rest unaffected
    inp, out, scale = run_paged([0, 50, 30], [0, 1, 2, 1, 1], [0, 49, 29, 10, 20], 4, 2, 128, 16,
                                True, 4, seed=16)
    inp["query_seq"][3] = 7
    inp["query_pos"][4] = -1
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                  64, 4)
    torch.cuda.synchronize()
    got = to64(out)
    assert np.isnan(got[[0, 3, 4]]).all()
    keep = [1, 2]
    ref = O.paged_attention(to64(inp["q"])[keep], to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), inp["seq_lens"].cpu().numpy(),
                            inp["query_seq"].cpu().numpy()[keep], inp["query_pos"].cpu().numpy()[keep],
                            scale, True)
    compare(got[keep], ref, torch.bfloat16, "valid rows next to empty ones")


def test_paged_invalid_table_entries_hide_their_keys():
    # logical pages 1 and 3 of a 64-key sequence point outside the cache: the
    # kernel must not read them and must hide their keys (non-causal, so the
    # result is the attention over logical pages 0 and 2 alone)
    inp, out, scale = run_paged([64], [0, 0], [63, 63], 4, 2, 128, 16, False, 2, seed=17,
                                tables=[[0, -1, 2, 99999]])
    valid = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                              np.array([[0, 2]]), np.array([32]), np.array([0, 0]),
                              np.array([31, 31]), scale, False)
    compare(to64(out), valid, torch.bfloat16, "invalid pages hidden")


def test_paged_decode_matches_dense_decode_bitwise():
    # Same keys, contiguous pages in order, splits of a multiple of 16 keys:
    # the paged and the dense decode run the same arithmetic.
    B, Hq, Hkv, Sk, D, ps = 3, 16, 4, 1024, 128, 64
    q, k, v = draw_qkv(B, Hq, Hkv, 1, Sk, D, torch.bfloat16, 18, DEV)
    kc = torch.cat([k[b].permute(1, 0, 2).reshape(Sk // ps, ps, Hkv, D) for b in range(B)]).contiguous()
    vc = torch.cat([v[b].permute(1, 0, 2).reshape(Sk // ps, ps, Hkv, D) for b in range(B)]).contiguous()
    tables = torch.arange(B * Sk // ps, dtype=torch.int32, device=DEV).view(B, Sk // ps)
    i32 = dict(dtype=torch.int32, device=DEV)
    lens = torch.full((B,), Sk, **i32)
    got = sd.sdpa_paged_attention(q[:, :, 0].contiguous(), kc, vc, tables, lens,
                                  torch.arange(B, **i32), torch.full((B,), Sk - 1, **i32), 0.09,
                                  True, Sk, 8)
    ref = sd.sdpa_decode(q, k, v, 0.09, None, 8)
    torch.cuda.synchronize()
    assert torch.equal(got, ref[:, :, 0])


def test_paged_deterministic():
    inp, a, scale = run_paged([5000, 3000], [0, 1], [4999, 2999], 32, 8, 128, 16, True, 32, seed=19)
    b = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                inp["block_tables"].shape[1] * 16, 32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size_paged_decode_whole_output():
    # the serving shape next to the dense decode workload: 64 sequences of
    # 32768 cached keys in 16-key pages, shuffled; every query against the
    # oracle (one query per thread, over that query's own pages)
    n, L = 64, 32768
    inp = draw_paged([L] * n, range(n), [L - 1] * n, 32, 8, 128, 16, torch.bfloat16, 20, DEV,
                     extra_pages=0)
    scale = 1.0 / math.sqrt(128)
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                  L, 32)
    torch.cuda.synchronize()
    tables = inp["block_tables"].cpu().numpy()
    qh, kc, vc = (inp[x].cpu() for x in ("q", "k_cache", "v_cache"))
    ref = np.empty((n, 32, 128))

    def one(t):
        pg = torch.as_tensor(tables[t]).long()
        ref[t:t + 1] = O.paged_attention(qh[t:t + 1].double().numpy(), kc[pg].double().numpy(),
                                         vc[pg].double().numpy(), np.arange(len(pg))[None, :],
                                         np.array([L]), np.array([0]), np.array([L - 1]), scale,
                                         True)

    run_threaded(one, range(n), workers=8)
    max_abs, rel = compare(to64(out), ref, torch.bfloat16, "paged decode whole output")
    print("paged decode whole output: max-abs %.3e rel-L2 %.3e" % (max_abs, rel))


# ------------------------------------------------------------ prefill chunks

def run_prefill(seq_lens, chunks, Hq, Hkv, D, page_size, causal, seed, tables=None, max_q=None,
                scale=None):
    nq = int(sum(chunks))
    inp = draw_paged(seq_lens, [0] * nq, [0] * nq, Hq, Hkv, D, page_size, torch.bfloat16, seed, DEV)
    if tables is not None:
        inp["block_tables"] = torch.tensor(tables, dtype=torch.int32, device=DEV)
    cu = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    max_q = max(chunks) if max_q is None else max_q
    out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], torch.tensor(cu, device=DEV), scale, causal,
                                max_q, inp["block_tables"].shape[1] * page_size)
    torch.cuda.synchronize()
    qs, qp = O.chunk_positions(cu, seq_lens)
    return inp, out, scale, cu, qs, qp


def check_prefill(seq_lens, chunks, Hq, Hkv, D, page_size, causal, seed, **kw):
    inp, out, scale, cu, qs, qp = run_prefill(seq_lens, chunks, Hq, Hkv, D, page_size, causal, seed,
                                              **kw)
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.asarray(seq_lens), qs, qp, scale,
                            causal)
    what = "prefill lens=%s chunks=%s ps=%d Hq=%d Hkv=%d D=%d causal=%d" % (
        seq_lens, chunks, page_size, Hq, Hkv, D, causal)
    return compare(to64(out), ref, torch.bfloat16, what)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("page_size", [16, 64])
def test_paged_prefill_full_sequences(D, page_size):
    lens = [300, 129, 1000]
    check_prefill(lens, lens, 8, 2, D, page_size, True, seed=D + page_size)


def test_paged_prefill_chunks_after_cache():
    # chunks appended after cached history, bottom-right aligned; one sequence
    # is a whole prefill, one a single decode-like token
    check_prefill([500, 2000, 64, 777], [37, 256, 64, 1], 4, 4, 128, 16, True, seed=31)
    check_prefill([500, 2000, 64, 777], [37, 256, 64, 1], 4, 4, 128, 32, False, seed=32)


def test_paged_prefill_ragged_chunk_sizes():
    chunks = [1, 127, 128, 129, 255, 257]
    lens = [c + 40 * i for i, c in enumerate(chunks)]
    check_prefill(lens, chunks, 16, 2, 128, 16, True, seed=33)


def test_paged_prefill_grid_larger_than_chunks():
    # max_q well above every chunk: the extra workgroups find no rows
    check_prefill([90, 300], [90, 20], 8, 8, 64, 16, True, seed=34, max_q=700)


def test_paged_prefill_invalid_table_entries_hide_their_keys():
    # non-causal chunk of 10 over a 64-key sequence whose logical pages 1 and
    # 3 point outside the cache: attention over pages 0 and 2 only
    inp, out, scale, cu, qs, qp = run_prefill([64], [10], 4, 2, 128, 16, False, seed=35,
                                              tables=[[0, -1, 2, 99999]])
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            np.array([[0, 2]]), np.array([32]), np.zeros(10, dtype=np.int64),
                            np.full(10, 31), scale, False)
    compare(to64(out), ref, torch.bfloat16, "prefill: invalid pages hidden")


def test_paged_prefill_matches_per_query_entry_point():
    lens, chunks = [700, 333], [200, 333]
    inp, out, scale, cu, qs, qp = run_prefill(lens, chunks, 8, 2, 128, 16, True, seed=36)
    i32 = dict(dtype=torch.int32, device=DEV)
    per_query = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                        inp["seq_lens"], torch.tensor(qs, **i32),
                                        torch.tensor(qp, **i32), scale, True,
                                        inp["block_tables"].shape[1] * 16, 8)
    torch.cuda.synchronize()
    compare(to64(out), to64(per_query), torch.bfloat16, "prefill vs per-query paged")


def test_paged_prefill_matches_dense_prefill_bitwise():
    # whole-sequence causal prefill on contiguous in-order pages runs the same
    # tiles, masks and arithmetic as the dense causal forward
    B, H, S, D, ps = 2, 4, 300, 128, 16
    q, k, v = draw_qkv(B, H, H, S, S, D, torch.bfloat16, 37, DEV)
    npg = -(-S // ps)
    pad = npg * ps - S

    def pages_of(t):
        t = torch.nn.functional.pad(t.permute(0, 2, 1, 3), (0, 0, 0, 0, 0, pad))  # [B, S+pad, H, D]
        return t.reshape(B * npg, ps, H, D).contiguous()

    kc, vc = pages_of(k), pages_of(v)
    tables = torch.arange(B * npg, dtype=torch.int32, device=DEV).view(B, npg)
    i32 = dict(dtype=torch.int32, device=DEV)
    qp = q.permute(0, 2, 1, 3).reshape(B * S, H, D).contiguous()
    got = sd.sdpa_paged_prefill(qp, kc, vc, tables, torch.full((B,), S, **i32),
                                torch.tensor([0, S, 2 * S], **i32), 0.07, True, S, npg * ps)
    ref = sd.sdpa_forward(q, k, v, 0.07, sd.MASK_CAUSAL)
    torch.cuda.synchronize()
    assert torch.equal(got.view(B, S, H, D).permute(0, 2, 1, 3), ref)


@pytest.mark.slow
def test_full_size_paged_prefill_whole_output():
    # the long causal prefill workload's shape (4 sequences x 4096, 16 heads,
    # D 128) as whole-sequence chunks over shuffled 16-key pages, every row
    # checked.  Each sequence's keys come through the oracle's page gather;
    # a whole-sequence causal chunk is then the dense causal forward of that
    # sequence (the reduction the oracle's own pins fix), evaluated per head
    # in row blocks.
    n, L, H, D = 4, 4096, 16, 128
    inp, out, scale, cu, qs, qp = run_prefill([L] * n, [L] * n, H, H, D, 16, True, seed=38)
    assert np.array_equal(qp, np.tile(np.arange(L), n))
    tables = inp["block_tables"].cpu().numpy()
    kc, vc = (inp[x].cpu().float().numpy() for x in ("k_cache", "v_cache"))
    qd = inp["q"].cpu().view(n, L, H, D).permute(0, 2, 1, 3)
    kd = torch.stack([torch.from_numpy(O.paged_gather(kc, tables[s], L, 16)) for s in range(n)])
    vd = torch.stack([torch.from_numpy(O.paged_gather(vc, tables[s], L, 16)) for s in range(n)])
    ref = oracle_forward_whole(O, qd, kd.permute(0, 2, 1, 3), vd.permute(0, 2, 1, 3), scale,
                               O.MASK_CAUSAL)
    got = to64(out).reshape(n, L, H, D).transpose(0, 2, 1, 3)
    max_abs, rel = compare(got, ref, torch.bfloat16, "paged prefill whole output")
    print("paged prefill whole output: max-abs %.3e rel-L2 %.3e" % (max_abs, rel))


# ------------------------------------------------- head dims above 256 (to 1024)
# The split pass runs on the head-dim-split kernel with the page policy.

@pytest.mark.parametrize("D", [264, 512, 1024])
@pytest.mark.parametrize("page_size,splits", [(16, 1), (32, 5), (64, 32)])
def test_paged_decode_headdim_split(D, page_size, splits):
    for causal in (True, False):
        check([300, 129, 1], [0, 1, 1, 2], [299, 128, 64, 0], 8, 2, D, page_size, causal, splits,
              seed=990 + D + page_size + causal)


def test_paged_headdim_split_empty_out_of_range_and_invalid_pages():
    D = 640
    inp, out, scale = run_paged([0, 50, 30], [0, 1, 2, 1, 1], [0, 49, 29, 10, 20], 4, 2, D, 16,
                                True, 4, seed=996)
    inp["query_seq"][3] = 7
    inp["query_pos"][4] = -1
    out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale, True,
                                  64, 4)
    torch.cuda.synchronize()
    got = to64(out)
    assert np.isnan(got[[0, 3, 4]]).all()
    keep = [1, 2]
    ref = O.paged_attention(to64(inp["q"])[keep], to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), inp["seq_lens"].cpu().numpy(),
                            inp["query_seq"].cpu().numpy()[keep], inp["query_pos"].cpu().numpy()[keep],
                            scale, True)
    compare(got[keep], ref, torch.bfloat16, "D=640: valid rows next to empty ones")
    inp, out, scale = run_paged([64], [0, 0], [63, 63], 4, 2, D, 16, False, 2, seed=997,
                                tables=[[0, -1, 2, 99999]])
    valid = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                              np.array([[0, 2]]), np.array([32]), np.array([0, 0]),
                              np.array([31, 31]), scale, False)
    compare(to64(out), valid, torch.bfloat16, "D=640: invalid pages hidden")


def test_paged_headdim_split_matches_dense_decode():
    # one query per sequence at its last position over 16-key pages equals the
    # dense decode of the same keys (both on the head-dim-split kernel)
    D, Hq, Hkv, lens = 512, 8, 2, [500, 77, 256]
    inp, out, scale = run_paged(lens, [0, 1, 2], [l - 1 for l in lens], Hq, Hkv, D, 16, True, 6,
                                seed=998)
    ref = oracle_of(inp, scale, True)
    compare(to64(out), ref, torch.bfloat16, "paged D=512 decode")


@pytest.mark.parametrize("D", [264, 512, 1024])
def test_paged_prefill_headdim_split(D):
    # whole sequences (ragged: 300 = 9 blocks of 32 + 12), chunks after cached
    # history (bottom-right aligned, a single token, causal and not), a grid
    # larger than the chunks, on the head-dim-split kernel
    check_prefill([300, 129, 100], [300, 129, 100], 8, 2, D, 16, True, seed=1010 + D)
    check_prefill([500, 300, 64, 777], [37, 100, 64, 1], 4, 4, D, 32, True, seed=1011 + D)
    check_prefill([500, 300, 64, 777], [37, 100, 64, 1], 4, 4, D, 16, False, seed=1012 + D)
    check_prefill([90, 300], [90, 20], 8, 8, D, 16, True, seed=1013 + D, max_q=300)


def test_paged_prefill_headdim_split_invalid_table_entries():
    D = 768
    inp, out, scale, cu, qs, qp = run_prefill([64], [10], 4, 2, D, 16, False, seed=1020,
                                              tables=[[0, -1, 2, 99999]])
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            np.array([[0, 2]]), np.array([32]), np.zeros(10, dtype=np.int64),
                            np.full(10, 31), scale, False)
    compare(to64(out), ref, torch.bfloat16, "prefill D=768: invalid pages hidden")


# ------------------------------------------------ value head dim Dv != D
# V [pages, page_size, Hkv, Dv] and the output [.., Hq, Dv] with Dv other than
# D (ruDNN user guide section 9): the general-width kernels, K and V with
# their own widths; above 128 value dims the prefill writes two 128-dim
# output slices.

DV_PAIRS = [(64, 128), (128, 64), (128, 256), (256, 64), (192, 96), (40, 200), (256, 136), (8, 16)]


def with_value_width(inp, Dv, dtype, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed + 7919)
    pages, ps, Hkv, _ = inp["k_cache"].shape
    inp["v_cache"] = torch.randn(pages, ps, Hkv, Dv, generator=g, device=DEV).to(dtype)
    return inp


@pytest.mark.parametrize("D,Dv", DV_PAIRS)
@pytest.mark.parametrize("splits", [1, 5])
def test_paged_attention_value_width(D, Dv, splits):
    lens, qs, qp = [300, 129, 1, 50], [0, 1, 2, 0, 3, 1], [299, 128, 0, 17, 49, 3]
    for causal in (False, True):
        seed = 2000 + D + Dv + splits + causal
        inp = with_value_width(draw_paged(lens, qs, qp, 8, 2, D, 16, torch.bfloat16, seed, DEV), Dv,
                               torch.bfloat16, seed)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                      inp["seq_lens"], inp["query_seq"], inp["query_pos"], scale,
                                      causal, inp["block_tables"].shape[1] * 16, splits)
        torch.cuda.synchronize()
        assert out.shape == (len(qs), 8, Dv)
        compare(to64(out), oracle_of(inp, scale, causal), torch.bfloat16,
                "paged D=%d Dv=%d splits=%d causal=%d" % (D, Dv, splits, causal))


@pytest.mark.parametrize("D,Dv", DV_PAIRS)
def test_paged_prefill_value_width(D, Dv):
    lens, chunks = [300, 129, 1000], [300, 40, 257]
    nq = sum(chunks)
    for causal in (False, True):
        seed = 2100 + D + Dv + causal
        inp = with_value_width(draw_paged(lens, [0] * nq, [0] * nq, 8, 2, D, 16, torch.bfloat16,
                                          seed, DEV), Dv, torch.bfloat16, seed)
        cu = torch.tensor(np.concatenate([[0], np.cumsum(chunks)]), dtype=torch.int32, device=DEV)
        scale = 1 / math.sqrt(D)
        out = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                    inp["seq_lens"], cu, scale, causal, max(chunks),
                                    inp["block_tables"].shape[1] * 16)
        torch.cuda.synchronize()
        assert out.shape == (nq, 8, Dv)
        qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
        ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                                inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, scale,
                                causal)
        compare(to64(out), ref, torch.bfloat16, "prefill D=%d Dv=%d causal=%d" % (D, Dv, causal))


def test_paged_value_width_fp16_and_prefill_matches_per_query():
    D, Dv = 128, 64
    lens, chunks = [700, 333], [200, 333]
    nq = sum(chunks)
    inp = with_value_width(draw_paged(lens, [0] * nq, [0] * nq, 8, 4, D, 32, torch.float16, 2200, DEV),
                           Dv, torch.float16, 2200)
    cu = torch.tensor([0, 200, 533], dtype=torch.int32, device=DEV)
    qs, qp = O.chunk_positions(cu.cpu().numpy(), np.array(lens))
    i32 = dict(dtype=torch.int32, device=DEV)
    pre = sd.sdpa_paged_prefill(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                inp["seq_lens"], cu, 0.1, True, 333, inp["block_tables"].shape[1] * 32)
    per = sd.sdpa_paged_attention(inp["q"], inp["k_cache"], inp["v_cache"], inp["block_tables"],
                                  inp["seq_lens"], torch.tensor(qs, **i32), torch.tensor(qp, **i32),
                                  0.1, True, inp["block_tables"].shape[1] * 32, 7)
    torch.cuda.synchronize()
    ref = O.paged_attention(to64(inp["q"]), to64(inp["k_cache"]), to64(inp["v_cache"]),
                            inp["block_tables"].cpu().numpy(), np.array(lens), qs, qp, 0.1, True)
    compare(to64(pre), ref, torch.float16, "fp16 prefill Dv=64")
    compare(to64(per), ref, torch.float16, "fp16 paged attention Dv=64")
