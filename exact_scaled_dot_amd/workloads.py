"""Seeded synthetic attention workloads.

This module only draws inputs: it holds none of the attention arithmetic, so
both the HIP library's tests and the CPU oracle can consume what it produces
without sharing any of the method's code.

Recipe (the same on every device): a torch.Generator on the target device,
seeded with the workload's seed, draws Q, K, V in that order as i.i.d. N(0, 1)
float32 values, which are then rounded to the workload dtype by torch's
float32 -> bfloat16 conversion (round to nearest even).  Key lengths come from
a separate CPU generator seeded with seed + 7919, uniform integers in the
inclusive range [lo, hi], so they are identical on every device.
"""

from dataclasses import dataclass
import math

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    dtype: torch.dtype
    causal: bool = False
    key_len_range: tuple = None      # (lo, hi) inclusive, or None for no padding
    decode: bool = False             # Sq == 1 split-KV decode
    num_splits: int = 1
    seed: int = 0

    @property
    def scale(self):
        return 1.0 / math.sqrt(self.D)

    @property
    def padded(self):
        return self.key_len_range is not None


# The five headline workloads: shapes, masks and dtypes of the attention the
# pages describe (single-head fp32, the small causal block of the tensai guide,
# long causal prefill, grouped K/V with key padding, grouped K/V decode).
WORKLOADS = {
    w.name: w for w in [
        Workload("fp32_single_head_s128_d64", 1, 1, 1, 128, 128, 64, torch.float32,
                 seed=1001),
        Workload("bf16_causal_b8_h4_s128_d64", 8, 4, 4, 128, 128, 64, torch.bfloat16,
                 causal=True, seed=1002),
        Workload("bf16_causal_b4_h16_s4096_d128", 4, 16, 16, 4096, 4096, 128, torch.bfloat16,
                 causal=True, seed=1003),
        Workload("bf16_gqa32x8_padded_b2_s8192_d128", 2, 32, 8, 8192, 8192, 128, torch.bfloat16,
                 key_len_range=(4096, 8192), seed=1004),
        Workload("bf16_gqa32x8_decode_b64_sk32768_d128", 64, 32, 8, 1, 32768, 128, torch.bfloat16,
                 decode=True, num_splits=32, seed=1005),
    ]
}


def draw_qkv(B, Hq, Hkv, Sq, Sk, D, dtype, seed, device="cpu"):
    """Q [B,Hq,Sq,D], K and V [B,Hkv,Sk,D]: i.i.d. N(0,1) rounded to dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = []
    for shape in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, D)):
        t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
        out.append(t.to(dtype) if dtype != torch.float32 else t)
        del t
    return tuple(out)


def draw_grad(shape, dtype, seed, device="cpu"):
    """Upstream gradient dO of the given shape: i.i.d. N(0,1) rounded to dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 15485863)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return t.to(dtype) if dtype != torch.float32 else t


def draw_bias(shape, dtype, seed, device="cpu"):
    """Additive mask tensor of the given shape: i.i.d. N(0, 4) rounded to dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 32452843)
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * 2.0
    return t.to(dtype) if dtype != torch.float32 else t


def draw_block(B, S, model, dtype, seed, device="cpu"):
    """Attention block inputs: x [B, S, model] i.i.d. N(0, 1) and four weights
    wq, wk, wv, wo [model, model] i.i.d. N(0, 1 / model) (so the projections
    keep unit variance), drawn in that order and rounded to dtype."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed + 49979687)
    out = [torch.randn((B, S, model), generator=gen, device=device, dtype=torch.float32)]
    for _ in range(4):
        out.append(torch.randn((model, model), generator=gen, device=device, dtype=torch.float32)
                   / math.sqrt(model))
    return tuple(t.to(dtype) if dtype != torch.float32 else t for t in out)


def draw_key_lens(B, lo, hi, seed, device="cpu"):
    """Per-batch valid key lengths, uniform integers in [lo, hi] (int32)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed + 7919)
    lens = torch.randint(lo, hi + 1, (B,), generator=gen, dtype=torch.int64)
    return lens.to(torch.int32).to(device)


def make_inputs(w, device="cpu", seed=None):
    """Inputs of workload w on device: dict with q, k, v, key_lens (or None)."""
    seed = w.seed if seed is None else seed
    q, k, v = draw_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.dtype, seed, device)
    key_lens = None
    if w.padded:
        key_lens = draw_key_lens(w.B, w.key_len_range[0], w.key_len_range[1], seed, device)
    return {"q": q, "k": k, "v": v, "key_lens": key_lens}


def to_f64_numpy(t):
    """Exact float64 copy of a float32 / bfloat16 tensor (for the CPU side)."""
    return t.detach().to("cpu", torch.float64).numpy()


def draw_paged(seq_lens, query_seq, query_pos, Hq, Hkv, D, page_size, dtype, seed, device="cpu",
               extra_pages=3):
    """Packed queries over a shuffled K/V page cache.

    seq_lens, query_seq, query_pos: host integer lists.  Sequence s owns
    ceil(seq_lens[s] / page_size) physical pages, dealt from a random
    permutation of all pages (CPU generator seeded with seed + 104729), and
    extra_pages pages belong to nobody; unused table entries are -1.  Q and
    the whole cache (unused slots included) are i.i.d. N(0, 1) float32 drawn in
    the order Q, K cache, V cache on a device generator seeded with seed, then
    rounded to dtype.  Returns a dict of device tensors plus the sizes.
    """
    seq_lens = [int(x) for x in seq_lens]
    need = [-(-n // page_size) for n in seq_lens]
    max_pages = max(1, max(need))
    pages = sum(need) + int(extra_pages)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    nq = len(query_seq)
    q = torch.randn(nq, Hq, D, generator=g, device=device, dtype=torch.float32).to(dtype)
    kc = torch.randn(pages, page_size, Hkv, D, generator=g, device=device, dtype=torch.float32).to(dtype)
    vc = torch.randn(pages, page_size, Hkv, D, generator=g, device=device, dtype=torch.float32).to(dtype)
    gc = torch.Generator(device="cpu")
    gc.manual_seed(seed + 104729)
    perm = torch.randperm(pages, generator=gc).to(torch.int32)
    tables = torch.full((len(seq_lens), max_pages), -1, dtype=torch.int32)
    nxt = 0
    for s, n in enumerate(need):
        tables[s, :n] = perm[nxt:nxt + n]
        nxt += n
    i32 = dict(dtype=torch.int32, device=device)
    return dict(q=q, k_cache=kc, v_cache=vc, block_tables=tables.to(device),
                seq_lens=torch.tensor(seq_lens, **i32), query_seq=torch.tensor(list(query_seq), **i32),
                query_pos=torch.tensor(list(query_pos), **i32), pages=pages, max_pages=max_pages,
                page_size=page_size)
