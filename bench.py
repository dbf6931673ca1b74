#!/usr/bin/env python3
"""Benchmark of libsdpa on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

One step is one pass of the whole hot path over synthetic inputs already
resident in HBM:
  * prefill, causal, bf16, B=4 Hq=Hkv=16 Sq=Sk=4096 D=128   (the headline)
  * prefill, grouped K/V 32/8 with key padding, bf16, B=2 S=8192 D=128
  * split-KV decode, bf16, B=64 Hq=32 Hkv=8 Sk=32768 D=128, 32 splits + merge
  * the same decode over a shuffled 16-key page cache, and the causal prefill
    as whole-sequence chunks over such a cache
  * the attention backward (dQ, dK, dV) of the causal prefill workload, from
    its forward output and log-sum-exp (computed once, before the timing),
    with the ordered reduction and with the atomic-dQ one, and the same
    backward with the per-head bias below, which also writes the bias
    gradient [4, 16, 4096, 4096] bf16 in full; and the backward of the
    256-wide-head prefill below (B=4 Hq=Hkv=8 S=4096 D=256, causal) on the
    head-dim-split backward kernels
  * the causal prefill with a general additive mask: a per-head bias tensor
    [1, 16, 4096, 4096] bf16 added to the scaled scores
  * the causal prefill with 1024-wide heads, bf16, B=1 Hq=Hkv=8 S=4096 D=1024
    (the same formula FLOPs again; the head dim is split across 8 waves)
  * the causal prefill with 256-wide heads, bf16, B=4 Hq=Hkv=8 S=4096 D=256
    (the same formula FLOPs as the headline; pairs of waves split the head
    dim and add each other's partial scores on chip), and the split-KV
    decode with 256-wide heads, B=32 Hq=32 Hkv=8 Sk=32768 (the decode's K+V
    bytes), 32 splits, and with 1024-wide heads, B=8 Hq=32 Hkv=8 Sk=32768 (the
    same K+V bytes again)
  * the multi-head attention block (q/k/v projections, causal attention,
    output projection) at the tensai guide's shape (batch 8, 128 tokens,
    model 256, 4 heads) and at the prefill's (batch 4, 4096 tokens, model
    2048, 16 heads of 128)
Each call is bracketed by HIP events on the stream it is launched on (torch's
current stream, which is the stream the binding hands to the library).

`value` is the causal prefill's TFLOP/s by the headline formula
4*B*Hq*Sq*Sk*D, halved when causal; `roofline` is that kernel's fraction of
the bf16 dense MFMA peak.  The decode result (HBM GB/s over the K+V+Q+O bytes
of one call, fraction of the 8 TB/s HBM peak) and the padded prefill are
reported in their own objects on the same line; the backward's TFLOP/s counts
2.5 times the forward formula (five products of the same shape against two).
`cpu_baseline` times the fp64
oracle on a bounded sample of the causal prefill workload on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s (+% bf16 MFMA peak); decode HBM GB/s (+% peak)"
BF16_MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
SQ_FILE = os.path.join(ROOT, "profiles", "sq_counters.json")
SMALL_FP32 = "fp32_single_head_s128_d64"
SMALL_CAUSAL = "bf16_causal_b8_h4_s128_d64"

PREFILL = "bf16_causal_b4_h16_s4096_d128"
PADDED = "bf16_gqa32x8_padded_b2_s8192_d128"
DECODE = "bf16_gqa32x8_decode_b64_sk32768_d128"
PAGE_SIZE = 16                      # paged decode: keys per cache page
# attention blocks: (batch, tokens, model width, heads)
BLOCKS = {"block": (4, 4096, 2048, 16), "block_small": (8, 128, 256, 4)}
WIDE = (4, 8, 4096, 256)            # wide heads: (batch, heads, tokens, head dim)
WIDEST = (1, 8, 4096, 1024)         # head-dim-split kernel: (batch, heads, tokens, head dim)
DECODE_WIDE = (32, 32, 8, 32768, 256)  # wide decode: (batch, Hq, Hkv, Sk, head dim)
DECODE_WIDEST = (8, 32, 8, 32768, 1024)  # head-dim-split decode (the same K+V bytes)


# Headers every kernel source includes: a change to them changes every kernel.
KERNEL_HEADERS = ("device_common.hpp", "launch.hpp")


def kernel_source_hash(name):
    """Hash of a kernel source together with the headers it includes."""
    h = hashlib.sha256()
    for part in (name,) + KERNEL_HEADERS:
        with open(os.path.join(ROOT, "exact_scaled_dot_amd", "csrc", part), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic(workload, source):
    """HBM bytes per launch from the committed counter summary, if still valid."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(source):
        return None  # the kernel changed since the counters were taken
    return rec.get("hbm_bytes_per_launch")


def pair_traffic(a, b, src_a, src_b=None):
    """HBM bytes of a split pass and its merge, if both records are valid."""
    parts = [stored_traffic(a, src_a), stored_traffic(b, src_b or src_a)]
    return None if None in parts else sum(parts)


def backward_traffic():
    """HBM bytes of one backward call (both passes), if both records are valid."""
    parts = [stored_traffic(k, "backward.hip") for k in ("backward_dq", "backward_dkdv")]
    return None if None in parts else sum(parts)


def wide_backward_traffic():
    """HBM bytes of one head-dim-split backward call (its three kernels), if valid."""
    parts = [stored_traffic(k, "backward_wide.hip")
             for k in ("backward_wide_stats", "backward_wide_dq", "backward_wide_dkdv")]
    return None if None in parts else sum(parts)


def bias_backward_traffic():
    """HBM bytes of one backward-with-bias call (both passes), if both records are valid."""
    parts = [stored_traffic(k, "backward.hip") for k in ("backward_bias_dq", "backward_bias_dkdv")]
    return None if None in parts else sum(parts)


def atomic_traffic():
    """HBM bytes of one atomic-dQ backward call (its three kernels), if valid."""
    parts = [stored_traffic(k, "backward.hip")
             for k in ("backward_atomic_prep", "backward_atomic_dkdv", "backward_atomic_convert")]
    return None if None in parts else sum(parts)


def block_traffic(tag):
    """HBM bytes of one attention-block call (its three kernels), if valid."""
    parts = [stored_traffic(tag + "_qkv", "gemm.hip"), stored_traffic(tag + "_attn", "forward.hip"),
             stored_traffic(tag + "_out", "gemm.hip")]
    return None if None in parts else sum(parts)


def block_flops(B, S, M, H, causal):
    """Four [B*S, M] x [M, M] projections plus the attention formula."""
    return 8.0 * B * S * M * M + formula_flops(B, H, S, S, M // H, causal)


def formula_flops(B, Hq, Sq, Sk, D, causal):
    f = 4.0 * B * Hq * Sq * Sk * D
    return f / 2 if causal else f


def timing(samples_ms):
    """Mean, median and minimum of per-call HIP-event times, in ms."""
    import statistics
    return {"ms": round(sum(samples_ms) / len(samples_ms), 4),
            "ms_median": round(statistics.median(samples_ms), 4),
            "ms_min": round(min(samples_ms), 4), "calls_timed": len(samples_ms)}


def stored_sq(workload, source):
    """Sustained clock and MFMA activity of a kernel from the committed SQ
    counter record (rocprofv3 --pmc passes), if it is still current."""
    try:
        with open(SQ_FILE) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != kernel_source_hash(source):
        return None
    return {k: rec[k] for k in ("clock_ghz", "mfma_busy", "mfma_coexec_of_busy",
                                "counter_duration_us") if k in rec}


def padded_algorithmic_flops(w, key_lens):
    # 4 * Hq * Sq * D per visible key, summed over the batch (no causal mask here)
    return 4.0 * w.Hq * w.Sq * w.D * float(sum(int(x) for x in key_lens))


def cpu_baseline(budget_s):
    """fp64 oracle on the first (batch, head) pairs of the causal prefill workload."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from exact_scaled_dot_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[PREFILL]
    inp = make_inputs(w, "cpu")
    q, k, v = (inp[x].to(torch.float64).numpy() for x in ("q", "k", "v"))
    heads, t0 = 0, time.perf_counter()
    while heads < w.B * w.Hq:
        b, h = divmod(heads, w.Hq)
        oracle.sdpa_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1], w.scale,
                            oracle.MASK_CAUSAL)
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    flops = heads * formula_flops(1, 1, w.Sq, w.Sk, w.D, True)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle",
            "sample": "%d of %d (batch, head) pairs of %s, %.1f s, fp64 NumPy/BLAS; affinity %d cores"
                      % (heads, w.B * w.Hq, w.name, dt, len(os.sched_getaffinity(0)))}


def cpu_baseline_padded(budget_s):
    """fp64 oracle on whole (batch, query head) pairs of the padded grouped
    prefill workload (its visible keys only count as work), until the budget
    is spent; with the whole workload's time extrapolated from that rate."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from exact_scaled_dot_amd.workloads import WORKLOADS, make_inputs

    w = WORKLOADS[PADDED]
    inp = make_inputs(w, "cpu")
    q, k, v = (inp[x].to(torch.float64).numpy() for x in ("q", "k", "v"))
    lens = inp["key_lens"].numpy()
    G = w.Hq // w.Hkv
    heads, flops, t0 = 0, 0.0, time.perf_counter()
    while heads < w.B * w.Hq:
        b, h = divmod(heads, w.Hq)
        oracle.sdpa_forward(q[b:b + 1, h:h + 1], k[b:b + 1, h // G:h // G + 1],
                            v[b:b + 1, h // G:h // G + 1], w.scale, oracle.MASK_KEY_PADDING,
                            lens[b:b + 1])
        flops += 4.0 * w.Sq * w.D * float(lens[b])
        heads += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    rate = flops / dt
    total = padded_algorithmic_flops(w, lens.tolist())
    return {"value": round(rate / 1e12, 6), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "whole_workload_s_extrapolated": round(total / rate, 1),
            "sample": "%d of %d (batch, query head) pairs of %s, %.1f s, fp64 NumPy/BLAS"
                      % (heads, w.B * w.Hq, w.name, dt)}


def ingest_counters(fetch_csv, write_csv, copy_bytes=1 << 30):
    """Turn two rocprofv3 --pmc runs of a full-step bench (FETCH_SIZE, then
    WRITE_SIZE; KiB per dispatch) into HBM bytes per launch for each workload,
    calibrated on the plain 1 GiB device copy that --copy-calibration adds, and
    tagged with the hash of the kernel source they were measured on."""
    import csv
    import statistics

    def per_kernel(path):
        rows = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.setdefault(r["Kernel_Name"], []).append(
                    (int(r["Dispatch_Id"]), float(r["Counter_Value"]) * 1024.0))
        return {k: [x for _, x in sorted(v)] for k, v in rows.items()}

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    copy = "__amd_rocclr_copyBuffer"
    f_scale = copy_bytes / max(fetch[copy])   # true bytes / counted bytes
    w_scale = copy_bytes / max(write[copy])
    out = {"_calibration": {"copy_bytes": copy_bytes, "fetch_scale": round(f_scale, 4),
                            "write_scale": round(w_scale, 4),
                            "note": "FETCH_SIZE/WRITE_SIZE KiB per dispatch x scale"}}

    def entry(kernel, src, reads, writes):
        r = statistics.median(reads) * f_scale
        w = statistics.median(writes) * w_scale
        return {"kernel": kernel, "source_sha256_16": kernel_source_hash(src),
                "read_bytes": round(r), "write_bytes": round(w),
                "hbm_bytes_per_launch": round(r + w)}

    fwd = "forward_bf16_kernel"
    if fwd in fetch:
        # a full step launches, in order: the causal prefill, the padded one,
        # the paged one, the bias prefill, the large block's attention and the
        # small block's (after the setup forwards that give the backward legs
        # their output and lse)
        fr, wr = fetch[fwd], write[fwd]
        setup = len(fr) % 6        # the backward legs' setup forwards come first
        fr, wr = fr[setup:], wr[setup:]
        for i, key in enumerate(("prefill", "padded", "paged_prefill", "bias", "block_attn",
                                 "block_small_attn")):
            out[key] = entry(fwd, "forward.hip", fr[i::6], wr[i::6])
    # the wide-head prefill (paired waves): once per step, after one setup
    # forward for the wide backward leg
    fp = "forward_pair_kernel"
    if fp in fetch:
        skip = 1 if len(fetch[fp]) > 1 else 0
        out["wide"] = entry(fp, "forward.hip", fetch[fp][skip:], write[fp][skip:])
    # the head-dim-split kernel: the widest prefill, then the widest decode's
    # split pass
    fw = "forward_wide_kernel"
    if fw in fetch:
        out["widest"] = entry(fw, "forward_wide.hip", fetch[fw][0::2], write[fw][0::2])
        out["decode_widest_split"] = entry(fw, "forward_wide.hip", fetch[fw][1::2], write[fw][1::2])
    # each block call: q/k/v projection GEMM, attention, output projection
    # GEMM; a step runs the large block, then the small one (names are
    # truncated, so the four GEMM dispatches of a step are told apart by order)
    gm = "gemm_kernel"
    if gm in fetch:
        for i, key in enumerate(("block_qkv", "block_out", "block_small_qkv", "block_small_out")):
            out[key] = entry(gm, "gemm.hip", fetch[gm][i::4], write[gm][i::4])
    # A full step runs the ordered backward, the atomic one and the one with a
    # bias, in that order: their dQ and dK/dV dispatches interleave.
    dq = "bwd_dq_kernel"
    if dq in fetch:
        out["backward_dq"] = entry(dq, "backward.hip", fetch[dq][0::2], write[dq][0::2])
        out["backward_bias_dq"] = entry(dq, "backward.hip", fetch[dq][1::2], write[dq][1::2])
    dk = "bwd_dkdv_kernel"
    if dk in fetch:
        for i, key in enumerate(("backward_dkdv", "backward_atomic_dkdv", "backward_bias_dkdv")):
            out[key] = entry(dk, "backward.hip", fetch[dk][i::3], write[dk][i::3])
    for key, name in (("backward_atomic_prep", "bwd_prep_kernel"),
                      ("backward_atomic_convert", "bwd_dq_convert_kernel")):
        if name in fetch:
            out[key] = entry(name, "backward.hip", fetch[name], write[name])
    # the head-dim-split backward (256-wide heads): its own three kernels
    for key, name in (("backward_wide_stats", "bwd_wide_stats_kernel"),
                      ("backward_wide_dq", "bwd_wide_dq_kernel"),
                      ("backward_wide_dkdv", "bwd_wide_dkdv_kernel")):
        if name in fetch:
            out[key] = entry(name, "backward_wide.hip", fetch[name], write[name])
    # A full step runs the dense decode, the paged one and the 256-wide one
    # (split and merge each), then the 1024-wide one (its own split kernel,
    # the same merge kernel): 3 split and 4 merge dispatches per step.
    sp, mg = "decode_split_bf16_kernel", "decode_merge_bf16_kernel"
    if sp in fetch:
        for i, key in enumerate(("decode_split", "paged_split", "decode_wide_split")):
            out[key] = entry(sp, "decode.hip", fetch[sp][i::3], write[sp][i::3])
    if mg in fetch:
        for i, key in enumerate(("decode_merge", "paged_merge", "decode_wide_merge",
                                 "decode_widest_merge")):
            out[key] = entry(mg, "decode.hip", fetch[mg][i::4], write[mg][i::4])
    return out


# Kernels whose SQ counters --ingest-sq records: workload -> (kernel, source)
SQ_KERNELS = {"prefill": ("forward_bf16_kernel", "forward.hip"),
              "padded": ("forward_bf16_kernel", "forward.hip")}


def ingest_sq(workload, csvs):
    """One record of SQ counters for a kernel from rocprofv3 --pmc passes of a
    one-call bench (--only WORKLOAD): the median of each counter over the
    kernel's dispatches, the dispatch duration from the counter passes' own
    timestamps, and from them the sustained clock (GRBM_GUI_ACTIVE counts GPU
    clocks summed over the 8 XCDs) and the MFMA busy fraction
    (SQ_VALU_MFMA_BUSY_CYCLES sums over the 1024 SIMDs)."""
    import csv
    import statistics
    kernel, src = SQ_KERNELS[workload]
    per, dur = {}, []
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                if kernel not in r["Kernel_Name"]:
                    continue
                per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                dur.append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    med = {k: statistics.median(v) for k, v in per.items()}
    d_ns = statistics.median(dur)
    rec = {"kernel": kernel, "source_sha256_16": kernel_source_hash(src),
           "counters": {k: med[k] for k in sorted(med)},
           "counter_duration_us": round(d_ns / 1e3, 2)}
    if "GRBM_GUI_ACTIVE" in med:
        xcd_cycles = med["GRBM_GUI_ACTIVE"] / 8
        rec["clock_ghz"] = round(xcd_cycles / d_ns, 3)
        if "SQ_VALU_MFMA_BUSY_CYCLES" in med:
            rec["mfma_busy"] = round(med["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / xcd_cycles, 4)
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in med and med.get("SQ_VALU_MFMA_BUSY_CYCLES"):
        rec["mfma_coexec_of_busy"] = round(med["SQ_VALU_MFMA_COEXEC_CYCLES"]
                                           / med["SQ_VALU_MFMA_BUSY_CYCLES"], 4)
    try:
        with open(SQ_FILE) as f:
            allrec = json.load(f)
    except (OSError, ValueError):
        allrec = {}
    allrec[workload] = rec
    with open(SQ_FILE, "w") as f:
        json.dump(allrec, f, indent=1)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    ap.add_argument("--small-iters", type=int, default=500,
                    help="timed calls of each small configuration (0: skip them)")
    ap.add_argument("--only", choices=["prefill", "padded", "decode", "paged", "paged_prefill",
                                       "backward", "backward_atomic", "backward_bias",
                                       "backward_wide", "bias",
                                       "wide", "widest", "decode_widest",
                                       "decode_wide", "block", "block_small"],
                    default=None,
                    help="run one call per step (for per-kernel profiling)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from two rocprofv3 --pmc runs and exit")
    ap.add_argument("--ingest-sq", nargs="+", metavar="ARG",
                    help="WORKLOAD CSV [CSV ...]: record SQ counters of a --only WORKLOAD run "
                         "in profiles/sq_counters.json and exit")
    args = ap.parse_args()

    if args.ingest_sq:
        print(json.dumps(ingest_sq(args.ingest_sq[0], args.ingest_sq[1:]), indent=1))
        return

    if args.ingest_counters:
        rec = ingest_counters(*args.ingest_counters)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
        print(json.dumps(rec, indent=1))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library runs on one device per process "
              "(got --gpus %d, WORLD_SIZE %d)" % (args.gpus, world), file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_scaled_dot_amd as sd
    from exact_scaled_dot_amd.workloads import (WORKLOADS, draw_bias, draw_block, draw_grad,
                                                 draw_paged, draw_qkv, make_inputs)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sd.load_library()

    wp, wg, wd = WORKLOADS[PREFILL], WORKLOADS[PADDED], WORKLOADS[DECODE]
    ip = make_inputs(wp, dev)
    ig = make_inputs(wg, dev)
    idd = make_inputs(wd, dev)
    out_p = torch.empty_like(ip["q"])
    out_g = torch.empty_like(ig["q"])
    out_d = torch.empty_like(idd["q"])
    ws = torch.empty(sd.sdpa_decode_workspace_size(wd.B, wd.Hq, wd.D, wd.num_splits),
                     dtype=torch.uint8, device=dev)
    lens_g = ig["key_lens"].cpu().tolist()
    # Paged decode: the decode workload's shape (B sequences of Sk cached keys,
    # Hq/Hkv heads, D) in shuffled 16-key pages, one query per sequence at its
    # last position, causal, same split count.
    ipg = None
    if args.only in (None, "paged"):
        ipg = draw_paged([wd.Sk] * wd.B, range(wd.B), [wd.Sk - 1] * wd.B, wd.Hq, wd.Hkv, wd.D,
                         PAGE_SIZE, wd.dtype, wd.seed, dev, extra_pages=0)
        out_pg = torch.empty_like(ipg["q"])
    # Paged prefill: the causal prefill workload's shape (B sequences of S
    # tokens, H heads, D) as whole-sequence chunks in shuffled 16-key pages.
    ipp = None
    if args.only in (None, "paged_prefill"):
        nq = wp.B * wp.Sq
        ipp = draw_paged([wp.Sk] * wp.B, [0] * nq, [0] * nq, wp.Hq, wp.Hkv, wp.D, PAGE_SIZE,
                         wp.dtype, wp.seed, dev, extra_pages=0)
        ipp["cu"] = torch.arange(0, nq + 1, wp.Sq, dtype=torch.int32, device=dev)
        out_pp = torch.empty_like(ipp["q"])
    # Backward: the causal prefill workload; its forward output and lse come
    # from one forward call here, outside the timed region.
    ibw = None
    if args.only in (None, "backward", "backward_atomic"):
        out_b, lse_b = sd.sdpa_forward_lse(ip["q"], ip["k"], ip["v"], wp.scale, sd.MASK_CAUSAL)
        ibw = {"out": out_b, "lse": lse_b,
               "dout": draw_grad(tuple(ip["q"].shape), wp.dtype, wp.seed, dev),
               "dq": torch.empty_like(ip["q"]), "dk": torch.empty_like(ip["k"]),
               "dv": torch.empty_like(ip["v"]),
               "ws": torch.empty(sd.sdpa_backward_atomic_workspace_size(wp.B, wp.Hq, wp.Sq, wp.D),
                                 dtype=torch.uint8, device=dev)}
    # Bias: the causal prefill workload with a per-head [1, Hq, Sq, Sk] bias.
    ibias = None
    if args.only in (None, "bias", "backward_bias"):
        ibias = {"bias": draw_bias((1, wp.Hq, wp.Sq, wp.Sk), wp.dtype, wp.seed, dev),
                 "out": torch.empty_like(ip["q"])}
    # Backward with that bias: output and lse from one biased forward here,
    # the bias gradient [B, Hq, Sq, Sk] written in full by every call.
    ibb = None
    if args.only in (None, "backward_bias"):
        out_bb, lse_bb = sd.sdpa_forward_bias(ip["q"], ip["k"], ip["v"], ibias["bias"], wp.scale,
                                              sd.MASK_CAUSAL, None, lse=True)
        ibb = {"out": out_bb, "lse": lse_bb,
               "dout": draw_grad(tuple(ip["q"].shape), wp.dtype, wp.seed, dev),
               "dq": torch.empty_like(ip["q"]), "dk": torch.empty_like(ip["k"]),
               "dv": torch.empty_like(ip["v"]),
               "dbias": torch.empty((wp.B, wp.Hq, wp.Sq, wp.Sk), dtype=wp.dtype, device=dev),
               "ws": torch.empty(sd.sdpa_backward_workspace_size(wp.B, wp.Hq, wp.Sq),
                                 dtype=torch.uint8, device=dev)}
    # Wide heads: the causal prefill's token count and model width in 8 heads
    # of 256.
    iwide = None
    if args.only in (None, "wide", "backward_wide"):
        iwide = dict(zip(("q", "k", "v"), draw_qkv(WIDE[0], WIDE[1], WIDE[1], WIDE[2], WIDE[2],
                                                   WIDE[3], wp.dtype, wp.seed + 31, dev)))
        iwide["out"] = torch.empty_like(iwide["q"])
    # Backward of the wide-head prefill (head-dim-split backward kernels):
    # output and lse from one forward here.
    ibwd = None
    if args.only in (None, "backward_wide"):
        out_w, lse_w = sd.sdpa_forward_lse(iwide["q"], iwide["k"], iwide["v"],
                                           1.0 / math.sqrt(WIDE[3]), sd.MASK_CAUSAL)
        ibwd = {"out": out_w, "lse": lse_w,
                "dout": draw_grad(tuple(iwide["q"].shape), wp.dtype, wp.seed + 41, dev),
                "dq": torch.empty_like(iwide["q"]), "dk": torch.empty_like(iwide["k"]),
                "dv": torch.empty_like(iwide["v"]),
                "ws": torch.empty(sd.sdpa_backward_workspace_size(WIDE[0], WIDE[1], WIDE[2]),
                                  dtype=torch.uint8, device=dev)}
    # Widest heads: the same tokens and batch*heads*head dim in 8 heads of 1024.
    iwst = None
    if args.only in (None, "widest"):
        iwst = dict(zip(("q", "k", "v"), draw_qkv(WIDEST[0], WIDEST[1], WIDEST[1], WIDEST[2],
                                                  WIDEST[2], WIDEST[3], wp.dtype, wp.seed + 37, dev)))
        iwst["out"] = torch.empty_like(iwst["q"])
    idws = None
    if args.only in (None, "decode_widest"):
        B, Hq, Hkv, Sk, D = DECODE_WIDEST
        idws = dict(zip(("q", "k", "v"), draw_qkv(B, Hq, Hkv, 1, Sk, D, wd.dtype, wd.seed + 41, dev)))
        idws["out"] = torch.empty_like(idws["q"])
        idws["ws"] = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, wd.num_splits),
                                 dtype=torch.uint8, device=dev)
    idw = None
    if args.only in (None, "decode_wide"):
        B, Hq, Hkv, Sk, D = DECODE_WIDE
        idw = dict(zip(("q", "k", "v"), draw_qkv(B, Hq, Hkv, 1, Sk, D, wd.dtype, wd.seed + 31, dev)))
        idw["out"] = torch.empty_like(idw["q"])
        idw["ws"] = torch.empty(sd.sdpa_decode_workspace_size(B, Hq, D, wd.num_splits),
                                dtype=torch.uint8, device=dev)
    # Attention blocks: x and four weights per shape (N(0,1) activations,
    # N(0, 1/model) weights), the output and the workspace allocated here.
    iblk = {}
    for name, (B, S, M, H) in BLOCKS.items():
        if args.only in (None, name):
            ins = draw_block(B, S, M, wp.dtype, wp.seed + 17, dev)
            iblk[name] = {"ins": ins, "y": torch.empty_like(ins[0]), "H": H,
                          "ws": torch.empty(sd.sdpa_block_workspace_size(B, S, M),
                                            dtype=torch.uint8, device=dev)}
    torch.cuda.synchronize()

    calls = {
        "prefill": lambda: sd.sdpa_forward(ip["q"], ip["k"], ip["v"], wp.scale, sd.MASK_CAUSAL,
                                           None, out_p),
        "padded": lambda: sd.sdpa_forward(ig["q"], ig["k"], ig["v"], wg.scale,
                                          sd.MASK_KEY_PADDING, ig["key_lens"], out_g),
        "decode": lambda: sd.sdpa_decode(idd["q"], idd["k"], idd["v"], wd.scale, None,
                                         wd.num_splits, ws, out_d),
        "paged": lambda: sd.sdpa_paged_attention(ipg["q"], ipg["k_cache"], ipg["v_cache"],
                                                 ipg["block_tables"], ipg["seq_lens"],
                                                 ipg["query_seq"], ipg["query_pos"], wd.scale,
                                                 True, wd.Sk, wd.num_splits, ws, out_pg),
        "paged_prefill": lambda: sd.sdpa_paged_prefill(ipp["q"], ipp["k_cache"], ipp["v_cache"],
                                                       ipp["block_tables"], ipp["seq_lens"],
                                                       ipp["cu"], wp.scale, True, wp.Sq, wp.Sk,
                                                       out_pp),
        "backward": lambda: sd.sdpa_backward(ip["q"], ip["k"], ip["v"], ibw["out"], ibw["dout"],
                                             ibw["lse"], wp.scale, sd.MASK_CAUSAL, None,
                                             ibw["dq"], ibw["dk"], ibw["dv"], ibw["ws"]),
    }
    calls["backward_atomic"] = lambda: sd.sdpa_backward(
        ip["q"], ip["k"], ip["v"], ibw["out"], ibw["dout"], ibw["lse"], wp.scale, sd.MASK_CAUSAL,
        None, ibw["dq"], ibw["dk"], ibw["dv"], ibw["ws"], atomic=True)
    calls["backward_bias"] = lambda: sd.sdpa_backward_bias(
        ip["q"], ip["k"], ip["v"], ibb["out"], ibb["dout"], ibb["lse"], ibias["bias"], wp.scale,
        sd.MASK_CAUSAL, None, ibb["dbias"], ibb["dq"], ibb["dk"], ibb["dv"], ibb["ws"])
    calls["backward_wide"] = lambda: sd.sdpa_backward(
        iwide["q"], iwide["k"], iwide["v"], ibwd["out"], ibwd["dout"], ibwd["lse"],
        1.0 / math.sqrt(WIDE[3]), sd.MASK_CAUSAL, None, ibwd["dq"], ibwd["dk"], ibwd["dv"],
        ibwd["ws"])
    calls["bias"] = lambda: sd.sdpa_forward_bias(ip["q"], ip["k"], ip["v"], ibias["bias"], wp.scale,
                                                 sd.MASK_CAUSAL, None, ibias["out"])
    calls["decode_wide"] = lambda: sd.sdpa_decode(idw["q"], idw["k"], idw["v"],
                                                  1.0 / math.sqrt(DECODE_WIDE[4]), None,
                                                  wd.num_splits, idw["ws"], idw["out"])
    calls["decode_widest"] = lambda: sd.sdpa_decode(idws["q"], idws["k"], idws["v"],
                                                    1.0 / math.sqrt(DECODE_WIDEST[4]), None,
                                                    wd.num_splits, idws["ws"], idws["out"])
    calls["wide"] = lambda: sd.sdpa_forward(iwide["q"], iwide["k"], iwide["v"],
                                            1.0 / math.sqrt(WIDE[3]), sd.MASK_CAUSAL, None,
                                            iwide["out"])
    calls["widest"] = lambda: sd.sdpa_forward(iwst["q"], iwst["k"], iwst["v"],
                                              1.0 / math.sqrt(WIDEST[3]), sd.MASK_CAUSAL, None,
                                              iwst["out"])
    for name in iblk:
        calls[name] = (lambda blk: lambda: sd.sdpa_block_forward(
            *blk["ins"], blk["H"], None, sd.MASK_CAUSAL, None, blk["y"], blk["ws"]))(iblk[name])
    order = ([args.only] if args.only else
             ["prefill", "padded", "decode", "paged", "paged_prefill", "backward", "backward_atomic",
              "backward_bias", "backward_wide", "bias", "wide", "widest", "decode_wide",
              "decode_widest", "block",
              "block_small"])

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    for _ in range(args.warmup):
        for name in order:
            calls[name]()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    ev = {name: [] for name in order}
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for name in order:
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            calls[name]()
            b.record(stream)
            ev[name].append((a, b))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    times = {name: [a.elapsed_time(b) for a, b in ev[name]] for name in order}
    ms = {name: sum(t) / len(t) for name, t in times.items()}

    # The small configurations (one fp32 head; the tensai guide's block-sized
    # causal attention): microseconds per call, so each is timed over many
    # calls of its own after the step loop (not part of a step).
    small = {}
    if args.only is None and args.small_iters > 0:
        for key, w in (("config1_fp32", WORKLOADS[SMALL_FP32]),
                       ("config2_causal_small", WORKLOADS[SMALL_CAUSAL])):
            inp = make_inputs(w, dev)
            o = torch.empty_like(inp["q"])
            kind = sd.MASK_CAUSAL if w.causal else sd.MASK_NONE
            call = (lambda i, o, w, kind: lambda: sd.sdpa_forward(
                i["q"], i["k"], i["v"], w.scale, kind, None, o))(inp, o, w, kind)
            for _ in range(50):
                call()
            torch.cuda.synchronize()
            evs = []
            for _ in range(args.small_iters):
                a = torch.cuda.Event(enable_timing=True)
                b = torch.cuda.Event(enable_timing=True)
                a.record(stream)
                call()
                b.record(stream)
                evs.append((a, b))
            torch.cuda.synchronize()
            small[key] = (w, [a.elapsed_time(b) for a, b in evs])

    rec = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall * 1e3 / args.steps, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}

    if "prefill" in ms:
        fl = formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["prefill"] * 1e-3) / 1e12
        traffic = stored_traffic("prefill", "forward.hip")
        rec.update({"value": round(tf, 3), "unit": "TFLOP/s"})
        rec["config"] = {"workload": wp.name, "B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Sq": wp.Sq,
                         "Sk": wp.Sk, "D": wp.D, "mask": "causal", "scale": wp.scale,
                         "step_calls": order}
        tp = timing(times["prefill"])
        rec["prefill_ms"] = tp["ms"]
        rec["prefill_ms_median"] = tp["ms_median"]
        rec["prefill_ms_min"] = tp["ms_min"]
        rec["roofline"] = {"bound": "mfma", "achieved": round(tf, 3),
                           "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": traffic,
                           "kernel": "forward_bf16_kernel<128>",
                           "flops_per_launch": fl,
                           "sq_counters": stored_sq("prefill", "forward.hip")}
    if "padded" in ms:
        fl = formula_flops(wg.B, wg.Hq, wg.Sq, wg.Sk, wg.D, False)
        fa = padded_algorithmic_flops(wg, lens_g)
        rec["padded"] = {"workload": wg.name, **timing(times["padded"]),
                         "tflops_formula": round(fl / (ms["padded"] * 1e-3) / 1e12, 3),
                         "tflops_algorithmic": round(fa / (ms["padded"] * 1e-3) / 1e12, 3),
                         "frac_algorithmic": round(fa / (ms["padded"] * 1e-3) / 1e12
                                                   / BF16_MFMA_PEAK_TFLOPS, 4),
                         "key_lens": lens_g,
                         "roofline": {"bound": "mfma",
                                      "achieved": round(fa / (ms["padded"] * 1e-3) / 1e12, 3),
                                      "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(fa / (ms["padded"] * 1e-3) / 1e12
                                                    / BF16_MFMA_PEAK_TFLOPS, 4),
                                      "traffic": stored_traffic("padded", "forward.hip"),
                                      "kernel": "forward_bf16_kernel<128>",
                                      "flops_per_launch": fa,
                                      "flops": "4*Hq*Sq*D per visible key (key_lens)",
                                      "sq_counters": stored_sq("padded", "forward.hip")}}
    if "decode" in ms:
        kv_bytes = 2 * wd.B * wd.Hkv * wd.Sk * wd.D * 2
        qo_bytes = 2 * wd.B * wd.Hq * wd.D * 2
        by = kv_bytes + qo_bytes
        gbs = by / (ms["decode"] * 1e-3) / 1e9
        rec["decode"] = {"workload": wd.name, **timing(times["decode"]), "value": round(gbs, 1),
                         "unit": "GB/s",
                         "tflops_formula": round(formula_flops(wd.B, wd.Hq, 1, wd.Sk, wd.D, False)
                                                 / (ms["decode"] * 1e-3) / 1e12, 3),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                      "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                      "frac": round(gbs / HBM_PEAK_GBS, 4),
                                      "traffic": stored_traffic("decode_split", "decode.hip"),
                                      "kernel": "decode_split_bf16_kernel<128> + merge",
                                      "bytes_per_launch": by}}
    if "paged" in ms:
        kv_bytes = 2 * wd.B * wd.Hkv * wd.Sk * wd.D * 2
        by = kv_bytes + 2 * wd.B * wd.Hq * wd.D * 2 + ipg["block_tables"].numel() * 4
        gbs = by / (ms["paged"] * 1e-3) / 1e9
        rec["paged"] = {"workload": "bf16_gqa32x8_paged_decode_b64_sk32768_d128_page16",
                        **timing(times["paged"]), "value": round(gbs, 1), "unit": "GB/s",
                        "page_size": PAGE_SIZE, "pages": ipg["pages"],
                        "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(gbs / HBM_PEAK_GBS, 4),
                                     "traffic": stored_traffic("paged_split", "decode.hip"),
                                     "kernel": "decode_split_bf16_kernel<128, paged> + merge",
                                     "bytes_per_launch": by}}
    if "paged_prefill" in ms:
        fl = formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["paged_prefill"] * 1e-3) / 1e12
        rec["paged_prefill"] = {"workload": "bf16_causal_paged_prefill_b4_h16_s4096_d128_page16",
                                **timing(times["paged_prefill"]), "value": round(tf, 3),
                                "unit": "TFLOP/s", "page_size": PAGE_SIZE,
                                "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                             "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                             "traffic": stored_traffic("paged_prefill",
                                                                       "forward.hip"),
                                             "kernel": "forward_bf16_kernel<128, paged>",
                                             "flops_per_launch": fl}}
    if "backward" in ms:
        fl = 2.5 * formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["backward"] * 1e-3) / 1e12
        rec["backward"] = {"workload": "bf16_causal_backward_b4_h16_s4096_d128",
                           **timing(times["backward"]), "value": round(tf, 3),
                           "unit": "TFLOP/s",
                           "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                        "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                        "traffic": backward_traffic(),
                                        "kernel": "bwd_dq_kernel<128> + bwd_dkdv_kernel<128>",
                                        "flops_per_launch": fl}}
    if "backward_atomic" in ms:
        fl = 2.5 * formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["backward_atomic"] * 1e-3) / 1e12
        rec["backward_atomic"] = {"workload": "bf16_causal_backward_atomic_b4_h16_s4096_d128",
                                  **timing(times["backward_atomic"]), "value": round(tf, 3),
                                  "unit": "TFLOP/s",
                                  "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                               "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                               "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                               "traffic": atomic_traffic(),
                                               "kernel": "bwd_prep + bwd_dkdv<128, atomic dQ> + "
                                                         "bwd_dq_convert",
                                               "flops_per_launch": fl}}
    if "backward_bias" in ms:
        fl = 2.5 * formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["backward_bias"] * 1e-3) / 1e12
        dbias_bytes = wp.B * wp.Hq * wp.Sq * wp.Sk * 2
        rec["backward_bias"] = {"workload": "bf16_causal_backward_bias_b4_h16_s4096_d128",
                                **timing(times["backward_bias"]), "value": round(tf, 3),
                                "unit": "TFLOP/s", "bias_shape": [1, wp.Hq, wp.Sq, wp.Sk],
                                "dbias_shape": [wp.B, wp.Hq, wp.Sq, wp.Sk],
                                "dbias_bytes_written": dbias_bytes,
                                "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                             "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                             "traffic": bias_backward_traffic(),
                                             "kernel": "bwd_dq_kernel<128, bias> + "
                                                       "bwd_dkdv_kernel<128, bias>",
                                             "flops_per_launch": fl}}
    if "bias" in ms:
        fl = formula_flops(wp.B, wp.Hq, wp.Sq, wp.Sk, wp.D, True)
        tf = fl / (ms["bias"] * 1e-3) / 1e12
        # bias bytes the kernel must read: the visible (causal) part of each
        # (batch, head)'s [Sq, Sk] slice, at 2 bytes, whole 64-key tiles
        nqb = wp.Sq // 128
        tiles = sum(2 * (qb + 1) for qb in range(nqb))          # 64-key tiles per (b, h)
        bias_bytes = wp.B * wp.Hq * 128 * 64 * 2 * tiles
        rec["bias"] = {"workload": "bf16_causal_bias_b4_h16_s4096_d128",
                       **timing(times["bias"]), "value": round(tf, 3), "unit": "TFLOP/s",
                       "bias_shape": [1, wp.Hq, wp.Sq, wp.Sk],
                       "bias_bytes_read": bias_bytes,
                       "bias_gbs": round(bias_bytes / (ms["bias"] * 1e-3) / 1e9, 1),
                       "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                    "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                    "traffic": stored_traffic("bias", "forward.hip"),
                                    "kernel": "forward_bf16_kernel<128, bias>",
                                    "flops_per_launch": fl}}
    if "wide" in ms:
        B, H, S, D = WIDE
        fl = formula_flops(B, H, S, S, D, True)
        tf = fl / (ms["wide"] * 1e-3) / 1e12
        rec["wide"] = {"workload": "bf16_causal_b%d_h%d_s%d_d%d" % (B, H, S, D),
                       **timing(times["wide"]), "value": round(tf, 3), "unit": "TFLOP/s",
                       "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                    "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                    "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                    "traffic": stored_traffic("wide", "forward.hip"),
                                    "kernel": "forward_pair_kernel<256>",
                                    "flops_per_launch": fl}}
    if "backward_wide" in ms:
        B, H, S, D = WIDE
        fl = 2.5 * formula_flops(B, H, S, S, D, True)
        tf = fl / (ms["backward_wide"] * 1e-3) / 1e12
        rec["backward_wide"] = {"workload": "bf16_causal_backward_b%d_h%d_s%d_d%d" % (B, H, S, D),
                                **timing(times["backward_wide"]), "value": round(tf, 3),
                                "unit": "TFLOP/s",
                                "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                             "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                             "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                             "traffic": wide_backward_traffic(),
                                             "kernel": "bwd_wide_stats_kernel + bwd_wide_dq_kernel<2>"
                                                       " + bwd_wide_dkdv_kernel<2>",
                                             "flops_per_launch": fl}}
    if "widest" in ms:
        B, H, S, D = WIDEST
        fl = formula_flops(B, H, S, S, D, True)
        tf = fl / (ms["widest"] * 1e-3) / 1e12
        rec["widest"] = {"workload": "bf16_causal_b%d_h%d_s%d_d%d" % (B, H, S, D),
                         **timing(times["widest"]), "value": round(tf, 3), "unit": "TFLOP/s",
                         "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                      "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                      "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                      "traffic": stored_traffic("widest", "forward_wide.hip"),
                                      "kernel": "forward_wide_kernel<8> (head dim split over 8 waves)",
                                      "flops_per_launch": fl}}
    if "decode_wide" in ms:
        B, Hq, Hkv, Sk, D = DECODE_WIDE
        by = 2 * B * Hkv * Sk * D * 2 + 2 * B * Hq * D * 2
        gbs = by / (ms["decode_wide"] * 1e-3) / 1e9
        rec["decode_wide"] = {"workload": "bf16_gqa32x8_decode_b%d_sk%d_d%d" % (B, Sk, D),
                              **timing(times["decode_wide"]), "value": round(gbs, 1),
                              "unit": "GB/s", "num_splits": wd.num_splits,
                              "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                           "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                           "frac": round(gbs / HBM_PEAK_GBS, 4),
                                           "traffic": pair_traffic("decode_wide_split",
                                                                   "decode_wide_merge", "decode.hip"),
                                           "kernel": "decode_split_bf16_kernel<256> + merge",
                                           "bytes_per_launch": by}}
    if "decode_widest" in ms:
        B, Hq, Hkv, Sk, D = DECODE_WIDEST
        by = 2 * B * Hkv * Sk * D * 2 + 2 * B * Hq * D * 2
        gbs = by / (ms["decode_widest"] * 1e-3) / 1e9
        rec["decode_widest"] = {"workload": "bf16_gqa32x8_decode_b%d_sk%d_d%d" % (B, Sk, D),
                                **timing(times["decode_widest"]), "value": round(gbs, 1),
                                "unit": "GB/s", "num_splits": wd.num_splits,
                                "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                             "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                             "frac": round(gbs / HBM_PEAK_GBS, 4),
                                             "traffic": pair_traffic("decode_widest_split",
                                                                     "decode_widest_merge",
                                                                     "forward_wide.hip", "decode.hip"),
                                             "kernel": "forward_wide_kernel<8, decode> + merge",
                                             "bytes_per_launch": by}}
    for name, (B, S, M, H) in BLOCKS.items():
        if name not in ms:
            continue
        fl = block_flops(B, S, M, H, True)
        tf = fl / (ms[name] * 1e-3) / 1e12
        rec[name] = {"workload": "bf16_causal_block_b%d_s%d_m%d_h%d" % (B, S, M, H),
                     **timing(times[name]), "value": round(tf, 3), "unit": "TFLOP/s",
                     "flops": "8*B*S*model^2 (four projections) + the causal attention formula",
                     "roofline": {"bound": "mfma", "achieved": round(tf, 3),
                                  "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                                  "traffic": block_traffic(name),
                                  "kernel": "gemm_kernel<q/k/v> + forward_bf16_kernel + "
                                            "gemm_kernel<out>",
                                  "flops_per_launch": fl}}
    for key, (w, t) in small.items():
        fl = formula_flops(w.B, w.Hq, w.Sq, w.Sk, w.D, w.causal)
        med = timing(t)["ms_median"]
        rec[key] = {"workload": w.name, "dtype": "f32" if w.dtype == torch.float32 else "bf16",
                    **timing(t), "us_median": round(med * 1e3, 2),
                    "us_min": round(min(t) * 1e3, 2),
                    "tflops_median": round(fl / (med * 1e-3) / 1e12, 4),
                    "note": "timed alone, per call, after the step loop; launch-bound"}
    if "value" not in rec:  # --only another call: report that call
        blk = [n for n in list(BLOCKS) + ["wide", "widest", "decode_wide", "decode_widest"] if n in rec]
        if blk:
            rec.update({"value": rec[blk[0]]["value"], "unit": rec[blk[0]]["unit"]})
            rec["config"] = {"workload": rec[blk[0]]["workload"]}
        elif "bias" in rec:
            rec.update({"value": rec["bias"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["bias"]["workload"]}
        elif "backward_bias" in rec:
            rec.update({"value": rec["backward_bias"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["backward_bias"]["workload"]}
        elif "backward_atomic" in rec:
            rec.update({"value": rec["backward_atomic"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["backward_atomic"]["workload"]}
        elif "backward_wide" in rec:
            rec.update({"value": rec["backward_wide"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["backward_wide"]["workload"]}
        elif "backward" in rec:
            rec.update({"value": rec["backward"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["backward"]["workload"]}
        elif "paged_prefill" in rec:
            rec.update({"value": rec["paged_prefill"]["value"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": rec["paged_prefill"]["workload"]}
        elif "paged" in rec:
            rec.update({"value": rec["paged"]["value"], "unit": "GB/s"})
            rec["config"] = {"workload": rec["paged"]["workload"]}
        elif "decode" in rec:
            rec.update({"value": rec["decode"]["value"], "unit": "GB/s"})
            rec["config"] = {"workload": wd.name}
        else:
            rec.update({"value": rec["padded"]["tflops_formula"], "unit": "TFLOP/s"})
            rec["config"] = {"workload": wg.name}

    del ip, ig, idd, ipg, ipp, ibw, ibias, ibb, iblk, iwide, iwst, idw, idws
    torch.cuda.empty_cache()
    if not args.no_cpu_baseline and args.only in (None, "prefill"):
        rec["cpu_baseline"] = cpu_baseline(args.cpu_budget)
    if not args.no_cpu_baseline and args.only in (None, "padded") and "padded" in rec:
        rec["padded"]["cpu_baseline"] = cpu_baseline_padded(args.cpu_budget / 2)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
