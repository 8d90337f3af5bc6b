"""Benchmark of the indexer hot path on one MI355X.

A step is one call of an exact Top-K entry point (every kernel of the path)
over one synthetic input batch already resident in HBM.  The timed region is
bracketed by device synchronisation; throughput counts visible (query, key)
pairs: key s is visible to a row at position p iff s <= p.

Prints ONE JSON line.  Default workload: the 128K chunked-prefill block (8192
rows at positions 122880..131071, 131072 keys, top-2048, bf16) through the
unpruned streaming Top-K (dsa_indexer_topk).  Reported beside it ("also"):
the certified-pruning path on the same block and on the 1M-key fp8 block
(with the unpruned 1M run, for the pruned/unpruned time ratio), the 128K
block with noisier queries (the filter-rate sensitivity), the 32K prefill,
decode, the projections and the sparse attention consumer.

The roofline object describes the dominant kernel of the timed path (the one
with the most device time): its duration is the mean of HIP events the
library records around each launch on the launch stream during the timed
steps; its work is the matrix-product FLOPs its launches execute (2*64*128
per fully scored pair; the pruned path's chunk screen 2*128*32 per bounded
pair), against MI355X's published dense MFMA peak for the dtype.  Beside
it, the rate the same score step sustains on this part with no memory
traffic (the library's probe on synthetic full-entropy operands): under a
full MFMA load the clock drops below the one the nominal peak assumes.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # MI355X dense MFMA, published
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
# HBM bytes per dispatch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs (KiB per
# dispatch, mean over dispatches), scaled by what the same counters read for a
# 1 GiB device copy (FETCH x2.000, WRITE x1.000).  Valid only for the kernel
# sources they were taken on: reported as null once the sources change.
FETCH_SCALE, WRITE_SCALE = 2.000, 1.000
MEASURED_KIB = {
    # (workload, kernel): (source digest, FETCH_SIZE KiB, WRITE_SIZE KiB), mean per dispatch
    ("chunked_prefill_128k", "k_topk_stream"): ("ed5c0288e30347f3", 2356716, 1326594),
    ("context_1m_fp8", "k_topk_stream"): ("ed5c0288e30347f3", 10755417, 3490426),
    ("prefill_32k", "k_topk_stream"): ("ed5c0288e30347f3", 5149960, 2898887),
    ("chunked_prefill_128k", "k_screen"): ("d2a4107fa2b71100", 59863, 12966),
    ("chunked_prefill_128k", "k_refine"): ("d2a4107fa2b71100", 178890, 37518),
    ("context_1m_fp8", "k_screen"): ("d2a4107fa2b71100", 133744, 65544),
    ("context_1m_fp8", "k_refine"): ("d2a4107fa2b71100", 206915, 35770),
    ("decode_64x128k", "k_scores"): ("08c4ecbd515913c3", 1067502, 33264),
    ("projection_prefill_128k", "k_proj_out"): ("c339d5bbec5abf88", 1073178, 553000),
    ("sparse_mla_128k", "k_sparse_mla"): ("2d225659671baf9a", 6519512, 1126288),
}
PAIR_FLOPS = 2 * 64 * 128  # full 64-head score of one pair
PAGES_SEEDS = 12288  # the pages' seed count (the library's default)
SCREEN_FLOPS = 2 * 128 * 32  # 32-row bound (30 retained heads, aux row, linear row) of one pair


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="chunked_prefill_128k")
    ap.add_argument("--path", choices=["auto", "topk", "pruned", "pruned_tau", "pruned_compact", "pruned_anchor"],
                    default="topk",
                    help="exact Top-K route of the main line (auto: pruned where the workload is a pruning one; "
                    "pruned_tau: the pruned path with every row's threshold starting at tau (12288 seeds); "
                    "pruned_compact: the pruned path with 32-bit candidate records; pruned_anchor: the pruned path "
                    "with seeds from anchor queries (12288 seeds: 6 anchor rows), starting at tau)")
    ap.add_argument(
        "--also",
        default="chunked_prefill_128k:pruned,chunked_prefill_128k:pruned_tau,chunked_prefill_128k:pruned_compact,"
        "chunked_prefill_128k:pruned_anchor,"
        "context_1m_fp8:topk,context_1m_fp8:pruned,context_1m_fp8:pruned_tau,context_1m_fp8:pruned_compact,"
        "context_1m_fp8:pruned_anchor,"
        "chunked_prefill_128k_noise02:pruned,prefill_32k:topk,"
        "decode_64x128k:topk,projection_prefill_128k:project,sparse_mla_128k:sparse_mla,"
        "sparse_mla_decode_64x128k:sparse_mla",
        help="comma list of extra workload[:path] runs (or 'none')",
    )
    ap.add_argument("--num-seeds", type=int, default=0,
                    help="seeds per sequence of the pruned paths (0: the workload's own count)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=1024, help="rows of the oracle sample (at most; see --cpu-seconds)")
    ap.add_argument("--cpu-seconds", type=float, default=25.0, help="stop the oracle sample after this much CPU time")
    ap.add_argument("--cpu-also", default="context_1m_fp8",
                    help="comma list of further workloads whose oracle is timed the same way (or 'none')")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device-to-device 3 times (counter calibration) and exit")
    ap.add_argument("--sustained-only", action="store_true",
                    help="only measure the score step's sustained MFMA rates (bf16, fp8), print them and exit")
    return ap.parse_args()


# Source files whose code a kernel is built from (its own file and the device
# headers it includes; kernels.h holds only host-side declarations, and no
# kernel takes one of its structs).  A stored counter reading is valid while
# their digest holds.
KERNEL_SOURCES = {
    "k_topk_stream": ["topk_stream.hip", "stream_common.h", "score_tile.h", "select.h"],
    "k_screen": ["topk_pruned.hip", "stream_common.h", "score_tile.h", "select.h"],
    "k_refine": ["topk_pruned.hip", "stream_common.h", "score_tile.h", "select.h"],
    "k_scores": ["scores.hip", "score_tile.h"],
    "k_proj_out": ["project.hip"],
    "k_sparse_mla": ["sparse_mla.hip"],
}


def _code_only(text):
    """Source text without comments, trailing blanks or empty lines."""
    import re

    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def source_digest(kernel):
    """Digest of the HIP code of one kernel (the key of MEASURED_KIB);
    comments do not enter it, so editing them keeps a reading valid."""
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "dsa_lightning_indexer_04_amd", "csrc")
    for f in sorted(KERNEL_SOURCES[kernel]):
        h.update(f.encode())
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    m = MEASURED_KIB.get((workload, kernel))
    if m is None or kernel not in KERNEL_SOURCES or m[0] != source_digest(kernel):
        return None
    return (m[1] * FETCH_SCALE + m[2] * WRITE_SCALE) * 1024


def copy_calibration(mib):
    """A plain copy of known size, for scaling FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": mib << 20, "copy_bytes_written": mib << 20, "launches": 3}), flush=True)


def sustained_rates(dtype, launches=5, warmup=2):
    """The score step's sustained MFMA rate on this part (TFLOP/s): the
    library's probe (dsa_indexer_mfma_ceiling) runs the streaming kernel's
    32-key block step on synthetic full-entropy operands in registers and LDS,
    without memory traffic or candidate bookkeeping, long enough (about 10 ms
    a launch) for the clock to settle.  mode 0: MFMAs and fragment reloads
    only; mode 1: with the ReLU-weighted head sum and the combine; mode 2
    (bf16): the head sum as (w/2)(x + |x|), one abs-FMA per head and key plus
    the linear term on 8 more 16x16x32 MFMAs per 32 keys (rate over the same
    64-head FLOPs)."""
    import torch
    from dsa_lightning_indexer_04_amd import _lib

    iters = 16000 if dtype == "bf16" else 32000
    wg = _lib.mfma_ceiling(dtype, 1, iters)
    out = torch.empty(wg * 256, dtype=torch.float32, device="cuda")
    flops = wg * 4 * iters * 2 * 64 * 32 * 128
    res = {"unit": "TFLOP/s", "workgroups": wg, "flops_per_launch": flops}
    modes = ((0, "mfma_only"), (1, "score_step")) + (((2, "score_step_abs_form"),) if dtype == "bf16" else ())
    for mode, key in modes:
        for _ in range(warmup):
            _lib.mfma_ceiling(dtype, mode, iters, out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            _lib.mfma_ceiling(dtype, mode, iters, out)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / launches
        res[key] = flops / (ms * 1e-3) / 1e12
        res[key + "_ms"] = ms
    return res


def run_workload(name, path, steps, warmup, num_seeds=0):
    import dataclasses

    import torch

    import dsa_lightning_indexer_04_amd as dsa
    from dsa_lightning_indexer_04_amd import _lib, inputs

    wl = inputs.WORKLOADS[name]
    if num_seeds:  # a seed count other than the workload's (pruned paths)
        wl = dataclasses.replace(wl, num_seeds=num_seeds)
    elif path in ("pruned_tau", "pruned_anchor"):
        # the pages' start (tau) and the anchor seeds take the pages' seed
        # count: tau is the K-th best seed score, so it needs seeds well
        # beyond K, which the raised start does not
        wl = dataclasses.replace(wl, num_seeds=PAGES_SEEDS)
    t0 = time.time()
    d = inputs.make_workload(wl)
    log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
    dev = torch.device("cuda:0")
    q, k, w, pos = (d[n].to(dev) for n in ("q", "k", "w", "pos"))
    qs = None if d["q_scale"] is None else d["q_scale"].to(dev)
    ks = None if d["k_scale"] is None else d["k_scale"].to(dev)
    del d
    use_pruned = path in ("pruned", "pruned_tau", "pruned_compact", "pruned_anchor") or (path == "auto" and wl.pruned)
    start = "tau" if path in ("pruned_tau", "pruned_anchor") else "raised"
    records = "compact" if path == "pruned_compact" else "exact"
    seeds_from = "anchor" if path == "pruned_anchor" else "even"
    inp = _lib.make_inputs_struct(q, k, w, pos, qs, ks)
    stats = None
    if use_pruned:
        opts = _lib.PruneOpts(wl.num_seeds, 0, None, None,
                              _lib.PRUNE_STARTS[start] | _lib.PRUNE_RECORDS[records] | _lib.PRUNE_SEEDS[seeds_from])
        ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK_PRUNED, inp, wl.topk, opts), dtype=torch.uint8,
                         device=dev)

        def call():
            return dsa.topk_pruned(q, k, w, pos, wl.topk, q_scale=qs, k_scale=ks, num_seeds=wl.num_seeds, start=start,
                                   records=records, seeds=seeds_from, return_scores=False, workspace=ws)

        _, _, st = dsa.topk_pruned(q, k, w, pos, wl.topk, q_scale=qs, k_scale=ks, num_seeds=wl.num_seeds,
                                   start=start, records=records, seeds=seeds_from, return_scores=False, workspace=ws,
                                   stats=True)
        scr = int(st["screened"].sum().item())
        sur = int(st["survivors"].sum().item())
        anchor_pairs = 0
        if seeds_from == "anchor":
            # every visible pair is a seed pair or screened (no row recovers
            # here); the anchor rows' own Top-K scores all their visible keys
            seeds = wl.visible_pairs - scr
            A = min(wl.num_q, max(1, wl.num_seeds // wl.topk))
            anchor_pairs = wl.batch * sum(min(wl.num_k, wl.pos_start + ((2 * i + 1) * wl.num_q) // (2 * A) + 1)
                                          for i in range(A))
        else:
            seeds = min(wl.num_seeds, wl.pos_start + 1) * wl.num_q * wl.batch  # evenly spaced, visible to every row
        stats = {"screened_pairs": scr, "survivor_pairs": sur, "seed_pairs": seeds, "anchor_pairs": anchor_pairs,
                 "filter_rate": 1.0 - sur / max(1, scr), "start": start, "records": records, "seeds": wl.num_seeds,
                 "seed_source": seeds_from,
                 "recovered_rows": int((st["recovered"] != 0).sum().item()),
                 "start_misses": int((st["recovered"] == 2).sum().item())}
    else:
        ws = torch.empty(_lib.workspace_bytes(_lib.DSA_OP_TOPK, inp, wl.topk), dtype=torch.uint8, device=dev)

        def call():
            return dsa.topk(q, k, w, pos, wl.topk, q_scale=qs, k_scale=ks, return_scores=False, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    _lib.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernels = _lib.profile_end()
    pairs = wl.visible_pairs
    res = {
        "workload": name,
        "path": (path if path.startswith("pruned") else "pruned") if use_pruned else "unpruned",
        "dtype": wl.dtype,
        "visible_pairs": pairs,
        "ms_per_step": wall * 1e3 / steps,
        "pairs_per_s": pairs / (wall / steps),
        "kernels_ms": {n: round(ms, 4) for n, (c, ms) in kernels.items()},
    }
    # per kernel: launches and device time per step, and the matrix-product
    # FLOPs its launches execute per step
    per_step = {n: {"launches": c / steps, "ms": c * ms / steps} for n, (c, ms) in kernels.items()}
    if use_pruned:
        # seeds: the streaming Top-K over the packed seed keys; the screen
        # bounds the other visible keys (32 plan rows each); the refine
        # rescores the survivors with all 64 heads
        work = {"k_topk_stream": stats["seed_pairs"] * PAIR_FLOPS,
                "k_topk_stream_anchors": stats["anchor_pairs"] * PAIR_FLOPS,
                "k_screen": stats["screened_pairs"] * SCREEN_FLOPS,
                "k_refine": stats["survivor_pairs"] * PAIR_FLOPS}
        res["prune"] = stats
    else:
        work = {n: pairs * PAIR_FLOPS for n in per_step if n in ("k_topk_stream", "k_scores")}
    for n, v in per_step.items():
        # HBM bytes from stored counter readings, or None (in the pruned path the
        # streaming kernel scores the packed seeds: no reading is stored for that)
        v["traffic_per_launch"] = None if (use_pruned and n == "k_topk_stream") else measured_traffic(name, n)
        # HBM rate of the kernel's counted traffic over its device time
        v["hbm_gbs"] = (v["traffic_per_launch"] * v["launches"] / (v["ms"] * 1e-3) / 1e9
                        if v["traffic_per_launch"] and v["ms"] > 0 else None)
        v["flops"] = work.get(n, 0)
        v["tflops"] = v["flops"] / (v["ms"] * 1e-3) / 1e12 if v["ms"] > 0 else 0.0
        v["frac"] = v["tflops"] / PEAK_TFLOPS[wl.dtype]
    res["kernels"] = per_step
    dom = max(per_step.items(), key=lambda kv: kv[1]["ms"])  # the kernel with the most device time
    dk, dv = dom
    flops = sum(work.values())
    res["dominant_kernel"] = dk
    res["dominant_ms"] = dv["ms"] / max(dv["launches"], 1e-9)  # mean per launch
    res["dominant_launches"] = dv["launches"]
    res["executed_flops"] = flops
    res["dominant_flops"] = dv["flops"] / max(dv["launches"], 1e-9)  # per launch
    res["achieved_tflops"] = dv["tflops"]
    res["effective_tflops"] = pairs * PAIR_FLOPS / (res["ms_per_step"] * 1e-3) / 1e12
    # every visible pair counted at 16,384 FLOP over the whole call's time (for a
    # pruned call this exceeds the work it executes)
    res["effective_frac"] = res["effective_tflops"] / PEAK_TFLOPS[wl.dtype]
    peak = PEAK_TFLOPS[wl.dtype]
    if wl.num_q == 1:
        # one query row per sequence (decode): every key row is read once and
        # serves 64 heads, far below the MFMA ridge point -> HBM-bound; the
        # algorithmic bytes are the keys (and fp8 scales), the query rows and
        # the weights
        key_bytes = wl.batch * wl.num_k * (256 if wl.dtype == "bf16" else 128 + 4)
        q_bytes = wl.batch * 64 * (256 if wl.dtype == "bf16" else 128) + wl.batch * 64 * 4
        alg = key_bytes + q_bytes
        sk = per_step.get("k_scores", dv)
        ms = sk["ms"] / max(sk["launches"], 1e-9)
        res["roofline"] = {"bound": "hbm", "achieved": alg / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "kernel": "k_scores", "bytes_per_launch": alg,
                           "traffic": measured_traffic(name, "k_scores")}
    else:
        res["roofline"] = {"bound": "mfma", "achieved": res["achieved_tflops"], "peak": peak, "unit": "TFLOP/s",
                           "kernel": dk, "flops_per_launch": res["dominant_flops"],
                           "traffic": measured_traffic(name, dk)}
    res["roofline"]["frac"] = res["roofline"]["achieved"] / res["roofline"]["peak"]
    log(f"[bench] {name} {res['path']}: {res['ms_per_step']:.3f} ms/step, {res['pairs_per_s']:.3e} pairs/s; "
        + ", ".join(f"{n} {v['ms']:.3f} ms" + (f" ({100 * v['frac']:.1f}%)" if v["flops"] else "")
                    for n, v in sorted(per_step.items(), key=lambda kv: -kv[1]["ms"]))
        + (f"; filter rate {100 * stats['filter_rate']:.1f}%; effective {100 * res['effective_frac']:.1f}% of "
           f"{wl.dtype} MFMA" if stats else ""))
    del q, k, w, pos, qs, ks, ws
    torch.cuda.empty_cache()
    return res


# Indexer projection workloads: tokens projected per step (DeepSeek-V3.2 sizes).
PROJ_WORKLOADS = {"projection_prefill_128k": 131072, "projection_chunk_8k": 8192}


def run_projection(name, steps, warmup):
    """The projection prologue: C^Q W_IQ, X [W_IK W_IW] (rocBLAS, bf16 -> fp32)
    and the per-token fp8 output pass, on T synthetic tokens."""
    import torch

    import dsa_lightning_indexer_04_amd as dsa
    from dsa_lightning_indexer_04_amd import _lib, inputs

    T = PROJ_WORKLOADS[name]
    L, D = inputs.PROJ_Q_LATENT, inputs.PROJ_HIDDEN
    t0 = time.time()
    d = inputs.make_projection_inputs(T, D, L, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
    args = (d["c_q"], d["x"], d["w_iq"], d["w_ik"], d["w_iw"])
    ws = torch.empty(_lib.project_workspace_bytes(_lib.make_proj_struct(*args)), dtype=torch.uint8, device="cuda")

    def call():
        return dsa.project(*args, out="fp8", workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    _lib.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernels = _lib.profile_end()
    ms = wall * 1e3 / steps
    flops = 2 * T * (L * 64 * 128 + D * 128 + D * 64)
    # tokens one launch of each kernel covers (the query GEMM and the output
    # pass run per token block, the key/weight GEMM once over all tokens)
    per_launch = {n: T * steps / c for n, (c, _) in kernels.items()}
    blk = per_launch.get("k_proj_out", T)
    gq = kernels.get("gemm_q_proj", (0, float("nan")))[1]
    gkw = kernels.get("gemm_kw_proj", (0, float("nan")))[1]
    po = kernels.get("k_proj_out", (0, float("nan")))[1]
    kw_tokens = per_launch.get("gemm_kw_proj", T)
    out_bytes = blk * ((64 * 128 + 128 + 64) * 4 + 64 * 128 + 128 + 64 * 4 + 8)  # fp32 staging in; codes, w, scales out
    res = {
        "workload": name,
        "path": "project",
        "dtype": "bf16",
        "tokens": T,
        "ms_per_step": ms,
        "tokens_per_s": T / (wall / steps),
        "tflops": flops / (ms * 1e-3) / 1e12,
        "kernels_ms": {n: round(v, 4) for n, (c, v) in kernels.items()},
        "roofline_gemm_q": {"bound": "mfma", "achieved": 2 * blk * L * 64 * 128 / (gq * 1e-3) / 1e12,
                            "peak": PEAK_TFLOPS["bf16"], "unit": "TFLOP/s", "kernel": "rocBLAS gemm (C^Q W_IQ)"},
        # 192 FLOP per byte of X: below the bf16 ridge (2500 TFLOP/s / 8 TB/s), so HBM-bound
        "roofline_gemm_kw": {"bound": "hbm", "achieved": kw_tokens * (D * 2 + 192 * 4) / (gkw * 1e-3) / 1e9,
                             "peak": PEAK_HBM_GBS, "unit": "GB/s", "kernel": "rocBLAS gemm (X [W_IK W_IW])",
                             "tflops": 2 * kw_tokens * D * 192 / (gkw * 1e-3) / 1e12},
        "roofline_out": {"bound": "hbm", "achieved": out_bytes / (po * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "kernel": "k_proj_out", "bytes_per_launch": out_bytes,
                         "traffic": measured_traffic(name, "k_proj_out")},
    }
    for key in ("roofline_gemm_q", "roofline_gemm_kw", "roofline_out"):
        res[key]["frac"] = res[key]["achieved"] / res[key]["peak"]
    log(f"[bench] {name}: {ms:.3f} ms/step, {res['tflops']:.0f} TFLOP/s overall; gemm_q {gq:.3f} ms "
        f"({100 * res['roofline_gemm_q']['frac']:.1f}% bf16), gemm_kw {gkw:.3f} ms "
        f"({100 * res['roofline_gemm_kw']['frac']:.1f}% HBM), k_proj_out {po:.3f} ms "
        f"({100 * res['roofline_out']['frac']:.1f}% HBM); {blk:.0f} tokens per query-GEMM block")
    del d, args, ws
    torch.cuda.empty_cache()
    return res


# Sparse MLA workloads: the indexer block whose Top-K the attention consumes.
MLA_WORKLOADS = {"sparse_mla_128k": "chunked_prefill_128k", "sparse_mla_decode_64x128k": "decode_64x128k"}
MLA_PAIR_FLOPS = 2 * 128 * (2 * 512 + 64)  # 2h(2 d_c + d_r) per selected pair


def run_sparse_mla(name, steps, warmup):
    """Core attention over the indexer's Top-K: the block's selections come
    from one dsa_indexer_topk call (untimed); q [Q,128,576] and the latent
    cache [N,576] are synthetic bf16."""
    import math

    import torch

    import dsa_lightning_indexer_04_amd as dsa
    from dsa_lightning_indexer_04_amd import _lib, inputs

    wl = inputs.WORKLOADS[MLA_WORKLOADS[name]]
    d = inputs.make_workload(wl)
    dev = torch.device("cuda:0")
    q8, k8, w, pos = (d[n].to(dev) for n in ("q", "k", "w", "pos"))
    idx, _ = dsa.topk(q8, k8, w, pos, wl.topk, return_scores=False)
    del q8, k8, w, d
    t0 = time.time()
    md = inputs.make_mla_inputs(wl.batch, wl.num_q, wl.num_k, seed=0, device="cuda")
    torch.cuda.synchronize()
    log(f"[bench] {name}: inputs drawn in {time.time() - t0:.1f}s")
    q, kv = md["q"], md["kv"]
    sm_scale = 1.0 / math.sqrt(576)
    ws = torch.empty(_lib.sparse_mla_workspace_bytes(_lib.make_mla_struct(q, kv, idx)), dtype=torch.uint8, device=dev)
    pairs = int((idx >= 0).sum().item())

    def call():
        return dsa.sparse_mla(q, kv, idx, sm_scale, workspace=ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    _lib.profile_begin()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernels = _lib.profile_end()
    ms = wall * 1e3 / steps
    km = kernels.get("k_sparse_mla", (0, float("nan")))[1]
    flops = pairs * MLA_PAIR_FLOPS
    rows = wl.batch * wl.num_q
    # gathered cache rows, the query block, the bf16 output and the lse
    alg_bytes = pairs * 576 * 2 + rows * 128 * 576 * 2 + rows * 128 * 512 * 2 + rows * 128 * 4
    res = {
        "workload": name,
        "path": "sparse_mla",
        "dtype": "bf16",
        "indexer_block": MLA_WORKLOADS[name],
        "selected_pairs": pairs,
        "ms_per_step": ms,
        "pairs_per_s": pairs / (wall / steps),
        "kernels_ms": {n: round(v, 4) for n, (c, v) in kernels.items()},
        # 278,528 FLOP per 1152-byte gathered row: ~228 FLOP/B with the query
        # and output, below the bf16 ridge (2500 TFLOP/s / 8 TB/s = 312): the
        # algorithmic bound is HBM (the MFMA fraction is reported beside it)
        "roofline": {"bound": "hbm", "achieved": alg_bytes / (km * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "kernel": "k_sparse_mla", "bytes_per_launch": alg_bytes,
                     "traffic": measured_traffic(name, "k_sparse_mla"),
                     "mfma_tflops": flops / (km * 1e-3) / 1e12, "mfma_frac": flops / (km * 1e-3) / 1e12 / PEAK_TFLOPS["bf16"],
                     "flops_per_launch": flops},
    }
    res["roofline"]["frac"] = res["roofline"]["achieved"] / res["roofline"]["peak"]
    log(f"[bench] {name}: {ms:.3f} ms/step, {res['pairs_per_s']:.3e} selected pairs/s; k_sparse_mla {km:.3f} ms at "
        f"{res['roofline']['achieved']:.0f} GB/s algorithmic ({100 * res['roofline']['frac']:.1f}% of HBM), "
        f"{res['roofline']['mfma_tflops']:.0f} TFLOP/s ({100 * res['roofline']['mfma_frac']:.1f}% of bf16 peak)")
    del q, kv, idx, ws, md
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name, rows_wanted, max_seconds):
    """Time the float64 oracle (scores + sort Top-K) on a bounded row sample:
    the last row, the first, then rows drawn by rng(0), until rows_wanted
    rows or max_seconds of oracle time; pairs/s of the sample."""
    from dsa_lightning_indexer_04_amd import inputs
    from oracle import indexer

    wl = inputs.WORKLOADS[name]
    d = inputs.make_workload(wl)
    qb, kb = inputs.to_bits(d["q"]), inputs.to_bits(d["k"])
    w = d["w"].numpy().astype(np.float64)
    pos = d["pos"].numpy()
    if wl.dtype == "bf16":
        kf = indexer.decode_bf16(kb[0])
    else:
        kf = indexer.decode_e4m3fn(kb[0]) * d["k_scale"].numpy()[0].astype(np.float64)[:, None]
    rng = np.random.default_rng(0)
    Q = wl.num_q
    threads = _blas_threads()
    order = [Q - 1, 0] + [int(t) for t in rng.permutation(Q) if t not in (0, Q - 1)]
    done_pairs, t_total, rows = 0, 0.0, 0
    for t in order:
        if rows >= rows_wanted or t_total > max_seconds:
            break
        t0 = time.perf_counter()
        if wl.dtype == "bf16":
            qf = indexer.decode_bf16(qb[0, t])
        else:
            qf = indexer.decode_e4m3fn(qb[0, t]) * float(d["q_scale"].numpy()[0, t])
        v = int(indexer.visible_count(pos[0, t], wl.num_k))
        s = indexer.index_score_row(qf, kf[:v], w[0, t])
        indexer.topk_row(s, wl.topk)
        t_total += time.perf_counter() - t0
        done_pairs += v
        rows += 1
    return {
        "value": done_pairs / t_total,
        "unit": "pairs/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} of {Q} query rows of {name} (last, first, then random by rng(0)), stopped at "
        f"{rows_wanted} rows or {max_seconds:.0f} s; float64 numpy scores + lexsort Top-K; {done_pairs} visible "
        f"pairs in {t_total:.1f} s; pairs/s of the sample (the whole block at this rate: "
        f"{wl.visible_pairs / (done_pairs / t_total):.0f} s)",
    }


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.sustained_only:
        res = {dt: sustained_rates(dt) for dt in ("bf16", "fp8")}
        for dt, r in res.items():
            for key in ("mfma_only", "score_step", "score_step_abs_form"):
                if key in r:
                    r[key + "_frac"] = r[key] / PEAK_TFLOPS[dt]
        print(json.dumps({"sustained_mfma": res}), flush=True)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; rows shard across GPUs with no "
                          "collective (see the design notes), so no multi-GPU figure is produced",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    import torch

    assert torch.cuda.is_available(), "bench needs a GPU"
    from dsa_lightning_indexer_04_amd import inputs

    main_res = run_workload(args.workload, args.path, args.steps, args.warmup, args.num_seeds)
    extra = {}
    if args.also and args.also != "none":
        for item in args.also.split(","):
            if not item:
                continue
            name, _, pth = item.partition(":")
            if name in PROJ_WORKLOADS:
                extra[item] = run_projection(name, max(3, args.steps // 2), max(1, args.warmup // 2))
                continue
            if name in MLA_WORKLOADS:
                extra[item] = run_sparse_mla(name, max(3, args.steps // 2), max(1, args.warmup // 2))
                continue
            extra[item] = run_workload(name, pth or args.path, max(3, args.steps // 2), max(1, args.warmup // 2),
                                       args.num_seeds)
    for wname in {args.workload} | {k.partition(":")[0] for k in extra}:
        runs = [r for r in [main_res, *extra.values()]
                if r["workload"] == wname and r["path"] not in ("project", "sparse_mla")]
        t = {r["path"]: r["ms_per_step"] for r in runs}
        if "unpruned" in t:
            for r in runs:
                if r["path"].startswith("pruned"):
                    r["pruned_over_unpruned_time"] = t[r["path"]] / t["unpruned"]
    peak = PEAK_TFLOPS[main_res["dtype"]]
    roofline = {
        "bound": "mfma",
        "achieved": main_res["achieved_tflops"],
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": main_res["achieved_tflops"] / peak,
        "traffic": measured_traffic(args.workload, main_res["dominant_kernel"]),
        "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE, copy-calibrated)",
        "kernel": main_res["dominant_kernel"],
        "launch_ms": main_res["dominant_ms"],
        "flops_per_launch": main_res["dominant_flops"],
    }
    sustained = {dt: sustained_rates(dt) for dt in ("bf16", "fp8")}
    st = sustained[main_res["dtype"]]
    roofline["sustained"] = {k: st[k] for k in ("mfma_only", "score_step", "unit")}
    roofline["frac_of_sustained_score_step"] = main_res["achieved_tflops"] / st["score_step"]
    for r in extra.values():  # other lines whose dominant kernel is the streaming Top-K
        if r.get("dominant_kernel") == "k_topk_stream" and r.get("dtype") in sustained:
            r["roofline"]["frac_of_sustained_score_step"] = (r["achieved_tflops"] /
                                                            sustained[r["dtype"]]["score_step"])
    for dt, r in sustained.items():
        log(f"[bench] sustained {dt}: MFMA only {r['mfma_only']:.0f} TFLOP/s "
            f"({100 * r['mfma_only'] / PEAK_TFLOPS[dt]:.1f}% of nominal), score step {r['score_step']:.0f} TFLOP/s "
            f"({100 * r['score_step'] / PEAK_TFLOPS[dt]:.1f}% of nominal)"
            + (f", |x| form {r['score_step_abs_form']:.0f} TFLOP/s "
               f"({100 * r['score_step_abs_form'] / PEAK_TFLOPS[dt]:.1f}%)" if "score_step_abs_form" in r else ""))
    cpu, cpu_more = None, {}
    if not args.no_cpu_baseline:
        log("[bench] timing the oracle on host cores ...")
        cpu = cpu_baseline(args.workload, args.cpu_rows, args.cpu_seconds)
        log(f"[bench] oracle: {cpu['value']:.3e} pairs/s on {cpu['cores']} threads ({cpu['sample'][:40]}...)")
        for name in (args.cpu_also.split(",") if args.cpu_also and args.cpu_also != "none" else []):
            cpu_more[name] = cpu_baseline(name, args.cpu_rows, args.cpu_seconds)
            log(f"[bench] oracle {name}: {cpu_more[name]['value']:.3e} pairs/s")
    wl = inputs.WORKLOADS[args.workload]
    line = {
        "metric": "indexer scored query-key pairs/s (+Top-K)",
        "value": main_res["pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": "synthetic",
        "config": {
            "workload": args.workload,
            "batch": wl.batch,
            "query_rows": wl.num_q,
            "keys": wl.num_k,
            "positions": f"{wl.pos_start}..{wl.pos_start + wl.num_q - 1}",
            "topk": wl.topk,
            "heads": 64,
            "head_dim": 128,
            "path": main_res["path"],
            "visible_pairs": main_res["visible_pairs"],
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
        "cpu_baselines_more": cpu_more,
        "sustained_mfma": sustained,
        "detail": main_res,
        "also": extra,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
