#!/usr/bin/env python3
"""Decode-step benchmark of the DSA hot path on one MI355X.

A step is one call of dsa_fused_decode: the fused Lightning Indexer (per-head
scores from the paged bf16 K cache, head-weighted sum, causal mask, Top-K) and
Sparse Flash Attention over the selected latent rows, for a batch of 32
sequences whose contexts are all 32768 tokens (one new token each), indexer 64
heads x 128, k = 2048, SFA 128 heads over 512 + 64 latent columns.  Inputs are
synthetic, seeded and resident in HBM; several value sets with the same layout
are rotated so that the ~354 MB step does not sit in the 256 MB last-level
cache between steps.

Prints one JSON line (see the fields below).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode tokens/s + µs/step (indexer+TopK+SFA) at 32k ctx; % HBM roofline"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "mxfp8": 5000.0, "f32": 157.3}

WORKLOADS = {
    "c2_decode_bf16": "decode, 32 sequences, contexts U[4096, 32768], bf16",
    "c2_decode_bf16_32k": "decode, 32 sequences, every context 32768, bf16",
    "c4_decode_fp8": "decode, 64 sequences, contexts U[16384, 65536], FP8 indexer",
    "c4_decode_mxfp8": "decode, 64 sequences, contexts U[16384, 65536], MXFP8 indexer",
    "c5_decode4": "4-token decode, 8 sequences at 131072 tokens, bf16",
    "c2_decode_fp8kv": "decode, 32 sequences, contexts U[4096, 32768], bf16, SFA KV cache FP8 "
                       "(one fp32 scale per 128-element tile)",
}


def _el(dtype):
    return {"f32": 4, "bf16": 2, "fp8": 1, "mxfp8": 1, "fp8_t128": 1}[dtype]


def algorithmic(case):
    """Bytes each step must move and flops it must do (per-head indexer)."""
    import numpy as np
    L = case.seq_lens_host.astype(np.int64)
    T = case.q_lens_host.astype(np.int64)
    ei, es = _el(case.idx_dtype), _el(case.sfa_dtype)
    keys = int(L.sum())
    k_scale = {"fp8": 4, "mxfp8": case.d_i // 32}.get(case.idx_dtype, 0)
    q_scale = {"fp8": 4, "mxfp8": case.d_i // 32}.get(case.idx_dtype, 0)
    tq = int(T.sum())
    idx_b = tq * case.topk * 4
    indexer_bytes = keys * (case.d_i * ei + k_scale) + tq * case.h_i * (case.d_i * ei + q_scale + 4) + idx_b
    rows = 0
    pairs = 0
    for b in range(case.batch):
        for i in range(int(T[b])):
            t = int(L[b] - T[b] + i)
            rows += min(case.topk, t + 1)
            pairs += t + 1
    # rows gathered once per sequence and step: the union over its queries is
    # bounded by the per-query count; for one query per sequence they coincide
    kv_scale = 4 * -(-case.d_qk // 128) if case.kv_dtype == "fp8_t128" else 0
    gather = rows * (case.d_qk * _el(case.kv_dtype) + kv_scale)
    sfa_bytes = gather + tq * case.h_s * (case.d_qk + case.d_v) * es + tq * case.h_s * 4 + idx_b
    indexer_flops = 2 * case.h_i * case.d_i * pairs
    sfa_flops = 2 * case.h_s * (case.d_qk + case.d_v) * rows
    return dict(indexer_bytes=indexer_bytes, sfa_bytes=sfa_bytes,
                fused_bytes=indexer_bytes + sfa_bytes - idx_b,
                indexer_flops=indexer_flops, sfa_flops=sfa_flops, keys=keys, rows=rows)


def time_calls(fn, steps, warmup, torch):
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s in range(steps):
        fn(s)
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms per call


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(case, budget_s):
    """The oracle as it stands, timed on this host on a bounded sample: the
    same seeded order of the workload's query tokens, with NumPy's BLAS on
    every core and on one thread, median of three runs each."""
    import numpy as np
    import oracle
    from oracle import dsa_oracle as od
    from threadpoolctl import threadpool_info, threadpool_limits
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    qs = [(b, i) for b in range(case.batch) for i in range(int(case.q_lens_host[b]))]
    # host copies of the pools are input staging, done before the clock starts
    for t in (case.k_pool, case.kv_pool, case.k_scale, case.block_table):
        if t is not None:
            od._np(t)
    order = np.random.default_rng(0).permutation(len(qs))
    per_run = budget_s / 6.0

    def one_run():
        done, t0 = 0, time.perf_counter()
        while True:
            oracle.run_query(case, *qs[order[done % len(qs)]])
            done += 1
            if time.perf_counter() - t0 > per_run:
                break
        return done, time.perf_counter() - t0

    runs = {}
    for label, limit in (("all", None), ("one", 1)):
        with threadpool_limits(limits=limit):
            runs[label] = [one_run() for _ in range(3)]
    rate = {k: float(np.median([d / e for d, e in v])) for k, v in runs.items()}
    n_all = sum(d for d, _ in runs["all"])
    return {"value": rate["all"], "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "one_thread_value": rate["one"],
            "cpu_model": _cpu_model(),
            "sample": f"seeded order over the {len(qs)} query tokens of the same workload (first seed), "
                      f"{per_run:.1f} s per run, median of 3 runs with BLAS on {threads} threads "
                      f"({n_all} tokens in all) and of 3 on 1 thread; float64 NumPy; "
                      f"host cores available {len(os.sched_getaffinity(0))}"}


PREFILL_WORKLOADS = {
    "c3_prefill_bf16": "one sequence, 32768 query tokens, causal, bf16, k=2048",
    "c3_prefill_fp8": "one sequence, 32768 query tokens, causal, FP8 indexer (1 % outliers), bf16 SFA, k=2048",
    "c3_prefill_mxfp8": "one sequence, 32768 query tokens, causal, MXFP8 indexer (1 % outliers), bf16 SFA, k=2048",
}


def prefill_line(torch, B, make_case, steps, name="c3_prefill_bf16"):
    """The 32768-token causal prefill: fused call time and MFMA fractions.  The
    indexer's flops are priced at its own dtype's peak (e4m3 for the quantised
    indexers), the SFA's at bf16; the fused fraction is the time both would
    take at their peaks over the measured time."""
    import numpy as np
    case = make_case(name, 3, device="cuda")
    call = B.Call(case)
    for op in (B.DSA_OP_FUSED_PREFILL, B.DSA_OP_INDEXER_TOPK, B.DSA_OP_SPARSE_ATTN):
        call.workspace(op)
    ms = time_calls(lambda s: call.fused_prefill(), steps, 1, torch)
    idx = call.indexer_topk().clone()
    ms_idx = time_calls(lambda s: call.indexer_topk(), steps, 1, torch)
    ms_sfa = time_calls(lambda s: call.sparse_attn(idx), steps, 1, torch)
    T = case.total_q
    t = np.arange(T, dtype=np.int64)
    rows = int(np.minimum(case.topk, t + 1).sum())
    pairs = int(((t + 1) * (t + 1 > case.topk)).sum())   # queries that need scores
    f_idx = 2 * case.h_i * case.d_i * pairs
    # with no activation on the per-head scores the head sum collapses into one
    # weighted query per token (sum_h w_h q_h, then one dot product per key):
    # the flops a collapsed indexer would need, printed so that the per-head
    # count is never read as required work
    f_idx_collapsed = 2 * case.d_i * pairs + 2 * case.h_i * case.d_i * int((t + 1 > case.topk).sum())
    f_sfa = 2 * case.h_s * (case.d_qk + case.d_v) * rows
    peak_i = MFMA_PEAK_TFLOPS["fp8" if case.idx_dtype in ("fp8", "mxfp8") else "bf16"] * 1e12
    peak_s = MFMA_PEAK_TFLOPS["bf16"] * 1e12
    out = {"workload": f"{name}: {PREFILL_WORKLOADS[name]}",
           "ms_per_call": ms, "tokens_per_s": T / (ms * 1e-3),
           "stages_ms": {"indexer_topk": ms_idx, "sparse_attn": ms_sfa},
           "algorithmic_flops": {"indexer_per_head": f_idx, "indexer_collapsed": f_idx_collapsed, "sfa": f_sfa},
           "mfma_frac": {"fused": (f_idx / peak_i + f_sfa / peak_s) / (ms * 1e-3),
                         "indexer": f_idx / (ms_idx * 1e-3) / peak_i, "sfa": f_sfa / (ms_sfa * 1e-3) / peak_s},
           "peak_tflops": {"indexer": peak_i / 1e12, "sfa": peak_s / 1e12}}
    del call, case
    torch.cuda.empty_cache()
    return out


def prolog_line(torch, B, make_case, steps, warmup):
    """The indexer prolog for the quantised decode workload's 64 new tokens
    (hidden rows of 7168, FP8 q and keys): projections, LayerNorm, dynamic
    quantisation and the key append, against the HBM roof (the weights dominate
    its bytes)."""
    from sparse_attention_04_amd.inputs import make_prolog
    case = make_case("c4_decode_fp8", 4, device="cuda")
    pros = [make_prolog(case, 80 + r, d_model=7168) for r in range(2)]
    call = B.Call(case)
    call.prolog(pros[0])
    ms = time_calls(lambda s: call.prolog(pros[s % 2]), steps, warmup, torch)
    T, H, D, dm = case.total_q, case.h_i, case.d_i, pros[0]["d_model"]
    wbytes = (H * D + D + H) * dm * 2
    nbytes = wbytes + T * dm * 2 + T * H * (D + 4 + 4) + T * (D + 4)
    out = {"workload": "c4 prolog: 64 new tokens, hidden 7168 -> q 64x128, k 128 (LayerNorm), w 64; FP8 q and keys, "
                       "keys appended to the paged cache", "ms_per_call": ms,
           "tokens_per_s": T / (ms * 1e-3), "algorithmic_bytes": nbytes,
           "hbm_frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    del call, case, pros
    torch.cuda.empty_cache()
    return out


def config_line(torch, B, make_case, name, steps, warmup, sets):
    """One more workload of the scope table: fused-call time and its rate
    against the roof that bounds it (HBM for decode, MFMA for prefill)."""
    seed = 5 if name.startswith("c5") else 2 if name.startswith("c2") else 4
    cases = [make_case(name, seed, device="cuda", value_seed=r + 1) for r in range(sets)]
    calls = [B.Call(c) for c in cases]
    prefill = cases[0].max_q_len > 4
    op = B.DSA_OP_FUSED_PREFILL if prefill else B.DSA_OP_FUSED_DECODE
    for c in calls:
        c.workspace(op)
    R = len(calls)
    fn = (lambda s: calls[s % R].fused_prefill()) if prefill else (lambda s: calls[s % R].fused_decode())
    ms = time_calls(fn, steps, warmup, torch)
    a = algorithmic(cases[0])
    out = {"workload": f"{name}: {CONFIGS_EXTRA[name]}", "ms_per_call": ms,
           "tokens_per_s": cases[0].total_q / (ms * 1e-3), "value_sets_rotated": R}
    if prefill:
        peak = MFMA_PEAK_TFLOPS["bf16"] * 1e12
        out["mfma_frac"] = (a["indexer_flops"] + a["sfa_flops"]) / (ms * 1e-3) / peak
    else:
        out["algorithmic_bytes"] = a["fused_bytes"]
        out["step_hbm_frac"] = a["fused_bytes"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS
    del calls, cases
    torch.cuda.empty_cache()
    return out


CONFIGS_EXTRA = {
    "c2_decode_bf16": "decode, 32 sequences, contexts U[4096, 32768], bf16",
    "c4_decode_fp8": "decode, 64 sequences, contexts U[16384, 65536], FP8 indexer, 1 % outliers",
    "c4_decode_mxfp8": "decode, 64 sequences, contexts U[16384, 65536], MXFP8 indexer, 1 % outliers",
    "c5_chunk_prefill": "chunked prefill, 8 sequences, 8192 new tokens after 122880 cached",
    "c5_decode4": "4-token decode, 8 sequences at 131072 tokens",
    "c2_decode_fp8kv": "decode, 32 sequences, contexts U[4096, 32768], SFA KV cache FP8 "
                       "(one fp32 scale per 128-element tile)",
}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2_decode_bf16_32k", choices=sorted(WORKLOADS))
    ap.add_argument("--sets", type=int, default=4, help="value sets rotated between steps")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--no-prefill", dest="prefill", action="store_false",
                    help="skip the 32k causal prefill measurement")
    ap.add_argument("--no-extra", dest="extra", action="store_false",
                    help="skip the C4 and C5 measurements")
    ap.add_argument("--only-config", default=None, choices=sorted(CONFIGS_EXTRA),
                    help="print only this workload's fused-call measurement (--steps calls)")
    ap.add_argument("--only-prolog", action="store_true",
                    help="print only the indexer prolog measurement")
    ap.add_argument("--only-prefill", action="store_true",
                    help="print only the 32k causal prefill measurement (--steps calls per stage)")
    ap.add_argument("--prefill-workload", default="c3_prefill_bf16", choices=sorted(PREFILL_WORKLOADS),
                    help="the prefill workload of --only-prefill")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 512 MiB device copy (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_04_amd import binding as B
    from sparse_attention_04_amd.inputs import make_case

    assert torch.cuda.is_available(), "bench.py needs the GPU"
    B.lib()
    if args.only_config:
        print(json.dumps(config_line(torch, B, make_case, args.only_config, args.steps, args.warmup,
                                     1 if args.only_config == "c5_chunk_prefill" else 2)), flush=True)
        return
    if args.only_prolog:
        print(json.dumps(prolog_line(torch, B, make_case, args.steps, args.warmup)), flush=True)
        return
    if args.only_prefill:
        print(json.dumps(prefill_line(torch, B, make_case, args.steps, args.prefill_workload)), flush=True)
        return
    seed = 2
    cases = [make_case(args.workload, seed, device="cuda", value_seed=seed + 100 * r) for r in range(args.sets)]
    calls = [B.Call(c) for c in cases]
    for c in calls:  # allocate every workspace before timing
        c.workspace(B.DSA_OP_FUSED_DECODE)
        c.workspace(B.DSA_OP_INDEXER_TOPK)
        c.workspace(B.DSA_OP_SPARSE_ATTN)
    case = cases[0]
    R = len(calls)

    ms_step = time_calls(lambda s: calls[s % R].fused_decode(), args.steps, args.warmup, torch)
    # per-stage times on the same stream (indexer incl. its workspace clear; SFA incl. combine)
    idx_sets = [c.indexer_topk().clone() for c in calls]
    ms_idx = time_calls(lambda s: calls[s % R].indexer_topk(), args.steps, args.warmup, torch)
    ms_sfa = time_calls(lambda s: calls[s % R].sparse_attn(idx_sets[s % R]), args.steps, args.warmup, torch)
    if args.calib_copy:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    a = algorithmic(case)
    tokens = case.total_q
    # The dominant kernel of the step.  dsa_fused_decode is the fused decode
    # kernel (indexer and attention in one launch) followed by the split
    # combine, so back-to-back calls timed with events on the stream they run
    # on give the pair's average duration (with the gaps); its algorithmic
    # bytes are the step's.  The separate stages (dsa_indexer_topk: one
    # launch of the decode indexer kernel; dsa_sparse_attn: attention and
    # combine) are timed the same way and reported beside it.
    fused = os.environ.get("DSA_FUSED_KERNEL", "1") != "0"
    step_kernels = ("fused_decode_kernel+sfa_combine_kernel" if fused else
                    "indexer_decode_kernel+sfa_bf16_kernel+sfa_combine_kernel")
    kern = {step_kernels: (ms_step, a["fused_bytes"]),
            "indexer_decode_kernel": (ms_idx, a["indexer_bytes"]),
            "sfa_bf16_kernel+sfa_combine_kernel": (ms_sfa, a["sfa_bytes"])}
    dom = max(kern, key=lambda k: kern[k][0])
    dms, dbytes = kern[dom]
    achieved = dbytes / (dms * 1e-3) / 1e9
    prof = os.path.join(ROOT, "profiles", "traffic.json")
    traffic = None
    if os.path.exists(prof):
        try:
            tr = json.load(open(prof))
            ent = tr.get(args.workload, {}).get(dom)
            if ent and ent.get("kernel_source_sha") == _kernel_sha():
                traffic = ent["bytes_per_launch"]
        except Exception:
            traffic = None
    line = {
        "metric": METRIC,
        "value": tokens / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "us_per_step": ms_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.idx_dtype if case.idx_dtype != "f32" else "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{args.workload}: {WORKLOADS[args.workload]}",
            "batch": case.batch, "query_tokens": tokens, "total_context_tokens": a["keys"],
            "indexer": f"{case.h_i} heads x {case.d_i}, {case.idx_dtype}, k={case.topk}",
            "sfa": f"{case.h_s} heads, latent {case.d_v} + rope {case.d_qk - case.d_v}, {case.sfa_dtype}",
            "page_size": case.page_size, "value_sets_rotated": R,
        },
        "stages_ms": {"fused_step": ms_step, "indexer_topk": ms_idx, "sparse_attn": ms_sfa},
        "step_kernels": step_kernels,
        "algorithmic": {"fused_step_bytes": a["fused_bytes"], "indexer_bytes": a["indexer_bytes"],
                        "sfa_bytes": a["sfa_bytes"], "indexer_flops_per_head": a["indexer_flops"],
                        "sfa_flops": a["sfa_flops"]},
        "step_hbm_frac": a["fused_bytes"] / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dbytes, "us_per_launch": dms * 1e3},
        "mfma_frac": {
            "indexer": a["indexer_flops"] / (ms_idx * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[case.idx_dtype],
            "sfa": a["sfa_flops"] / (ms_sfa * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS[case.sfa_dtype],
        },
    }
    headline = args.workload == "c2_decode_bf16_32k"
    if headline and args.prefill:
        line["prefill_32k"] = prefill_line(torch, B, make_case, 3)
        if args.extra:
            line["prefill_32k_quantised_indexer"] = {
                n: prefill_line(torch, B, make_case, 3, n) for n in ("c3_prefill_fp8", "c3_prefill_mxfp8")}
    if headline and args.extra:
        line["prolog"] = prolog_line(torch, B, make_case, 50, 5)
    if headline and args.extra:
        line["other_configs"] = {
            n: config_line(torch, B, make_case, n, *((3, 1, 1) if n == "c5_chunk_prefill" else (50, 5, 2)))
            for n in CONFIGS_EXTRA}
    if args.cpu_budget > 0:
        line["cpu_baseline"] = cpu_baseline(case, args.cpu_budget)
    print(json.dumps(line), flush=True)


def _kernel_sha():
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_attention_04_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


if __name__ == "__main__":
    main()
