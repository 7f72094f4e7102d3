"""Benchmark of the index-selection sparse attention layer on one MI355X.

A step is one call of li_topk_sfa (indexer scores -> Top-K -> sparse MLA
attention) over one batch of synthetic decode queries: by default 64
sequences at context 32768, paged 64-token blocks, 64x128 bf16 indexer,
K = 2048, 128-head 512+64 bf16 MLA.  Inputs are generated on the GPU before
timing and stay resident in HBM.

Prints ONE JSON line with the layer throughput (query rows per second), the
roofline of the dominant kernel (timed live with HIP events on its stream),
per-stage timings, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn layer tokens/s (indexer+TopK+SFA) at L=32K; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl, b):
    """Algorithmic bytes / flops per launch of each stage (what the method must
    move or compute; the dense attention it avoids is not counted).  Cached
    keys and latent rows count once per sequence: rows of one sequence share
    them (prefill), and the union of a sequence's selected rows is bounded by
    both the selections and the visible context."""
    R = b.R
    pos = [int(p) for p in b.row_pos.tolist()]
    seq = [int(s) for s in b.row_seq.tolist()]
    ke = 1 if wl.indexer_dtype in ("fp8", "mxfp8") else 2
    ks = {"fp8": 4, "mxfp8": wl.D_I // 32}.get(wl.indexer_dtype, 0)   # scale bytes per key (or query head)
    ve = 1 if wl.kv_dtype in ("fp8", "fp8_tile128") else 2
    vs = {"fp8": 4, "fp8_tile128": 4 * ((wl.D_qk + 127) // 128)}.get(wl.kv_dtype, 0)   # scale bytes per row
    vis = sum(p + 1 for p in pos)
    sel = sum(min(wl.K, p + 1) for p in pos)
    seq_vis, seq_sel = {}, {}
    for s, p in zip(seq, pos):
        seq_vis[s] = max(seq_vis.get(s, 0), p + 1)
        seq_sel[s] = seq_sel.get(s, 0) + min(wl.K, p + 1)
    keys = sum(seq_vis.values())
    rows = sum(min(seq_sel[s], seq_vis[s]) for s in seq_vis)
    qs = wl.H_I * ks if wl.indexer_dtype == "mxfp8" else ks
    li_bytes = keys * (wl.D_I * ke + ks) + R * (wl.H_I * (wl.D_I * ke + 4) + qs)
    li_flops = 2.0 * wl.H_I * wl.D_I * vis
    sfa_bytes = rows * (wl.D_qk * ve + vs) + R * wl.H * (wl.D_qk * 2 + wl.D_v * 2 + 4) + sel * 4
    sfa_flops = 2.0 * wl.H * sel * (wl.D_qk + wl.D_v)
    topk_bytes = vis * 4 + R * wl.K * 4
    lt_bytes = li_bytes + R * wl.K * 4    # fused: keys and queries in, index lists out, no scores
    return dict(li=(li_bytes, li_flops), topk=(topk_bytes, 0.0), sfa=(sfa_bytes, sfa_flops),
                lt=(lt_bytes, li_flops))


KERNEL_SOURCES = {
    "li_score": ["li_score.hip", "li_dec.hpp", "common.hpp"],
    "li_topk": ["li_topk.hip", "li_dec.hpp", "common.hpp"],
    "topk_select": ["topk.hip", "common.hpp"],
    "sparse_mla_attn": ["sparse_mla.hip", "common.hpp"],
}


def source_hash(stage: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[stage]:
        with open(os.path.join(ROOT, "indexer_selected_sparse_li_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_path(stage: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"{stage}_{workload}_traffic.md")


def stored_traffic(stage: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = traffic_path(stage, workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    try:
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        d = json.loads(blob)
    except Exception:
        return None
    if d.get("source_hash") != source_hash(stage):
        return None
    return d.get("hbm_bytes_per_launch")


# kernels one call of each stage launches (name substrings)
STAGE_KERNELS = {
    "li_score": ["li_score"],
    "topk_select": ["topk"],
    "li_topk": ["li_topk_kernel", "lt_clear_kernel"],
    "sparse_mla_attn": ["sfa_mla_kernel", "sfa_kernel<", "sfa_combine_kernel"],
}


def pmc_per_dispatch(csv_path: str, counter: str, kernel_substrs):
    """Sum over the stage's kernels of the median per-dispatch counter value."""
    import csv
    per = {}
    with open(csv_path) as fh:
        for row in csv.DictReader(fh):
            if row["Counter_Name"] != counter:
                continue
            for k in kernel_substrs:
                if k in row["Kernel_Name"]:
                    per.setdefault(k, []).append(float(row["Counter_Value"]))
                    break
    if not per:
        raise SystemExit(f"no {counter} rows for {kernel_substrs} in {csv_path}")
    total, n = 0.0, 0
    for vals in per.values():
        vals.sort()
        total += vals[len(vals) // 2]
        n = max(n, len(vals))
    return total, n, sorted(per)


def write_traffic_summary(args):
    """Turn four rocprofv3 --pmc CSVs (kernel FETCH_SIZE / WRITE_SIZE, copy
    FETCH_SIZE / WRITE_SIZE) into a profiles/ summary with the scaled bytes."""
    stage, wl_name = args.stage, args.workload
    copy_bytes = args.copy_bytes
    kf, nkf, knames = pmc_per_dispatch(args.fetch_csv, "FETCH_SIZE", STAGE_KERNELS[stage])
    kw, nkw, _ = pmc_per_dispatch(args.write_csv, "WRITE_SIZE", STAGE_KERNELS[stage])
    cf, _, _ = pmc_per_dispatch(args.copy_fetch_csv, "FETCH_SIZE", [""])
    cw, _, _ = pmc_per_dispatch(args.copy_write_csv, "WRITE_SIZE", [""])
    kname = " + ".join(k.rstrip("<") for k in knames)
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch = kf * 1024.0 * f_scale
    write = kw * 1024.0 * w_scale
    d = dict(stage=stage, workload=wl_name, source_hash=source_hash(stage),
             fetch_kib_raw=kf, write_kib_raw=kw, copy_fetch_kib_raw=cf, copy_write_kib_raw=cw,
             copy_bytes=copy_bytes, fetch_scale=round(f_scale, 4), write_scale=round(w_scale, 4),
             hbm_bytes_per_launch=int(fetch + write), fetch_bytes=int(fetch), write_bytes=int(write))
    path = traffic_path(stage, wl_name)
    with open(path, "w") as fh:
        fh.write(f"# HBM traffic of {stage} ({kname}) on {wl_name}\n\n")
        fh.write("Median per dispatch over the profiled launches (summed over the kernels one call\n"
                 "of the stage launches), rocprofv3 --pmc counters in KiB.\n")
        fh.write("Each counter is scaled by what it reads for a plain device copy of known size\n")
        fh.write(f"(torch copy of {copy_bytes} bytes: expected = copy_bytes / 1024 KiB).\n\n")
        fh.write("Commands (run from the repository root on the GPU box):\n\n")
        for c in args.commands or []:
            fh.write(f"    {c}\n")
        fh.write("\n```json\n" + json.dumps(d, indent=1) + "\n```\n")
    print(f"wrote {path}: {d['hbm_bytes_per_launch'] / 1e6:.1f} MB per launch "
          f"(fetch scale {f_scale:.3f}, write scale {w_scale:.3f})")


def write_mfma_summary(args):
    """Turn one rocprofv3 --pmc CSV (SQ_INSTS_VALU_MFMA_MOPS_BF16, _F8, and the
    derived MfmaUtil) into a profiles/ summary of MFMA work and utilisation."""
    import csv
    stage, wl_name = args.stage, args.workload
    per = {}
    with open(args.mfma_csv) as fh:
        for row in csv.DictReader(fh):
            for k in STAGE_KERNELS[stage]:
                if k in row["Kernel_Name"]:
                    d = per.setdefault(k, {})
                    d.setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
                    dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-3
                    d.setdefault("_us", []).append(dur)
                    break
    if not per:
        raise SystemExit(f"no rows for {STAGE_KERNELS[stage]} in {args.mfma_csv}")

    def med(v):
        v = sorted(v)
        return v[len(v) // 2]

    rows = []
    for k, d in sorted(per.items()):
        us = med(d["_us"])
        bf = med(d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0.0])) * 512
        f8 = med(d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", [0.0])) * 512
        util = med(d["MfmaUtil"]) if "MfmaUtil" in d else None
        tf = (bf + f8) / (us * 1e-6) / 1e12 if us > 0 else 0.0
        pk = (bf / BF16_PEAK_TFLOPS + f8 / FP8_PEAK_TFLOPS) / max(bf + f8, 1.0)   # 1/TFLOP-weighted peak
        frac = tf * pk if bf + f8 > 0 else 0.0
        rows.append(dict(kernel=k.rstrip("<"), dispatch_us=round(us, 2), mfma_bf16_flop=int(bf),
                         mfma_fp8_flop=int(f8), achieved_tflops=round(tf, 2), frac_of_peak=round(frac, 4),
                         mfma_busy_pct=None if util is None else round(util, 2)))
    path = os.path.join(ROOT, "profiles", f"{stage}_{wl_name}_mfma.md")
    with open(path, "w") as fh:
        fh.write(f"# MFMA work and utilisation of {stage} on {wl_name}\n\n")
        fh.write("Median per dispatch, rocprofv3 --pmc. Flops = SQ_INSTS_VALU_MFMA_MOPS_* x 512 (rocprofv3's\n"
                 "MfmaFlops definition); dispatch time from the same run's timestamps (counter collection\n"
                 "serialises dispatches, so it runs slightly long); peak 2.5 PFLOP/s bf16, 5.0 fp8 dense.\n"
                 "mfma_busy_pct is rocprofv3's derived MfmaUtil (MFMA-busy cycles over active cycles x SIMDs).\n\n")
        fh.write("Command (run from the repository root on the GPU box):\n\n")
        for c in args.commands or []:
            fh.write(f"    {c}\n")
        fh.write("\n| kernel | us | bf16 MFMA GFLOP | fp8 MFMA GFLOP | TFLOP/s | % of MFMA peak | MFMA busy % |\n")
        fh.write("|---|---|---|---|---|---|---|\n")
        for r in rows:
            fh.write(f'| {r["kernel"]} | {r["dispatch_us"]} | {r["mfma_bf16_flop"] / 1e9:.2f} | '
                     f'{r["mfma_fp8_flop"] / 1e9:.2f} | {r["achieved_tflops"]} | {r["frac_of_peak"] * 100:.1f} | '
                     f'{r["mfma_busy_pct"]} |\n')
        fh.write("\n```json\n" + json.dumps(dict(stage=stage, workload=wl_name, source_hash=source_hash(stage),
                                                  kernels=rows), indent=1) + "\n```\n")
    print(f"wrote {path}")


def kernel_short_name(n: str) -> str:
    """lisfa::kernel<args> from a demangled name, or from a mangled one that the
    profiler left as is (template arguments: integer, bool, float, __bf16)."""
    if not n.startswith("_ZN5lisfa"):
        return n.split("(")[0].replace("void ", "")
    import re
    m = re.match(r"_ZN5lisfa(\d+)", n)
    k = m.end() + int(m.group(1))
    base, rest, args = n[m.end():k], n[k:], []
    if rest.startswith("I"):
        i = 1
        while i < len(rest) and rest[i] != "E":
            t = re.match(r"L[ib](-?\d+)E|DF16b|f|i", rest[i:])
            if t is None:
                break
            tok = t.group(0)
            args.append(t.group(1) if t.group(1) is not None else {"DF16b": "__bf16", "f": "float", "i": "int"}[tok])
            i += len(tok)
    return f"lisfa::{base}<{', '.join(args)}>" if args else f"lisfa::{base}"


def write_kernel_stats(args):
    """Turn a rocprofv3 --kernel-trace --stats kernel_stats.csv (and, with
    --bench-json, the line of a plain bench.py run in the same GPU session)
    into profiles/layer_<workload>_kernel_stats.md."""
    import csv
    rows = []
    with open(args.stats_csv) as fh:
        for r in csv.DictReader(fh):
            if "lisfa" not in r["Name"]:
                continue
            name = kernel_short_name(r["Name"])
            rows.append((name, int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    rows.sort(key=lambda x: -x[2] * x[1])
    path = os.path.join(ROOT, "profiles", f"layer_{args.workload}_kernel_stats.md")
    with open(path, "w") as fh:
        fh.write(f"# Kernel trace: the layer on {args.workload}\n\n")
        fh.write("Commands (repository root, GPU box):\n\n")
        for c in args.commands or []:
            fh.write(f"    {c}\n")
        fh.write("\nThe profiled bench.py run makes warmup + steps fused layer calls, then steps cold layer "
                 "calls (each after an\nL2 / MALL flush), then warmup + steps calls of each stage alone (the "
                 "stage timing): 2 + 10 + 10 + 2 + 10 = 34\ncalls of every kernel.\n\n")
        fh.write("| kernel | calls | average us | min us | max us |\n|---|---|---|---|---|\n")
        for r in rows:
            fh.write(f"| `{r[0]}` | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} |\n")
        if args.bench_json:
            d = json.loads(open(args.bench_json).read().strip().splitlines()[-1])
            fh.write("\nThe plain bench.py run of the same GPU session (no profiler attached), its own HIP-event "
                     "timing of each stage:\n\n")
            fh.write("| stage | us | algorithmic bytes | roofline fraction |\n|---|---|---|---|\n")
            for k, v in d["stages"].items():
                rf = v["roofline"]
                fh.write(f"| {k} | {v['us']} | {v['algorithmic_bytes']} | {rf['frac']} ({rf['bound']}) |\n")
            fh.write(f"\nLayer: {d['ms_per_step'] * 1e3:.1f} us per step cold ({d['value']:.0f} query rows/s), "
                     f"{d['ms_per_step_hot'] * 1e3:.1f} us hot.  Line roofline: {d['roofline']['kernel']} "
                     f"{d['roofline']['achieved']} GB/s = {d['roofline']['frac']} of peak, traffic "
                     f"{d['roofline']['traffic']} B per launch.\n")
    print(f"wrote {path}")


def time_on_stream(fn, stream, warmup, steps, graph=False):
    """Seconds per call of fn(stream).  With graph=True the calls are captured
    into one HIP graph first, so the time excludes the host's per-call cost."""
    import torch
    for _ in range(warmup):
        fn(stream)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            st = torch.cuda.current_stream()
            for _ in range(steps):
                fn(st)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
            start.record(stream)
            g.replay()
            end.record(stream)
        torch.cuda.synchronize()
        del g
    else:
        start.record(stream)
        for _ in range(steps):
            fn(stream)
        end.record(stream)
        torch.cuda.synchronize()
    return start.elapsed_time(end) / steps * 1e-3  # seconds per call


def cpu_baseline(b, budget_s: float):
    """The oracle, as is, on the first rows of the same batch until about
    budget_s seconds of CPU work; tokens/s = rows / oracle seconds."""
    import numpy as np
    import oracle as O
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = os.cpu_count() or 1
    inp = W.to_numpy(b)
    rows, t_used = 0, 0.0
    while t_used < budget_s and rows < 64 * b.R:
        t0 = time.perf_counter()
        O.layer_row(inp, rows % b.R)
        t_used += time.perf_counter() - t0
        rows += 1
    return dict(value=rows / t_used, unit="tokens/s", cores=int(cores), kind="oracle",
                sample=f"{rows} query-row evaluations cycling over the {b.R} rows of the same batch "
                       f"(scores over the full context, selection, attention; float64 NumPy, "
                       f"{t_used:.1f} s of oracle time)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_paged_64x32768")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-each", type=float, default=4.0,
                    help="with --report-all: seconds of oracle time per workload")
    ap.add_argument("--stage-steps", type=int, default=None)
    ap.add_argument("--only", choices=["li_score", "topk_select", "li_topk", "sparse_mla_attn", "layer"],
                    help="profiling mode: run just this stage (no JSON line)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="profiling mode: run a plain device copy of --copy-bytes bytes")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--write-traffic-summary", action="store_true")
    ap.add_argument("--stage", default="li_score")
    ap.add_argument("--fetch-csv")
    ap.add_argument("--write-csv")
    ap.add_argument("--copy-fetch-csv")
    ap.add_argument("--copy-write-csv")
    ap.add_argument("--commands", nargs="*")
    ap.add_argument("--report-all", action="store_true",
                    help="time every workload (hot and cold), one JSON line each")
    ap.add_argument("--write-mfma-summary", action="store_true")
    ap.add_argument("--write-kernel-stats", action="store_true")
    ap.add_argument("--stats-csv")
    ap.add_argument("--bench-json")
    ap.add_argument("--mfma-csv")
    ap.add_argument("--report-cp", action="store_true",
                    help="time one GPU's context-parallel share and the Zigzag prefill balance")
    ap.add_argument("--report-prolog", action="store_true", help="time the indexer prolog kernels")
    ap.add_argument("--report-cold", action="store_true",
                    help="time the layer's stages hot and cold (after an L2 / MALL eviction)")
    ap.add_argument("--report-md", help="with --report-all / --report-cp: write a markdown table here")
    args = ap.parse_args()
    if args.write_traffic_summary:
        write_traffic_summary(args)
        return
    if args.write_mfma_summary:
        write_mfma_summary(args)
        return
    if args.write_kernel_stats:
        write_kernel_stats(args)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer's multi-GPU sharding is a design, not part of this build)", file=sys.stderr)
        sys.exit(2)

    import torch
    import indexer_selected_sparse_li_amd as lisfa
    import workloads as W

    lisfa.load()
    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.empty(args.copy_bytes, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_bytes} bytes x {args.steps}")
        return
    if args.report_all:
        report_all(args)
        return
    if args.report_cp:
        report_cp(args)
        return
    if args.report_prolog:
        report_prolog(args)
        return
    if args.report_cold:
        report_cold(args)
        return
    wl = W.get(args.workload)
    res, b = run_workload(args, wl, cold=not args.only)
    if res is None:
        return
    if not args.no_cpu_baseline:
        log("[bench] cpu oracle baseline")
        res["cpu_baseline"] = cpu_baseline(b, args.cpu_budget)
    print(json.dumps(res), flush=True)


def run_workload(args, wl, cold=False, graph=False):
    """Generate one workload on the GPU and time the layer and its stages.
    Returns (result dict, batch); (None, batch) in the profiling modes."""
    import torch
    import indexer_selected_sparse_li_amd as lisfa
    import workloads as W

    log(f"[bench] generating {wl.name} on the GPU")
    b = W.make_batch(wl, device="cuda")
    torch.cuda.synchronize()
    R = b.R
    kc = lisfa.KVCache(data=b.k_data, scale=b.k_scale, scale_group=1, block_table=b.block_table,
                       block_size=wl.block_size, seq_base=b.seq_base)
    vc = lisfa.KVCache(data=b.kv_data, scale=b.kv_scale, scale_group=wl.kv_scale_group,
                       block_table=b.block_table, block_size=wl.block_size, seq_base=b.seq_base)
    rpg = (16 if R % 16 == 0 else 8 if R % 8 == 0 else 1) if wl.mode == "prefill" else 1
    out = torch.empty(R, wl.H, wl.D_v, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(R, wl.H, dtype=torch.float32, device="cuda")
    idx = torch.empty(R, wl.K, dtype=torch.int32, device="cuda")
    ws = torch.empty(lisfa.workspace_size(2, R, b.max_visible, wl.K, wl.H, wl.D_v), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()

    def step_on(st):
        lisfa.li_topk_sfa(b.q_idx, b.w, kc, b.q, vc, b.row_seq, b.row_pos, wl.K, b.max_visible, out, lse,
                          idx_out=idx, q_scale=b.q_scale, rows_per_group=rpg,
                          softmax_scale=wl.softmax_scale, workspace=ws, stream=st)

    def step():
        step_on(stream)

    if args.only:
        ld_o = (b.max_visible + 63) // 64 * 64
        scores_o = torch.empty(R, ld_o, dtype=torch.float32, device="cuda")
        sfa_ws_o = torch.empty(max(1, lisfa.workspace_size(1, R, 0, wl.K, wl.H, wl.D_v)), dtype=torch.uint8,
                               device="cuda")
        fns = {
            "layer": step,
            "li_score": lambda: lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, scores_o, b.max_visible,
                                               q_scale=b.q_scale, rows_per_group=rpg, stream=stream),
            "topk_select": lambda: lisfa.topk_select(scores_o, b.row_pos, wl.K, idx, stream=stream),
            "li_topk": lambda: lisfa.li_topk(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, idx, b.max_visible,
                                             q_scale=b.q_scale, rows_per_group=rpg, workspace=ws, stream=stream),
            "sparse_mla_attn": lambda: lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx, out, lse,
                                                             softmax_scale=wl.softmax_scale, workspace=sfa_ws_o,
                                                             stream=stream),
        }
        if args.only in ("topk_select", "sparse_mla_attn"):
            fns["li_score"]()
            fns["topk_select"]()
        for _ in range(args.warmup + args.steps):
            fns[args.only]()
        torch.cuda.synchronize()
        log(f"[bench] ran {args.only} x {args.warmup + args.steps}")
        return None, b

    # the whole layer, timed: barrier + synchronize on both sides
    log(f"[bench] warmup {args.warmup}, timed {args.steps}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps
    value = R / (ms_step * 1e-3)
    log(f"[bench] layer {ms_step * 1e3:.1f} us/step (wall {wall / args.steps * 1e6:.1f} us)")

    ms_cold = None
    if cold:
        # each step after a 512 MiB write, which evicts the L2s and the 256 MB MALL
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        for i, (e0, e1) in enumerate(evs):
            flush.fill_(i & 255)
            e0.record(stream)
            step()
            e1.record(stream)
        torch.cuda.synchronize()
        ms_cold = sum(e0.elapsed_time(e1) for e0, e1 in evs) / args.steps
        del flush
        log(f"[bench] layer cold {ms_cold * 1e3:.1f} us/step")

    ms_graph = None
    if graph:
        ms_graph = graph_replay_ms(step_on, (idx, out, lse), stream, args.steps)
        log(f"[bench] layer graph replay {ms_graph * 1e3:.1f} us/step")

    # stages on their own, same stream, same inputs
    ss = args.stage_steps or args.steps
    ld = (b.max_visible + 63) // 64 * 64
    scores = torch.empty(R, ld, dtype=torch.float32, device="cuda")
    sfa_ws = torch.empty(max(1, lisfa.workspace_size(1, R, 0, wl.K, wl.H, wl.D_v)), dtype=torch.uint8,
                         device="cuda")
    t_li = time_on_stream(lambda st: lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, scores,
                                                    b.max_visible, q_scale=b.q_scale, rows_per_group=rpg,
                                                    stream=st), stream, 2, ss, graph)
    t_tk = time_on_stream(lambda st: lisfa.topk_select(scores, b.row_pos, wl.K, idx, stream=st),
                          stream, 2, ss, graph)
    # the index step as the layer runs it: one fused launch when li_topk_plan says so
    lt_wg = lisfa.li_topk_plan(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, b.max_visible, q_scale=b.q_scale,
                               rows_per_group=rpg, layer=True)
    t_lt = time_on_stream(lambda st: lisfa.li_topk(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, idx,
                                                   b.max_visible, q_scale=b.q_scale, rows_per_group=rpg,
                                                   workspace=ws, stream=st), stream, 2, ss, graph)
    t_sfa = time_on_stream(lambda st: lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx, out, lse,
                                                            softmax_scale=wl.softmax_scale, workspace=sfa_ws,
                                                            stream=st), stream, 2, ss, graph)
    alg = algorithmic(wl, b)

    def peak_tflops(name):
        # the indexer's contraction runs on fp8 MFMA for fp8 keys; sparse MLA always on bf16 MFMA
        fp8 = name in ("li", "lt") and wl.indexer_dtype in ("fp8", "mxfp8")
        return FP8_PEAK_TFLOPS if fp8 else BF16_PEAK_TFLOPS

    def roof(name, t, bound):
        by, fl = alg[name]
        if bound == "hbm":
            ach = by / t / 1e9
            return dict(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                        frac=round(ach / HBM_PEAK_GBS, 4))
        ach = fl / t / 1e12
        pk = peak_tflops(name)
        return dict(bound="mfma", achieved=round(ach, 2), peak=pk, unit="TFLOP/s", frac=round(ach / pk, 4))

    def bound_of(name):
        by, fl = alg[name]
        if name == "topk" or fl == 0:
            return "hbm"
        return "mfma" if fl / max(by, 1) > peak_tflops(name) * 1e12 / (HBM_PEAK_GBS * 1e9) else "hbm"

    fused = lt_wg > 0
    in_layer = {"li_score": not fused, "topk_select": not fused, "li_topk": fused, "sparse_mla_attn": True}
    stages = {}
    for name, t in (("li_score", t_li), ("topk_select", t_tk), ("li_topk", t_lt), ("sparse_mla_attn", t_sfa)):
        key = {"li_score": "li", "topk_select": "topk", "li_topk": "lt", "sparse_mla_attn": "sfa"}[name]
        r = roof(key, t, bound_of(key))
        stages[name] = dict(us=round(t * 1e6, 2), algorithmic_bytes=int(alg[key][0]),
                            algorithmic_flops=int(alg[key][1]), roofline=r, in_layer=in_layer[name])
    dominant = max((k for k in stages if stages[k]["in_layer"]), key=lambda k: stages[k]["us"])
    roofline = dict(stages[dominant]["roofline"])
    roofline["kernel"] = dominant
    roofline["traffic"] = stored_traffic(dominant, wl.name)

    # headline: cold steps (every step after a flush of the L2s and the MALL)
    # when measured, else back-to-back ("hot") steps
    ms_head = ms_cold if ms_cold is not None else ms_step
    res = {
        "metric": METRIC, "value": round(R / (ms_head * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_head, 4),
        "timing": "cold: each timed step follows a 512 MiB write that evicts the L2s and the MALL"
                  if ms_cold is not None else "hot: back-to-back steps",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": wl.kv_dtype,
        "data": "synthetic (seeded; inputs resident in HBM)",
        "config": {"workload": wl.name, "rows": R, "context": b.max_visible, "K": wl.K,
                   "indexer": f"{wl.H_I}x{wl.D_I} {wl.indexer_dtype}",
                   "mla": f"{wl.H} heads {wl.D_latent}+{wl.D_rope} {wl.kv_dtype}",
                   "cache": f"paged {wl.block_size}" if wl.paged else "contiguous",
                   "index_step": (f"li_topk fused, {lt_wg} workgroups per row, scores on chip" if fused
                                  else "li_score + topk_select, scores through the workspace"),
                   "parallelism": "single GPU"},
        "roofline": roofline,
        "stages": stages,
    }
    res["ms_per_step_hot"] = round(ms_step, 4)
    res["value_hot"] = round(value, 1)
    if ms_cold is not None:
        res["ms_per_step_cold"] = round(ms_cold, 4)
        res["value_cold"] = round(R / (ms_cold * 1e-3), 1)
    if ms_graph is not None:
        res["ms_per_step_graph"] = round(ms_graph, 4)
        res["value_graph"] = round(R / (ms_graph * 1e-3), 1)
    return res, b


def graph_replay_ms(step_on, outs, stream, steps):
    """Capture one layer call into a HIP graph and time its replays.  Every
    replay is checked bit for bit against the eager result first (the kernels
    are deterministic), with eager work and synchronizations in between."""
    import torch
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step_on(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step_on(torch.cuda.current_stream())
    torch.cuda.synchronize()
    for i in range(3):
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, ref):
            if not torch.equal(t.view(torch.uint8) if t.dtype == torch.bfloat16 else t,
                               r.view(torch.uint8) if r.dtype == torch.bfloat16 else r):
                raise SystemExit(f"graph replay {i} differs from the eager call")
        step_on(stream)
        torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        ev0.record(stream)
        for _ in range(steps):
            g.replay()
        ev1.record(stream)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    del g
    return ms


def report_all(args):
    """Every workload of the registry, one JSON line each (hot and cold layer
    timings, per-stage times and rooflines); optionally a markdown table."""
    import torch
    import workloads as W
    lines = []
    for name in REPORT_ORDER:
        wl = W.get(name)
        res, b = run_workload(args, wl, cold=True, graph=True)
        if not args.no_cpu_baseline:
            # the oracle on the same batch, in the same run (bounded sample)
            log(f"[bench] cpu oracle baseline for {wl.name}")
            res["cpu_baseline"] = cpu_baseline(b, args.cpu_budget_each)
            res["vs_cpu_oracle"] = res["value"] / res["cpu_baseline"]["value"]
        del b
        torch.cuda.empty_cache()
        lines.append(res)
        print(json.dumps(res), flush=True)
    if args.report_md:
        write_report_md(args.report_md, lines, args)


def _cp_caches(lisfa, b, shard):
    wl = b.wl
    kc = lisfa.KVCache(data=b.k_data, scale=b.k_scale, scale_group=1, block_table=shard["block_table"],
                       block_size=wl.block_size, seq_base=shard["seq_base"])
    vc = lisfa.KVCache(data=b.kv_data, scale=b.kv_scale, scale_group=wl.kv_scale_group,
                       block_table=shard["block_table"], block_size=wl.block_size, seq_base=shard["seq_base"])
    return kc, vc


def cp_share_timing(args, wl, G):
    """One GPU's share of a decode context split over G GPUs (rank 0's
    contiguous range of every sequence): local scores, local candidates, the
    merge of the G gathered candidate lists, partial attention over the
    selected rows it holds, and the LSE combine of the G gathered partials.
    The other ranks' candidates and partials (what the two gathers would
    bring) are computed first, untimed; the gathers themselves are not part
    of one GPU.  Each step is graph-captured and timed on its own."""
    import torch
    import indexer_selected_sparse_li_amd as lisfa
    import workloads as W
    log(f"[bench] context-parallel share of {wl.name}, G={G}")
    b = W.make_batch(wl, device="cuda")
    R, K = b.R, wl.K
    stream = torch.cuda.current_stream()
    shards = W.context_shards(b, G)
    st = []
    for s in shards:
        kc, vc = _cp_caches(lisfa, b, s)
        ld = max(64, -(-s["max_vis"] // 64) * 64)
        scores = torch.empty((R, ld), dtype=torch.float32, device="cuda")
        lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, s["row_pos"], scores, s["max_vis"], q_scale=b.q_scale)
        cp = torch.empty((R, K), dtype=torch.int32, device="cuda")
        cs = torch.empty((R, K), dtype=torch.float32, device="cuda")
        lisfa.topk_candidates(scores, s["row_pos"], K, cp, cs, pos_offset=s["pos_offset"])
        st.append(dict(kc=kc, vc=vc, scores=scores, cp=cp, cs=cs))
    cand_pos = torch.cat([x["cp"] for x in st], 1).contiguous()
    cand_score = torch.cat([x["cs"] for x in st], 1).contiguous()
    idx = torch.empty((R, K), dtype=torch.int32, device="cuda")
    lisfa.topk_merge(cand_score, cand_pos, K, idx, ordered=True)
    pout = torch.empty((G, R, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    plse = torch.empty((G, R, wl.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(1, lisfa.workspace_size(4, R, 0, K, wl.H, wl.D_v)), dtype=torch.uint8, device="cuda")
    for g, (s, x) in enumerate(zip(shards, st)):
        lisfa.sparse_mla_attn_partial(b.q, x["vc"], b.row_seq, idx, pout[g], plse[g], shard_range=s["range"],
                                      softmax_scale=wl.softmax_scale, workspace=ws)
    out = torch.empty((R, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((R, wl.H), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    s0, x0 = shards[0], st[0]
    tws = torch.empty(max(1, lisfa.workspace_size(3, R, x0["scores"].shape[1], K, 0, 0)), dtype=torch.uint8,
                      device="cuda")
    cp0 = torch.empty((R, K), dtype=torch.int32, device="cuda")
    cs0 = torch.empty((R, K), dtype=torch.float32, device="cuda")
    po0 = torch.empty((R, wl.H, wl.D_v), dtype=torch.float32, device="cuda")
    pl0 = torch.empty((R, wl.H), dtype=torch.float32, device="cuda")
    idx0 = torch.empty((R, K), dtype=torch.int32, device="cuda")
    steps = [
        ("li_score (local)", lambda q: lisfa.li_score(b.q_idx, b.w, x0["kc"], b.row_seq, s0["row_pos"], x0["scores"],
                                                      s0["max_vis"], q_scale=b.q_scale, stream=q)),
        ("topk_candidates", lambda q: lisfa.topk_candidates(x0["scores"], s0["row_pos"], K, cp0, cs0,
                                                             pos_offset=s0["pos_offset"], workspace=tws, stream=q)),
        ("topk_merge", lambda q: lisfa.topk_merge(cand_score, cand_pos, K, idx0, ordered=True, stream=q)),
        ("sparse_mla_attn_partial", lambda q: lisfa.sparse_mla_attn_partial(
            b.q, x0["vc"], b.row_seq, idx, po0, pl0, shard_range=s0["range"], softmax_scale=wl.softmax_scale,
            workspace=ws, stream=q)),
        ("lse_combine", lambda q: lisfa.lse_combine(pout, plse, out, lse, stream=q)),
    ]
    times = {}
    for name, fn in steps:
        times[name] = time_on_stream(fn, stream, 2, args.steps, graph=True) * 1e6
    total = sum(times.values())
    vis_local = int((s0["row_pos"].to(torch.int64) + 1).clamp(min=0).sum().item())
    ke = 1 if wl.indexer_dtype in ("fp8", "mxfp8") else 2
    ks = {"fp8": 4, "mxfp8": wl.D_I // 32}.get(wl.indexer_dtype, 0)
    li_bytes = vis_local * (wl.D_I * ke + ks) + R * (wl.H_I * (wl.D_I * ke + 4) + ks)
    res = dict(workload=wl.name, G=G, rank=0, rows=R, local_positions=vis_local,
               us={k: round(v, 2) for k, v in times.items()}, share_us=round(total, 2),
               rows_per_s=round(R / (total * 1e-6), 1),
               li_score_local_hbm_frac=round(li_bytes / (times["li_score (local)"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4))
    log(f"[bench] share {res}")
    return res


def zigzag_balance(args, wl, G):
    """Causal prefill rows split over G GPUs in order and by the Zigzag
    partition: the fused layer's time on each GPU's rows."""
    import torch
    import indexer_selected_sparse_li_amd as lisfa
    import workloads as W
    log(f"[bench] zigzag balance on {wl.name}, G={G}")
    b = W.make_batch(wl, device="cuda")
    n = b.R
    kc = lisfa.KVCache(data=b.k_data, scale=b.k_scale, scale_group=1, block_table=b.block_table,
                       block_size=wl.block_size, seq_base=b.seq_base)
    vc = lisfa.KVCache(data=b.kv_data, scale=b.kv_scale, scale_group=wl.kv_scale_group,
                       block_table=b.block_table, block_size=wl.block_size, seq_base=b.seq_base)
    stream = torch.cuda.current_stream()
    res = {}
    for part in ("in-order", "zigzag"):
        per = []
        for g in range(G):
            if part == "zigzag":
                rng = lisfa.zigzag_share(n, G, g)
            else:
                rng = [(g * n // G, (g + 1) * n // G)]
            rows = torch.cat([torch.arange(a, c) for a, c in rng]).cuda()
            m = rows.numel()
            sub = dict(q_idx=b.q_idx[rows].contiguous(), w=b.w[rows].contiguous(), q=b.q[rows].contiguous(),
                       row_seq=b.row_seq[rows].contiguous(), row_pos=b.row_pos[rows].contiguous())
            out = torch.empty((m, wl.H, wl.D_v), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((m, wl.H), dtype=torch.float32, device="cuda")
            ws = torch.empty(lisfa.workspace_size(2, m, b.max_visible, wl.K, wl.H, wl.D_v), dtype=torch.uint8,
                             device="cuda")
            fn = (lambda q, sub=sub, out=out, lse=lse, ws=ws: lisfa.li_topk_sfa(
                sub["q_idx"], sub["w"], kc, sub["q"], vc, sub["row_seq"], sub["row_pos"], wl.K, b.max_visible,
                out, lse, rows_per_group=8, softmax_scale=wl.softmax_scale, workspace=ws, stream=q))
            per.append(round(time_on_stream(fn, stream, 1, max(2, args.steps // 4)) * 1e3, 3))
            del ws, out, lse, sub
        res[part] = dict(ms=per, max_over_min=round(max(per) / min(per), 3), max_ms=max(per))
        log(f"[bench] {part}: {res[part]}")
    return dict(workload=wl.name, G=G, rows=n, **res)


def report_cp(args):
    """Context-parallel measurements: one GPU's decode share, and the Zigzag
    load balance of causal prefill rows; a markdown table if asked."""
    import workloads as W
    shares = [cp_share_timing(args, W.get("fp8_decode_16x131072"), 8),
              cp_share_timing(args, W.get("decode_paged_64x32768"), 8)]
    pre = W.get("prefill_4096q_l65536").with_(name="prefill_16384q_from0", seq_len=16384, q_rows=16384)
    zz = zigzag_balance(args, pre, 4)
    print(json.dumps(dict(shares=shares, zigzag=zz)), flush=True)
    if args.report_md:
        with open(args.report_md, "w") as fh:
            fh.write("# Context-parallel share on one MI355X\n\n")
            fh.write("One GPU's share of a context split (rank 0 of G). Every step is captured in a HIP graph and\n"
                     "timed on its own with HIP events; the candidates and partials of the other ranks (what the\n"
                     "two gathers between GPUs would bring) are computed beforehand, untimed. The gathers are not\n"
                     "part of one GPU. rows/s = rows / share time, i.e. the whole job's rate when all G GPUs run\n"
                     "their shares at once, gathers excluded.\n\n")
            fh.write("Command (from the repository root):\n\n")
            fh.write(f"    python3 bench.py --report-cp --steps {args.steps} --report-md "
                     f"{os.path.relpath(args.report_md, ROOT)}\n\n")
            names = list(shares[0]["us"])
            fh.write("| workload | G | rows | local positions | " + " | ".join(f"{k} us" for k in names) +
                     " | share us | rows/s | local li_score % HBM |\n")
            fh.write("|---" * (7 + len(names)) + "|\n")
            for s in shares:
                fh.write(f'| {s["workload"]} | {s["G"]} | {s["rows"]} | {s["local_positions"]} | ' +
                         " | ".join(str(s["us"][k]) for k in names) +
                         f' | {s["share_us"]} | {s["rows_per_s"]:.0f} | {s["li_score_local_hbm_frac"] * 100:.1f} |\n')
            fh.write(f'\nZigzag balance: {zz["rows"]} causal prefill rows (positions 0..{zz["rows"] - 1}) on '
                     f'{zz["G"]} GPUs, fused layer time per GPU (ms):\n\n')
            fh.write("| partition | " + " | ".join(f"GPU {g}" for g in range(zz["G"])) + " | max / min |\n")
            fh.write("|---" * (zz["G"] + 2) + "|\n")
            for part in ("in-order", "zigzag"):
                fh.write(f"| {part} | " + " | ".join(str(x) for x in zz[part]["ms"]) +
                         f' | {zz[part]["max_over_min"]} |\n')
        log(f"[bench] wrote {args.report_md}")


def report_cold(args):
    """The layer's stages hot and cold on a few workloads: each stage on its
    own, back-to-back (hot) and after a 512 MiB write that evicts the L2s and
    the MALL (cold), then the layer's three stages in turn with HIP events at
    the stage boundaries, cold and hot.  Eager launches on one stream."""
    import torch
    import indexer_selected_sparse_li_amd as lisfa
    import workloads as W
    names = [args.workload] if args.workload != "decode_paged_64x32768" else [
        "decode_paged_64x32768", "decode_paged_64x32768_mxfp8", "batched_paged_64x4k_32k", "fp8_decode_16x131072"]
    stream = torch.cuda.current_stream()
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    n = args.steps

    def ev():
        return torch.cuda.Event(enable_timing=True)

    rows = []
    for name in names:
        wl = W.get(name)
        log(f"[bench] cold/hot stages of {name}")
        b = W.make_batch(wl, device="cuda")
        R = b.R
        kc = lisfa.KVCache(data=b.k_data, scale=b.k_scale, scale_group=1, block_table=b.block_table,
                           block_size=wl.block_size, seq_base=b.seq_base)
        vc = lisfa.KVCache(data=b.kv_data, scale=b.kv_scale, scale_group=wl.kv_scale_group,
                           block_table=b.block_table, block_size=wl.block_size, seq_base=b.seq_base)
        out = torch.empty(R, wl.H, wl.D_v, dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(R, wl.H, dtype=torch.float32, device="cuda")
        idx = torch.empty(R, wl.K, dtype=torch.int32, device="cuda")
        ld = (b.max_visible + 63) // 64 * 64
        scores = torch.empty(R, ld, dtype=torch.float32, device="cuda")
        sws = torch.empty(max(1, lisfa.workspace_size(1, R, 0, wl.K, wl.H, wl.D_v)), dtype=torch.uint8,
                          device="cuda")
        lws = torch.empty(max(1, lisfa.workspace_size(5, R, b.max_visible, wl.K, 0, 0)), dtype=torch.uint8,
                          device="cuda")
        fns = {
            "li_score": lambda: lisfa.li_score(b.q_idx, b.w, kc, b.row_seq, b.row_pos, scores, b.max_visible,
                                               q_scale=b.q_scale, stream=stream),
            "topk_select": lambda: lisfa.topk_select(scores, b.row_pos, wl.K, idx, stream=stream),
            "li_topk": lambda: lisfa.li_topk(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, idx, b.max_visible,
                                             q_scale=b.q_scale, workspace=lws, stream=stream),
            "sparse_mla_attn": lambda: lisfa.sparse_mla_attn(b.q, vc, b.row_seq, idx, out, lse,
                                                             softmax_scale=wl.softmax_scale, workspace=sws,
                                                             stream=stream),
        }
        fused = lisfa.li_topk_plan(b.q_idx, b.w, kc, b.row_seq, b.row_pos, wl.K, b.max_visible,
                                   q_scale=b.q_scale, layer=True) > 0
        # the layer's own sequence of stages
        stages = [(k, fns[k]) for k in (("li_topk", "sparse_mla_attn") if fused
                                        else ("li_score", "topk_select", "sparse_mla_attn"))]
        for f in fns.values():
            f()
        torch.cuda.synchronize()
        alone = {}
        for sname, f in fns.items():
            for _ in range(args.warmup):
                f()
            e0, e1 = ev(), ev()
            e0.record(stream)
            for _ in range(n):
                f()
            e1.record(stream)
            torch.cuda.synchronize()
            hot = e0.elapsed_time(e1) / n * 1e3
            es = []
            for i in range(n):
                flush.fill_(i & 255)
                a, c = ev(), ev()
                a.record(stream)
                f()
                c.record(stream)
                es.append((a, c))
            torch.cuda.synchronize()
            alone[sname] = (hot, sum(a.elapsed_time(c) for a, c in es) / n * 1e3)
        split = {}
        for mode in ("cold", "hot"):
            es = []
            for i in range(n):
                if mode == "cold":
                    flush.fill_(i & 255)
                e = [ev() for _ in range(len(stages) + 1)]
                e[0].record(stream)
                for j, (_, f) in enumerate(stages):
                    f()
                    e[j + 1].record(stream)
                es.append(e)
            torch.cuda.synchronize()
            split[mode] = [sum(e[j].elapsed_time(e[j + 1]) for e in es) / n * 1e3 for j in range(len(stages))]
        nrow0 = len(rows)
        for j, (sname, _) in enumerate(stages):
            rows.append((name, sname, alone[sname][0], alone[sname][1], split["hot"][j], split["cold"][j]))
        for sname in fns:   # stages the layer does not run here, alone only
            if sname not in dict(stages):
                rows.append((name, sname + " (not in the layer)", alone[sname][0], alone[sname][1],
                             float("nan"), float("nan")))
        rows.append((name, "layer", sum(alone[k][0] for k, _ in stages), sum(alone[k][1] for k, _ in stages),
                     sum(split["hot"]), sum(split["cold"])))
        for r in rows[nrow0:]:
            log(f"[bench] {r[0]} {r[1]}: alone hot {r[2]:.1f} cold {r[3]:.1f} us; in the layer hot {r[4]:.1f} "
                f"cold {r[5]:.1f} us")
        del b, kc, vc, scores
        torch.cuda.empty_cache()
    print(json.dumps([dict(workload=r[0], stage=r[1], alone_hot_us=round(r[2], 1), alone_cold_us=round(r[3], 1),
                           layer_hot_us=round(r[4], 1), layer_cold_us=round(r[5], 1)) for r in rows]), flush=True)
    if args.report_md:
        with open(args.report_md, "w") as fh:
            fh.write("# The layer's stages hot and cold (one MI355X)\n\n")
            fh.write("Each stage alone: back-to-back calls (hot), and calls that each follow a 512 MiB write that\n"
                     "evicts the L2s and the MALL (cold). In the layer: the layer's stages in turn (li_topk +\n"
                     "sparse_mla_attn where the fused index step takes the shape, else li_score + topk_select +\n"
                     "sparse_mla_attn) with HIP events at the stage boundaries, hot and cold (the flush before each\n"
                     f"layer step). Eager launches on one stream, {n} timed calls each.\n\n")
            fh.write("Command (from the repository root):\n\n")
            fh.write(f"    python3 bench.py --report-cold --steps {n} --report-md "
                     f"{os.path.relpath(args.report_md, ROOT)}\n\n")
            fh.write("| workload | stage | alone hot us | alone cold us | in the layer hot us | in the layer cold us |\n"
                     "|---|---|---|---|---|---|\n")
            for r in rows:
                fh.write(f"| {r[0]} | {r[1]} | {r[2]:.1f} | {r[3]:.1f} | {r[4]:.1f} | {r[5]:.1f} |\n")


def report_prolog(args):
    """The indexer prolog kernels on a decode step (64 query rows, 64 new
    keys) and a prefill chunk (4096 of each): query quantisation (fp8 per row
    and MXFP8) and key LayerNorm + store (bf16, fp8, MXFP8 paged caches).
    Each call graph-captured and timed on its own; bytes = bf16 inputs read +
    codes and scales written."""
    import torch
    import indexer_selected_sparse_li_amd as lisfa
    stream = torch.cuda.current_stream()
    rows = []
    for n in (64, 4096):
        g = torch.Generator(device="cuda").manual_seed(n)
        q = torch.randn(n, 64, 128, device="cuda", generator=g).to(torch.bfloat16)
        for fmt in ("fp8", "mxfp8"):
            qo = torch.empty(n, 64, 128, dtype=torch.uint8, device="cuda")
            qs = (torch.empty(n, dtype=torch.float32, device="cuda") if fmt == "fp8"
                  else torch.empty(n, 64, 4, dtype=torch.uint8, device="cuda"))
            t = time_on_stream(lambda st: lisfa.indexer_q_quant(q, fmt, qo, qs, stream=st), stream, 2, args.steps,
                               graph=True)
            by = q.numel() * 2 + qo.numel() + qs.numel() * qs.element_size()
            rows.append(("indexer_q_quant", fmt, n, t * 1e6, by))
        k = torch.randn(n, 128, device="cuda", generator=g).to(torch.bfloat16)
        gamma = torch.rand(128, device="cuda", generator=g) + 0.5
        beta = torch.randn(128, device="cuda", generator=g) * 0.1
        nblk = 2 * (n // 64 + 1)
        bt = torch.randperm(nblk, device="cuda", generator=g).to(torch.int32).view(1, nblk)
        seq = torch.zeros(n, dtype=torch.int32, device="cuda")
        pos = torch.arange(n, dtype=torch.int32, device="cuda")
        for fmt in ("bf16", "fp8", "mxfp8"):
            if fmt == "bf16":
                data, scale = torch.empty(nblk * 64, 128, dtype=torch.bfloat16, device="cuda"), None
            else:
                data = torch.empty(nblk * 64, 128, dtype=torch.uint8, device="cuda")
                scale = (torch.empty(nblk * 64, dtype=torch.float32, device="cuda") if fmt == "fp8"
                         else torch.empty(nblk * 64, 4, dtype=torch.uint8, device="cuda"))
            kc = lisfa.KVCache(data=data, scale=scale, block_table=bt, block_size=64)
            t = time_on_stream(lambda st: lisfa.indexer_k_store(k, seq, pos, kc, gamma=gamma, beta=beta, stream=st),
                               stream, 2, args.steps, graph=True)
            elt = 2 if fmt == "bf16" else 1
            sc = {"bf16": 0, "fp8": 4, "mxfp8": 4}[fmt]
            by = k.numel() * 2 + n * (128 * elt + sc) + 2 * 128 * 4 + n * 8
            rows.append(("indexer_k_store (LayerNorm)", fmt, n, t * 1e6, by))
    # the whole prolog: key store and query quantisation in turn on one
    # stream, or on two side streams side by side (graph-captured, so the
    # replay runs the two branches concurrently)
    both = []
    for n in (64, 4096):
        g = torch.Generator(device="cuda").manual_seed(n + 1)
        q = torch.randn(n, 64, 128, device="cuda", generator=g).to(torch.bfloat16)
        k = torch.randn(n, 128, device="cuda", generator=g).to(torch.bfloat16)
        gamma = torch.rand(128, device="cuda", generator=g) + 0.5
        beta = torch.randn(128, device="cuda", generator=g) * 0.1
        nblk = 2 * (n // 64 + 1)
        bt = torch.randperm(nblk, device="cuda", generator=g).to(torch.int32).view(1, nblk)
        seq = torch.zeros(n, dtype=torch.int32, device="cuda")
        pos = torch.arange(n, dtype=torch.int32, device="cuda")
        for fmt in ("fp8", "mxfp8"):
            qo = torch.empty(n, 64, 128, dtype=torch.uint8, device="cuda")
            qs = (torch.empty(n, dtype=torch.float32, device="cuda") if fmt == "fp8"
                  else torch.empty(n, 64, 4, dtype=torch.uint8, device="cuda"))
            data = torch.empty(nblk * 64, 128, dtype=torch.uint8, device="cuda")
            scale = (torch.empty(nblk * 64, dtype=torch.float32, device="cuda") if fmt == "fp8"
                     else torch.empty(nblk * 64, 4, dtype=torch.uint8, device="cuda"))
            kc = lisfa.KVCache(data=data, scale=scale, block_table=bt, block_size=64)
            t = {}
            for mode in ("serial", "streams", "fused"):
                t[mode] = time_on_stream(lambda st: lisfa.indexer_prolog(q, fmt, qo, qs, k, seq, pos, kc, gamma=gamma,
                                                                         beta=beta, mode=mode, stream=st),
                                         stream, 2, args.steps, graph=True)
            both.append((fmt, n, t["serial"] * 1e6, t["streams"] * 1e6, t["fused"] * 1e6))
    for r in rows:
        log(f"[bench] {r[0]} {r[1]} n={r[2]}: {r[3]:.2f} us, {r[4] / r[3] / 1e3:.2f} GB/s")
    for b_ in both:
        log(f"[bench] prolog {b_[0]} n={b_[1]}: serial {b_[2]:.2f} us, two streams {b_[3]:.2f} us, "
            f"one launch {b_[4]:.2f} us")
    print(json.dumps([dict(kernel=r[0], format=r[1], rows=r[2], us=round(r[3], 2), bytes=r[4]) for r in rows]),
          flush=True)
    if args.report_md:
        with open(args.report_md, "w") as fh:
            fh.write("# Indexer prolog kernels on one MI355X\n\n")
            fh.write("Query quantisation of [n, 64, 128] bf16 queries and LayerNorm + store of n new 128-wide keys\n"
                     "into a paged key cache (random 64-token blocks). Each call captured in a HIP graph and timed\n"
                     "on its own with HIP events; bytes = bf16 inputs read + codes and scales written.\n\n")
            fh.write("Command (from the repository root):\n\n")
            fh.write(f"    python3 bench.py --report-prolog --steps {args.steps} --report-md "
                     f"{os.path.relpath(args.report_md, ROOT)}\n\n")
            fh.write("| kernel | format | rows | us | GB/s | % of HBM peak |\n|---|---|---|---|---|---|\n")
            for r in rows:
                gbs = r[4] / r[3] / 1e3
                fh.write(f"| {r[0]} | {r[1]} | {r[2]} | {r[3]:.2f} | {gbs:.1f} | {gbs / HBM_PEAK_GBS * 100:.1f} |\n")
            fh.write("\nThe whole prolog of a step (key LayerNorm + store and query quantisation) with n new keys\n"
                     "and n query rows, graph-captured: the two calls in turn on one stream (serial); the two on\n"
                     "side streams that fork from and join back into the launch stream (two streams); the C ABI's\n"
                     "`indexer_prolog`, one launch whose workgroups split between query rows and keys (one\n"
                     "launch).  All three write the same bytes\n"
                     "(`tests/test_gpu_prolog.py::test_prolog_overlap_bit_identical`).\n\n")
            fh.write("| format | n | serial us | two streams us | one launch us |\n|---|---|---|---|---|\n")
            for b_ in both:
                fh.write(f"| {b_[0]} | {b_[1]} | {b_[2]:.2f} | {b_[3]:.2f} | {b_[4]:.2f} |\n")
        log(f"[bench] wrote {args.report_md}")


REPORT_ORDER = ["tiny_l256", "decode_l8192", "batched_paged_64x4k_32k", "prefill_4096q_l65536",
                "fp8_decode_16x131072", "decode_paged_1x32768", "decode_paged_64x32768",
                "decode_paged_64x32768_mxfp8", "decode_paged_64x32768_fp8tilekv"]


def write_report_md(path, lines, args):
    def st(r, k):
        s = r["stages"][k]
        rf = s["roofline"]
        return f'{s["us"]:.1f} ({rf["frac"] * 100:.1f} % {rf["bound"].upper()})'
    with open(path, "w") as fh:
        fh.write("# Layer throughput on every workload (one MI355X)\n\n")
        fh.write("HIP-event timings on the launch stream; a step is one li_topk_sfa call over the whole batch.\n"
                 "Cold = each step after a 512 MiB write that evicts the L2s and the MALL; hot = back-to-back\n"
                 "calls from Python; graph = the same call captured once in a HIP graph and replayed (no\n"
                 "host overhead per call; every replay checked against the eager result first).\n"
                 "Stage times are hot, each stage launched on its own (graph-captured); the fraction is of the stage's binding\n"
                 "roofline (HBM 8 TB/s; MFMA bf16 2.5 PFLOP/s, fp8 5.0) on algorithmic bytes or flops.\n"
                 "The layer's index step is li_topk (scores and Top-K in one launch, the scores on chip) where\n"
                 "li_topk_plan takes the shape, else li_score + topk_select; both are timed on every workload.\n\n")
        fh.write("Command (from the repository root):\n\n")
        fh.write(f"    python3 bench.py --report-all --steps {args.steps} --warmup {args.warmup} "
                 f"--report-md {os.path.relpath(path, ROOT)}\n\n")
        fh.write("| workload | rows | layer cold us | tokens/s cold | layer hot us | tokens/s hot | "
                 "graph replay us | tokens/s graph | li_topk us | li_score us | topk_select us | "
                 "sparse_mla_attn us | oracle tokens/s (threads) |\n")
        fh.write("|---|---|---|---|---|---|---|---|---|---|---|---|---|\n")
        for r in lines:
            cb = r.get("cpu_baseline")
            orc = f'{cb["value"]:.3g} ({cb["cores"]})' if cb else "not run"
            fh.write(f'| {r["config"]["workload"]} | {r["config"]["rows"]} | '
                     f'{r["ms_per_step_cold"] * 1e3:.1f} | {r["value_cold"]:.0f} | '
                     f'{r["ms_per_step_hot"] * 1e3:.1f} | {r["value_hot"]:.0f} | '
                     f'{r["ms_per_step_graph"] * 1e3:.1f} | {r["value_graph"]:.0f} | '
                     f'{st(r, "li_topk")}{"" if r["stages"]["li_topk"]["in_layer"] else " (separate kernels)"} | '
                     f'{st(r, "li_score")} | {st(r, "topk_select")} | {st(r, "sparse_mla_attn")} | {orc} |\n')
        if any(r.get("cpu_baseline") for r in lines):
            fh.write("\nOracle: the CPU oracle (float64 NumPy, scores over the full visible context, selection, "
                     "attention) on the first rows of the same batch in the same run, about "
                     f"{args.cpu_budget_each:g} s per workload (at least one row); threads = the BLAS pool's size. "
                     "A baseline, not the target.\n")
    log(f"[bench] wrote {path}")


if __name__ == "__main__":
    main()
