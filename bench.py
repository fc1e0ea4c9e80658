"""Benchmark of the gated DSA forward hot path on one MI355X.

A step is one dsa_fused_fwd call (key LayerNorm, indexer + top-k, sparse latent attention, V
up-projection and gate) over one batch of synthetic input. The default workload is the long-context
one: a single 131,072-token document (top-2048, 96 heads, indexer 64 heads x 128, latent 512+64),
seed 5. All inputs are resident in device memory before timing starts.

Prints one JSON line: throughput (query tokens/s) of the default workload, the roofline of its
dominant kernel (the one with the longest stage time: the indexer at this size), the other
workloads (T=4,096, T=8,192, eight packed documents) as extra fields, and the CPU oracle timed on a
bounded, evenly spaced sample of rows.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "query tokens/sec for indexer+top-2048+sparse MLA fwd; % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
CSRC = os.path.join(ROOT, "dsa_indexer_top_index_amd", "csrc")
KERNEL_SRC = {
    "k_index_topk": os.path.join(CSRC, "k_index.hip"),
    "k_sparse_mla": os.path.join(CSRC, "k_mla.hip"),
    "k_up_gate": os.path.join(CSRC, "k_up.hip"),
}
# The rocprofv3 names of the three path kernels as the bench's workloads launch them (BF16 indexer,
# 96 heads), matched exactly: the backward's k_sparse_mla_bwd and the FP8 indexer instance are other kernels.
KERNEL_NAME = {
    "k_index_topk": "k_index_topk<64, 128, false, false>",
    "k_sparse_mla": "k_sparse_mla<96>",
    "k_up_gate": "k_up_gate(",
}
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 1 << 30         # plain device copy used to scale the HBM byte counters
D_MODEL = 7168               # hidden size of the model (KimiK3TextConfig), the width of o_proj's output
COPY_LAUNCHES = 5

WORKLOAD_TEXT = {
    "t131072": "single document T=131072, top-2048, 96 heads, indexer 64x128 with key LayerNorm, latent 512+64, "
               "W_UV 96x512x128, per-head gate",
    "t4096": "single document T=4096, top-2048, 96 heads, indexer 64x128 with key LayerNorm, latent 512+64, "
             "W_UV 96x512x128, per-head gate",
    "t8192": "single document T=8192, top-2048, 96 heads, indexer 64x128, latent 512+64",
    "packed": "8 packed documents (lengths U[1024,8192], seed 4), top-2048, 96 heads, indexer 64x128, latent 512+64",
    "tiny": "single document T=1024, top-256, 16 heads, indexer 4x64, latent 512+64",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def work_counts(cfg):
    """(sum of k_eff over rows, causal pairs of all rows, causal pairs of the rows the indexer scores,
    i.e. rows with more than k causal keys)."""
    cu = cfg.cu_seqlens
    keff = all_pairs = sel_pairs = 0
    for d in range(cfg.n_docs):
        L = int(cu[d + 1] - cu[d])
        n = np.arange(1, L + 1, dtype=np.int64)
        keff += int(np.minimum(n, cfg.topk).sum())
        all_pairs += int(n.sum())
        sel_pairs += int(n[n > cfg.topk].sum())
    return keff, all_pairs, sel_pairs


def alg_work(cfg):
    """Algorithmic flops per launch of each kernel and the attention's logical gather bytes:
    indexer 2*H_I*d_I per scored causal pair; attention 2*H*(576+512) per selected key;
    up-projection 2*H*512*128 per row; gather 1,152 B per selected key."""
    keff, all_pairs, sel_pairs = work_counts(cfg)
    return {
        "k_index_topk": 2.0 * cfg.H_I * cfg.d_I * sel_pairs,
        "k_sparse_mla": 2.0 * cfg.H * (576 + 512) * keff,
        "k_up_gate": 2.0 * cfg.H * 512 * 128 * cfg.T,
        "gather_bytes": 1152.0 * keff,
        "keff_sum": keff, "all_pairs": all_pairs, "scored_pairs": sel_pairs,
    }


def src_hash(path):
    """Hash of a kernel source's code: comments and layout are left out, so that editing a comment
    does not invalidate counters taken on the same code."""
    import re
    t = open(path).read()
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return hashlib.sha256(" ".join(t.split()).encode()).hexdigest()[:16]


def pmc_hbm_path(kernel, workload):
    return os.path.join(PROFILES, f"pmc_hbm_{kernel}_{workload}.json")


def traffic_from_profile(kernel, workload):
    """HBM bytes per whole-workload launch of `kernel` on `workload` from its committed counter summary,
    or None when there is none or the kernel's code has changed since the counters were taken."""
    path = pmc_hbm_path(kernel, workload)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel") != kernel or d.get("workload") != workload or d.get("instance") != KERNEL_NAME[kernel]:
        return None
    if d.get("kernel_code_sha256_16") != src_hash(KERNEL_SRC[kernel]):
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_rows(d):
    """Rows of every rocprofv3 counter-collection CSV under directory d."""
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)):
        rows += list(csv.DictReader(open(f)))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def _dispatches(rows, kernel):
    """{dispatch id: duration (ns)} of the path kernel `kernel` (its exact instance name)."""
    return {r["Dispatch_Id"]: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            for r in rows if KERNEL_NAME[kernel] in r["Kernel_Name"]}


def _whole_workload(dur):
    """The dispatches of one kernel that run at least 0.8 times as long as its longest one: the bench's
    stage window launches each path kernel once over all rows, while the fused step (and the backward's
    recompute) launch the attention and the up-projection per 2,048-row chunk, at most two thirds of
    the work of any bench workload (the last chunk at T=4,096)."""
    longest = max(dur.values())
    return {d for d, t in dur.items() if t >= 0.8 * longest}


def _per_dispatch_kib(rows, kernel, counter):
    """Values of `counter` (KiB; summed over the counter's instances) of the whole-workload launches of
    the path kernel `kernel`."""
    keep = _whole_workload(_dispatches(rows, kernel)) if _dispatches(rows, kernel) else set()
    per = {}
    for r in rows:
        if r["Dispatch_Id"] in keep and KERNEL_NAME[kernel] in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return list(per.values())


def pmc_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, workload, commands):
    """HBM bytes per whole-workload launch of each path kernel from FETCH_SIZE / WRITE_SIZE counter
    runs, each scaled by what the same counter reads for a plain device copy of known size; one
    summary per kernel."""
    import testgen as tg
    cfg = tg.get_config(workload)
    work = alg_work(cfg)
    cal_bytes = COPY_LAUNCHES * COPY_BYTES  # every copy dispatch of the calibration run together
    cal_f, cal_w = _counter_rows(cal_fetch_dir), _counter_rows(cal_write_dir)
    cf_kib = sum(float(r["Counter_Value"]) for r in cal_f if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == "FETCH_SIZE")
    cw_kib = sum(float(r["Counter_Value"]) for r in cal_w if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == "WRITE_SIZE")
    f_scale = cal_bytes / (cf_kib * 1024.0)
    w_scale = cal_bytes / (cw_kib * 1024.0)
    frows, wrows = _counter_rows(fetch_dir), _counter_rows(write_dir)
    out = {}
    for kernel in KERNEL_SRC:
        fv = _per_dispatch_kib(frows, kernel, "FETCH_SIZE")
        wv = _per_dispatch_kib(wrows, kernel, "WRITE_SIZE")
        if not fv or not wv:  # every path kernel runs in every bench workload
            raise SystemExit(f"no launches of {KERNEL_NAME[kernel]} in the counter runs")
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        fetch_b, write_b = f_kib * 1024.0 * f_scale, w_kib * 1024.0 * w_scale
        res = {
            "kernel": kernel, "instance": KERNEL_NAME[kernel], "workload": workload,
            "kernel_code_sha256_16": src_hash(KERNEL_SRC[kernel]),
            "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [len(fv), len(wv)],
            "dispatch_rule": "the kernel's launches over the whole workload only (at least 0.8 of its longest launch: "
                             "the bench's stage window; the fused step's row-chunk launches are left out)",
            "copy_calibration": {"bytes_each_way_all_copies": cal_bytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                                 "fetch_scale": f_scale, "write_scale": w_scale},
            "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
            "hbm_bytes_per_launch": fetch_b + write_b, "commands": commands,
        }
        if kernel == "k_sparse_mla":
            res["gather_logical_bytes_per_launch"] = work["gather_bytes"]
        with open(pmc_hbm_path(kernel, workload), "w") as fh:
            json.dump(res, fh, indent=1)
        out[kernel] = res
    print(json.dumps(out, indent=1))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4   # 256 CUs x 4 SIMDs
XCDS = 8


def pmc_mfma_summary(mfma_dir, workload, commands):
    """Per-kernel MFMA counters of the whole-workload launches of a bench run: bf16 MFMA flops the
    hardware executed (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against the algorithmic flops, the rate both
    give over the dispatch time, and the share of SIMD cycles the matrix cores were busy."""
    import testgen as tg
    rows = _counter_rows(mfma_dir)
    cfg = tg.get_config(workload)
    work = alg_work(cfg)
    out = {"workload": workload, "counters": list(MFMA_COUNTERS), "simds": SIMDS, "kernels": {},
           "kernel_code_sha256_16": {k: src_hash(v) for k, v in KERNEL_SRC.items()},
           "alg_flop_note": "indexer: 2*H_I*d_I per causal pair of the rows it scores (n_t > k); attention: "
                            "2*H*(576+512) per selected key; up-projection: 2*H*512*128 per row",
           "commands": commands}
    for name in KERNEL_SRC:
        per = {}
        for r in rows:
            if KERNEL_NAME[name] in r["Kernel_Name"]:
                d = per.setdefault(r["Dispatch_Id"], {"t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ds = [d for d in per.values() if all(c in d for c in MFMA_COUNTERS)]
        if not ds:
            raise SystemExit(f"no launches of {KERNEL_NAME[name]} in the counter run")
        keep = _whole_workload({i: int(d["t"] * 1e9) for i, d in enumerate(ds)})
        ds = [d for i, d in enumerate(ds) if i in keep]
        t = float(np.mean([d["t"] for d in ds]))
        mops = float(np.mean([d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds]))
        busy = float(np.mean([d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds]))
        gui = float(np.mean([d["GRBM_GUI_ACTIVE"] for d in ds]))
        hw_flop = mops * 512.0
        alg_flop = work[name]
        out["kernels"][name] = {
            "instance": KERNEL_NAME[name], "dispatches": len(ds), "mean_dispatch_us": t * 1e6,
            "hw_bf16_mfma_flop": hw_flop, "alg_flop": alg_flop, "hw_over_alg": hw_flop / alg_flop,
            "hw_tflops": hw_flop / t / 1e12, "alg_tflops": alg_flop / t / 1e12,
            "alg_frac_of_peak": alg_flop / t / 1e12 / PEAK_BF16_TFLOPS,
            "mfma_busy_cycles": busy, "grbm_gui_active": gui,
            # GRBM_GUI_ACTIVE comes summed over the XCDs; per-XCD active cycles x all SIMDs
            "mfma_busy_frac": busy / (gui / XCDS * SIMDS),
            "implied_clock_ghz": gui / XCDS / t / 1e9,
        }
    path = os.path.join(PROFILES, f"pmc_mfma_{workload}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def stats_summary(stats_dir, workload, command, bench_log):
    """Markdown summary of a `rocprofv3 --kernel-trace --stats` run of this bench: the statistics of
    every kernel, the mean duration of the whole-workload launches of the three path kernels, and the
    bench line the same command printed (its HIP-event stage times)."""
    import csv
    import glob
    stats = list(csv.DictReader(open(glob.glob(os.path.join(stats_dir, "**", "*kernel_stats.csv"), recursive=True)[0])))
    trace = list(csv.DictReader(open(glob.glob(os.path.join(stats_dir, "**", "*kernel_trace.csv"), recursive=True)[0])))
    line = None
    for l in open(bench_log):
        if l.startswith("{"):
            line = json.loads(l)
    lines = [f"# rocprofv3 kernel statistics: fused forward, {WORKLOAD_TEXT[workload]}", "",
             "Command (on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; R is the repository root):",
             "", "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share |", "|---|---|---|---|---|---|"]
    for r in stats:
        lines.append(f"| `{r['Name'][:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f}% |")
    lines += ["", "Launches over the whole workload (at least 0.8 of the kernel's longest launch: the bench's stage "
              "window launches each path kernel once over all rows, the fused step runs the attention and the "
              "up-projection per row chunk), against the HIP-event stage times of the bench line printed by the "
              "same command:", "",
              "| kernel (instance) | launches | trace average (us) | bench, HIP events (us) |", "|---|---|---|---|"]
    ev = {"k_index_topk": ("index_topk_ms", "key LayerNorm prologue + indexer"), "k_sparse_mla": ("attention_ms", "attention"),
          "k_up_gate": ("up_gate_ms", "up-projection + gate")}
    for k, (field, what) in ev.items():
        d = {r["Dispatch_Id"]: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in trace
             if KERNEL_NAME[k] in r["Kernel_Name"]}
        if not d:
            continue
        full = [d[i] for i in _whole_workload(d)]
        b = f"{line['stages'][field] * 1e3:.1f} ({what})" if line else "n/a"
        lines.append(f"| `{KERNEL_NAME[k].rstrip('(')}` | {len(full)} | {np.mean(full):.1f} | {b} |")
    if line:
        st = line["stages"]
        lines += ["", f"Bench line of the same command: {st['value']:.0f} query tokens/s, {st['ms_per_step']:.3f} ms per "
                  f"fused step (profiled, few steps); indexer {st['indexer_frac_scored_rows']:.3f} and attention "
                  f"{st['attention_frac']:.3f} of dense bf16 MFMA peak.",
                  "", "Kernel code hashes (sha256[:16] of the source without comments): " +
                  ", ".join(f"{k} {src_hash(v)}" for k, v in KERNEL_SRC.items()) + "."]
    print("\n".join(lines))


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, keys, stride):
    """The oracle, built for this host (-O3 -march=native, same floating-point semantics), on every
    stride-th row ending at the last: top-k with FP32 scores, then attention, up-projection and gate
    accumulated in float. The rows are evenly spaced, so their mean cost is the workload's mean cost
    per row, and rows per second extrapolate to the whole workload."""
    import oracle
    import testgen as tg

    t0 = time.perf_counter()
    oracle.use_native()
    build_s = time.perf_counter() - t0
    rows = np.arange(cfg.T - 1, -1, -stride)[::-1]
    t0 = time.perf_counter()
    LNk = oracle.key_layernorm(keys["k_I"], cfg.ln_eps)
    qr = tg.query_rows(cfg, rows)
    gen_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx, theta, keff = oracle.topk(rows, qr["q_I"].reshape(len(rows), cfg.H_I, cfg.d_I), qr["w"], LNk,
                                   cfg.cu_seqlens, cfg.topk)
    t1 = time.perf_counter()
    oracle.sparse_mla_f32(rows, qr["q"].reshape(len(rows), cfg.H, 576), keys["kv"], idx, keys["W_UV"],
                          qr["gate"].reshape(len(rows), cfg.H), cfg.softmax_scale)
    el = time.perf_counter() - t0
    return {
        "value": len(rows) / el, "unit": "query tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": f"{len(rows)} of {cfg.T} rows (every {stride}th row, ending at the last) of the same workload, "
                  f"extrapolated to it (evenly spaced rows have its mean cost per row): top-k with FP32 scores "
                  f"({t1 - t0:.1f}s), then attention + up-projection + gate accumulated in float "
                  f"({el - (t1 - t0):.1f}s), {el:.1f}s wall; plain C++ oracle built -O3 -march=native "
                  f"-ffp-contract=off with OpenMP over rows ({build_s:.1f}s build); key LayerNorm and input "
                  f"drawing ({gen_s:.1f}s) excluded",
        "cpu_model": cpu_model(),
    }


def run_workload(name, steps, warmup, cold_steps, want_inputs=False):
    """Times `steps` fused steps of one workload after `warmup`, then the three stages in a second
    window of the same length with HIP events on the launch stream, then `cold_steps` whole steps
    each after a 512 MB cache flush. Returns a result dict (and the host key-side inputs)."""
    import torch

    import dsa_indexer_top_index_amd as dsa
    import testgen as tg
    from tests import gpu_util as gu

    cfg = tg.get_config(name)
    log(f"[bench] {name}: generating inputs (T={cfg.T})")
    keys, dev = gu.device_inputs(cfg)
    shape = gu.shape_of(cfg, dev.get("cu_seqlens"))
    ws = dsa.alloc_workspace(shape)
    T = cfg.T
    topk_idx = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, cfg.H, 128), dtype=torch.bfloat16, device="cuda")

    def step():
        dsa.dsa_fused_fwd(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"],
                          topk_idx, out, ws)

    log(f"[bench] {name}: {warmup} warm-up and {steps} timed steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / steps * 1e3

    # Per-stage launch durations: HIP events on the stream the kernels run on, around the same
    # entry points the fused step is made of (the attention and the up-projection separately, with
    # o_lat for every row in a buffer of its own).
    log(f"[bench] {name}: stage timing")
    stream = torch.cuda.current_stream()
    o_lat = torch.empty((T, cfg.H, 512), dtype=torch.bfloat16, device="cuda")
    n_stage = max(steps, 3)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_stage)]
    for i in range(n_stage):
        ev[i][0].record(stream)
        dsa.dsa_index_topk(shape, dev["q_I"], dev["k_I"], dev["w"], topk_idx, ws)
        ev[i][1].record(stream)
        dsa.dsa_sparse_attention_latent(shape, dev["q"], dev["kv"], topk_idx, o_lat)
        ev[i][2].record(stream)
        dsa.dsa_up_gate(shape, o_lat, dev["W_UV"], dev["gate"], out)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    del o_lat
    warm_steps = [e[0].elapsed_time(e[3]) for e in ev]
    # The FP8 indexer (an alternative to the BF16 one, same outputs' shape), timed the same way.
    t_idx8 = t_idx_ln = ln_same = None
    if cfg.H_I == 64 and cfg.d_I == 128:
        idx8 = torch.empty_like(topk_idx)
        ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_stage)]
        for i in range(n_stage):
            ev8[i][0].record(stream)
            dsa.dsa_index_topk_fp8(shape, dev["q_I"], dev["k_I"], dev["w"], idx8, ws)
            ev8[i][1].record(stream)
        torch.cuda.synchronize()
        t_idx8 = float(np.mean([e[0].elapsed_time(e[1]) for e in ev8]))
        # The indexer with the key LayerNorm fused into its key-chunk loads (same results as the BF16
        # indexer, checked here on the whole output).
        ev_ln = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_stage)]
        for i in range(n_stage):
            ev_ln[i][0].record(stream)
            dsa.dsa_index_topk_fused_ln(shape, dev["q_I"], dev["k_I"], dev["w"], idx8, ws)
            ev_ln[i][1].record(stream)
        torch.cuda.synchronize()
        t_idx_ln = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_ln]))
        ln_same = bool(torch.equal(idx8, topk_idx))
        del idx8
    # The steps on either side of the path: the W_UK absorption that produces q, and o_proj after the
    # gate (hidden size 7168), on seeded synthetic operands of their shapes.
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed)
    q_nope = torch.randn((T, cfg.H, 128), generator=gen, device="cuda").to(torch.bfloat16)
    q_pe = torch.randn((T, cfg.H, 64), generator=gen, device="cuda").to(torch.bfloat16)
    W_UK = (0.02 * torch.randn((cfg.H, 512, 128), generator=gen, device="cuda")).to(torch.bfloat16)
    W_o = (0.01 * torch.randn((D_MODEL, cfg.H * 128), generator=gen, device="cuda")).to(torch.bfloat16)
    y = torch.empty((T, D_MODEL), dtype=torch.bfloat16, device="cuda")
    q_abs = dev["q"]  # the absorbed query overwrites q, which nothing reads after this point
    eva = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_stage)]
    for i in range(n_stage):
        eva[i][0].record(stream)
        dsa.dsa_q_absorb(shape, q_nope, q_pe, W_UK, q_abs)
        eva[i][1].record(stream)
        dsa.dsa_o_proj(shape, out.view(T, cfg.H * 128), W_o, y)
        eva[i][2].record(stream)
    torch.cuda.synchronize()
    t_abs = float(np.mean([e[0].elapsed_time(e[1]) for e in eva]))
    t_op = float(np.mean([e[1].elapsed_time(e[2]) for e in eva]))
    del q_nope, q_pe, W_UK, W_o, y
    # The backward of the attention, up-projection and gate (96 heads), on the fused step's indices,
    # out and lse, with a seeded synthetic dout.
    t_bwd = None
    if cfg.H == 96:
        lse = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
        dsa.dsa_fused_fwd(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"],
                          topk_idx, out, ws, lse=lse)
        dout = torch.randn((T, cfg.H, 128), generator=gen, device="cuda").to(torch.bfloat16)
        wsb = dsa.alloc_bwd_workspace(shape)
        dq = torch.empty((T, cfg.H, 576), dtype=torch.float32, device="cuda")
        dkv = torch.empty((T, 576), dtype=torch.float32, device="cuda")
        dW = torch.empty((cfg.H, 512, 128), dtype=torch.float32, device="cuda")
        dg = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
        n_bwd = 3 if T > 65536 else n_stage
        evb = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_bwd)]
        for i in range(n_bwd):
            evb[i][0].record(stream)
            dsa.dsa_sparse_mla_bwd(shape, dev["q"], dev["kv"], topk_idx, dev["W_UV"], dev["gate"], out, lse, dout, dq,
                                   dkv, dW, dg, wsb)
            evb[i][1].record(stream)
        torch.cuda.synchronize()
        t_bwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evb]))
        # the same backward given the forward's o_lat (kept from the latent attention call), which
        # it then reads instead of running the attention again
        o_lat = torch.empty((T, cfg.H, 512), dtype=torch.bfloat16, device="cuda")
        dsa.dsa_sparse_attention_latent(shape, dev["q"], dev["kv"], topk_idx, o_lat)
        for i in range(n_bwd):
            evb[i][0].record(stream)
            dsa.dsa_sparse_mla_bwd_saved(shape, dev["q"], dev["kv"], topk_idx, dev["W_UV"], dev["gate"], out, lse, o_lat,
                                         dout, dq, dkv, dW, dg, wsb)
            evb[i][1].record(stream)
        torch.cuda.synchronize()
        t_bwd_saved = float(np.mean([e[0].elapsed_time(e[1]) for e in evb]))
        del lse, dout, wsb, dq, dkv, dW, dg, o_lat
    cold = []
    if cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(cold_steps)]
        for i in range(cold_steps):
            flush.fill_(i & 0x7f)
            evc[i][0].record(stream)
            step()
            evc[i][1].record(stream)
        torch.cuda.synchronize()
        cold = [e[0].elapsed_time(e[1]) for e in evc]
        del flush
    t_idx = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    t_up = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))
    w = alg_work(cfg)
    frac = lambda flop, ms: flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    up_bytes = T * cfg.H * (512 + 128) * 2 + T * cfg.H * 2 + cfg.H * 512 * 128 * 2
    att_traffic = traffic_from_profile("k_sparse_mla", name)
    res = {
        "workload": name, "T": T, "docs": cfg.n_docs, "value": round(T * steps / el, 1),
        "ms_per_step": round(ms_step, 4),
        "index_topk_ms": round(t_idx, 4), "attention_ms": round(t_att, 4), "up_gate_ms": round(t_up, 4),
        # fractions of dense bf16 MFMA peak over the algorithmic flops of each stage
        "indexer_frac_scored_rows": round(frac(w["k_index_topk"], t_idx), 4),
        "attention_frac": round(frac(w["k_sparse_mla"], t_att), 4),
        "sparse_mla_frac_incl_up_gate": round(frac(w["k_sparse_mla"] + w["k_up_gate"], t_att + t_up), 4),
        "gather_logical_gbs": round(w["gather_bytes"] / (t_att * 1e-3) / 1e9, 1),
        "attention_hbm_gbs": round(att_traffic / (t_att * 1e-3) / 1e9, 1) if att_traffic else None,
        "up_gate_gbs": round(up_bytes / (t_up * 1e-3) / 1e9, 1),
        "path_tflops": round((w["k_index_topk"] + w["k_sparse_mla"] + w["k_up_gate"]) / (ms_step * 1e-3) / 1e12, 2),
        "warm_ms_per_step_median": round(float(np.median(warm_steps)), 4),
        "warm_ms_per_step_min": round(float(np.min(warm_steps)), 4),
        "cold_cache_ms_per_step_median": round(float(np.median(cold)), 4) if cold else None,
        "scored_pairs": w["scored_pairs"], "keff_sum": w["keff_sum"],
    }
    abs_bytes = T * cfg.H * (128 + 64 + 576) * 2 + cfg.H * 512 * 128 * 2
    op_flop = 2.0 * T * cfg.H * 128 * D_MODEL
    res.update({
        # adjacent steps: W_UK absorption (HBM-bound: bytes moved) and o_proj (an MFMA GEMM)
        "q_absorb_ms": round(t_abs, 4), "q_absorb_gbs": round(abs_bytes / (t_abs * 1e-3) / 1e9, 1),
        "o_proj_ms": round(t_op, 4), "o_proj_tflops": round(op_flop / (t_op * 1e-3) / 1e12, 1),
        "o_proj_frac": round(op_flop / (t_op * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    })
    if t_bwd is not None:
        # backward flops: S recompute (576), dP (512), dq (576), dkv (576 + 512) per selected key and head,
        # the forward attention again for o_lat (1,088), and do_lat and dW_UV (2 * 512 * 128 each) per row and head
        bwd_flop = 2.0 * cfg.H * (576 + 512 + 576 + 576 + 512 + 1088) * w["keff_sum"] + 2.0 * 2 * cfg.H * 512 * 128 * T
        res.update({"bwd_ms": round(t_bwd, 4), "bwd_tflops": round(bwd_flop / (t_bwd * 1e-3) / 1e12, 1),
                    "bwd_frac": round(bwd_flop / (t_bwd * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
        # with the forward's o_lat given: no attention recompute (its 1,088 flop per selected key and head)
        saved_flop = bwd_flop - 2.0 * cfg.H * 1088 * w["keff_sum"]
        res.update({"bwd_saved_olat_ms": round(t_bwd_saved, 4),
                    "bwd_saved_olat_frac": round(saved_flop / (t_bwd_saved * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)})
    if t_idx8 is not None:
        res.update({
            # FP8 indexer: the same algorithmic flops against the dense fp8 MFMA peak
            "index_topk_fp8_ms": round(t_idx8, 4),
            "indexer_fp8_frac_of_fp8_peak": round(w["k_index_topk"] / (t_idx8 * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4),
            "indexer_fp8_speedup_over_bf16": round(t_idx / t_idx8, 3),
            "fp8_indexer_path_tokens_per_s": round(T / ((t_idx8 + t_att + t_up) * 1e-3), 1),
            # key LayerNorm fused into the indexer's key-chunk loads: time, and whether its indices
            # equal the BF16 indexer's on every row
            "index_topk_fused_ln_ms": round(t_idx_ln, 4),
            "fused_ln_over_prologue": round(t_idx_ln / t_idx, 3),
            "fused_ln_indices_equal": ln_same,
        })
    log(f"[bench] {name}: {res['value']:.0f} tokens/s, {ms_step:.3f} ms/step (indexer {t_idx:.3f}, "
        f"attention {t_att:.3f}, up/gate {t_up:.3f} ms; fp8 indexer {t_idx8 if t_idx8 is None else round(t_idx8, 3)} ms)")
    del dev, ws, topk_idx, out
    torch.cuda.empty_cache()
    return (res, cfg, keys) if want_inputs else res


def roofline_of(res, cfg):
    """Roofline block of the stage with the longest time: achieved = algorithmic flops per launch /
    mean launch duration (HIP events), against the dense bf16 MFMA peak."""
    w = alg_work(cfg)
    stages = {"k_index_topk": res["index_topk_ms"], "k_sparse_mla": res["attention_ms"], "k_up_gate": res["up_gate_ms"]}
    kernel = max(stages, key=stages.get)
    ms = stages[kernel]
    if kernel == "k_up_gate":
        up_bytes = cfg.T * cfg.H * (512 + 128) * 2 + cfg.T * cfg.H * 2 + cfg.H * 512 * 128 * 2
        ach = up_bytes / (ms * 1e-3) / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic_from_profile(kernel, cfg.name),
                "alg_bytes_per_launch": up_bytes, "launch_ms": round(ms, 4)}
    ach = w[kernel] / (ms * 1e-3) / 1e12
    note = {
        "k_index_topk": "16,384 flop (2*H_I*d_I) per causal (query, key) pair of the rows with more than k causal "
                        "keys; the event interval also holds the key LayerNorm prologue",
        "k_sparse_mla": "208,896 flop (2*H*(576+512)) per selected key",
    }[kernel]
    return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4), "traffic": traffic_from_profile(kernel, cfg.name),
            "alg_flop_per_launch": w[kernel], "alg_flop_rule": note, "launch_ms": round(ms, 4)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="t131072", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--also", default="t4096,t8192,packed",
                    help="comma-separated workloads timed after the main one and reported as extra fields ('' for none)")
    ap.add_argument("--also-steps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=3,
                    help="steps timed one by one after a 512 MB cache flush (0: none)")
    ap.add_argument("--cpu-stride", type=int, default=0, help="row stride of the CPU sample (0: by workload)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write each kernel's HBM bytes per launch from rocprofv3 counter runs of --workload")
    ap.add_argument("--pmc-commands", default="", help="the profiling commands, recorded in the summary")
    ap.add_argument("--pmc-mfma-summary", metavar="MFMA_DIR",
                    help="write per-kernel MFMA counters from a rocprofv3 run of " + ", ".join(MFMA_COUNTERS))
    ap.add_argument("--stats-summary", nargs=2, metavar=("STATS_DIR", "BENCH_LOG"),
                    help="print a markdown summary of a rocprofv3 --kernel-trace --stats run of --workload")
    args = ap.parse_args()

    if args.stats_summary:
        stats_summary(args.stats_summary[0], args.workload, args.pmc_commands, args.stats_summary[1])
        return

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, workload=args.workload, commands=args.pmc_commands)
        return
    if args.pmc_mfma_summary:
        pmc_mfma_summary(args.pmc_mfma_summary, workload=args.workload, commands=args.pmc_commands)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    if args.copy_calibration:
        a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        b = torch.empty_like(a)
        for _ in range(COPY_LAUNCHES):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": COPY_BYTES, "copy_bytes_written": COPY_BYTES, "launches": COPY_LAUNCHES}))
        return

    main_res, cfg, keys = run_workload(args.workload, args.steps, args.warmup, args.cold_steps, want_inputs=True)
    roof = roofline_of(main_res, cfg)
    others = {}
    for name in [x for x in args.also.split(",") if x and x != args.workload]:
        others[name] = run_workload(name, args.also_steps, max(args.warmup, 10), 0)
    cpu = None
    if not args.no_cpu_baseline:
        stride = args.cpu_stride or (256 if cfg.T >= 65536 else 4)
        log(f"[bench] timing the CPU oracle on every {stride}th row")
        cpu = cpu_baseline(cfg, keys, stride)
    res = {
        "metric": METRIC, "value": main_res["value"], "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": main_res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[cfg.name], "T": cfg.T, "docs": cfg.n_docs, "topk": cfg.topk, "H": cfg.H,
                   "H_I": cfg.H_I, "d_I": cfg.d_I, "seed": cfg.seed},
        "roofline": roof, "stages": main_res, "other_workloads": others, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
