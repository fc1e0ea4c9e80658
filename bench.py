"""Benchmark of the gated DSA forward hot path on one MI355X.

A step is one dsa_fused_fwd call (key LayerNorm, indexer + top-k, sparse latent attention, V
up-projection and gate) over one batch of synthetic input. The default workload is a single
4,096-token document (top-2048, 96 heads, indexer 64 heads x 128, latent 512+64), seed 2. All
inputs are resident in device memory before timing starts.

Prints one JSON line: throughput (query tokens/s), the roofline of the dominant kernel (the sparse
latent attention kernel at this size), and the CPU oracle timed on a bounded sample of rows.
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
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
ATTN_SRC = os.path.join(ROOT, "dsa_indexer_top_index_amd", "csrc", "k_mla.hip")
IDX_SRC = os.path.join(ROOT, "dsa_indexer_top_index_amd", "csrc", "k_index.hip")
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_sparse_attention_t4096.json")
COPY_BYTES = 1 << 30         # plain device copy used to scale the HBM byte counters
COPY_LAUNCHES = 5

WORKLOAD_TEXT = {
    "t4096": "single document T=4096, top-2048, 96 heads, indexer 64x128 with key LayerNorm, latent 512+64, "
             "W_UV 96x512x128, per-head gate",
    "t8192": "single document T=8192, top-2048, 96 heads, indexer 64x128, latent 512+64",
    "packed": "8 packed documents (lengths U[1024,8192], seed 4), top-2048, 96 heads, indexer 64x128, latent 512+64",
    "t131072": "single document T=131072, top-2048, 96 heads, indexer 64x128, latent 512+64",
    "tiny": "single document T=1024, top-256, 16 heads, indexer 4x64, latent 512+64",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def sum_keff(cfg):
    cu = cfg.cu_seqlens
    total = 0
    sel_pairs = 0
    all_pairs = 0
    for d in range(cfg.n_docs):
        L = int(cu[d + 1] - cu[d])
        n = np.arange(1, L + 1, dtype=np.int64)
        total += int(np.minimum(n, cfg.topk).sum())
        all_pairs += int(n.sum())
        sel_pairs += int(n[n > cfg.topk].sum())
    return total, all_pairs, sel_pairs


def src_hash(path):
    """Hash of a kernel source's code: comments and layout are left out, so that editing a comment
    does not invalidate counters taken on the same code."""
    import re
    t = open(path).read()
    t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
    t = re.sub(r"//[^\n]*", " ", t)
    return hashlib.sha256(" ".join(t.split()).encode()).hexdigest()[:16]


def traffic_from_profile(launch_bytes_alg):
    """HBM bytes per attention launch from the committed counter summary, if it still matches the kernel."""
    if not os.path.exists(PMC_FILE):
        return None
    d = json.load(open(PMC_FILE))
    if d.get("kernel_code_sha256_16") != src_hash(ATTN_SRC):
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


def _per_dispatch_kib(rows, name_part, counter):
    """Per-dispatch values of `counter` (KiB; summed over the counter's instances) for kernels
    whose name contains name_part."""
    per = {}
    for r in rows:
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernels matching {name_part!r}")
    return list(per.values())


def pmc_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, commands):
    """HBM bytes per attention launch from FETCH_SIZE / WRITE_SIZE counter runs, each scaled by
    what the same counter reads for a plain device copy of known size."""
    copy_name = "copyBuffer"
    cal_bytes = COPY_LAUNCHES * COPY_BYTES  # every copy dispatch of the calibration run together
    fv = _per_dispatch_kib(_counter_rows(fetch_dir), "k_sparse_mla", "FETCH_SIZE")
    wv = _per_dispatch_kib(_counter_rows(write_dir), "k_sparse_mla", "WRITE_SIZE")
    f_kib, nf = sum(fv) / len(fv), len(fv)
    w_kib, nw = sum(wv) / len(wv), len(wv)
    cf_kib = sum(_per_dispatch_kib(_counter_rows(cal_fetch_dir), copy_name, "FETCH_SIZE"))
    cw_kib = sum(_per_dispatch_kib(_counter_rows(cal_write_dir), copy_name, "WRITE_SIZE"))
    f_scale = cal_bytes / (cf_kib * 1024.0)
    w_scale = cal_bytes / (cw_kib * 1024.0)
    fetch_b = f_kib * 1024.0 * f_scale
    write_b = w_kib * 1024.0 * w_scale
    res = {
        "kernel": "k_sparse_mla", "workload": "t4096", "kernel_code_sha256_16": src_hash(ATTN_SRC),
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib, "dispatches": [nf, nw],
        "copy_calibration": {"bytes_each_way_all_copies": cal_bytes, "fetch_kib": cf_kib, "write_kib": cw_kib,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "hbm_fetch_bytes_per_launch": fetch_b, "hbm_write_bytes_per_launch": write_b,
        "hbm_bytes_per_launch": fetch_b + write_b, "commands": commands,
    }
    with open(PMC_FILE, "w") as fh:
        json.dump(res, fh, indent=1)
    print(json.dumps(res, indent=1))


MFMA_COUNTERS = ("SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
SIMDS = 256 * 4   # 256 CUs x 4 SIMDs
XCDS = 8


def pmc_mfma_summary(mfma_dir, commands):
    """Per-kernel MFMA counters of a bench run (t4096): bf16 MFMA flops the hardware executed
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) against the algorithmic flops, the rate both give over
    the dispatch time, and the share of SIMD cycles the matrix cores were busy."""
    import testgen as tg
    rows = _counter_rows(mfma_dir)
    cfg = tg.get_config("t4096")
    keff_sum, all_pairs, sel_pairs = sum_keff(cfg)
    alg = {
        "k_sparse_mla": 2.0 * cfg.H * (576 + 512) * keff_sum,
        "k_index_topk": 2.0 * cfg.H_I * cfg.d_I * all_pairs,   # every causal pair (the spec's count)
        "k_up_gate": 2.0 * cfg.H * 512 * 128 * cfg.T,
    }
    out = {"workload": "t4096", "counters": list(MFMA_COUNTERS), "simds": SIMDS, "kernels": {},
           "kernel_code_sha256_16": {"attention": src_hash(ATTN_SRC), "indexer": src_hash(IDX_SRC)},
           "commands": commands}
    for name, alg_flop in alg.items():
        per = {}
        for r in rows:
            if name in r["Kernel_Name"]:
                d = per.setdefault(r["Dispatch_Id"], {"t": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        ds = [d for d in per.values() if all(c in d for c in MFMA_COUNTERS)]
        if not ds:
            raise SystemExit(f"no complete counter rows for {name}")
        t = float(np.mean([d["t"] for d in ds]))
        mops = float(np.mean([d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds]))
        busy = float(np.mean([d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds]))
        gui = float(np.mean([d["GRBM_GUI_ACTIVE"] for d in ds]))
        hw_flop = mops * 512.0
        out["kernels"][name] = {
            "dispatches": len(ds), "mean_dispatch_us": t * 1e6,
            "hw_bf16_mfma_flop": hw_flop, "alg_flop": alg_flop, "hw_over_alg": hw_flop / alg_flop,
            "hw_tflops": hw_flop / t / 1e12, "alg_tflops": alg_flop / t / 1e12,
            "hw_frac_of_peak": hw_flop / t / 1e12 / PEAK_BF16_TFLOPS,
            "mfma_busy_cycles": busy, "grbm_gui_active": gui,
            # GRBM_GUI_ACTIVE comes summed over the XCDs; per-XCD active cycles x all SIMDs
            "mfma_busy_frac": busy / (gui / XCDS * SIMDS),
            "implied_clock_ghz": gui / XCDS / t / 1e9,
        }
    path = os.path.join(ROOT, "profiles", "pmc_mfma_t4096.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


def cpu_baseline(cfg, keys, stride):
    import oracle
    import testgen as tg

    rows = np.arange(cfg.T - 1, -1, -stride)[::-1]
    t0 = time.perf_counter()
    LNk = oracle.key_layernorm(keys["k_I"], cfg.ln_eps)
    qr = tg.query_rows(cfg, rows)
    gen_s = time.perf_counter() - t0
    t0 = time.perf_counter()
    idx, theta, keff = oracle.topk(rows, qr["q_I"].reshape(len(rows), cfg.H_I, cfg.d_I), qr["w"], LNk,
                                   cfg.cu_seqlens, cfg.topk)
    oracle.sparse_mla(rows, qr["q"].reshape(len(rows), cfg.H, 576), keys["kv"], idx, keys["W_UV"],
                      qr["gate"].reshape(len(rows), cfg.H), cfg.softmax_scale)
    el = time.perf_counter() - t0
    return {
        "value": len(rows) / el, "unit": "query tokens/s", "cores": oracle.num_threads(), "kind": "oracle",
        "sample": f"{len(rows)} of {cfg.T} rows (every {stride}th row, ending at the last), top-k + attention + "
                  f"up-projection + gate in the plain C++ oracle (FP32 scores, FP64 attention); LayerNorm of all "
                  f"keys ({gen_s:.1f}s with input drawing) excluded; {el:.1f}s wall",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="t4096", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cold-steps", type=int, default=10,
                    help="steps timed one by one after a 512 MB cache flush (0: none)")
    ap.add_argument("--cpu-stride", type=int, default=4)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"),
                    help="write the attention kernel's HBM bytes per launch from rocprofv3 counter runs")
    ap.add_argument("--pmc-commands", default="", help="the profiling commands, recorded in the summary")
    ap.add_argument("--pmc-mfma-summary", metavar="MFMA_DIR",
                    help="write per-kernel MFMA counters from a rocprofv3 run of " + ", ".join(MFMA_COUNTERS))
    args = ap.parse_args()

    if args.pmc_summary:
        pmc_summary(*args.pmc_summary, commands=args.pmc_commands)
        return
    if args.pmc_mfma_summary:
        pmc_mfma_summary(args.pmc_mfma_summary, commands=args.pmc_commands)
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

    import dsa_indexer_top_index_amd as dsa
    import testgen as tg
    from tests import gpu_util as gu

    cfg = tg.get_config(args.workload)
    log(f"[bench] generating {cfg.name} inputs (T={cfg.T})")
    keys, dev = gu.device_inputs(cfg)
    shape = gu.shape_of(cfg, dev.get("cu_seqlens"))
    ws = dsa.alloc_workspace(shape)
    T = cfg.T
    topk_idx = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, cfg.H, 128), dtype=torch.bfloat16, device="cuda")
    o_lat = torch.empty((T, cfg.H, 512), dtype=torch.bfloat16, device="cuda")

    def step():
        dsa.dsa_fused_fwd(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"],
                          topk_idx, out, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el / args.steps * 1e3
    value = T * args.steps / el

    # Per-stage launch durations, HIP events on the stream the kernels run on.
    stream = torch.cuda.current_stream()
    n_stage = max(args.steps, 3)
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
    warm_steps = [e[0].elapsed_time(e[3]) for e in ev]
    # The same steps with L2 and the Infinity Cache flushed before each one (a 512 MB write,
    # outside the timed interval): the cold-cache protocol.
    cold_steps = []
    if args.cold_steps > 0:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        evc = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.cold_steps)]
        for i in range(args.cold_steps):
            flush.fill_(i & 0x7f)
            evc[i][0].record(stream)
            step()
            evc[i][1].record(stream)
        torch.cuda.synchronize()
        cold_steps = [e[0].elapsed_time(e[1]) for e in evc]
        del flush
    t_idx = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    t_att = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    t_up = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))

    keff_sum, all_pairs, sel_pairs = sum_keff(cfg)
    att_flop = 2.0 * cfg.H * (576 + 512) * keff_sum          # QK^T over 576 dims + PV over 512, per selected key
    idx_flop_sel = 2.0 * cfg.H_I * cfg.d_I * sel_pairs       # scores the selection needs (rows with n_t > k)
    idx_flop_all = 2.0 * cfg.H_I * cfg.d_I * all_pairs       # every causal pair, short rows included
    up_flop = 2.0 * cfg.H * 512 * 128 * T
    up_bytes = T * cfg.H * (512 + 128) * 2 + T * cfg.H * 2 + cfg.H * 512 * 128 * 2
    att_tflops = att_flop / (t_att * 1e-3) / 1e12
    total_flop = att_flop + idx_flop_sel + up_flop
    traffic = traffic_from_profile(None)
    roof = {
        "kernel": "k_sparse_mla (dsa_sparse_attention_latent)",
        "bound": "mfma", "achieved": round(att_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
        "frac": round(att_tflops / PEAK_BF16_TFLOPS, 4),
        "traffic": traffic,
        "alg_flop_per_launch": att_flop, "launch_ms": round(t_att, 4),
    }
    mla_frac = (att_flop + up_flop) / ((t_att + t_up) * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
    stages = {
        "index_topk_ms": round(t_idx, 4), "attention_ms": round(t_att, 4), "up_gate_ms": round(t_up, 4),
        # fractions of bf16 MFMA peak: the indexer over every causal pair (16,384 flop each), and sparse
        # MLA over QK^T + PV of the selected keys plus W_UV (attention + up-projection/gate kernels)
        "indexer_frac_all_pairs": round(idx_flop_all / (t_idx * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "sparse_mla_frac_incl_up_gate": round(mla_frac, 4),
        "indexer_tflops_needed_rows": round(idx_flop_sel / (t_idx * 1e-3) / 1e12, 2),
        "indexer_tflops_all_pairs": round(idx_flop_all / (t_idx * 1e-3) / 1e12, 2),
        "indexer_frac_needed_rows": round(idx_flop_sel / (t_idx * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "up_gate_gbs": round(up_bytes / (t_up * 1e-3) / 1e9, 1),
        "path_tflops": round(total_flop / (ms_step * 1e-3) / 1e12, 2),
        # per-step times of the three kernels back to back (warm), and of whole steps after a cache flush
        "warm_ms_per_step_median": round(float(np.median(warm_steps)), 4),
        "warm_ms_per_step_min": round(float(np.min(warm_steps)), 4),
        "cold_cache_ms_per_step_median": round(float(np.median(cold_steps)), 4) if cold_steps else None,
        "cold_cache_ms_per_step_min": round(float(np.min(cold_steps)), 4) if cold_steps else None,
    }
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a row sample")
        cpu = cpu_baseline(cfg, keys, args.cpu_stride)
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "query tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[cfg.name], "T": T, "docs": cfg.n_docs, "topk": cfg.topk, "H": cfg.H,
                   "H_I": cfg.H_I, "d_I": cfg.d_I, "seed": cfg.seed},
        "roofline": roof, "stages": stages, "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
