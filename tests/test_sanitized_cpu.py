"""The CPU code of the checker (the oracle, oracle/oracle.cpp, and the input generator,
testgen/testgen.c) built with AddressSanitizer and UndefinedBehaviorSanitizer and run through every
oracle entry point on small packed inputs, in a child process that preloads the ASan runtime. Any
out-of-bounds access, use after free or undefined behaviour (signed overflow, misaligned or null
access, invalid shift) aborts the child, and the test fails with its report."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import sys
import numpy as np
sys.path.insert(0, sys.argv[1])
import oracle, testgen as tg
oracle.use_library(sys.argv[2])
tg.use_library(sys.argv[3])

# two packed documents, the second shorter than k (every key kept), a 16-head and a 96-head shape;
# every array passed is its own allocation (slices are copied), so a read past its end leaves it
for cfg in (tg.Config("san16", 31, [300, 90], topk=128, H=16, H_I=4, d_I=64, w_scale=0.5),
            tg.Config("san96", 32, [200, 61], topk=96, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                      W_UV_std=0.02)):
    inp = tg.make_inputs(cfg)
    T, H = cfg.T, cfg.H
    rows = np.arange(T)
    g = np.random.default_rng(3).uniform(0.5, 1.5, cfg.d_I).astype(np.float32)
    b = np.random.default_rng(4).uniform(-0.2, 0.2, cfg.d_I).astype(np.float32)
    LNk = oracle.key_layernorm(inp["k_I"], cfg.ln_eps, g, b)
    LNk = oracle.key_layernorm(inp["k_I"], cfg.ln_eps)
    idx, theta, keff = oracle.topk(rows, inp["q_I"], inp["w"], LNk, inp["cu_seqlens"], cfg.topk)
    oracle.index_scores(inp["q_I"][T - 1].copy(), inp["w"][T - 1].copy(), LNk, oracle.doc_begin(inp["cu_seqlens"], T - 1),
                        T - 1)
    oracle.index_score_scale(inp["q_I"][5].copy(), inp["w"][5].copy(), LNk, 0, 5)
    oracle.sparse_mla(rows, inp["q"], inp["kv"], idx, inp["W_UV"], inp["gate"], cfg.softmax_scale)
    oracle.sparse_mla_f32(rows, inp["q"], inp["kv"], idx, inp["W_UV"], inp["gate"], cfg.softmax_scale)
    oracle.dense_causal(rows[:40].copy(), inp["q"][:40].copy(), inp["kv"], inp["cu_seqlens"], inp["W_UV"],
                        inp["gate"][:40].copy(), cfg.softmax_scale)
    sink = np.linspace(-2.0, 2.0, H).astype(np.float32)
    gate_e = np.repeat(inp["gate"][:, :, None], 128, axis=2)
    oracle.sparse_mla_variant(rows, inp["q"], inp["kv"], idx, inp["W_UV"], gate_e, cfg.softmax_scale,
                              gate_per_dim=True, sink=sink)
    f64 = lambda a: tg.bf16_to_f32(a).astype(np.float64)
    dout = f64(tg.normal_bf16(cfg.seed, 70, 0, T * H * 128, 1.0).reshape(T, H, 128))
    oracle.sparse_mla_bwd(f64(inp["q"]), f64(inp["kv"]), idx, f64(inp["W_UV"]), f64(inp["gate"]),
                          cfg.softmax_scale, dout)
    oracle.sparse_mla_bwd(f64(inp["q"]), f64(inp["kv"]), idx, f64(inp["W_UV"]), f64(gate_e), cfg.softmax_scale,
                          dout, gate_per_dim=True, sink=sink.astype(np.float64))
    if cfg.d_I == 128:
        q8, eq = oracle.quantize_fp8_rows(inp["q_I"].reshape(T, cfg.H_I, cfg.d_I))
        k8, ek = oracle.quantize_fp8_rows(LNk)
        oracle.topk_fp8(rows, q8, eq, inp["w"], k8, ek, inp["cu_seqlens"], cfg.topk)
    q_nope = tg.normal_bf16(cfg.seed, 80, 0, T * H * 128, 1.0).reshape(T, H, 128)
    q_pe = tg.normal_bf16(cfg.seed, 81, 0, T * H * 64, 1.0).reshape(T, H, 64)
    W_UK = tg.normal_bf16(cfg.seed, 82, 0, H * 512 * 128, 0.02).reshape(H, 512, 128)
    oracle.q_absorb(q_nope, q_pe, W_UK, want_f64=True)
    x = tg.normal_bf16(cfg.seed, 83, 0, 8 * H * 128, 0.5).reshape(8, H * 128)
    W_o = tg.normal_bf16(cfg.seed, 84, 0, 256 * H * 128, 0.01).reshape(256, H * 128)
    oracle.o_proj(x, W_o, want_f64=True)
for c in range(256):
    oracle.e4m3_encode(oracle.e4m3_decode(c) if c not in (0x7F, 0xFF) else 0.0)
print("sanitized run complete", flush=True)
'''


def _asan_runtime():
    try:
        path = subprocess.check_output(["gcc", "-print-file-name=libasan.so"], text=True).strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("g++") is None or _asan_runtime() is None, reason="no g++ with an ASan runtime")
def test_oracle_and_generator_under_address_and_ub_sanitizers(tmp_path):
    sys.path.insert(0, ROOT)
    import oracle
    import testgen as tg
    olib = oracle.build_sanitized(str(tmp_path / "liboracle_san.so"))
    tlib = tg.build_sanitized(str(tmp_path / "libtestgen_san.so"))
    env = dict(os.environ, LD_PRELOAD=_asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT, olib, tlib], env=env, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0 and "sanitized run complete" in r.stdout, (r.returncode, r.stdout[-2000:],
                                                                         r.stderr[-4000:])
