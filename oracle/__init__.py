"""Python access to the CPU oracle (``oracle.cpp``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the package smoke check and by the
benchmark's CPU-baseline leg. The product path never imports this module.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.cpp")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

# -ffp-contract=off: no fused multiply-adds, so every sum is evaluated as written. The parity build
# targets the generic x86-64 ISA so that the library built here also runs on other hosts.
CXXFLAGS = ["-O2", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]
# The CPU-baseline build: the same source and floating-point semantics, optimised for the host that
# runs it (built there, into a temporary directory, each time it is timed).
NATIVE_CXXFLAGS = ["-O3", "-march=native", "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["g++", *CXXFLAGS, _SRC, "-o", _LIB_PATH + ".tmp"], check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None


def build_native() -> str:
    """Compiles the oracle with NATIVE_CXXFLAGS for this host into a fresh temporary directory."""
    import tempfile
    d = tempfile.mkdtemp(prefix="oracle_native_")
    path = os.path.join(d, "liboracle_native.so")
    subprocess.run(["g++", *NATIVE_CXXFLAGS, _SRC, "-o", path], check=True)
    return path


# The sanitizer build (tests only): AddressSanitizer and UndefinedBehaviorSanitizer, stopping at the
# first report. The process that loads it must preload the ASan runtime.
SANITIZE_CXXFLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                     "-std=c++17", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared"]


def build_sanitized(path: str) -> str:
    subprocess.run(["g++", *SANITIZE_CXXFLAGS, _SRC, "-o", path], check=True)
    return path


def use_library(path: str):
    """Switches this module to another build of the same source (the sanitizer test's)."""
    global _lib
    _lib = _load(path)
    return _lib


def use_native():
    """Switches this module to a host-optimised build of the same source (for timing only)."""
    global _lib
    _lib = _load(build_native())
    return _lib


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = _load(_LIB_PATH)
    return _lib


def _load(path):
    L = ctypes.CDLL(path)
    p, i32, i64, d = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    L.oracle_num_threads.restype = ctypes.c_int
    L.oracle_doc_begin.argtypes = [p, i32, i64]
    L.oracle_doc_begin.restype = i64
    L.oracle_key_layernorm.argtypes = [p, i64, i32, p, p, d, p, p]
    L.oracle_index_scores.argtypes = [p, p, i32, i32, p, i64, i64, p]
    L.oracle_index_score_scale.argtypes = [p, p, i32, i32, p, i64, i64, p]
    L.oracle_topk.argtypes = [i64, p, p, p, i32, i32, p, p, i32, i32, p, p, p]
    L.oracle_sparse_mla.argtypes = [i64, p, p, p, i64, p, i32, p, p, i32, d, p, p, p, p, p]
    L.oracle_dense_causal.argtypes = [i64, p, p, p, i64, p, i32, p, p, i32, d, p]
    L.oracle_sparse_mla_f32.argtypes = [i64, p, p, p, i64, p, i32, p, p, i32, d, p]
    L.oracle_sparse_mla_variant.argtypes = [i64, p, p, p, i64, p, i32, p, p, i32, d, i32, p, p, p, p, p, p]
    L.oracle_quantize_fp8_rows.argtypes = [p, i64, i32, p, p]
    L.oracle_q_absorb.argtypes = [i64, p, p, p, i32, p, p]
    L.oracle_o_proj.argtypes = [i64, p, p, i32, i32, p, p]
    L.oracle_sparse_mla_f64in.argtypes = [i64, p, p, i64, p, i32, p, p, i32, d, p, p]
    L.oracle_sparse_mla_f64in_variant.argtypes = [i64, p, p, i64, p, i32, p, p, i32, d, i32, p, p, p]
    L.oracle_sparse_mla_bwd_variant.argtypes = [i64, p, p, i64, p, i32, p, p, i32, d, i32, p, p, p, p, p, p, p]
    L.oracle_sparse_mla_bwd.argtypes = [i64, p, p, i64, p, i32, p, p, i32, d, p, p, p, p, p]
    L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.oracle_e4m3_decode.restype = d
    L.oracle_e4m3_encode.argtypes = [d]
    L.oracle_e4m3_encode.restype = ctypes.c_uint8
    L.oracle_fp8_scale_exponent.argtypes = [d]
    L.oracle_fp8_scale_exponent.restype = i32
    L.oracle_index_scores_fp8.argtypes = [p, p, p, i32, i32, p, p, i64, i64, p]
    L.oracle_topk_fp8.argtypes = [i64, p, p, p, p, i32, i32, p, p, p, i32, i32, p, p, p]
    return L


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data


def _opt(a, dtype):
    if a is None:
        return None, None
    return _c(a, dtype)


def key_layernorm(k_I, eps=1e-5, gamma=None, beta=None, want_pre=False):
    k_I, pk = _c(k_I, np.uint16)
    T, d_I = k_I.shape
    out = np.empty_like(k_I)
    pre = np.empty((T, d_I), dtype=np.float64) if want_pre else None
    g, pg = _opt(gamma, np.float32)
    b, pb = _opt(beta, np.float32)
    lib().oracle_key_layernorm(pk, T, d_I, pg, pb, eps, out.ctypes.data, pre.ctypes.data if want_pre else None)
    return (out, pre) if want_pre else out


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def doc_begin(cu_seqlens, t):
    cu, pc = _c(cu_seqlens, np.int32)
    return int(lib().oracle_doc_begin(pc, len(cu) - 1, t))


def index_scores(qI_row, w_row, LNk, s0, s1):
    """FP32 scores of one query (qI_row [H_I,d_I], w_row [H_I]) over keys s0..s1 inclusive."""
    q, pq = _c(qI_row, np.uint16)
    w, pw = _c(w_row, np.uint16)
    L, pl = _c(LNk, np.uint16)
    H_I, d_I = q.shape
    out = np.empty(s1 - s0 + 1, dtype=np.float32)
    lib().oracle_index_scores(pq, pw, H_I, d_I, pl, s0, s1, out.ctypes.data)
    return out


def index_score_scale(qI_row, w_row, LNk, s0, s1):
    q, pq = _c(qI_row, np.uint16)
    w, pw = _c(w_row, np.uint16)
    L, pl = _c(LNk, np.uint16)
    H_I, d_I = q.shape
    out = np.empty(s1 - s0 + 1, dtype=np.float64)
    lib().oracle_index_score_scale(pq, pw, H_I, d_I, pl, s0, s1, out.ctypes.data)
    return out


def topk(rows, qI_rows, w_rows, LNk, cu_seqlens, k):
    """Top-k indices of the listed global rows; returns (idx [n,k] int32, theta [n], keff [n])."""
    rows, pr = _c(rows, np.int64)
    q, pq = _c(qI_rows, np.uint16)
    w, pw = _c(w_rows, np.uint16)
    L, pl = _c(LNk, np.uint16)
    cu, pc = _c(cu_seqlens, np.int32)
    n = len(rows)
    H_I, d_I = q.shape[-2], q.shape[-1]
    idx = np.empty((n, k), dtype=np.int32)
    theta = np.empty(n, dtype=np.float32)
    keff = np.empty(n, dtype=np.int32)
    lib().oracle_topk(n, pr, pq, pw, H_I, d_I, pl, pc, len(cu) - 1, k, idx.ctypes.data, theta.ctypes.data,
                      keff.ctypes.data)
    return idx, theta, keff


def sparse_mla(rows, q_rows, kv, idx, W_UV, gate_rows, scale):
    """Returns dict with o_pre, out (float64), out_bf16, lse, psum for the listed rows."""
    rows, pr = _c(rows, np.int64)
    q, pq = _c(q_rows, np.uint16)
    kvc, pkv = _c(kv, np.uint16)
    ix, pi = _c(idx, np.int32)
    W, pw = _c(W_UV, np.uint16)
    g, pg = _c(gate_rows, np.uint16)
    n, H = q.shape[0], q.shape[1]
    k = ix.shape[1]
    res = {
        "o_pre": np.empty((n, H, 128)), "out": np.empty((n, H, 128)),
        "out_bf16": np.empty((n, H, 128), dtype=np.uint16), "lse": np.empty((n, H)), "psum": np.empty((n, H)),
    }
    lib().oracle_sparse_mla(n, pr, pq, pkv, kvc.shape[0], pi, k, pw, pg, H, scale,
                            res["o_pre"].ctypes.data, res["out"].ctypes.data, res["out_bf16"].ctypes.data,
                            res["lse"].ctypes.data, res["psum"].ctypes.data)
    return res


def sparse_mla_variant(rows, q_rows, kv, idx, W_UV, gate, scale, gate_per_dim=False, sink=None):
    """Gate/sink variants: gate [n,H] or, with gate_per_dim, [n,H,128]; sink [H] float (natural-log
    units) or None. Returns the same dict as sparse_mla."""
    rows, pr = _c(rows, np.int64)
    q, pq = _c(q_rows, np.uint16)
    kvc, pkv = _c(kv, np.uint16)
    ix, pi = _c(idx, np.int32)
    W, pw = _c(W_UV, np.uint16)
    g, pg = _c(gate, np.uint16)
    sk, ps = _opt(sink, np.float64)
    n, H = q.shape[0], q.shape[1]
    assert g.size == n * H * (128 if gate_per_dim else 1)
    res = {
        "o_pre": np.empty((n, H, 128)), "out": np.empty((n, H, 128)),
        "out_bf16": np.empty((n, H, 128), dtype=np.uint16), "lse": np.empty((n, H)), "psum": np.empty((n, H)),
    }
    lib().oracle_sparse_mla_variant(n, pr, pq, pkv, kvc.shape[0], pi, ix.shape[1], pw, pg, H, scale,
                                    1 if gate_per_dim else 0, ps, res["o_pre"].ctypes.data, res["out"].ctypes.data,
                                    res["out_bf16"].ctypes.data, res["lse"].ctypes.data, res["psum"].ctypes.data)
    return res


def sparse_mla_f32(rows, q_rows, kv, idx, W_UV, gate_rows, scale):
    """The attention, up-projection and gate accumulated in float (timing only); returns out [n,H,128]."""
    rows, pr = _c(rows, np.int64)
    q, pq = _c(q_rows, np.uint16)
    kvc, pkv = _c(kv, np.uint16)
    ix, pi = _c(idx, np.int32)
    W, pw = _c(W_UV, np.uint16)
    g, pg = _c(gate_rows, np.uint16)
    n, H = q.shape[0], q.shape[1]
    out = np.empty((n, H, 128))
    lib().oracle_sparse_mla_f32(n, pr, pq, pkv, kvc.shape[0], pi, ix.shape[1], pw, pg, H, scale, out.ctypes.data)
    return out


def dense_causal(rows, q_rows, kv, cu_seqlens, W_UV, gate_rows, scale):
    rows, pr = _c(rows, np.int64)
    q, pq = _c(q_rows, np.uint16)
    kvc, pkv = _c(kv, np.uint16)
    cu, pc = _c(cu_seqlens, np.int32)
    W, pw = _c(W_UV, np.uint16)
    g, pg = _c(gate_rows, np.uint16)
    n, H = q.shape[0], q.shape[1]
    out = np.empty((n, H, 128))
    lib().oracle_dense_causal(n, pr, pq, pkv, kvc.shape[0], pc, len(cu) - 1, pw, pg, H, scale, out.ctypes.data)
    return out


def forward(cfg, inputs, rows):
    """Whole path for the listed rows of a testgen workload: (idx, theta, keff, mla-dict)."""
    LNk = key_layernorm(inputs["k_I"], cfg.ln_eps)
    rows = np.asarray(rows, dtype=np.int64)
    idx, theta, keff = topk(rows, inputs["q_I"][rows], inputs["w"][rows], LNk, inputs["cu_seqlens"], cfg.topk)
    mla = sparse_mla(rows, inputs["q"][rows], inputs["kv"], idx, inputs["W_UV"], inputs["gate"][rows],
                     cfg.softmax_scale)
    return idx, theta, keff, mla


# ---- FP8 indexer (E4M3 with power-of-two row scales)

def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def fp8_scale_exponent(amax: float) -> int:
    return int(lib().oracle_fp8_scale_exponent(float(amax)))


def quantize_fp8_rows(x):
    """x: bf16 bits [..., d]; returns (E4M3 codes [..., d] uint8, scale exponents [...] int32)."""
    x, px = _c(x, np.uint16)
    d = x.shape[-1]
    n = x.size // d
    q8 = np.empty(x.shape, dtype=np.uint8)
    e = np.empty(x.shape[:-1], dtype=np.int32)
    lib().oracle_quantize_fp8_rows(px, n, d, q8.ctypes.data, e.ctypes.data)
    return q8, e


def index_scores_fp8(q8_row, eq, w_row, k8, ek, s0, s1):
    q, pq = _c(q8_row, np.uint8)
    e, pe = _c(eq, np.int32)
    w, pw = _c(w_row, np.uint16)
    K, pk = _c(k8, np.uint8)
    E, pE = _c(ek, np.int32)
    H_I, d_I = q.shape
    out = np.empty(s1 - s0 + 1, dtype=np.float32)
    lib().oracle_index_scores_fp8(pq, pe, pw, H_I, d_I, pk, pE, s0, s1, out.ctypes.data)
    return out


def topk_fp8(rows, q8_rows, eq_rows, w_rows, k8, ek, cu_seqlens, k):
    """FP8-indexer top-k of the listed global rows; returns (idx [n,k] int32, theta [n], keff [n])."""
    rows, pr = _c(rows, np.int64)
    q, pq = _c(q8_rows, np.uint8)
    e, pe = _c(eq_rows, np.int32)
    w, pw = _c(w_rows, np.uint16)
    K, pk = _c(k8, np.uint8)
    E, pE = _c(ek, np.int32)
    cu, pc = _c(cu_seqlens, np.int32)
    n = len(rows)
    H_I, d_I = q.shape[-2], q.shape[-1]
    idx = np.empty((n, k), dtype=np.int32)
    theta = np.empty(n, dtype=np.float32)
    keff = np.empty(n, dtype=np.int32)
    lib().oracle_topk_fp8(n, pr, pq, pe, pw, H_I, d_I, pk, pE, pc, len(cu) - 1, k, idx.ctypes.data,
                          theta.ctypes.data, keff.ctypes.data)
    return idx, theta, keff


# ---- adjacent steps

def q_absorb(q_nope, q_pe, W_UK, want_f64=False):
    """q_nope [n,H,128], q_pe [n,H,64], W_UK [H,512,128] (bf16 bits) -> q [n,H,576] bf16 bits
    (and the unrounded latent part [n,H,512] in float64)."""
    qn, pn = _c(q_nope, np.uint16)
    qp, pp = _c(q_pe, np.uint16)
    W, pw = _c(W_UK, np.uint16)
    n, H = qn.shape[0], qn.shape[1]
    out = np.empty((n, H, 576), dtype=np.uint16)
    f = np.empty((n, H, 512)) if want_f64 else None
    lib().oracle_q_absorb(n, pn, pp, pw, H, out.ctypes.data, f.ctypes.data if want_f64 else None)
    return (out, f) if want_f64 else out


def o_proj(x, W_o, want_f64=False):
    """x [n,K], W_o [N,K] (bf16 bits) -> y [n,N] bf16 bits (and the unrounded values in float64)."""
    xc, px = _c(x, np.uint16)
    W, pw = _c(W_o, np.uint16)
    n, K = xc.shape[0], int(np.prod(xc.shape[1:]))
    N = W.shape[0]
    assert W.shape[1] == K
    y = np.empty((n, N), dtype=np.uint16)
    f = np.empty((n, N)) if want_f64 else None
    lib().oracle_o_proj(n, px, pw, K, N, y.ctypes.data, f.ctypes.data if want_f64 else None)
    return (y, f) if want_f64 else y


# ---- backward (inputs as float64 arrays; bf16 inputs are converted exactly by the caller)

def sparse_mla_f64in(q, kv, idx, W_UV, gate, scale, gate_per_dim=False, sink=None):
    """Forward with double inputs: q [n,H,576], kv [T,576], idx [n,k], W_UV [H,512,128], gate [n,H]
    (or [n,H,128] with gate_per_dim), sink [H] or None. Returns (out [n,H,128], lse [n,H])."""
    q, pq = _c(q, np.float64)
    kvc, pkv = _c(kv, np.float64)
    ix, pi = _c(idx, np.int32)
    W, pw = _c(W_UV, np.float64)
    g, pg = _c(gate, np.float64)
    n, H = q.shape[0], q.shape[1]
    out = np.empty((n, H, 128))
    lse = np.empty((n, H))
    if not gate_per_dim and sink is None:
        lib().oracle_sparse_mla_f64in(n, pq, pkv, kvc.shape[0], pi, ix.shape[1], pw, pg, H, scale, out.ctypes.data,
                                      lse.ctypes.data)
    else:
        sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
        lib().oracle_sparse_mla_f64in_variant(n, pq, pkv, kvc.shape[0], pi, ix.shape[1], pw, pg, H, scale,
                                              1 if gate_per_dim else 0, None if sk is None else sk.ctypes.data,
                                              out.ctypes.data, lse.ctypes.data)
    return out, lse


def sparse_mla_bwd(q, kv, idx, W_UV, gate, scale, dout, gate_per_dim=False, sink=None):
    """Gradients of L = sum(dout * out): returns dict dq [n,H,576], dkv [T,576], dW_UV [H,512,128], dgate
    [n,H] (or [n,H,128] with gate_per_dim) and, with a sink [H], dsink [H]."""
    q, pq = _c(q, np.float64)
    kvc, pkv = _c(kv, np.float64)
    ix, pi = _c(idx, np.int32)
    W, pw = _c(W_UV, np.float64)
    g, pg = _c(gate, np.float64)
    do, pd = _c(dout, np.float64)
    n, H = q.shape[0], q.shape[1]
    T = kvc.shape[0]
    res = {"dq": np.empty((n, H, 576)), "dkv": np.zeros((T, 576)), "dW_UV": np.zeros((H, 512, 128)),
           "dgate": np.empty((n, H, 128) if gate_per_dim else (n, H))}
    if not gate_per_dim and sink is None:
        lib().oracle_sparse_mla_bwd(n, pq, pkv, T, pi, ix.shape[1], pw, pg, H, scale, pd, res["dq"].ctypes.data,
                                    res["dkv"].ctypes.data, res["dW_UV"].ctypes.data, res["dgate"].ctypes.data)
        return res
    sk = None if sink is None else np.ascontiguousarray(sink, dtype=np.float64)
    if sk is not None:
        res["dsink"] = np.zeros(H)
    lib().oracle_sparse_mla_bwd_variant(n, pq, pkv, T, pi, ix.shape[1], pw, pg, H, scale, 1 if gate_per_dim else 0,
                                        None if sk is None else sk.ctypes.data, pd, res["dq"].ctypes.data,
                                        res["dkv"].ctypes.data, res["dW_UV"].ctypes.data, res["dgate"].ctypes.data,
                                        None if sk is None else res["dsink"].ctypes.data)
    return res
