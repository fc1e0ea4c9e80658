"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Only number drawing and input preparation live here (no step of the method): the C library
``libtestgen.so`` draws counter-based values, so any single row of any tensor can be
regenerated on its own. Workload shapes and value distributions follow the validation sizes
of the Kimi-K3.1-Pro model-coverage page ("Validation and Training": 4,096- and 8,192-token
single documents), its long-context claim (model table, context length), and the MLA fields of
``KimiK3TextConfig`` on the kimi_k3 API index page (96 heads, kv_lora_rank 512, 64 unrotated
dims, v_head_dim 128).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtestgen.so")

# Tensor tags: each tensor draws from its own stream.
TAG_QI, TAG_KI, TAG_W, TAG_Q, TAG_KV, TAG_WUV, TAG_GATE, TAG_DOCLEN = 1, 2, 3, 4, 5, 6, 7, 8

D_L, D_V, D_O = 576, 512, 128


def build(force: bool = False) -> str:
    if force or not os.path.exists(_LIB_PATH):
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c11",
               os.path.join(_HERE, "testgen.c"), "-o", _LIB_PATH + ".tmp", "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


_lib = None
_lib_path = None  # a different build of the same source to load instead (the sanitizer test's)


def build_sanitized(path: str) -> str:
    """The generator built with AddressSanitizer and UndefinedBehaviorSanitizer (tests only; the
    process that loads it must preload the ASan runtime)."""
    cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fPIC", "-shared", "-fopenmp", "-std=c11", os.path.join(_HERE, "testgen.c"), "-o", path, "-lm"]
    subprocess.run(cmd, check=True)
    return path


def use_library(path: str) -> None:
    """Loads `path` (a build of testgen.c) instead of the default build."""
    global _lib, _lib_path
    _lib, _lib_path = None, path


def lib():
    global _lib
    if _lib is None:
        L = ctypes.CDLL(_lib_path if _lib_path else build())
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        L.tg_normal_bf16.argtypes = [u64, u64, i64, i64, ctypes.c_double, p]
        L.tg_uniform_bf16.argtypes = [u64, u64, i64, i64, ctypes.c_double, p]
        L.tg_uniform_int.argtypes = [u64, u64, i64, i64, i64, p]
        L.tg_rms_rows_bf16.argtypes = [p, i64, i64, ctypes.c_float]
        L.tg_words.argtypes = [u64, u64, i64, i64, p]
        L.tg_mix64_public.argtypes = [u64]
        L.tg_mix64_public.restype = u64
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    assert a.flags.c_contiguous
    return a.ctypes.data


def normal_bf16(seed: int, tag: int, start: int, n: int, scale: float, out: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16) if out is None else out
    lib().tg_normal_bf16(seed, tag, start, n, float(scale), _ptr(out))
    return out


def uniform_bf16(seed: int, tag: int, start: int, n: int, scale: float, out: np.ndarray | None = None) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16) if out is None else out
    lib().tg_uniform_bf16(seed, tag, start, n, float(scale), _ptr(out))
    return out


def uniform_int(seed: int, tag: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int64)
    lib().tg_uniform_int(seed, tag, n, lo, hi, _ptr(out))
    return out


def rms_rows_bf16(rows: np.ndarray, dim: int, eps: float = 1e-5) -> np.ndarray:
    lib().tg_rms_rows_bf16(_ptr(rows), rows.size // dim, dim, ctypes.c_float(eps))
    return rows


def bf16_to_f32(a: np.ndarray) -> np.ndarray:
    return (a.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 bit patterns with round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


@dataclass
class Config:
    """One synthetic workload. Distributions are scales of N(0,1) or U[0,1)."""
    name: str
    seed: int
    doc_lens: list
    topk: int
    H: int
    H_I: int
    d_I: int
    q_I_std: float = 1.0
    k_I_std: float = 1.0
    w_scale: float = 1.0          # w ~ U[0,1) * w_scale
    q_std: float = 1.0
    W_UV_std: float = 1.0
    gate_std: float = 1.0
    ln_eps: float = 1e-5
    softmax_scale: float = 1.0 / math.sqrt(192.0)
    extra: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return int(sum(self.doc_lens))

    @property
    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.doc_lens)]).astype(np.int32)

    @property
    def n_docs(self) -> int:
        return len(self.doc_lens)


def _packed_lengths(seed: int) -> list:
    return [int(x) for x in uniform_int(seed, TAG_DOCLEN, 8, 1024, 8192)]


def get_config(name: str) -> Config:
    big = dict(topk=2048, H=96, H_I=64, d_I=128, w_scale=1.0 / 8.0, q_std=1.0 / 24.0, W_UV_std=0.02)
    if name == "tiny":
        return Config("tiny", 1, [1024], topk=256, H=16, H_I=4, d_I=64, w_scale=0.5)
    if name == "t4096":
        return Config("t4096", 2, [4096], **big)
    if name == "t8192":
        return Config("t8192", 3, [8192], **big)
    if name == "packed":
        d = dict(big)
        d["q_std"] = 1.0
        return Config("packed", 4, _packed_lengths(4), **d)
    if name == "t131072":
        return Config("t131072", 5, [131072], **big)
    if name == "dense2048":
        return Config("dense2048", 6, [2048], **big)
    raise KeyError(name)


CONFIG_NAMES = ["tiny", "t4096", "t8192", "packed", "t131072", "dense2048"]


def _rows_of(seed: int, tag: int, rows, row_elems: int, scale: float, kind: str) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((len(rows), row_elems), dtype=np.uint16)
    # Consecutive runs of rows are drawn in one call.
    i = 0
    while i < len(rows):
        j = i
        while j + 1 < len(rows) and rows[j + 1] == rows[j] + 1:
            j += 1
        n = (j - i + 1) * row_elems
        start = int(rows[i]) * row_elems
        buf = out[i:j + 1].reshape(-1)
        if kind == "normal":
            normal_bf16(seed, tag, start, n, scale, buf)
        else:
            uniform_bf16(seed, tag, start, n, scale, buf)
        i = j + 1
    return out


def query_rows(cfg: Config, rows) -> dict:
    """Query-side tensors (q_I, w, q, gate) for the given global rows only."""
    return {
        "q_I": _rows_of(cfg.seed, TAG_QI, rows, cfg.H_I * cfg.d_I, cfg.q_I_std, "normal"),
        "w": _rows_of(cfg.seed, TAG_W, rows, cfg.H_I, cfg.w_scale, "uniform"),
        "q": _rows_of(cfg.seed, TAG_Q, rows, cfg.H * D_L, cfg.q_std, "normal"),
        "gate": _rows_of(cfg.seed, TAG_GATE, rows, cfg.H, cfg.gate_std, "normal"),
    }


def key_side(cfg: Config) -> dict:
    """Key-side tensors over all T tokens (k_I, kv) and the up-projection W_UV."""
    T = cfg.T
    k_I = normal_bf16(cfg.seed, TAG_KI, 0, T * cfg.d_I, cfg.k_I_std).reshape(T, cfg.d_I)
    kv = normal_bf16(cfg.seed, TAG_KV, 0, T * D_L, 1.0).reshape(T, D_L)
    rms_rows_bf16(kv, D_L)
    W_UV = normal_bf16(cfg.seed, TAG_WUV, 0, cfg.H * D_V * D_O, cfg.W_UV_std).reshape(cfg.H, D_V, D_O)
    return {"k_I": k_I, "kv": kv, "W_UV": W_UV}


def make_inputs(cfg: Config, with_query: bool = True) -> dict:
    """Every tensor of one workload, as bf16 bit patterns (numpy uint16)."""
    d = key_side(cfg)
    T = cfg.T
    if with_query:
        d["q_I"] = normal_bf16(cfg.seed, TAG_QI, 0, T * cfg.H_I * cfg.d_I, cfg.q_I_std).reshape(T, cfg.H_I, cfg.d_I)
        d["w"] = uniform_bf16(cfg.seed, TAG_W, 0, T * cfg.H_I, cfg.w_scale).reshape(T, cfg.H_I)
        d["q"] = normal_bf16(cfg.seed, TAG_Q, 0, T * cfg.H * D_L, cfg.q_std).reshape(T, cfg.H, D_L)
        d["gate"] = normal_bf16(cfg.seed, TAG_GATE, 0, T * cfg.H, cfg.gate_std).reshape(T, cfg.H)
    d["cu_seqlens"] = cfg.cu_seqlens
    return d
