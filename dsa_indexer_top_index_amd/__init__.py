"""Python binding of libdsa.so (include/dsa.h): argument marshalling only.

Every step of the path runs in the library's HIP kernels; PyTorch provides device memory and the
current stream. There is no fallback: if the library is missing, importing the entry points
raises.

Entry points (same names as the C ABI):
  dsa_workspace_size(shape) -> int
  dsa_check_shape(shape) -> int status
  dsa_index_topk(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None)
  dsa_sparse_mla_fwd(shape, q, kv, topk_idx, W_UV, gate, out, workspace, lse=None)
  dsa_sparse_attention_latent(shape, q, kv, topk_idx, o_lat, lse=None)
  dsa_up_gate(shape, o_lat, W_UV, gate, out)
  dsa_fused_fwd(shape, q_I, k_I, w, q, kv, W_UV, gate, topk_idx, out, workspace,
                ln_gamma=None, ln_beta=None, lse=None)
  dsa_index_topk_noalloc(shape, q_I, k_I, w, topk_idx, ln_gamma=None, ln_beta=None)
  dsa_index_topk_fp8(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None)
  dsa_index_topk_fused_ln(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None)
  dsa_quantize_fp8(x, q8, scale)
  dsa_q_absorb(shape, q_nope, q_pe, W_UK, q)
  dsa_o_proj(shape, x, W_o, y)
  dsa_sparse_mla_bwd(shape, q, kv, topk_idx, W_UV, gate, out, lse, dout, dq, dkv, dW_UV, dgate, workspace)
  dsa_sparse_mla_fwd_ex / dsa_fused_fwd_ex: the same with gate_per_dim=False, sink=None (elementwise
  gate [rows,H,128] and per-head sink logits [H] float32)
  dsa_sparse_mla_bwd_ex(shape, ..., dgate, workspace, gate_per_dim=False, sink=None, dsink=None)
  dsa_sparse_attention_latent_ex(shape, q, kv, topk_idx, o_lat, lse=None, sink=None)
  dsa_sparse_mla_bwd_saved(shape, q, kv, topk_idx, W_UV, gate, out, lse, o_lat, dout, dq, dkv, dW_UV, dgate,
                           workspace, gate_per_dim=False, sink=None, dsink=None)
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_LAUNCH, DSA_ERR_TOO_LARGE = range(6)
NOALLOC_MAX_T, NOALLOC_MAX_DOCS = 131072, 64   # limits of dsa_index_topk_noalloc


class DsaError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} (status {status})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("T", ctypes.c_int32),
        ("n_docs", ctypes.c_int32),
        ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
        ("cu_seqlens_dev", ctypes.c_void_p),
        ("q_begin", ctypes.c_int32),
        ("q_end", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("H_I", ctypes.c_int32),
        ("d_I", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("ln_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float),
    ]


class Variant(ctypes.Structure):
    """dsa_mla_variant: elementwise gate and/or per-head sink (include/dsa.h)."""
    _fields_ = [("gate_per_dim", ctypes.c_int32), ("sink", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER(Shape)
        v = ctypes.c_void_p
        L.dsa_status_string.argtypes = [ctypes.c_int]
        L.dsa_status_string.restype = ctypes.c_char_p
        L.dsa_check_shape.argtypes = [P]
        L.dsa_check_shape.restype = ctypes.c_int
        L.dsa_workspace_size.argtypes = [P]
        L.dsa_workspace_size.restype = ctypes.c_size_t
        L.dsa_index_topk.argtypes = [P, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_index_topk.restype = ctypes.c_int
        L.dsa_sparse_mla_fwd.argtypes = [P, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_sparse_mla_fwd.restype = ctypes.c_int
        L.dsa_sparse_attention_latent.argtypes = [P, v, v, v, v, v, v]
        L.dsa_sparse_attention_latent.restype = ctypes.c_int
        L.dsa_up_gate.argtypes = [P, v, v, v, v, v]
        L.dsa_up_gate.restype = ctypes.c_int
        L.dsa_fused_fwd.argtypes = [P, v, v, v, v, v, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_fused_fwd.restype = ctypes.c_int
        L.dsa_index_topk_noalloc.argtypes = [P, v, v, v, v, v, v, v]
        L.dsa_index_topk_noalloc.restype = ctypes.c_int
        L.dsa_index_topk_fp8.argtypes = [P, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_index_topk_fp8.restype = ctypes.c_int
        L.dsa_index_topk_fused_ln.argtypes = [P, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_index_topk_fused_ln.restype = ctypes.c_int
        L.dsa_quantize_fp8.argtypes = [ctypes.c_int64, v, v, v, v]
        L.dsa_quantize_fp8.restype = ctypes.c_int
        L.dsa_bwd_workspace_size.argtypes = [P]
        L.dsa_bwd_workspace_size.restype = ctypes.c_size_t
        L.dsa_sparse_mla_bwd.argtypes = [P, v, v, v, v, v, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_sparse_mla_bwd.restype = ctypes.c_int
        L.dsa_o_proj.argtypes = [P, v, v, ctypes.c_int32, v, v]
        L.dsa_o_proj.restype = ctypes.c_int
        L.dsa_q_absorb.argtypes = [P, v, v, v, v, v]
        L.dsa_q_absorb.restype = ctypes.c_int
        V = ctypes.POINTER(Variant)
        L.dsa_sparse_mla_fwd_ex.argtypes = [P, V, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_sparse_mla_fwd_ex.restype = ctypes.c_int
        L.dsa_fused_fwd_ex.argtypes = [P, V, v, v, v, v, v, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_fused_fwd_ex.restype = ctypes.c_int
        L.dsa_sparse_mla_bwd_ex.argtypes = [P, V, v, v, v, v, v, v, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_sparse_mla_bwd_ex.restype = ctypes.c_int
        L.dsa_sparse_attention_latent_ex.argtypes = [P, V, v, v, v, v, v, v]
        L.dsa_sparse_attention_latent_ex.restype = ctypes.c_int
        L.dsa_sparse_mla_bwd_saved.argtypes = [P, V, v, v, v, v, v, v, v, v, v, v, v, v, v, v, v, ctypes.c_size_t, v]
        L.dsa_sparse_mla_bwd_saved.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def make_shape(T, topk, H_I, d_I, H, cu_seqlens=None, cu_seqlens_dev=None, q_begin=0, q_end=0,
               ln_eps=1e-5, softmax_scale=1.0 / math.sqrt(192.0)) -> Shape:
    """cu_seqlens: host sequence of n_docs+1 ints (None = one document);
    cu_seqlens_dev: the same values as an int32 device tensor (required when n_docs > 1)."""
    s = Shape()
    s.T = int(T)
    if cu_seqlens is None:
        s.n_docs = 1
        s.cu_seqlens_host = None
        s._cu_keep = None
    else:
        arr = (ctypes.c_int32 * len(cu_seqlens))(*[int(x) for x in cu_seqlens])
        s._cu_keep = arr
        s.n_docs = len(cu_seqlens) - 1
        s.cu_seqlens_host = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    if cu_seqlens_dev is not None:
        _check(cu_seqlens_dev, torch.int32, "cu_seqlens_dev")
        s._cu_dev_keep = cu_seqlens_dev
        s.cu_seqlens_dev = cu_seqlens_dev.data_ptr()
    else:
        s.cu_seqlens_dev = None
    s.q_begin, s.q_end = int(q_begin), int(q_end)
    s.topk, s.H_I, s.d_I, s.H = int(topk), int(H_I), int(d_I), int(H)
    s.ln_eps, s.softmax_scale = float(ln_eps), float(softmax_scale)
    return s


def _check(t, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be in device memory")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _p(t, dtype, name, optional=False, numel=None):
    """Device pointer of t after dtype/device/contiguity checks and, if numel is given, a size check:
    an undersized buffer would otherwise become an out-of-bounds device access."""
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    _check(t, dtype, name)
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} has {t.numel()} elements, the shape needs {numel}")
    return t.data_ptr()


def _rows(shape: Shape) -> int:
    return (shape.q_end or shape.T) - shape.q_begin


def _sizes(shape: Shape) -> dict:
    """Element counts of every tensor argument for this shape (include/dsa.h)."""
    r, T = _rows(shape), shape.T
    return {
        "q_I": r * shape.H_I * shape.d_I, "k_I": T * shape.d_I, "w": r * shape.H_I, "ln": shape.d_I,
        "topk_idx": r * shape.topk, "q": r * shape.H * 576, "kv": T * 576, "W_UV": shape.H * 512 * 128,
        "gate": r * shape.H, "out": r * shape.H * 128, "lse": r * shape.H, "o_lat": r * shape.H * 512,
    }


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _raise(st, where):
    if st != DSA_OK:
        raise DsaError(st, where)


def dsa_check_shape(shape: Shape) -> int:
    return lib().dsa_check_shape(ctypes.byref(shape))


def dsa_workspace_size(shape: Shape) -> int:
    return int(lib().dsa_workspace_size(ctypes.byref(shape)))


def alloc_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    n = dsa_workspace_size(shape)
    if n == 0:
        _raise(dsa_check_shape(shape), "dsa_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dsa_index_topk(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None):
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_index_topk(
        ctypes.byref(shape), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]),
        _p(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _raise(st, "dsa_index_topk")


def dsa_index_topk_fp8(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None):
    """dsa_index_topk with the FP8 indexer (E4M3 operands, power-of-two row scales; H_I=64, d_I=128)."""
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_index_topk_fp8(
        ctypes.byref(shape), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]),
        _p(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _raise(st, "dsa_index_topk_fp8")


def dsa_index_topk_fused_ln(shape, q_I, k_I, w, topk_idx, workspace, ln_gamma=None, ln_beta=None):
    """dsa_index_topk with the key LayerNorm fused into the indexer's key-chunk loads (H_I=64, d_I=128;
    k_I 16-byte aligned). Same results."""
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_index_topk_fused_ln(
        ctypes.byref(shape), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]),
        _p(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _raise(st, "dsa_index_topk_fused_ln")


def dsa_q_absorb(shape, q_nope, q_pe, W_UK, q):
    """q [rows,H,576] from q_nope [rows,H,128], q_pe [rows,H,64] and W_UK [H,512,128] (all bf16)."""
    bf, r, H = torch.bfloat16, _rows(shape), shape.H
    st = lib().dsa_q_absorb(ctypes.byref(shape), _p(q_nope, bf, "q_nope", numel=r * H * 128),
                            _p(q_pe, bf, "q_pe", numel=r * H * 64), _p(W_UK, bf, "W_UK", numel=H * 512 * 128),
                            _p(q, bf, "q", numel=r * H * 576), _stream())
    _raise(st, "dsa_q_absorb")


def alloc_bwd_workspace(shape: Shape, device="cuda") -> torch.Tensor:
    n = int(lib().dsa_bwd_workspace_size(ctypes.byref(shape)))
    if n == 0:
        _raise(dsa_check_shape(shape), "dsa_bwd_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def dsa_sparse_mla_bwd(shape, q, kv, topk_idx, W_UV, gate, out, lse, dout, dq, dkv, dW_UV, dgate, workspace):
    """Gradients of sum(dout * out) for dsa_sparse_mla_fwd (H = 96): dq [rows,H,576], dkv [T,576],
    dW_UV [H,512,128], dgate [rows,H], float32."""
    bf, f, n = torch.bfloat16, torch.float32, _sizes(shape)
    st = lib().dsa_sparse_mla_bwd(
        ctypes.byref(shape), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(W_UV, bf, "W_UV", numel=n["W_UV"]),
        _p(gate, bf, "gate", numel=n["gate"]), _p(out, bf, "out", numel=n["out"]), _p(lse, f, "lse", numel=n["lse"]),
        _p(dout, bf, "dout", numel=n["out"]), _p(dq, f, "dq", numel=n["q"]), _p(dkv, f, "dkv", numel=n["kv"]),
        _p(dW_UV, f, "dW_UV", numel=n["W_UV"]), _p(dgate, f, "dgate", numel=n["gate"]),
        _p(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _raise(st, "dsa_sparse_mla_bwd")


def dsa_o_proj(shape, x, W_o, y):
    """y [rows, d_model] = x [rows, H*128] W_o^T, W_o [d_model, H*128] (bf16)."""
    bf, r, K = torch.bfloat16, _rows(shape), shape.H * 128
    d_model = W_o.shape[0]
    st = lib().dsa_o_proj(ctypes.byref(shape), _p(x, bf, "x", numel=r * K), _p(W_o, bf, "W_o", numel=d_model * K),
                          d_model, _p(y, bf, "y", numel=r * d_model), _stream())
    _raise(st, "dsa_o_proj")


def dsa_quantize_fp8(x, q8, scale):
    """Rows of 128 bf16 values (x [n,128]) -> E4M3 codes q8 [n,128] uint8 and scale [n] float32."""
    rows = x.numel() // 128
    st = lib().dsa_quantize_fp8(rows, _p(x, torch.bfloat16, "x", numel=rows * 128), _p(q8, torch.uint8, "q8", numel=rows * 128),
                                _p(scale, torch.float32, "scale", numel=rows), _stream())
    _raise(st, "dsa_quantize_fp8")


def dsa_index_topk_noalloc(shape, q_I, k_I, w, topk_idx, ln_gamma=None, ln_beta=None):
    """dsa_index_topk without a workspace: the library's fixed per-GPU scratch is used instead
    (T <= NOALLOC_MAX_T, at most NOALLOC_MAX_DOCS documents). Allocates nothing."""
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_index_topk_noalloc(
        ctypes.byref(shape), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _stream())
    _raise(st, "dsa_index_topk_noalloc")


def dsa_sparse_mla_fwd(shape, q, kv, topk_idx, W_UV, gate, out, workspace, lse=None):
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_sparse_mla_fwd(
        ctypes.byref(shape), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(W_UV, bf, "W_UV", numel=n["W_UV"]),
        _p(gate, bf, "gate", numel=n["gate"]), _p(out, bf, "out", numel=n["out"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _p(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream())
    _raise(st, "dsa_sparse_mla_fwd")


def dsa_sparse_attention_latent(shape, q, kv, topk_idx, o_lat, lse=None):
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_sparse_attention_latent(
        ctypes.byref(shape), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(o_lat, bf, "o_lat", numel=n["o_lat"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _stream())
    _raise(st, "dsa_sparse_attention_latent")


def dsa_up_gate(shape, o_lat, W_UV, gate, out):
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_up_gate(ctypes.byref(shape), _p(o_lat, bf, "o_lat", numel=n["o_lat"]),
                           _p(W_UV, bf, "W_UV", numel=n["W_UV"]), _p(gate, bf, "gate", numel=n["gate"]),
                           _p(out, bf, "out", numel=n["out"]), _stream())
    _raise(st, "dsa_up_gate")


def dsa_fused_fwd(shape, q_I, k_I, w, q, kv, W_UV, gate, topk_idx, out, workspace, ln_gamma=None, ln_beta=None,
                  lse=None):
    bf, n = torch.bfloat16, _sizes(shape)
    st = lib().dsa_fused_fwd(
        ctypes.byref(shape), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(W_UV, bf, "W_UV", numel=n["W_UV"]), _p(gate, bf, "gate", numel=n["gate"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(out, bf, "out", numel=n["out"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _p(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream())
    _raise(st, "dsa_fused_fwd")


def _variant(shape, gate_per_dim, sink):
    """(Variant, element count of the gate) for the _ex entry points."""
    var = Variant()
    var.gate_per_dim = 1 if gate_per_dim else 0
    var.sink = _p(sink, torch.float32, "sink", True, shape.H)
    return var, _rows(shape) * shape.H * (128 if gate_per_dim else 1)


def dsa_sparse_mla_fwd_ex(shape, q, kv, topk_idx, W_UV, gate, out, workspace, lse=None, gate_per_dim=False,
                          sink=None):
    """dsa_sparse_mla_fwd with the gate/sink variant: gate [rows,H] or, with gate_per_dim, [rows,H,128];
    sink: float32 [H] (natural-log units) or None."""
    bf, n = torch.bfloat16, _sizes(shape)
    var, n_gate = _variant(shape, gate_per_dim, sink)
    st = lib().dsa_sparse_mla_fwd_ex(
        ctypes.byref(shape), ctypes.byref(var), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(W_UV, bf, "W_UV", numel=n["W_UV"]),
        _p(gate, bf, "gate", numel=n_gate), _p(out, bf, "out", numel=n["out"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _p(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream())
    _raise(st, "dsa_sparse_mla_fwd_ex")


def _bwd_variant_call(name, shape, q, kv, topk_idx, W_UV, gate, out, lse, o_lat, dout, dq, dkv, dW_UV, dgate,
                      workspace, gate_per_dim, sink, dsink):
    bf, f, n = torch.bfloat16, torch.float32, _sizes(shape)
    var, n_gate = _variant(shape, gate_per_dim, sink)
    head = [ctypes.byref(shape), ctypes.byref(var), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
            _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(W_UV, bf, "W_UV", numel=n["W_UV"]),
            _p(gate, bf, "gate", numel=n_gate), _p(out, bf, "out", numel=n["out"]), _p(lse, f, "lse", numel=n["lse"])]
    if name == "dsa_sparse_mla_bwd_saved":
        head.append(_p(o_lat, bf, "o_lat", numel=n["o_lat"]))
    st = getattr(lib(), name)(
        *head, _p(dout, bf, "dout", numel=n["out"]), _p(dq, f, "dq", numel=n["q"]), _p(dkv, f, "dkv", numel=n["kv"]),
        _p(dW_UV, f, "dW_UV", numel=n["W_UV"]), _p(dgate, f, "dgate", numel=n_gate),
        _p(dsink, f, "dsink", True, shape.H), _p(workspace, torch.uint8, "workspace"), workspace.numel(), _stream())
    _raise(st, name)


def dsa_sparse_mla_bwd_ex(shape, q, kv, topk_idx, W_UV, gate, out, lse, dout, dq, dkv, dW_UV, dgate, workspace,
                          gate_per_dim=False, sink=None, dsink=None):
    """dsa_sparse_mla_bwd for the gate/sink variant of dsa_sparse_mla_fwd_ex: gate and dgate [rows,H] or,
    with gate_per_dim, [rows,H,128]; with sink [H] float32, dsink [H] float32 receives its gradient."""
    _bwd_variant_call("dsa_sparse_mla_bwd_ex", shape, q, kv, topk_idx, W_UV, gate, out, lse, None, dout, dq, dkv,
                      dW_UV, dgate, workspace, gate_per_dim, sink, dsink)


def dsa_sparse_mla_bwd_saved(shape, q, kv, topk_idx, W_UV, gate, out, lse, o_lat, dout, dq, dkv, dW_UV, dgate,
                             workspace, gate_per_dim=False, sink=None, dsink=None):
    """dsa_sparse_mla_bwd_ex given the forward's latent attention output o_lat [rows,H,512] bf16 (from
    dsa_sparse_attention_latent(_ex) with the same variant), which it reads instead of recomputing."""
    _bwd_variant_call("dsa_sparse_mla_bwd_saved", shape, q, kv, topk_idx, W_UV, gate, out, lse, o_lat, dout, dq,
                      dkv, dW_UV, dgate, workspace, gate_per_dim, sink, dsink)


def dsa_sparse_attention_latent_ex(shape, q, kv, topk_idx, o_lat, lse=None, sink=None):
    """dsa_sparse_attention_latent with per-head sink logits [H] float32 (natural-log units) or None."""
    bf, n = torch.bfloat16, _sizes(shape)
    var, _ = _variant(shape, False, sink)
    st = lib().dsa_sparse_attention_latent_ex(
        ctypes.byref(shape), ctypes.byref(var), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(o_lat, bf, "o_lat", numel=n["o_lat"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _stream())
    _raise(st, "dsa_sparse_attention_latent_ex")


def dsa_fused_fwd_ex(shape, q_I, k_I, w, q, kv, W_UV, gate, topk_idx, out, workspace, ln_gamma=None, ln_beta=None,
                     lse=None, gate_per_dim=False, sink=None):
    """dsa_fused_fwd with the gate/sink variant of steps 4-5 (see dsa_sparse_mla_fwd_ex)."""
    bf, n = torch.bfloat16, _sizes(shape)
    var, n_gate = _variant(shape, gate_per_dim, sink)
    st = lib().dsa_fused_fwd_ex(
        ctypes.byref(shape), ctypes.byref(var), _p(q_I, bf, "q_I", numel=n["q_I"]), _p(k_I, bf, "k_I", numel=n["k_I"]),
        _p(ln_gamma, torch.float32, "ln_gamma", True, n["ln"]), _p(ln_beta, torch.float32, "ln_beta", True, n["ln"]),
        _p(w, bf, "w", numel=n["w"]), _p(q, bf, "q", numel=n["q"]), _p(kv, bf, "kv", numel=n["kv"]),
        _p(W_UV, bf, "W_UV", numel=n["W_UV"]), _p(gate, bf, "gate", numel=n_gate),
        _p(topk_idx, torch.int32, "topk_idx", numel=n["topk_idx"]), _p(out, bf, "out", numel=n["out"]),
        _p(lse, torch.float32, "lse", True, n["lse"]), _p(workspace, torch.uint8, "workspace"), workspace.numel(),
        _stream())
    _raise(st, "dsa_fused_fwd_ex")
