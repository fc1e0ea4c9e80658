"""C ABI checks that need no GPU: the library loads, exports every function include/dsa.h declares,
and the host-side argument checks return the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

import dsa_indexer_top_index_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert names == ["dsa_bwd_workspace_size", "dsa_check_shape", "dsa_fused_fwd", "dsa_fused_fwd_ex", "dsa_index_topk",
                     "dsa_index_topk_fp8", "dsa_index_topk_fused_ln", "dsa_index_topk_noalloc", "dsa_o_proj", "dsa_q_absorb",
                     "dsa_quantize_fp8",
                     "dsa_sparse_attention_latent", "dsa_sparse_attention_latent_ex", "dsa_sparse_mla_bwd",
                     "dsa_sparse_mla_bwd_ex", "dsa_sparse_mla_bwd_saved", "dsa_sparse_mla_fwd",
                     "dsa_sparse_mla_fwd_ex",
                     "dsa_status_string", "dsa_up_gate", "dsa_workspace_size"]
    L = dsa.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings():
    for st in range(6):
        assert dsa.status_string(st)
    assert "allocation-free" in dsa.status_string(dsa.DSA_ERR_TOO_LARGE)
    assert dsa.status_string(99) == "unknown status"


def _shape(**kw):
    base = dict(T=4096, topk=2048, H_I=64, d_I=128, H=96)
    base.update(kw)
    return dsa.make_shape(**base)


def test_supported_shapes_and_workspace():
    assert dsa.dsa_check_shape(_shape()) == dsa.DSA_OK
    assert dsa.dsa_check_shape(_shape(T=1024, topk=256, H_I=4, d_I=64, H=16)) == dsa.DSA_OK
    # LN(k_I) ((T + 128 padding rows) x d_I bf16), 256 candidate-slot flags (1 KB), 256 candidate
    # slots of 8 rows x 4,160 int32 token indices, the FP8 indexer's operands (E4M3 codes of LN(k_I)
    # and q_I, one float scale per 128-value row), and the latent output of one row chunk (rows x H x
    # 512 bf16, at most 2,048 rows); each region starts 256-byte aligned
    al = lambda x: (x + 255) // 256 * 256
    flags, slots = 1024, 256 * 8 * 2 * 4672 * 4  # per row: 4,672 score keys and 4,672 token indices

    def fp8(T, rows, H_I, d_I):
        return al((T + 128) * d_I) + al((T + 128) * 4) + al(rows * H_I * d_I) + al(rows * H_I * 4)
    ws = dsa.dsa_workspace_size(_shape())
    assert ws == (4096 + 128) * 128 * 2 + flags + slots + fp8(4096, 4096, 64, 128) + 2048 * 96 * 512 * 2
    big = dsa.dsa_workspace_size(_shape(T=131072))
    assert big == (131072 + 128) * 128 * 2 + flags + slots + fp8(131072, 131072, 64, 128) + 2048 * 96 * 512 * 2
    assert dsa.dsa_workspace_size(_shape(topk=0)) == 0
    tiny = dsa.dsa_workspace_size(_shape(T=1024, topk=256, H_I=4, d_I=64, H=16))
    assert tiny == (1024 + 128) * 64 * 2 + flags + slots + fp8(1024, 1024, 4, 64) + 1024 * 16 * 512 * 2
    one = dsa.dsa_workspace_size(_shape(T=1024, topk=256, H_I=4, d_I=64, H=16, q_begin=1000, q_end=1001))
    assert one == al((1024 + 128) * 64 * 2) + flags + slots + fp8(1024, 1, 4, 64) + 16 * 512 * 2


@pytest.mark.parametrize("kw,status", [
    (dict(topk=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(topk=2049), dsa.DSA_ERR_UNSUPPORTED),
    (dict(H_I=32), dsa.DSA_ERR_UNSUPPORTED),
    (dict(d_I=96), dsa.DSA_ERR_UNSUPPORTED),
    (dict(H=128), dsa.DSA_ERR_UNSUPPORTED),
    (dict(T=0), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_begin=5, q_end=5), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_begin=-1), dsa.DSA_ERR_INVALID_ARG),
    (dict(q_end=4097), dsa.DSA_ERR_INVALID_ARG),
    (dict(ln_eps=0.0), dsa.DSA_ERR_INVALID_ARG),
    (dict(softmax_scale=float("nan")), dsa.DSA_ERR_INVALID_ARG),
    (dict(cu_seqlens=[0, 100, 100, 4096]), dsa.DSA_ERR_INVALID_ARG),   # empty document
    (dict(cu_seqlens=[0, 100, 4000]), dsa.DSA_ERR_INVALID_ARG),        # does not end at T
    (dict(cu_seqlens=[1, 100, 4096]), dsa.DSA_ERR_INVALID_ARG),        # does not start at 0
])
def test_invalid_shapes(kw, status):
    s = _shape(**kw)
    if "cu_seqlens" in kw:
        s.cu_seqlens_dev = 16  # a non-null stand-in; never dereferenced by the host checks
    assert dsa.dsa_check_shape(s) == status


def test_multi_document_needs_device_offsets():
    s = _shape(cu_seqlens=[0, 1000, 4096])
    assert dsa.dsa_check_shape(s) == dsa.DSA_ERR_INVALID_ARG
    s.cu_seqlens_dev = 256
    assert dsa.dsa_check_shape(s) == dsa.DSA_OK


def test_entry_points_reject_before_any_hip_call():
    """Null pointers, misalignment and small workspaces are caught on the host (no GPU here)."""
    L = dsa.lib()
    s = _shape()
    P = ctypes.byref(s)
    fake = 1 << 20  # aligned, never dereferenced: every call below fails its host checks first
    n = dsa.dsa_workspace_size(s)
    assert L.dsa_index_topk(P, None, fake, None, None, fake, fake, fake, n, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk(P, fake + 2, fake, None, None, fake, fake, fake, n, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk(P, fake, fake, None, None, fake, fake, None, n, None) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_index_topk(P, fake, fake, None, None, fake, fake, fake, n - 1, None) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_index_topk(P, fake, fake, None, None, fake, fake, fake + 16, n, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_sparse_mla_fwd(P, fake, None, fake, fake, fake, fake, None, fake, n, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_sparse_mla_fwd(P, fake, fake + 8, fake, fake, fake, fake, None, fake, n, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_fused_fwd(P, fake, fake, None, None, fake, fake, fake, fake, fake, fake, None, None, fake, n,
                           None) == dsa.DSA_ERR_INVALID_ARG
    bad = _shape(H=8)
    assert L.dsa_fused_fwd(ctypes.byref(bad), fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake, None,
                           fake, n, None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.dsa_check_shape(None) == dsa.DSA_ERR_INVALID_ARG


def test_python_binding_rejects_undersized_tensors():
    """The binding checks each tensor's element count against the shape before calling the library
    (an undersized buffer would become an out-of-bounds device access). CPU tensors are rejected
    too, before any size check can pass, so nothing here reaches the GPU."""
    import torch
    s = _shape(T=64, topk=16, H_I=4, d_I=64, H=16)
    sz = dsa._sizes(s)
    assert sz["q_I"] == 64 * 4 * 64 and sz["out"] == 64 * 16 * 128 and sz["topk_idx"] == 64 * 16
    part = _shape(T=64, topk=16, H_I=4, d_I=64, H=16, q_begin=10, q_end=20)
    assert dsa._sizes(part)["q"] == 10 * 16 * 576 and dsa._sizes(part)["kv"] == 64 * 576
    t = torch.empty(3, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dsa._p(t, torch.bfloat16, "x")   # host memory
    fake = torch.empty(5, dtype=torch.bfloat16)
    # exercise the size rule alone on a tensor that passes the other checks
    orig = dsa._check
    try:
        dsa._check = lambda *a: None
        with pytest.raises(ValueError, match="elements"):
            dsa._p(fake, torch.bfloat16, "q", numel=6)
        assert dsa._p(fake, torch.bfloat16, "q", numel=5) == fake.data_ptr()
    finally:
        dsa._check = orig


def test_noalloc_entry_point_host_checks():
    """dsa_index_topk_noalloc rejects shapes beyond its fixed scratch (T > 131072, more than 64
    documents) and bad pointers on the host, before any HIP call."""
    L = dsa.lib()
    fake = 1 << 20
    ok = _shape(T=131072)
    assert dsa.dsa_check_shape(ok) == dsa.DSA_OK
    big = _shape(T=131073)
    assert L.dsa_index_topk_noalloc(ctypes.byref(big), fake, fake, None, None, fake, fake, None) == dsa.DSA_ERR_TOO_LARGE
    cu = list(range(0, 65 * 64, 64)) + [65 * 64 + 10]   # 65 documents
    many = _shape(T=cu[-1], cu_seqlens=cu)
    many.cu_seqlens_dev = 256
    assert dsa.dsa_check_shape(many) == dsa.DSA_OK
    assert L.dsa_index_topk_noalloc(ctypes.byref(many), fake, fake, None, None, fake, fake, None) == dsa.DSA_ERR_TOO_LARGE
    assert L.dsa_index_topk_noalloc(ctypes.byref(ok), None, fake, None, None, fake, fake, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk_noalloc(ctypes.byref(ok), fake, fake, None, None, fake, fake + 4, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk_noalloc(ctypes.byref(_shape(H=8)), fake, fake, None, None, fake, fake, None) == dsa.DSA_ERR_UNSUPPORTED


def test_variant_host_checks():
    """The gate/sink variant is checked on the host: gate_per_dim must be 0 or 1, an elementwise gate
    16-byte aligned, the sink 4-byte aligned."""
    L = dsa.lib()
    s = _shape()
    P = ctypes.byref(s)
    fake = 1 << 20
    n = dsa.dsa_workspace_size(s)
    var = dsa.Variant()
    var.gate_per_dim, var.sink = 2, None
    args = (fake, fake, fake, fake, fake, fake, None, fake, n, None)
    assert L.dsa_sparse_mla_fwd_ex(P, ctypes.byref(var), *args) == dsa.DSA_ERR_INVALID_ARG
    var.gate_per_dim = 1
    bad_gate = (fake, fake, fake, fake, fake + 2, fake, None, fake, n, None)
    assert L.dsa_sparse_mla_fwd_ex(P, ctypes.byref(var), *bad_gate) == dsa.DSA_ERR_INVALID_ARG
    var.gate_per_dim, var.sink = 0, fake + 2
    assert L.dsa_sparse_mla_fwd_ex(P, ctypes.byref(var), *args) == dsa.DSA_ERR_INVALID_ARG
    var.sink = None
    assert L.dsa_sparse_mla_fwd_ex(P, ctypes.byref(var), fake, fake, fake, fake, fake, fake, None, None, n,
                                   None) == dsa.DSA_ERR_WORKSPACE


def test_fp8_entry_points_host_checks():
    """The FP8 indexer takes only the 64x128 indexer shape; the quantiser checks its pointers."""
    L = dsa.lib()
    fake = 1 << 20
    tiny = _shape(T=1024, topk=256, H_I=4, d_I=64, H=16)
    n = dsa.dsa_workspace_size(tiny)
    assert L.dsa_index_topk_fp8(ctypes.byref(tiny), fake, fake, None, None, fake, fake, fake, n, None) == dsa.DSA_ERR_UNSUPPORTED
    s = _shape()
    assert L.dsa_index_topk_fp8(ctypes.byref(s), fake, fake, None, None, fake, fake, fake, 16, None) == dsa.DSA_ERR_WORKSPACE
    assert L.dsa_quantize_fp8(-1, fake, fake, fake, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(4, None, fake, fake, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_quantize_fp8(4, fake, fake + 8, fake, None) == dsa.DSA_ERR_INVALID_ARG


def test_fused_ln_indexer_host_checks():
    """The fused-LN indexer takes only the 64x128 indexer shape, a 16-byte aligned k_I and the workspace."""
    L = dsa.lib()
    fake = 1 << 20
    tiny = _shape(T=1024, topk=256, H_I=4, d_I=64, H=16)
    n = dsa.dsa_workspace_size(tiny)
    args = lambda k_I, ws_bytes: (fake, k_I, None, None, fake, fake, fake, ws_bytes, None)
    assert L.dsa_index_topk_fused_ln(ctypes.byref(tiny), *args(fake, n)) == dsa.DSA_ERR_UNSUPPORTED
    s = _shape()
    n = dsa.dsa_workspace_size(s)
    assert L.dsa_index_topk_fused_ln(ctypes.byref(s), *args(fake + 2, n)) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk_fused_ln(ctypes.byref(s), *args(None, n)) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_index_topk_fused_ln(ctypes.byref(s), *args(fake, n - 1)) == dsa.DSA_ERR_WORKSPACE


def test_backward_host_checks():
    """The backward takes 96 heads only, checks its pointers and its (larger) workspace."""
    L = dsa.lib()
    fake = 1 << 20
    s = _shape(T=1024)
    nb = L.dsa_bwd_workspace_size(ctypes.byref(s))
    # the forward's workspace, then per chunk of (here all) 1,024 rows: do, do_lat, delta, g (dS' and P
    # of the 96 heads for every selected key, k rounded up to 32), the bf16 dkv contribution of every
    # (row, selected key) pair, and the counting sort of the pairs by key (count, start, list, and
    # the scan's sums over tiles of 4,096 keys), and the sink's per-(row, head) gradient terms
    al = lambda x: (x + 255) // 256 * 256
    cr, g_stride, T, k = 1024 * 96, (s.topk + 31) // 32 * 32, s.T, s.topk
    assert nb == (dsa.dsa_workspace_size(s) + al(cr * 128 * 2) + al(cr * 512 * 2) + al(cr * 4)
                  + al(1024 * g_stride * 192 * 2) + al(1024 * k * 576 * 2) + al(T * 4) + al((T + 1) * 4)
                  + al(1024 * k * 4) + al((T + 4095) // 4096 * 4) + al(cr * 4))
    # longer inputs are taken in chunks of 2,048 rows, so the chunk regions stop growing there
    s2 = _shape(T=8192)
    g2, c2, T2 = (s2.topk + 31) // 32 * 32, 2048 * 96, 8192
    assert L.dsa_bwd_workspace_size(ctypes.byref(s2)) == (
        dsa.dsa_workspace_size(s2) + al(c2 * 128 * 2) + al(c2 * 512 * 2) + al(c2 * 4) + al(2048 * g2 * 192 * 2)
        + al(2048 * s2.topk * 576 * 2) + al(T2 * 4) + al((T2 + 1) * 4) + al(2048 * s2.topk * 4)
        + al((T2 + 4095) // 4096 * 4) + al(c2 * 4))
    args = [fake] * 12
    assert L.dsa_sparse_mla_bwd(ctypes.byref(_shape(T=1024, topk=256, H_I=4, d_I=64, H=16)), *args, fake, nb,
                                None) == dsa.DSA_ERR_UNSUPPORTED
    assert L.dsa_sparse_mla_bwd(ctypes.byref(s), *args, fake, nb - 1, None) == dsa.DSA_ERR_WORKSPACE
    bad = list(args)
    bad[7] = None  # dout
    assert L.dsa_sparse_mla_bwd(ctypes.byref(s), *bad, fake, nb, None) == dsa.DSA_ERR_INVALID_ARG
    # the variant form: a sink needs dsink and dsink needs a sink; a per-element dgate must be 16-byte aligned
    var = dsa.Variant()
    var.gate_per_dim, var.sink = 0, fake
    assert L.dsa_sparse_mla_bwd_ex(ctypes.byref(s), ctypes.byref(var), *args, None, fake, nb, None) == dsa.DSA_ERR_INVALID_ARG
    var.sink = None
    assert L.dsa_sparse_mla_bwd_ex(ctypes.byref(s), ctypes.byref(var), *args, fake, fake, nb, None) == dsa.DSA_ERR_INVALID_ARG
    var.gate_per_dim = 1
    odd = list(args)
    odd[11] = fake + 4  # dgate
    assert L.dsa_sparse_mla_bwd_ex(ctypes.byref(s), ctypes.byref(var), *odd, None, fake, nb, None) == dsa.DSA_ERR_INVALID_ARG
    var.gate_per_dim = 2
    assert L.dsa_sparse_mla_bwd_ex(ctypes.byref(s), ctypes.byref(var), *args, None, fake, nb, None) == dsa.DSA_ERR_INVALID_ARG
    assert L.dsa_sparse_mla_bwd_ex(ctypes.byref(s), ctypes.byref(var), *args, None, fake, nb - 1, None) == dsa.DSA_ERR_INVALID_ARG
    # the form with the forward's o_lat: it must be given, 16-byte aligned, and the workspace is the same
    var.gate_per_dim = 0
    saved = lambda o_lat, n_ws: L.dsa_sparse_mla_bwd_saved(ctypes.byref(s), ctypes.byref(var), *args[:7], o_lat,
                                                          *args[7:], None, fake, n_ws, None)
    assert saved(None, nb) == dsa.DSA_ERR_INVALID_ARG
    assert saved(fake + 8, nb) == dsa.DSA_ERR_INVALID_ARG
    assert saved(fake, nb - 1) == dsa.DSA_ERR_WORKSPACE
    # the latent attention with a variant checks the variant's fields
    var.gate_per_dim, var.sink = 2, None
    assert L.dsa_sparse_attention_latent_ex(ctypes.byref(s), ctypes.byref(var), fake, fake, fake, fake, None,
                                            None) == dsa.DSA_ERR_INVALID_ARG
    var.gate_per_dim, var.sink = 0, fake + 2
    assert L.dsa_sparse_attention_latent_ex(ctypes.byref(s), ctypes.byref(var), fake, fake, fake, fake, None,
                                            None) == dsa.DSA_ERR_INVALID_ARG
