"""GPU parity of the gate and sink variants (archdiff.com "Kimi K3.1 Pro" blueprint, entry "Output
gate + sink"): an elementwise gate [rows, H, 128] and a per-head sink logit in the softmax
denominator, through dsa_fused_fwd_ex and dsa_sparse_mla_fwd_ex, against the oracle's variant
computed on the GPU's own indices. Sinks include one far above every logit of its head (the kernel's
rescaled branch), one far below (no effect) and one that takes all the weight."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_indexer_top_index_amd as dsa
import oracle
import testgen as tg
from tests import gpu_util as gu
from tests.parity import check_outputs

pytestmark = pytest.mark.gpu


def _cfg(H):
    if H == 96:
        return tg.Config("variant96", 71, [1500], topk=256, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                         W_UV_std=0.02)
    return tg.Config("variant16", 72, [900, 300], topk=128, H=16, H_I=4, d_I=64, w_scale=0.5)


def _sink(H):
    s = np.random.default_rng(5).normal(0, 2, H)
    s[0] = 60.0     # above every logit by far more than 2^64 in base 2: the rescaled branch
    s[1] = -1.0e4   # no effect
    s[2] = 1.0e4    # takes all the weight: output 0, lse = sink
    return s


def _lse_ok(got, ref):
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= 5e-3 * max(1.0, np.abs(ref[fin]).max() * 1e-3)


@pytest.mark.parametrize("mode", ["sink", "gate-per-dim", "both"])
@pytest.mark.parametrize("H", [96, 16])
def test_fused_variants(H, mode):
    cfg = _cfg(H)
    print(f"[gpu] fused variant {mode}: T={cfg.T} docs={cfg.n_docs} k={cfg.topk} H={H}", flush=True)
    sys.stdout.flush()
    inp = tg.make_inputs(cfg)
    T = cfg.T
    per_dim = mode in ("gate-per-dim", "both")
    gate = tg.normal_bf16(cfg.seed, 50, 0, T * H * 128, 1.0).reshape(T, H, 128) if per_dim else inp["gate"]
    sink = _sink(H) if mode in ("sink", "both") else None
    dev = gu.to_device(dict(inp, gate=gate))
    shape = gu.shape_of(cfg, dev["cu_seqlens"])
    ws = dsa.alloc_workspace(shape)
    idx_t = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.empty((T, H), dtype=torch.float32, device="cuda")
    sink_t = None if sink is None else torch.from_numpy(sink.astype(np.float32)).cuda()
    dsa.dsa_fused_fwd_ex(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"], idx_t,
                         out_t, ws, lse=lse_t, gate_per_dim=per_dim, sink=sink_t)
    # the default variant must be untouched by the new entry point: same indices as dsa_fused_fwd
    idx_ref = torch.empty_like(idx_t)
    out_def = torch.empty_like(out_t)
    dsa.dsa_fused_fwd(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"],
                      gu.bf16_np_to_tensor(inp["gate"]), idx_ref, out_def, ws)
    torch.cuda.synchronize()
    idx = idx_t.cpu().numpy()
    assert np.array_equal(idx, idx_ref.cpu().numpy())
    rows = np.arange(T)
    ref = oracle.sparse_mla_variant(rows, inp["q"], inp["kv"], idx, inp["W_UV"], gate, cfg.softmax_scale,
                                    gate_per_dim=per_dim, sink=None if sink is None else sink.astype(np.float32).astype(np.float64))
    got = gu.bf16_tensor_to_f32(out_t)
    ok, err, mx = check_outputs(got, ref["out"])
    assert ok, (err, mx)
    _lse_ok(lse_t.cpu().numpy(), ref["lse"])
    if sink is not None:
        # each special head against its own scale: rescaled branch (tiny but nonzero outputs), no
        # effect, and all weight to the sink
        ok0, e0, m0 = check_outputs(got[:, 0], ref["out"][:, 0])
        assert ok0 and m0 > 0, (e0, m0)
        assert np.all(got[:, 2] == 0) and np.all(lse_t.cpu().numpy()[:, 2] == np.float32(1.0e4))
    print(f"[gpu] fused variant {mode} H={H}: out rel err {err / mx:.2e}", flush=True)


def test_sink_with_caller_indices_and_empty_row():
    """dsa_sparse_mla_fwd_ex with a sink: a row with no usable index gives zeros and lse = sink."""
    cfg = _cfg(96)
    inp = tg.make_inputs(cfg)
    T, k, H = cfg.T, cfg.topk, cfg.H
    rng = np.random.default_rng(9)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        n = min(k, t + 1)
        idx[t, :n] = np.sort(rng.choice(t + 1, n, replace=False))
    idx[7, :] = -1
    sink = _sink(H)
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_workspace(shape)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    print("[gpu] sparse_mla_fwd_ex with a sink and caller indices", flush=True)
    dsa.dsa_sparse_mla_fwd_ex(shape, dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), dev["W_UV"], dev["gate"], out,
                              ws, lse=lse, sink=torch.from_numpy(sink.astype(np.float32)).cuda())
    torch.cuda.synchronize()
    ref = oracle.sparse_mla_variant(np.arange(T), inp["q"], inp["kv"], idx, inp["W_UV"], inp["gate"],
                                    cfg.softmax_scale, sink=sink.astype(np.float32).astype(np.float64))
    got = gu.bf16_tensor_to_f32(out)
    ok, err, mx = check_outputs(got, ref["out"])
    assert ok, (err, mx)
    assert np.all(got[7] == 0)
    l = lse.cpu().numpy()
    assert np.allclose(l[7], sink.astype(np.float32), rtol=0, atol=1e-4)
    _lse_ok(l, ref["lse"])
