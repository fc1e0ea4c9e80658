"""GPU parity of the sparse MLA backward on the native 96 heads (model-coverage page: the backward runs
96 heads without padding; hard top-k carries no gradient) against the oracle's double-precision
backward, through the C ABI. The indices, out and lse come from the GPU forward; the oracle takes the
same bf16 values as exact doubles. Each gradient must satisfy the output rule
max |g - g_ref| <= 2e-2 * max |g_ref| (the GPU rounds do, do_lat, P and dS to bf16 for its MFMAs and
takes D = sum dout * out from the bf16 out)."""
from __future__ import annotations

import math
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

TAG_DOUT = 70


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _f64(a):
    return tg.bf16_to_f32(a).astype(np.float64)


def _run_bwd(cfg, inp, idx_t, out_t, lse_t, dout):
    T, H = cfg.T, cfg.H
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg, dev["cu_seqlens"])
    ws = dsa.alloc_bwd_workspace(shape)
    dq = torch.empty((T, H, 576), dtype=torch.float32, device="cuda")
    dkv = torch.empty((T, 576), dtype=torch.float32, device="cuda")
    dW = torch.empty((H, 512, 128), dtype=torch.float32, device="cuda")
    dg = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_bwd(shape, dev["q"], dev["kv"], idx_t, dev["W_UV"], dev["gate"], out_t, lse_t,
                           gu.bf16_np_to_tensor(dout), dq, dkv, dW, dg, ws)
    torch.cuda.synchronize()
    return {"dq": dq.cpu().numpy(), "dkv": dkv.cpu().numpy(), "dW_UV": dW.cpu().numpy(), "dgate": dg.cpu().numpy()}


def _compare(name, got, inp, idx, dout, cfg):
    ref = oracle.sparse_mla_bwd(_f64(inp["q"]), _f64(inp["kv"]), idx, _f64(inp["W_UV"]), _f64(inp["gate"]),
                                cfg.softmax_scale, _f64(dout))
    msgs = []
    for k in ["dq", "dkv", "dW_UV", "dgate"]:
        ok, err, mx = check_outputs(got[k], ref[k])
        msgs.append(f"{k} {err / mx:.2e}")
        assert ok, (name, k, err, mx)
    _say(f"[gpu] backward {name}: max error / max |ref|: " + ", ".join(msgs))


@pytest.mark.parametrize("case", ["single", "packed", "odd-k"])
def test_backward_after_fused_forward(case):
    if case == "single":
        cfg = tg.Config("bwd", 101, [700], topk=256, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24, W_UV_std=0.02)
    elif case == "odd-k":
        # k = 100: the last 32-key tile of a full row reaches past k (the next row's pairs)
        cfg = tg.Config("bwd-oddk", 105, [500], topk=100, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                        W_UV_std=0.02)
    else:
        cfg = tg.Config("bwd-packed", 102, [300, 1, 40, 500], topk=128, H=96, H_I=64, d_I=128, w_scale=1 / 8,
                        q_std=1 / 24, W_UV_std=0.02)
    _say(f"[gpu] backward {case}: T={cfg.T} docs={cfg.n_docs} k={cfg.topk}")
    inp = tg.make_inputs(cfg)
    dev = gu.to_device(inp)
    res = gu.run_fused(cfg, dev, with_lse=True)
    torch.cuda.synchronize()
    dout = tg.normal_bf16(cfg.seed, TAG_DOUT, 0, cfg.T * cfg.H * 128, 1.0).reshape(cfg.T, cfg.H, 128)
    got = _run_bwd(cfg, inp, res["topk_idx"], res["out"], res["lse"], dout)
    _compare(case, got, inp, res["topk_idx"].cpu().numpy(), dout, cfg)


def _bwd_sink(H):
    s = np.random.default_rng(6).normal(0, 1, H)  # comparable with the logits: the sink takes a real share
    s[0] = 60.0     # far above every logit: the forward's rescaled branch, the keys keep almost no weight
    s[1] = -1.0e4   # no effect: its gradient is exactly 0
    return s.astype(np.float32)


@pytest.mark.parametrize("mode", ["gate-per-dim", "sink", "both"])
def test_backward_variants(mode):
    """The backward of the gate and sink variants (dsa_sparse_mla_bwd_ex) after dsa_fused_fwd_ex on two
    packed documents: every gradient, dsink included, against the oracle's variant backward."""
    cfg = tg.Config("bwd-var", 104, [600, 200], topk=128, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    T, H = cfg.T, cfg.H
    per_dim, with_sink = mode != "sink", mode != "gate-per-dim"
    _say(f"[gpu] backward variant {mode}: T={T} docs={cfg.n_docs} k={cfg.topk}")
    inp = tg.make_inputs(cfg)
    gate = tg.normal_bf16(cfg.seed, 50, 0, T * H * 128, 1.0).reshape(T, H, 128) if per_dim else inp["gate"]
    sink = _bwd_sink(H) if with_sink else None
    dev = gu.to_device(dict(inp, gate=gate))
    shape = gu.shape_of(cfg, dev["cu_seqlens"])
    ws = dsa.alloc_workspace(shape)
    idx_t = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.empty((T, H), dtype=torch.float32, device="cuda")
    sink_t = torch.from_numpy(sink).cuda() if with_sink else None
    dsa.dsa_fused_fwd_ex(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"], idx_t,
                         out_t, ws, lse=lse_t, gate_per_dim=per_dim, sink=sink_t)
    dout = tg.normal_bf16(cfg.seed, TAG_DOUT, 0, T * H * 128, 1.0).reshape(T, H, 128)
    wsb = dsa.alloc_bwd_workspace(shape)
    dq = torch.empty((T, H, 576), dtype=torch.float32, device="cuda")
    dkv = torch.empty((T, 576), dtype=torch.float32, device="cuda")
    dW = torch.empty((H, 512, 128), dtype=torch.float32, device="cuda")
    dg = torch.empty(gate.shape, dtype=torch.float32, device="cuda")
    dsink = torch.empty(H, dtype=torch.float32, device="cuda") if with_sink else None
    dsa.dsa_sparse_mla_bwd_ex(shape, dev["q"], dev["kv"], idx_t, dev["W_UV"], dev["gate"], out_t, lse_t,
                              gu.bf16_np_to_tensor(dout), dq, dkv, dW, dg, wsb, gate_per_dim=per_dim, sink=sink_t,
                              dsink=dsink)
    torch.cuda.synchronize()
    ref = oracle.sparse_mla_bwd(_f64(inp["q"]), _f64(inp["kv"]), idx_t.cpu().numpy(), _f64(inp["W_UV"]), _f64(gate),
                                cfg.softmax_scale, _f64(dout), gate_per_dim=per_dim,
                                sink=sink.astype(np.float64) if with_sink else None)
    got = {"dq": dq.cpu().numpy(), "dkv": dkv.cpu().numpy(), "dW_UV": dW.cpu().numpy(), "dgate": dg.cpu().numpy()}
    if with_sink:
        got["dsink"] = dsink.cpu().numpy()
        assert got["dsink"][1] == 0.0
    msgs = []
    for k in got:
        ok, err, mx = check_outputs(got[k], ref[k])
        msgs.append(f"{k} {err / mx:.2e}")
        assert ok, (mode, k, err, mx)
    _say(f"[gpu] backward variant {mode}: max error / max |ref|: " + ", ".join(msgs))


@pytest.mark.parametrize("mode", ["plain", "sink"])
def test_backward_saved_olat(mode):
    """dsa_sparse_mla_bwd_saved with the forward's o_lat from dsa_sparse_attention_latent_ex, on 4,200 rows
    (three backward chunks of up to 2,048 rows): every output equals dsa_sparse_mla_bwd_ex's (dq, dgate
    and dsink bit for bit; dkv and dW_UV, whose sums run in an order that atomics decide, to 1e-5 of their
    largest value). With o_lat doubled (exact in bf16) dW_UV doubles and nothing else moves, so the saved
    rows are what dW_UV reads, chunk by chunk. The latent attention's lse equals the fused forward's."""
    cfg = tg.Config("bwd-saved", 105, [2500, 1700], topk=128, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    T, H = cfg.T, cfg.H
    with_sink = mode == "sink"
    _say(f"[gpu] backward with saved o_lat ({mode}): T={T} docs={cfg.n_docs} k={cfg.topk}")
    inp = tg.make_inputs(cfg)
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg, dev["cu_seqlens"])
    ws = dsa.alloc_workspace(shape)
    sink_t = torch.from_numpy(_bwd_sink(H)).cuda() if with_sink else None
    idx_t = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out_t = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse_t = torch.empty((T, H), dtype=torch.float32, device="cuda")
    dsa.dsa_fused_fwd_ex(shape, dev["q_I"], dev["k_I"], dev["w"], dev["q"], dev["kv"], dev["W_UV"], dev["gate"], idx_t,
                         out_t, ws, lse=lse_t, sink=sink_t)
    o_lat = torch.empty((T, H, 512), dtype=torch.bfloat16, device="cuda")
    lse2 = torch.empty_like(lse_t)
    dsa.dsa_sparse_attention_latent_ex(shape, dev["q"], dev["kv"], idx_t, o_lat, lse=lse2, sink=sink_t)
    dout_t = gu.bf16_np_to_tensor(tg.normal_bf16(cfg.seed, TAG_DOUT, 0, T * H * 128, 1.0).reshape(T, H, 128))
    wsb = dsa.alloc_bwd_workspace(shape)

    def grads(fn, *olat):
        g = {"dq": torch.empty((T, H, 576), dtype=torch.float32, device="cuda"),
             "dkv": torch.empty((T, 576), dtype=torch.float32, device="cuda"),
             "dW_UV": torch.empty((H, 512, 128), dtype=torch.float32, device="cuda"),
             "dgate": torch.empty((T, H), dtype=torch.float32, device="cuda")}
        if with_sink:
            g["dsink"] = torch.empty(H, dtype=torch.float32, device="cuda")
        fn(shape, dev["q"], dev["kv"], idx_t, dev["W_UV"], dev["gate"], out_t, lse_t, *olat, dout_t, g["dq"], g["dkv"],
           g["dW_UV"], g["dgate"], wsb, sink=sink_t, dsink=g.get("dsink"))
        torch.cuda.synchronize()
        return {k: v.cpu().numpy() for k, v in g.items()}

    ref = grads(dsa.dsa_sparse_mla_bwd_ex)
    got = grads(dsa.dsa_sparse_mla_bwd_saved, o_lat)
    got2 = grads(dsa.dsa_sparse_mla_bwd_saved, o_lat * 2)
    assert torch.equal(lse2, lse_t)
    for k in ref:
        if k in ("dkv", "dW_UV"):
            mx = np.abs(ref[k]).max()
            assert mx > 0 and np.abs(got[k] - ref[k]).max() <= 1e-5 * mx, k
        else:
            assert np.array_equal(got[k], ref[k]), k
        if k == "dW_UV":
            assert np.abs(got2[k] - 2 * ref[k]).max() <= 2e-5 * mx, k
        elif k == "dkv":
            assert np.abs(got2[k] - ref[k]).max() <= 1e-5 * mx, k
        else:
            assert np.array_equal(got2[k], ref[k]), k
    _say(f"[gpu] backward with saved o_lat ({mode}): equal to the recomputing backward")


def test_backward_row_ranges_sum_to_the_whole():
    """The backward over query-row ranges (dsa_shape's q_begin/q_end, one range per rank when the rows
    are sharded): on two packed documents split at a row inside the first document, each range's dq
    and dgate equal those rows of the whole-range run bit for bit, and the two ranges' dkv and dW_UV
    (partial sums over their rows, which ranks would add up) sum to the whole run's within FP32
    reordering (1e-5 of the largest value)."""
    cfg = tg.Config("bwd-ranges", 106, [2600, 900], topk=256, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    T, H, k = cfg.T, cfg.H, cfg.topk
    _say(f"[gpu] backward over row ranges: T={T} docs={cfg.n_docs} k={k}")
    inp = tg.make_inputs(cfg)
    dev = gu.to_device(inp)
    res = gu.run_fused(cfg, dev, with_lse=True)
    idx_t, out_t, lse_t = res["topk_idx"], res["out"], res["lse"]
    dout_t = gu.bf16_np_to_tensor(tg.normal_bf16(cfg.seed, TAG_DOUT, 0, T * H * 128, 1.0).reshape(T, H, 128))

    def bwd(b, e):
        shape = gu.shape_of(cfg, dev["cu_seqlens"], q_begin=b, q_end=e)
        n = e - b
        g = {"dq": torch.empty((n, H, 576), dtype=torch.float32, device="cuda"),
             "dkv": torch.empty((T, 576), dtype=torch.float32, device="cuda"),
             "dW_UV": torch.empty((H, 512, 128), dtype=torch.float32, device="cuda"),
             "dgate": torch.empty((n, H), dtype=torch.float32, device="cuda")}
        dsa.dsa_sparse_mla_bwd(shape, dev["q"][b:e].contiguous(), dev["kv"], idx_t[b:e].contiguous(), dev["W_UV"],
                               dev["gate"][b:e].contiguous(), out_t[b:e].contiguous(), lse_t[b:e].contiguous(),
                               dout_t[b:e].contiguous(), g["dq"], g["dkv"], g["dW_UV"], g["dgate"],
                               dsa.alloc_bwd_workspace(shape))
        torch.cuda.synchronize()
        return {key: v.cpu().numpy() for key, v in g.items()}

    whole = bwd(0, T)
    cut = 1300
    lo, hi = bwd(0, cut), bwd(cut, T)
    assert np.array_equal(lo["dq"], whole["dq"][:cut]) and np.array_equal(hi["dq"], whole["dq"][cut:])
    assert np.array_equal(lo["dgate"], whole["dgate"][:cut]) and np.array_equal(hi["dgate"], whole["dgate"][cut:])
    for key in ("dkv", "dW_UV"):
        mx = np.abs(whole[key]).max()
        err = np.abs(lo[key].astype(np.float64) + hi[key] - whole[key]).max()
        assert mx > 0 and err <= 1e-5 * mx, (key, err, mx)
    _say("[gpu] backward over row ranges: the ranges' gradients make up the whole run's")


def test_backward_caller_indices():
    """Caller indices with duplicates, -1 and out-of-range entries, and a row with no usable index."""
    cfg = tg.Config("bwd-idx", 103, [400], topk=64, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    inp = tg.make_inputs(cfg)
    T, k, H = cfg.T, cfg.topk, cfg.H
    rng = np.random.default_rng(4)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        keff = min(k, t + 1)
        row = rng.integers(0, t + 1, keff).astype(np.int32)
        kill = rng.random(keff) < 0.15
        row[kill] = rng.choice([-1, -5, T, T + 9], kill.sum())
        idx[t, :keff] = row
    idx[9, :] = -1
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_workspace(shape)
    idx_t = torch.from_numpy(idx).cuda()
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    _say("[gpu] backward with caller indices")
    dsa.dsa_sparse_mla_fwd(shape, dev["q"], dev["kv"], idx_t, dev["W_UV"], dev["gate"], out, ws, lse=lse)
    dout = tg.normal_bf16(cfg.seed, TAG_DOUT, 0, T * H * 128, 1.0).reshape(T, H, 128)
    got = _run_bwd(cfg, inp, idx_t, out, lse, dout)
    assert np.all(got["dq"][9] == 0) and np.all(got["dgate"][9] == 0)
    _compare("caller indices", got, inp, idx, dout, cfg)


def test_backward_t4096_sampled_rows():
    """Full-size T=4096, top-2048: dq and dgate of sampled rows (each depends on its own row only), and
    the dkv rows of keys 4088..4095, which by causality only rows 4088..4095 can select, so the oracle's
    backward of those eight rows gives them in full. dW_UV sums over every row and is checked for
    finiteness only at this size (the small cases above compare it in full)."""
    cfg = tg.get_config("t4096")
    keys, dev = gu.device_inputs(cfg)
    res = gu.run_fused(cfg, dev, with_lse=True)
    torch.cuda.synchronize()
    dout = tg.normal_bf16(cfg.seed, TAG_DOUT, 0, cfg.T * cfg.H * 128, 1.0).reshape(cfg.T, cfg.H, 128)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_bwd_workspace(shape)
    T, H = cfg.T, cfg.H
    dq = torch.empty((T, H, 576), dtype=torch.float32, device="cuda")
    dkv = torch.empty((T, 576), dtype=torch.float32, device="cuda")
    dW = torch.empty((H, 512, 128), dtype=torch.float32, device="cuda")
    dg = torch.empty((T, H), dtype=torch.float32, device="cuda")
    _say("[gpu] backward t4096")
    dsa.dsa_sparse_mla_bwd(shape, dev["q"], dev["kv"], res["topk_idx"], dev["W_UV"], dev["gate"], res["out"],
                           res["lse"], gu.bf16_np_to_tensor(dout), dq, dkv, dW, dg, ws)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 2048, 3000] + list(range(4088, 4096)))
    qr = tg.query_rows(cfg, rows)
    idx = res["topk_idx"].cpu().numpy()[rows]
    ref = oracle.sparse_mla_bwd(_f64(qr["q"].reshape(len(rows), H, 576)), _f64(keys["kv"]), idx, _f64(keys["W_UV"]),
                                _f64(qr["gate"].reshape(len(rows), H)), cfg.softmax_scale, _f64(dout[rows]))
    for k, g in [("dq", dq.cpu().numpy()[rows]), ("dgate", dg.cpu().numpy()[rows])]:
        ok, err, mx = check_outputs(g, ref[k])
        assert ok, (k, err, mx)
    ok, err, mx = check_outputs(dkv.cpu().numpy()[4088:], ref["dkv"][4088:])
    assert ok, ("dkv of the last keys", err, mx)
    assert np.all(np.isfinite(dkv.cpu().numpy())) and np.all(np.isfinite(dW.cpu().numpy()))


def test_backward_four_row_chunks_caller_indices():
    """T=6,200 runs the backward in four 2,048-row chunks, so both double-buffered g / do_lat buffers are
    reused while the other chunk's dkv contraction may still run on the library's second stream; every
    gradient is compared in full. Caller indices (k=16, some invalid) keep the oracle's cost small."""
    cfg = tg.Config("bwd-chunks", 104, [6200], topk=16, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    inp = tg.make_inputs(cfg)
    T, k, H = cfg.T, cfg.topk, cfg.H
    rng = np.random.default_rng(6)
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        keff = min(k, t + 1)
        row = rng.integers(0, t + 1, keff).astype(np.int32)
        row[rng.random(keff) < 0.1] = -1
        idx[t, :keff] = row
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_workspace(shape)
    idx_t = torch.from_numpy(idx).cuda()
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    _say("[gpu] backward over four row chunks")
    dsa.dsa_sparse_mla_fwd(shape, dev["q"], dev["kv"], idx_t, dev["W_UV"], dev["gate"], out, ws, lse=lse)
    dout = tg.normal_bf16(cfg.seed, TAG_DOUT, 0, T * H * 128, 1.0).reshape(T, H, 128)
    got = _run_bwd(cfg, inp, idx_t, out, lse, dout)
    _compare("four row chunks", got, inp, idx, dout, cfg)


def _dout_device(cfg, chunk_rows=4096):
    """The seeded dout of every row, drawn in row chunks straight into device memory (the same values
    as one draw over all rows: the generator is counter-based)."""
    T, per = cfg.T, cfg.H * 128
    t = torch.empty((T, per), dtype=torch.bfloat16, device="cuda")
    for r0 in range(0, T, chunk_rows):
        n = min(chunk_rows, T - r0)
        t[r0:r0 + n] = gu.bf16_np_to_tensor(tg.normal_bf16(cfg.seed, TAG_DOUT, r0 * per, n * per, 1.0).reshape(n, per))
    return t.view(T, cfg.H, 128)


def _dout_rows(cfg, rows):
    per = cfg.H * 128
    return np.stack([tg.normal_bf16(cfg.seed, TAG_DOUT, int(r) * per, per, 1.0) for r in rows]).reshape(len(rows), cfg.H, 128)


def test_backward_t131072_sampled_rows_and_identities():
    """Full-size T=131,072, top-2048, in the bench's launch configuration:
    - dq and dgate of sampled rows against the oracle (each depends on its own row only): both sides of
      the backward's 1,024-row chunk boundaries and of the forward's 2,048-row ones, the middle, the end;
    - the complete dkv rows of the last eight keys (only the last eight rows can select them);
    - on the full gradients, the closed forms of L = sum(dout * out) that the oracle's backward is
      pinned to: <dW_UV[h], W_UV[h]> = sum_r <dout[r,h], out[r,h]> per head, and
      sum_key <dkv, kv> - sum_(r,h) <dq, q> = sum_(r,h) <dout, out>; and dgate = (1 - sigmoid(gate)) *
      <dout, out> on every row. These compare the backward with the forward's out, so they check the
      whole dkv and dW_UV sums (every pair of every row) at this size, in float64 over the GPU's values.
      The GPU's roundings to bf16 (P, dS', do, do_lat: about 4e-3 relative, unbiased) add errors of
      random sign, so the bound is 0.05 of the root sum of squares of the per-key, per-(row, head) and
      per-row terms, not of their absolute sums: dropping a few per mille of the pairs from dkv would
      exceed it."""
    cfg = tg.get_config("t131072")
    T, H = cfg.T, cfg.H
    _say(f"[gpu] backward t131072: inputs")
    keys, dev = gu.device_inputs(cfg)
    res = gu.run_fused(cfg, dev, with_lse=True)
    dout_t = _dout_device(cfg)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_bwd_workspace(shape)
    dq = torch.empty((T, H, 576), dtype=torch.float32, device="cuda")
    dkv = torch.empty((T, 576), dtype=torch.float32, device="cuda")
    dW = torch.empty((H, 512, 128), dtype=torch.float32, device="cuda")
    dg = torch.empty((T, H), dtype=torch.float32, device="cuda")
    _say("[gpu] backward t131072: dsa_sparse_mla_bwd")
    dsa.dsa_sparse_mla_bwd(shape, dev["q"], dev["kv"], res["topk_idx"], dev["W_UV"], dev["gate"], res["out"],
                           res["lse"], dout_t, dq, dkv, dW, dg, ws)
    torch.cuda.synchronize()
    del ws
    _say("[gpu] backward t131072: sampled rows against the oracle")
    rows = np.array([0, 1, 1023, 1024, 2047, 2048, 65535, 65536, 98304, 130047, 130048] + list(range(T - 8, T)))
    rows_t = torch.from_numpy(rows).cuda()
    qr = tg.query_rows(cfg, rows)
    idx = res["topk_idx"][rows_t].cpu().numpy()
    ref = oracle.sparse_mla_bwd(_f64(qr["q"].reshape(len(rows), H, 576)), _f64(keys["kv"]), idx, _f64(keys["W_UV"]),
                                _f64(qr["gate"].reshape(len(rows), H)), cfg.softmax_scale, _f64(_dout_rows(cfg, rows)))
    for k, g in [("dq", dq[rows_t].cpu().numpy()), ("dgate", dg[rows_t].cpu().numpy())]:
        ok, err, mx = check_outputs(g, ref[k])
        assert ok, (k, err, mx)
    ok, err, mx = check_outputs(dkv[T - 8:].cpu().numpy(), ref["dkv"][T - 8:])
    assert ok, ("dkv of the last keys", err, mx)
    _say("[gpu] backward t131072: identities on the full gradients")
    # D[r, h] = <dout, out> in float64, row chunk by row chunk; sum_(r,h) <dq, q> likewise
    D = torch.empty((T, H), dtype=torch.float64, device="cuda")
    dq_q = torch.zeros((), dtype=torch.float64, device="cuda")
    dq_q_sq = torch.zeros((), dtype=torch.float64, device="cuda")
    for r0 in range(0, T, 8192):
        sl = slice(r0, min(r0 + 8192, T))
        D[sl] = (dout_t[sl].double() * res["out"][sl].double()).sum(dim=2)
        p = (dq[sl].double() * dev["q"][sl].double()).sum(dim=2)  # <dq[r,h], q[r,h]>
        dq_q += p.sum()
        dq_q_sq += (p ** 2).sum()
    dq_q, dq_q_sq = float(dq_q), float(dq_q_sq)
    per_key = (dkv.double() * dev["kv"].double()).sum(dim=1)  # <dkv[key], kv[key]>
    lhs, rhs = float(per_key.sum() - dq_q), float(D.sum())
    rss = math.sqrt(float((per_key ** 2).sum() + dq_q_sq + (D ** 2).sum()))
    tol = 0.05 * rss
    _say(f"[gpu] backward t131072: sum <dkv, kv> - sum <dq, q> = {lhs:.6e}, sum <dout, out> = {rhs:.6e}, "
         f"difference {abs(lhs - rhs) / rss:.2e} of the root sum of squares")
    assert abs(lhs - rhs) <= tol, ("sum <dkv, kv> - sum <dq, q>", lhs, rhs, tol)
    lhs_w = (dW.double() * dev["W_UV"].double()).sum(dim=(1, 2))
    rhs_w, rss_w = D.sum(dim=0), (D ** 2).sum(dim=0).sqrt()
    worst = float(((lhs_w - rhs_w).abs() / rss_w).max())
    _say(f"[gpu] backward t131072: <dW_UV[h], W_UV[h]> worst difference {worst:.2e} of the root sum of squares")
    assert worst <= 0.05, ("<dW_UV[h], W_UV[h]>", worst)
    sig = torch.sigmoid(dev["gate"].double())
    dg_ref = (1 - sig) * D
    err = float((dg.double() - dg_ref).abs().max())
    assert err <= 1e-4 * float(dg_ref.abs().max()), ("dgate on every row", err)
    assert bool(torch.isfinite(dkv).all()) and bool(torch.isfinite(dW).all())
