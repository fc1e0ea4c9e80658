"""GPU parity of the steps on either side of the path: the W_UK absorption that produces the latent
query (model-coverage page, Implementation Limits, 2nd bullet; KimiK3TextConfig MLA fields), through
the C ABI, against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_indexer_top_index_amd as dsa
import oracle
import testgen as tg
from tests import gpu_util as gu
from tests.parity import check_index_row, check_outputs, gamma

pytestmark = pytest.mark.gpu

TAG_QNOPE, TAG_QPE, TAG_WUK = 60, 61, 62


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _absorb_inputs(seed, rows, H):
    q_nope = tg.normal_bf16(seed, TAG_QNOPE, 0, rows * H * 128, 1.0).reshape(rows, H, 128)
    q_pe = tg.normal_bf16(seed, TAG_QPE, 0, rows * H * 64, 1.0 / 24).reshape(rows, H, 64)
    W_UK = tg.normal_bf16(seed, TAG_WUK, 0, H * 512 * 128, 0.02).reshape(H, 512, 128)
    return q_nope, q_pe, W_UK


@pytest.mark.parametrize("rows,H", [(1000, 96), (333, 16), (1, 96)])
def test_q_absorb_within_one_bf16_step(rows, H):
    """Every latent element is one of the two bf16 neighbours of the exact value (FP32 accumulation is
    far finer than a bf16 step; the second term covers values that cancel to near zero), and the 64
    unrotated dims are copied bit for bit. Ragged row counts cover partial 256-row workgroups."""
    _say(f"[gpu] q absorb rows={rows} H={H}")
    q_nope, q_pe, W_UK = _absorb_inputs(90 + H, rows, H)
    cfg = tg.Config("absorb", 1, [max(rows, 1)], topk=1, H=H, H_I=4, d_I=64)
    shape = gu.shape_of(cfg)
    q = torch.empty((rows, H, 576), dtype=torch.bfloat16, device="cuda")
    dsa.dsa_q_absorb(shape, gu.bf16_np_to_tensor(q_nope), gu.bf16_np_to_tensor(q_pe), gu.bf16_np_to_tensor(W_UK), q)
    torch.cuda.synchronize()
    got = q.view(torch.int16).cpu().numpy().view(np.uint16)
    ref, exact = oracle.q_absorb(q_nope, q_pe, W_UK, want_f64=True)
    assert np.array_equal(got[:, :, 512:], q_pe)
    g = tg.bf16_to_f32(got[:, :, :512]).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    absdot = np.einsum("nhd,hcd->nhc", np.abs(tg.bf16_to_f32(q_nope).astype(np.float64)),
                       np.abs(tg.bf16_to_f32(W_UK).astype(np.float64)))
    assert np.all(np.abs(g - exact) <= ulp + 2 * gamma(128) * absdot)
    same = np.mean(got[:, :, :512] == ref[:, :, :512])
    _say(f"[gpu] q absorb rows={rows} H={H}: {same:.4f} of elements equal the oracle's rounding")


def test_absorbed_query_through_the_fused_forward():
    """q from dsa_q_absorb drives dsa_fused_fwd; outputs match the oracle path fed by the oracle's own
    absorption (differences: the bf16 roundings of q, within the output rule)."""
    cfg = tg.Config("absorb-fused", 93, [900], topk=256, H=96, H_I=64, d_I=128, w_scale=1 / 8, W_UV_std=0.02)
    inp = tg.make_inputs(cfg)
    T, H = cfg.T, cfg.H
    q_nope, q_pe, W_UK = _absorb_inputs(93, T, H)
    shape = gu.shape_of(cfg)
    dev = gu.to_device(inp)
    q = torch.empty((T, H, 576), dtype=torch.bfloat16, device="cuda")
    dsa.dsa_q_absorb(shape, gu.bf16_np_to_tensor(q_nope), gu.bf16_np_to_tensor(q_pe), gu.bf16_np_to_tensor(W_UK), q)
    ws = dsa.alloc_workspace(shape)
    idx = torch.empty((T, cfg.topk), dtype=torch.int32, device="cuda")
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    _say("[gpu] absorbed query through dsa_fused_fwd")
    dsa.dsa_fused_fwd(shape, dev["q_I"], dev["k_I"], dev["w"], q, dev["kv"], dev["W_UV"], dev["gate"], idx, out, ws)
    torch.cuda.synchronize()
    q_ref = oracle.q_absorb(q_nope, q_pe, W_UK)
    rows = np.arange(T)
    ref = oracle.sparse_mla(rows, q_ref, inp["kv"], idx.cpu().numpy(), inp["W_UV"], inp["gate"], cfg.softmax_scale)
    ok, err, mx = check_outputs(gu.bf16_tensor_to_f32(out), ref["out"])
    assert ok, (err, mx)


TAG_X, TAG_WO = 63, 64


@pytest.mark.parametrize("rows,H,d_model", [(1000, 96, 7168), (300, 16, 512), (1, 96, 256)])
def test_o_proj_within_one_bf16_step(rows, H, d_model):
    """y = x W_o^T: every checked element is one of the two bf16 neighbours of the exact value, up to
    the FP32 accumulation bound over K = H * 128 terms. Rows are checked in full for the small shape and
    sampled (first, last, partial tile, random) for the production one."""
    K = H * 128
    _say(f"[gpu] o_proj rows={rows} K={K} d_model={d_model}")
    x = tg.normal_bf16(95, TAG_X, 0, rows * K, 0.5).reshape(rows, K)
    W = tg.normal_bf16(95, TAG_WO, 0, d_model * K, 0.01).reshape(d_model, K)
    cfg = tg.Config("oproj", 1, [rows], topk=1, H=H, H_I=4, d_I=64)
    shape = gu.shape_of(cfg)
    y = torch.empty((rows, d_model), dtype=torch.bfloat16, device="cuda")
    dsa.dsa_o_proj(shape, gu.bf16_np_to_tensor(x), gu.bf16_np_to_tensor(W), y)
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    if rows > 400:
        rng = np.random.default_rng(2)
        sel = np.array(sorted(set([0, 1, 255, 256, 511, 767, 768, rows - 1] + rng.integers(0, rows, 40).tolist())))
    else:
        sel = np.arange(rows)
    ref, exact = oracle.o_proj(x[sel], W, want_f64=True)
    g = tg.bf16_to_f32(got[sel]).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(exact))[1] - 8)
    absdot = np.abs(tg.bf16_to_f32(x[sel]).astype(np.float64)) @ np.abs(tg.bf16_to_f32(W).astype(np.float64)).T
    assert np.all(np.abs(g - exact) <= ulp + 2 * gamma(K) * absdot)
    _say(f"[gpu] o_proj rows={rows} K={K}: {np.mean(got[sel] == ref):.4f} of checked elements equal the oracle's rounding")


def _fused_ln_pair(cfg, inp, g=None, bb=None):
    """Indices of every row from dsa_index_topk and from dsa_index_topk_fused_ln on the same inputs."""
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg, dev.get("cu_seqlens"))
    ws = dsa.alloc_workspace(shape)
    gt = None if g is None else torch.from_numpy(g).cuda()
    bt = None if bb is None else torch.from_numpy(bb).cuda()
    ref = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device="cuda")
    got = torch.full((cfg.T, cfg.topk), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_index_topk(shape, dev["q_I"], dev["k_I"], dev["w"], ref, ws, ln_gamma=gt, ln_beta=bt)
    dsa.dsa_index_topk_fused_ln(shape, dev["q_I"], dev["k_I"], dev["w"], got, ws, ln_gamma=gt, ln_beta=bt)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("case", ["t4096", "t4096-affine", "t8192", "ragged-docs", "const-and-neg-zero"])
def test_fused_ln_indexer_equals_prologue_path(case):
    """dsa_index_topk_fused_ln normalises every key it stages inside the indexer (archdiff blueprint:
    LayerNorm on the indexer key), in double with one rounding to bf16 like the prologue, whose LN(k_I)
    equals the oracle's bit for bit (test_key_layernorm_bit_exact_with_affine). Equal LN bits give equal
    scores, so every row's indices must equal dsa_index_topk's exactly, ties and -1 padding included.
    Cases: the T=4,096 and T=8,192 workloads (the latter with mid-stream selections), an affine weight
    and bias, three documents with a ragged total (the last chunk's raw loads past T), and keys with
    constant rows (zero variance) and negative zeros."""
    g = bb = None
    if case in ("t4096", "t8192"):
        cfg = tg.get_config(case)
    elif case == "t4096-affine":
        cfg = tg.get_config("t4096")
        rng = np.random.default_rng(5)
        g = rng.uniform(0.5, 1.5, cfg.d_I).astype(np.float32)
        bb = rng.uniform(-0.2, 0.2, cfg.d_I).astype(np.float32)
    elif case == "ragged-docs":
        cfg = tg.Config(case, 71, [2500, 1371, 3003], topk=512, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                        W_UV_std=0.02)
    else:
        cfg = tg.Config(case, 72, [1800], topk=300, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                        W_UV_std=0.02)
    inp = tg.make_inputs(cfg)
    if case == "const-and-neg-zero":
        inp["k_I"][::5] = tg.f32_to_bf16(np.full((len(inp["k_I"][::5]), cfg.d_I), 0.75, np.float32))
        inp["k_I"][1::5, ::3] = np.uint16(0x8000)
    _say(f"[gpu] fused-LN indexer {case}: T={cfg.T} docs={cfg.n_docs} k={cfg.topk}")
    ref, got = _fused_ln_pair(cfg, inp, g, bb)
    bad = (ref != got).any(dim=1).nonzero().flatten().tolist()
    assert not bad, f"rows differing from the prologue path: {bad[:10]} ({len(bad)} rows)"
    if case == "const-and-neg-zero":
        # and against the oracle on a spread of rows (the prologue path's own parity covers the rest)
        LNk = oracle.key_layernorm(inp["k_I"], cfg.ln_eps)
        rows = np.arange(cfg.topk, cfg.T, 97)
        o_idx, theta, keff = oracle.topk(rows, inp["q_I"][rows], inp["w"][rows], LNk, cfg.cu_seqlens, cfg.topk)
        g_idx = got.cpu().numpy()
        for j, t in enumerate(rows):
            b = oracle.doc_begin(cfg.cu_seqlens, t)
            msg = check_index_row(g_idx[t], o_idx[j], keff[j], b, t, cfg.topk, inp["q_I"][t], inp["w"][t], LNk, theta[j])
            assert msg is None, msg
