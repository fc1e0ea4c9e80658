"""GPU parity of the FP8 indexer (model-coverage page, Implementation Limits, 2nd bullet; the recipe
is this build's reading: power-of-two row scales, OCP E4M3 with ties to even, exact products summed
in FP32) against the oracle's FP8 top-k, through the C ABI.

The operand quantisation is compared bit for bit (codes and scales), on constructed rows that put
values exactly on every rounding midpoint of E4M3, one bf16 step off them, on subnormals and on zero
and tiny rows, and on the quantised LN(k_I) the indexer leaves in its workspace. Index rows use the
near-tie rule of tests/parity.py on the oracle's FP8 scores."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_indexer_top_index_amd as dsa
import oracle
import testgen as tg
from tests import gpu_util as gu
from tests.parity import check_index_row, format_stats, new_stats
from tests.test_gpu_parity import _check_structure

pytestmark = pytest.mark.gpu

bf = tg.f32_to_bf16


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _quant_rows():
    """Rows of 128 bf16 values: each rounding case of E4M3 at several row scales."""
    codes = np.arange(0x7F)
    vals = np.array([oracle.e4m3_decode(c) for c in codes])
    mids = (vals[:-1] + vals[1:]) / 2                      # 126 exact ties
    rng = np.random.default_rng(21)
    rows = []
    for e in (-20, -3, 0, 4):
        s = 2.0 ** e
        for chunk in (mids[:63], mids[63:]):
            r = np.zeros(128)
            r[0] = 448 * s                                   # fixes the row's scale 2^e
            r[1:1 + len(chunk)] = chunk * s * rng.choice([-1, 1], len(chunk))
            r[1 + len(chunk):] = vals[rng.integers(0, 0x7F, 127 - len(chunk))] * s   # exact codes
            rows.append(r)
        # one bf16 step either side of each midpoint
        for sign in (-1, 1):
            r = np.zeros(128)
            r[0] = -448 * s
            m = mids[rng.integers(0, len(mids), 127)]
            step = 2.0 ** (np.floor(np.log2(m)) - 7)        # bf16 has 8 significant bits
            r[1:] = (m + sign * step) * s
            rows.append(r)
    rows.append(np.zeros(128))
    tiny = np.zeros(128)
    tiny[:5] = [2.0 ** -130, -2.0 ** -131, 2.0 ** -133, 3 * 2.0 ** -132, 2.0 ** -126]
    rows.append(tiny)
    x = np.stack(rows).astype(np.float32)
    x = np.concatenate([x, rng.standard_normal((1000, 128)).astype(np.float32) * np.ldexp(1.0, rng.integers(-8, 9, (1000, 1))).astype(np.float32)])
    xb = bf(x)
    assert np.array_equal(tg.bf16_to_f32(xb)[:len(rows)], x[:len(rows)])  # the constructed values are exact in bf16
    return xb


def test_quantize_fp8_bit_exact():
    x = _quant_rows()
    _say(f"[gpu] dsa_quantize_fp8 on {len(x)} rows")
    xt = gu.bf16_np_to_tensor(x)
    q8 = torch.empty((len(x), 128), dtype=torch.uint8, device="cuda")
    sc = torch.empty(len(x), dtype=torch.float32, device="cuda")
    dsa.dsa_quantize_fp8(xt, q8, sc)
    torch.cuda.synchronize()
    ref_q, ref_e = oracle.quantize_fp8_rows(x)
    got_q = q8.cpu().numpy()
    bad = np.argwhere(got_q != ref_q)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:5].tolist()}: gpu {got_q[tuple(bad[0])]:#x} " \
                          f"oracle {ref_q[tuple(bad[0])]:#x}"
    assert np.array_equal(sc.cpu().numpy(), np.ldexp(np.float32(1), ref_e).astype(np.float32))


def _fp8_cases():
    mid = tg.Config("fp8-mid", 81, [2203], topk=512, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                    W_UV_std=0.02)
    packed = tg.Config("fp8-packed", 82, [700, 1, 33, 900, 256, 257, 1400], topk=256, H=96, H_I=64, d_I=128,
                       w_scale=1 / 8, q_std=1.0, W_UV_std=0.02)
    return {"mid": (mid, None), "mid-affine": (mid, "affine"), "packed-small": (packed, None),
            "t4096": (tg.get_config("t4096"), "sample"), "t131072": (tg.get_config("t131072"), "sample")}


def _ws_fp8_keys(ws, cfg):
    """The indexer's E4M3 codes and scales of LN(k_I) in the workspace (regions after LNk, the slot
    flags and the candidate slots)."""
    al = lambda v: (v + 255) // 256 * 256
    off = al((cfg.T + 128) * cfg.d_I * 2) + 1024 + 256 * 8 * 2 * 4672 * 4
    k8 = ws[off: off + cfg.T * cfg.d_I].cpu().numpy().reshape(cfg.T, cfg.d_I)
    off_s = off + al((cfg.T + 128) * cfg.d_I)
    sk = ws[off_s: off_s + 4 * cfg.T].view(torch.float32).cpu().numpy()
    return k8, sk


@pytest.mark.parametrize("case", ["mid", "mid-affine", "packed-small", "t4096", "t131072"])
def test_fp8_indexer_parity(case):
    """mid-affine: the key LayerNorm with a weight and a bias, which the quantisation then sees."""
    cfg, mode = _fp8_cases()[case]
    _say(f"[gpu] fp8 indexer {case}: T={cfg.T} docs={cfg.n_docs} k={cfg.topk}")
    keys, dev = gu.device_inputs(cfg)
    shape = gu.shape_of(cfg, dev["cu_seqlens"])
    ws = dsa.alloc_workspace(shape)
    ln_g = ln_b = None
    if mode == "affine":
        rng = np.random.default_rng(12)
        ln_g = rng.uniform(0.5, 1.5, cfg.d_I).astype(np.float32)
        ln_b = rng.uniform(-0.2, 0.2, cfg.d_I).astype(np.float32)
    ln_kw = {} if ln_g is None else {"ln_gamma": torch.from_numpy(ln_g).cuda(), "ln_beta": torch.from_numpy(ln_b).cuda()}
    idx_t = torch.empty((cfg.T, cfg.topk), dtype=torch.int32, device="cuda")
    dsa.dsa_index_topk_fp8(shape, dev["q_I"], dev["k_I"], dev["w"], idx_t, ws, **ln_kw)
    idx2 = torch.empty_like(idx_t)
    dsa.dsa_index_topk_fp8(shape, dev["q_I"], dev["k_I"], dev["w"], idx2, ws, **ln_kw)
    torch.cuda.synchronize()
    assert torch.equal(idx_t, idx2), "FP8 indexer is not deterministic"
    idx = idx_t.cpu().numpy()
    _check_structure(cfg, idx)
    LNk = oracle.key_layernorm(keys["k_I"], cfg.ln_eps, ln_g, ln_b)
    k8, ek = oracle.quantize_fp8_rows(LNk)
    g8, gsk = _ws_fp8_keys(ws, cfg)
    assert np.array_equal(g8, k8) and np.array_equal(gsk, np.ldexp(np.float32(1), ek).astype(np.float32))
    if mode == "sample":
        rng = np.random.default_rng(1)
        bounds = [x for j in range(1, cfg.T // 2048) for x in (2048 * j - 1, 2048 * j)]
        extra = [0, 1, 2047, 2048, 2049, cfg.T - 2, cfg.T - 1] + (bounds[::4] if cfg.T > 8192 else list(range(3584, 4096, 16)))
        rows = np.array(sorted(set(x for x in extra if 0 <= x < cfg.T) | set(rng.integers(0, cfg.T, 16).tolist())))
    else:
        rows = np.arange(cfg.T)
    qr = tg.query_rows(cfg, rows)
    q_I = qr["q_I"].reshape(len(rows), cfg.H_I, cfg.d_I)
    w = qr["w"].reshape(len(rows), cfg.H_I)
    q8, eq = oracle.quantize_fp8_rows(q_I)
    o_idx, theta, keff = oracle.topk_fp8(rows, q8, eq, w, k8, ek, cfg.cu_seqlens, cfg.topk)
    dec = np.array([oracle.e4m3_decode(c) if c not in (0x7F, 0xFF) else 0.0 for c in range(256)])

    def scores(qr_, wr, L, b, t):
        return oracle.index_scores_fp8(qr_[0], qr_[1], wr, k8, ek, b, t)

    def scale(qr_, wr, L, b, t):
        qd = dec[qr_[0]] * np.ldexp(1.0, qr_[1])[:, None]
        kd = dec[k8[b:t + 1]] * np.ldexp(1.0, ek[b:t + 1])[:, None]
        return (np.abs(tg.bf16_to_f32(wr)).astype(np.float64)[None, :] * (np.abs(kd) @ np.abs(qd).T)).sum(1)

    st = new_stats()
    bad = []
    for j, t in enumerate(rows):
        b = oracle.doc_begin(cfg.cu_seqlens, t)
        msg = check_index_row(idx[t], o_idx[j], keff[j], b, t, cfg.topk, (q8[j], eq[j]), w[j], None, theta[j],
                              stats=st, score_fn=scores, scale_fn=scale, dims=(cfg.H_I, cfg.d_I))
        if msg:
            bad.append(msg)
    _say(f"[gpu] fp8 {case} index rule: {format_stats(st)}")
    assert not bad, f"{len(bad)} rows fail, first: {bad[:3]}"
    # how far the FP8 selection is from the BF16 one on the same rows (information only)
    o16, _, _ = oracle.topk(rows, q_I, w, LNk, cfg.cu_seqlens, cfg.topk)
    sel = keff > 0
    ov = np.mean([len(set(o16[j][:keff[j]]) & set(o_idx[j][:keff[j]])) / keff[j] for j in range(len(rows)) if sel[j]])
    _say(f"[gpu] fp8 {case}: mean overlap with the BF16 selection {ov:.4f}")
    del dev, ws
    torch.cuda.empty_cache()
