"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Index rule and output rule: see tests/parity.py. Outputs are compared with the oracle's attention
computed on the GPU's own indices, so a legitimate near-tie swap cannot fail the output check.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import dsa_indexer_top_index_amd as dsa
import oracle
import testgen as tg
from tests import gpu_util as gu
from tests.parity import (check_index_row, check_outputs, format_stats, gamma, lower_index_rule_violations,
                          new_stats)

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _check_rows(cfg, keys, qrows, rows, idx_gpu, out_gpu, lse_gpu=None, LNk=None):
    """keys: host k_I/kv/W_UV; qrows: tg.query_rows for `rows`; idx_gpu/out_gpu: host arrays for `rows`."""
    cu = cfg.cu_seqlens
    LNk = oracle.key_layernorm(keys["k_I"], cfg.ln_eps) if LNk is None else LNk
    q_I = qrows["q_I"].reshape(len(rows), cfg.H_I, cfg.d_I)
    w = qrows["w"].reshape(len(rows), cfg.H_I)
    o_idx, theta, keff = oracle.topk(rows, q_I, w, LNk, cu, cfg.topk)
    bad = []
    st = new_stats()
    for j, t in enumerate(rows):
        b = oracle.doc_begin(cu, t)
        msg = check_index_row(idx_gpu[j], o_idx[j], keff[j], b, t, cfg.topk, q_I[j], w[j], LNk, theta[j], stats=st)
        if msg:
            bad.append(msg)
    _say(f"[gpu] {cfg.name} index rule: {format_stats(st)}")
    assert not bad, f"{len(bad)} index rows fail, first: {bad[:3]}"
    q = qrows["q"].reshape(len(rows), cfg.H, 576)
    gate = qrows["gate"].reshape(len(rows), cfg.H)
    ref = oracle.sparse_mla(rows, q, keys["kv"], idx_gpu, keys["W_UV"], gate, cfg.softmax_scale)
    ok, err, mx = check_outputs(out_gpu, ref["out"])
    assert ok, f"output max err {err} > 2e-2 * {mx}"
    if lse_gpu is not None:
        assert np.array_equal(np.isneginf(lse_gpu), np.isneginf(ref["lse"]))
        fin = np.isfinite(ref["lse"])
        assert np.abs(lse_gpu[fin] - ref["lse"][fin]).max() < 5e-3
    same = np.array([set(idx_gpu[j]) == set(o_idx[j]) for j in range(len(rows))])
    return same.mean(), err / mx


_cache = {}


def _inputs(name_or_cfg):
    cfg = tg.get_config(name_or_cfg) if isinstance(name_or_cfg, str) else name_or_cfg
    if cfg.name not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _say(f"[gpu] generating inputs for {cfg.name} (T={cfg.T})")
        keys, dev = gu.device_inputs(cfg)
        _cache[cfg.name] = (cfg, keys, dev)
    return _cache[cfg.name]


def _check_structure(cfg, idx):
    """Every row: min(k, n_t) distinct causal indices of its document in ascending order, then -1."""
    T, k = idx.shape
    t = np.arange(T)
    b = np.zeros(T, dtype=np.int64)
    cu = cfg.cu_seqlens
    for d in range(cfg.n_docs):
        b[cu[d]:cu[d + 1]] = cu[d]
    keff = np.minimum(k, t - b + 1)
    pos = np.arange(k)[None, :]
    live = pos < keff[:, None]
    assert np.all(idx[~live] == -1), "entries past min(k, n_t) are not -1"
    assert np.all(np.where(live, idx >= b[:, None], True)), "index before the document start"
    assert np.all(np.where(live, idx <= t[:, None], True)), "index after the query token"
    inc = np.diff(idx.astype(np.int64), axis=1) > 0
    assert np.all(np.where(live[:, 1:], inc, True)), "row not strictly ascending"


def _run_and_check(cfg, keys, dev, rows, with_lse=True):
    _say(f"[gpu] fused forward {cfg.name}: T={cfg.T} docs={cfg.n_docs} k={cfg.topk} H={cfg.H}")
    res = gu.run_fused(cfg, dev, with_lse=with_lse)
    torch.cuda.synchronize()
    idx = res["topk_idx"].cpu().numpy()
    _check_structure(cfg, idx)
    out = gu.bf16_tensor_to_f32(res["out"])
    lse = res["lse"].cpu().numpy() if with_lse else None
    rows = np.asarray(rows, dtype=np.int64)
    qrows = tg.query_rows(cfg, rows)
    frac, rel = _check_rows(cfg, keys, qrows, rows, idx[rows], out[rows], None if lse is None else lse[rows])
    _say(f"[gpu] {cfg.name}: {len(rows)} rows ok, identical index sets {frac:.3f}, out rel err {rel:.2e}")
    return res, idx, out


# ------------------------------------------------------------------ element-by-element, small sizes

def test_tiny_all_rows():
    cfg, keys, dev = _inputs("tiny")
    _run_and_check(cfg, keys, dev, np.arange(cfg.T))


MID = tg.Config("mid", 7, [2203], topk=512, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24, W_UV_std=0.02)
PACKED_SMALL = tg.Config("packed-small", 8, [700, 1, 33, 900, 256, 257, 1400], topk=256, H=96, H_I=64, d_I=128,
                         w_scale=1 / 8, q_std=1.0, W_UV_std=0.02)


def test_mid_production_shapes_all_rows():
    """96 heads, 64x128 indexer, k=512, T=2203: every row, ragged final query block and key chunk."""
    cfg, keys, dev = _inputs(MID)
    _run_and_check(cfg, keys, dev, np.arange(cfg.T))


def test_packed_small_all_rows():
    """Packed documents (lengths 700, 1, 33, 900, 256, 257, 1400), k=256: every row."""
    cfg, keys, dev = _inputs(PACKED_SMALL)
    _run_and_check(cfg, keys, dev, np.arange(cfg.T))


# ------------------------------------------------------------------ full sizes, sampled rows

def _sample(cfg, extra, n=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(int(x) for x in extra if 0 <= x < cfg.T)
    rows |= set(int(x) for x in rng.integers(0, cfg.T, n))
    return np.array(sorted(rows))


def test_t4096_full_size():
    """Sampled rows plus every 8th row of 3584..4095 (rows whose candidate lists first fill near
    their last key chunk) and of the last 128 rows; the structure of every row."""
    cfg, keys, dev = _inputs("t4096")
    band = list(range(3584, 4096, 8)) + list(range(cfg.T - 128, cfg.T, 8))
    rows = _sample(cfg, [0, 1, 2047, 2048, 2049, cfg.T // 2, cfg.T - 2, cfg.T - 1] + band)
    _run_and_check(cfg, keys, dev, rows)


def test_t8192_full_size():
    """Rows whose candidate lists first overflow (n_t around 3,840..3,904 keys, i.e. the list capacity
    plus one or two chunks), rows that select several times mid-stream (the last 512 rows), the
    longest rows, and a random sample; the structure of every row."""
    cfg, keys, dev = _inputs("t8192")
    first_fill = list(range(3800, 3940, 4))
    many_sel = list(range(cfg.T - 512, cfg.T, 16)) + list(range(cfg.T - 16, cfg.T))
    rows = _sample(cfg, [0, 1, 2047, 2048, 2049, 4095, 4096, 6000] + first_fill + many_sel, n=16)
    _run_and_check(cfg, keys, dev, rows)


def test_dense_check_t2048_equals_dense_attention():
    """T = k = 2048: every row keeps every causal key; outputs equal dense causal attention."""
    cfg, keys, dev = _inputs("dense2048")
    res = gu.run_fused(cfg, dev)
    torch.cuda.synchronize()
    idx = res["topk_idx"].cpu().numpy()
    for t in range(cfg.T):
        assert np.array_equal(idx[t, :t + 1], np.arange(t + 1)) and np.all(idx[t, t + 1:] == -1)
    rows = np.array([0, 1, 5, 1024, 2047])
    qr = tg.query_rows(cfg, rows)
    dense = oracle.dense_causal(rows, qr["q"].reshape(len(rows), cfg.H, 576), keys["kv"], cfg.cu_seqlens,
                                keys["W_UV"], qr["gate"].reshape(len(rows), cfg.H), cfg.softmax_scale)
    ok, err, mx = check_outputs(gu.bf16_tensor_to_f32(res["out"])[rows], dense)
    assert ok, (err, mx)


def test_packed_full_size():
    cfg, keys, dev = _inputs("packed")
    cu = cfg.cu_seqlens
    extra = []
    for d in range(cfg.n_docs):
        b, e = int(cu[d]), int(cu[d + 1])
        extra += [b, b + 1, min(b + 2047, e - 1), min(b + 2048, e - 1), e - 1]
    rows = _sample(cfg, extra, n=8)
    _run_and_check(cfg, keys, dev, rows)


def test_long_context_131072_sampled():
    """Both sides of every 2,048-row boundary (this covers the attention's row chunks, whatever their
    power-of-two size from 2,048 up), the first selected rows, the last 8 rows and a random sample;
    indices, outputs and lse against the oracle, and the structure of every row."""
    cfg, keys, dev = _inputs("t131072")
    bounds = [x for j in range(1, cfg.T // 2048) for x in (2048 * j - 1, 2048 * j)]
    rows = _sample(cfg, [0, 1, 2049, 2050] + bounds + list(range(cfg.T - 8, cfg.T)), n=16)
    assert len(rows) >= 128
    _run_and_check(cfg, keys, dev, rows, with_lse=True)
    _cache.clear()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ edge cases

def test_determinism_and_row_range():
    """Two runs are bit-identical; a query-row range [q_begin, q_end) equals that slice of the full run."""
    cfg, keys, dev = _inputs("t4096")
    a = gu.run_fused(cfg, dev)
    b = gu.run_fused(cfg, dev)
    torch.cuda.synchronize()
    assert torch.equal(a["topk_idx"], b["topk_idx"])
    assert torch.equal(a["out"].view(torch.int16), b["out"].view(torch.int16))
    part = gu.run_fused(cfg, dev, q_begin=1000, q_end=3001)
    torch.cuda.synchronize()
    assert torch.equal(part["topk_idx"], a["topk_idx"][1000:3001])
    assert torch.equal(part["out"].view(torch.int16), a["out"][1000:3001].view(torch.int16))


def test_key_layernorm_bit_exact_with_affine():
    """The LN(k_I) the indexer consumes (first workspace region) equals the oracle's bf16 LN bit for bit."""
    cfg = tg.get_config("t4096")
    keys = tg.key_side(cfg)
    rng = np.random.default_rng(5)
    gamma = rng.uniform(0.5, 1.5, cfg.d_I).astype(np.float32)
    beta = rng.uniform(-0.2, 0.2, cfg.d_I).astype(np.float32)
    for g, bb in [(None, None), (gamma, beta)]:
        shape = gu.shape_of(cfg, q_begin=cfg.T - 4, q_end=cfg.T)
        ws = dsa.alloc_workspace(shape)
        q_I = gu.bf16_np_to_tensor(tg.query_rows(cfg, range(cfg.T - 4, cfg.T))["q_I"])
        w = gu.bf16_np_to_tensor(tg.query_rows(cfg, range(cfg.T - 4, cfg.T))["w"])
        idx = torch.empty((4, cfg.topk), dtype=torch.int32, device="cuda")
        dsa.dsa_index_topk(shape, q_I, gu.bf16_np_to_tensor(keys["k_I"]), w, idx, ws,
                           ln_gamma=None if g is None else torch.from_numpy(g).cuda(),
                           ln_beta=None if bb is None else torch.from_numpy(bb).cuda())
        torch.cuda.synchronize()
        lnk_gpu = ws[: cfg.T * cfg.d_I * 2].view(torch.int16).cpu().numpy().view(np.uint16).reshape(cfg.T, cfg.d_I)
        lnk_ref = oracle.key_layernorm(keys["k_I"], cfg.ln_eps, g, bb)
        assert np.array_equal(lnk_gpu, lnk_ref)


def _small_cfg(name, seed, lens, topk, H=16, H_I=4, d_I=64, **kw):
    return tg.Config(name, seed, lens, topk=topk, H=H, H_I=H_I, d_I=d_I, w_scale=kw.pop("w_scale", 0.5), **kw)


@pytest.mark.parametrize("case", ["T1", "k1", "k3-negw", "ties", "const-keys", "few-keys", "few-keys-96"])
def test_edge_cases(case):
    if case == "T1":
        cfg = _small_cfg("T1", 40, [1], topk=1, H=96, H_I=64, d_I=128)
    elif case == "k1":
        cfg = _small_cfg("k1", 41, [300], topk=1)
    elif case == "k3-negw":
        cfg = _small_cfg("k3", 42, [97, 200], topk=3, w_scale=-1.0)
    elif case == "few-keys-96":
        cfg = _small_cfg(case, 46, [1500, 700], topk=300, H=96, H_I=64, d_I=128, w_scale=1 / 8, q_std=1 / 24,
                         W_UV_std=0.02)
    else:
        cfg = _small_cfg(case, 43, [333], topk=40)
    inp = tg.make_inputs(cfg)
    if case == "ties":  # duplicated key rows: equal scores, resolved to the lower index
        inp["k_I"][1::3] = inp["k_I"][0::3][: len(inp["k_I"][1::3])]
    if case == "const-keys":  # LN of a constant row is 0: every score is exactly +0
        inp["k_I"][:] = tg.f32_to_bf16(np.full(inp["k_I"].shape, 0.5, np.float32))
    if case.startswith("few-keys"):  # 7 distinct key rows repeated: every k-th score is an exact tie
        inp["k_I"][:] = inp["k_I"][np.arange(cfg.T) % 7]
    dev = gu.to_device(inp)
    _say(f"[gpu] edge case {case}: T={cfg.T} k={cfg.topk}")
    res = gu.run_fused(cfg, dev, with_lse=True)
    torch.cuda.synchronize()
    rows = np.arange(cfg.T)
    keys = {k: inp[k] for k in ["k_I", "kv", "W_UV"]}
    qrows = {k: inp[k].reshape(cfg.T, -1) for k in ["q_I", "w", "q", "gate"]}
    idx = res["topk_idx"].cpu().numpy()
    _check_rows(cfg, keys, qrows, rows, idx, gu.bf16_tensor_to_f32(res["out"]), res["lse"].cpu().numpy())
    if case in ("ties", "const-keys") or case.startswith("few-keys"):
        # Equal scores must go to the lower index: no kept key may follow a dropped key of equal
        # oracle score (the duplicated keys get bit-identical scores on both sides).
        LNk = oracle.key_layernorm(inp["k_I"], cfg.ln_eps)
        o_idx, theta, keff = oracle.topk(rows, inp["q_I"], inp["w"], LNk, cfg.cu_seqlens, cfg.topk)
        viol = []
        for t in rows:
            b = oracle.doc_begin(cfg.cu_seqlens, t)
            if t - b + 1 <= cfg.topk:
                continue
            S = oracle.index_scores(inp["q_I"][t], inp["w"][t], LNk, b, t)
            viol += [(int(t),) + v for v in lower_index_rule_violations(idx[t], S, b, t)]
        assert not viol, f"lower-index tie rule broken: {viol[:5]}"
        if case == "const-keys":
            assert np.array_equal(idx, o_idx)
        if case.startswith("few-keys"):
            # At most seven distinct scores per row, and the k-th one is shared by a large group of
            # keys, so the tie rule alone decides which of the group are kept. Where every other
            # distinct score lies far from theta (beyond the near-tie band, or beyond the FP32 floor
            # when theta is 0) the set is fixed exactly and must equal the oracle's.
            exact, long_rows = 0, 0
            for j, t in enumerate(rows):
                b = oracle.doc_begin(cfg.cu_seqlens, t)
                if t - b + 1 <= cfg.topk:
                    continue
                long_rows += 1
                S = oracle.index_scores(inp["q_I"][t], inp["w"][t], LNk, b, t).astype(np.float64)
                th = float(theta[j])
                others = np.unique(S[S != th])
                sep = 1e-3 * abs(th) if th != 0 else 2 * gamma(cfg.d_I + cfg.H_I) * float(
                    oracle.index_score_scale(inp["q_I"][t], inp["w"][t], LNk, b, t).max())
                if others.size == 0 or np.min(np.abs(others - th)) > sep:
                    exact += 1
                    assert np.array_equal(idx[t], o_idx[j]), f"row {t}: tie group resolved differently"
            _say(f"[gpu] {case}: {exact} of {long_rows} selecting rows fixed by the tie rule, all equal to the oracle")
            assert exact >= 0.9 * long_rows


def test_sparse_mla_caller_indices():
    """dsa_sparse_mla_fwd with caller indices: -1, out-of-range entries and duplicates; only the first
    min(k, n_t) entries of a row are read."""
    cfg = _small_cfg("mla-idx", 44, [500], topk=64, H=96)
    inp = tg.make_inputs(cfg)
    rng = np.random.default_rng(3)
    T, k = cfg.T, cfg.topk
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        keff = min(k, t + 1)
        row = rng.integers(0, t + 1, keff).astype(np.int32)  # duplicates allowed
        kill = rng.random(keff) < 0.2
        row[kill] = rng.choice([-1, -7, T, T + 100], kill.sum())
        idx[t, :keff] = row
    idx[7, :] = -1  # a row with no usable entry: zeros, lse -inf
    dev = gu.to_device(inp)
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_workspace(shape)
    out = torch.empty((T, cfg.H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, cfg.H), dtype=torch.float32, device="cuda")
    _say("[gpu] sparse_mla_fwd with caller indices")
    dsa.dsa_sparse_mla_fwd(shape, dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), dev["W_UV"], dev["gate"], out,
                           ws, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.sparse_mla(np.arange(T), inp["q"], inp["kv"], idx, inp["W_UV"], inp["gate"], cfg.softmax_scale)
    got = gu.bf16_tensor_to_f32(out)
    ok, err, mx = check_outputs(got, ref["out"])
    assert ok, (err, mx)
    lse_g = lse.cpu().numpy()
    empty = np.isneginf(ref["lse"])
    assert empty[7].all() and np.all(got[7] == 0)
    assert np.array_equal(np.isneginf(lse_g), empty)
    assert np.abs(lse_g[~empty] - ref["lse"][~empty]).max() < 5e-3


@pytest.mark.parametrize("H", [96, 16])
def test_sparse_mla_logit_growth_redo(H):
    """Rows whose logits grow far beyond the first key tile's maximum (more than 2^64 in base 2):
    the kernel redoes such a row against exact per-head maxima. One head's query is twice the
    latent row of the query token itself, which is the last selected key of its row; the result
    must still match the oracle, and the construction is checked to reach the redo condition."""
    cfg = _small_cfg(f"growth{H}", 45 + H, [300], topk=96, H=H)
    inp = tg.make_inputs(cfg)
    T, k, big = cfg.T, cfg.topk, 5
    kv32 = tg.bf16_to_f32(inp["kv"]).astype(np.float64)
    q = inp["q"].copy()
    q[:, big, :] = tg.f32_to_bf16((2.0 * kv32).astype(np.float32))  # exact: a power-of-two scale
    idx = np.full((T, k), -1, np.int32)
    for t in range(T):
        keff = min(k, t + 1)
        idx[t, :keff] = np.arange(t - keff + 1, t + 1, dtype=np.int32)  # ascending, the token itself last
    # base-2 logits of the big head: first 16-key tile's maximum against the token's own key
    log2e = 1.0 / np.log(2.0)
    qb = tg.bf16_to_f32(q[:, big, :]).astype(np.float64)
    gaps = []
    for t in range(16, T):
        first = idx[t, :16]
        m0 = (cfg.softmax_scale * log2e * (kv32[first] @ qb[t])).max()
        gaps.append(cfg.softmax_scale * log2e * (kv32[t] @ qb[t]) - m0)
    gaps = np.array(gaps)
    assert (gaps > 64.0).sum() > 200 and gaps.max() < 127.0, (gaps.min(), gaps.max())
    dev = gu.to_device(dict(inp, q=q))
    shape = gu.shape_of(cfg)
    ws = dsa.alloc_workspace(shape)
    out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, H), dtype=torch.float32, device="cuda")
    _say(f"[gpu] sparse_mla_fwd logit-growth redo, H={H}")
    dsa.dsa_sparse_mla_fwd(shape, dev["q"], dev["kv"], torch.from_numpy(idx).cuda(), dev["W_UV"], dev["gate"], out,
                           ws, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.sparse_mla(np.arange(T), q, inp["kv"], idx, inp["W_UV"], inp["gate"], cfg.softmax_scale)
    ok, err, mx = check_outputs(gu.bf16_tensor_to_f32(out), ref["out"])
    assert ok, (err, mx)
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() < 5e-3
