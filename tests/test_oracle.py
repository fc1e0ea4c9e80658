"""Pins for the CPU oracle: each test checks it against something other than itself.

Pages cited: the Kimi-K3.1-Pro model-coverage page ("KC"), the archdiff "Kimi K3.1 Pro" blueprint
("AD"), and the kimi_k3 API index ("API").
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import testgen as tg
from tests.parity import check_index_row, gamma

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
bf = tg.f32_to_bf16
f32 = tg.bf16_to_f32


def _bf(a):
    return bf(np.asarray(a, dtype=np.float32))


# ---------------------------------------------------------------- generator (not the method)

def test_generator_rows_are_counter_based():
    cfg = tg.get_config("tiny")
    full = tg.make_inputs(cfg)
    rows = [0, 1, 2, 511, 1023]
    part = tg.query_rows(cfg, rows)
    for name in ["q_I", "w", "q", "gate"]:
        assert np.array_equal(part[name].reshape(len(rows), -1), full[name][rows].reshape(len(rows), -1))


def test_generator_distributions():
    x = f32(tg.normal_bf16(9, 1, 0, 200000, 1.0))
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    u = f32(tg.uniform_bf16(9, 3, 0, 200000, 0.125))
    assert u.min() >= 0 and u.max() <= 0.125 and abs(u.mean() - 0.0625) < 0.001
    kv = f32(tg.key_side(tg.get_config("tiny"))["kv"])
    rms = np.sqrt((kv.astype(np.float64) ** 2).mean(1))
    assert np.all(np.abs(rms - 1) < 0.01)


def test_packed_lengths_in_range():
    c = tg.get_config("packed")
    assert len(c.doc_lens) == 8 and all(1024 <= n <= 8192 for n in c.doc_lens)
    assert c.T == sum(c.doc_lens) and max(c.doc_lens) > 2048


# ---------------------------------------------------------------- LayerNorm on the indexer key (AD)

def test_layernorm_matches_torch_float64():
    """P9: before rounding, the oracle's LN equals torch's layer_norm in float64."""
    k_I = tg.normal_bf16(3, 2, 0, 300 * 128, 1.0).reshape(300, 128)
    LNk, pre = oracle.key_layernorm(k_I, 1e-5, want_pre=True)
    x = torch.from_numpy(f32(k_I).astype(np.float64))
    ref = torch.nn.functional.layer_norm(x, (128,), eps=1e-5).numpy()
    assert np.abs(pre - ref).max() < 1e-12
    # Rounding: LNk is a bf16 value within half a bf16 ulp of the double value (round to nearest).
    y = f32(LNk).astype(np.float64)
    ulp = np.ldexp(1.0, (np.frexp(np.abs(pre))[1] - 8))
    assert np.all(np.abs(y - pre) <= ulp / 2 + 1e-300)


def test_layernorm_affine_and_closed_forms():
    d = 64
    rows = np.zeros((3, d), dtype=np.float32)
    rows[0] = 1.5                                   # constant row -> all zeros
    rows[1] = np.where(np.arange(d) % 2 == 0, 2.0, -2.0)  # mean 0, var 4 -> +-2/sqrt(4+eps)
    rows[2] = np.arange(d) - 31.5                   # symmetric ramp
    k_I = _bf(rows)
    gamma_ = np.full(d, 2.0, np.float32)
    beta_ = np.full(d, -0.5, np.float32)
    LNk, pre = oracle.key_layernorm(k_I, 1e-5, gamma_, beta_, want_pre=True)
    assert np.all(pre[0] == -0.5)
    expect = 2.0 * np.where(np.arange(d) % 2 == 0, 1, -1) * 2 / math.sqrt(4 + 1e-5) - 0.5
    assert np.abs(pre[1] - expect).max() < 1e-12
    var = ((np.arange(d) - 31.5) ** 2).mean()
    assert np.abs(pre[2] - (2 * (np.arange(d) - 31.5) / math.sqrt(var + 1e-5) - 0.5)).max() < 1e-12


# ---------------------------------------------------------------- indexer scores (KC bullet 2)

def test_hand_worked_indexer_example():
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    k_I = _bf(g["k_I"])
    LNk = oracle.key_layernorm(k_I, 1e-5)
    assert np.array_equal(f32(LNk), np.array(g["LNk_expected"], np.float32))
    cu = np.array([0, 5], np.int32)
    for case in g["cases"]:
        q = _bf(case["q_I"])
        w = _bf(case["w"])
        t = case["t"]
        S = oracle.index_scores(q, w, LNk, 0, t)
        assert np.array_equal(S, np.array(case["scores_expected"], np.float32)), case["name"]
        for k, exp_idx in case["topk"].items():
            k = int(k)
            idx, theta, keff = oracle.topk([t], q[None], w[None], LNk, cu, k)
            want = exp_idx + [-1] * (k - len(exp_idx)) if len(exp_idx) < k else exp_idx
            assert list(idx[0]) == want, (case["name"], k)
            if str(k) in case["theta"]:
                assert theta[0] == case["theta"][str(k)]


def test_scores_one_hot_closed_form():
    """q_I[h] = c_h e_{i_h} and one-hot w: S(s) = w * max(c * LNk[s, i], 0) exactly."""
    H_I, d_I, T = 4, 64, 40
    LNk = _bf(np.random.default_rng(0).standard_normal((T, d_I)))
    for h_star, i_star, c, wv in [(0, 0, 1.0, 1.0), (3, 63, -2.0, 0.5), (2, 17, 4.0, -1.5)]:
        q = np.zeros((H_I, d_I), np.float32)
        for h in range(H_I):
            q[h, (h * 7) % d_I] = 3.0          # other heads are live but carry zero weight
        q[h_star] = 0
        q[h_star, i_star] = c
        w = np.zeros(H_I, np.float32)
        w[h_star] = wv
        S = oracle.index_scores(_bf(q), _bf(w), LNk, 0, T - 1)
        want = np.float32(wv) * np.maximum(np.float32(c) * f32(LNk[:, i_star]), 0)
        assert np.array_equal(S, want.astype(np.float32))


def test_scores_exact_within_fp32_bound():
    """Scores equal the exact value (rational arithmetic) within the FP32 accumulation bound."""
    from fractions import Fraction
    rng = np.random.default_rng(1)
    H_I, d_I = 4, 64
    LNk = _bf(rng.standard_normal((6, d_I)))
    q = _bf(rng.standard_normal((H_I, d_I)))
    w = _bf(rng.uniform(-1, 1, H_I))
    S = oracle.index_scores(q, w, LNk, 0, 5)
    sc = oracle.index_score_scale(q, w, LNk, 0, 5)
    qf, wf, kf = f32(q), f32(w), f32(LNk)
    for s in range(6):
        exact = Fraction(0)
        for h in range(H_I):
            dot = sum(Fraction(float(qf[h, i])) * Fraction(float(kf[s, i])) for i in range(d_I))
            exact += Fraction(float(wf[h])) * max(dot, Fraction(0))
        assert abs(float(S[s]) - float(exact)) <= gamma(d_I + H_I) * sc[s] + 1e-30


def test_score_scale_exact_rational():
    """oracle_index_score_scale equals sum_h |w_h| sum_i |q_I[h,i] LNk[s,i]| computed in exact rational
    arithmetic, to double rounding (it sets the parity floor where the k-th score is exactly 0)."""
    from fractions import Fraction
    rng = np.random.default_rng(4)
    for H_I, d_I in [(4, 64), (64, 128)]:
        n = 5
        LNk = _bf(rng.standard_normal((n, d_I)))
        q = _bf(rng.standard_normal((H_I, d_I)))
        w = _bf(rng.uniform(-1, 1, H_I))        # negative weights count by magnitude
        sc = oracle.index_score_scale(q, w, LNk, 1, n - 1)
        assert sc.shape == (n - 1,)
        qf, wf, kf = f32(q), f32(w), f32(LNk)
        for s in range(1, n):
            exact = Fraction(0)
            for h in range(H_I):
                dot = sum(abs(Fraction(float(qf[h, i])) * Fraction(float(kf[s, i]))) for i in range(d_I))
                exact += abs(Fraction(float(wf[h]))) * dot
            assert abs(Fraction(float(sc[s - 1])) - exact) <= Fraction(1, 2 ** 40) * exact
    # one-hot closed form: a single nonzero product
    q = np.zeros((4, 64), np.float32)
    q[2, 5] = -3.0
    w = np.array([9, 9, -0.5, 9], np.float32)
    LNk = np.zeros((2, 64), np.float32)
    LNk[1, 5] = 1.25
    assert list(oracle.index_score_scale(_bf(q), _bf(w), _bf(LNk), 0, 1)) == [0.0, 0.5 * 3.0 * 1.25]


def test_lower_index_rule_helper():
    """The tie-rule check used by the GPU tests flags a kept higher index over a dropped equal lower one."""
    from tests.parity import lower_index_rule_violations
    S = np.array([5, 3, 3, 3, 1, 3], np.float32)   # keys 10..15
    assert lower_index_rule_violations([10, 11, 12, -1], S, 10, 15) == []
    assert lower_index_rule_violations([10, 11, 13, -1], S, 10, 15) == [(11, 3.0)]
    assert lower_index_rule_violations([10, 11, 12, 13, 15], S, 10, 15) == []
    assert lower_index_rule_violations([10, 15], S, 10, 15) == [(11, 3.0)]
    assert lower_index_rule_violations([10, 14], S, 10, 15) == []


def test_scores_scaling_and_head_permutation():
    """P8: scaling q_I or w by 2 doubles S exactly; permuting heads keeps S within the FP32 bound."""
    rng = np.random.default_rng(2)
    H_I, d_I, T = 4, 64, 50
    LNk = oracle.key_layernorm(_bf(rng.standard_normal((T, d_I))))
    q = _bf(rng.standard_normal((H_I, d_I)))
    w = _bf(rng.uniform(0, 0.5, H_I))
    S = oracle.index_scores(q, w, LNk, 0, T - 1)
    assert np.array_equal(oracle.index_scores(_bf(2 * f32(q)), w, LNk, 0, T - 1), 2 * S)
    assert np.array_equal(oracle.index_scores(q, _bf(2 * f32(w)), LNk, 0, T - 1), 2 * S)
    perm = [2, 0, 3, 1]
    Sp = oracle.index_scores(q[perm], w[perm], LNk, 0, T - 1)
    sc = oracle.index_score_scale(q, w, LNk, 0, T - 1)
    assert np.all(np.abs(Sp - S) <= 2 * gamma(d_I + H_I) * sc)


# ---------------------------------------------------------------- hard top-k (KC summary, bullets 3-4)

def _brute_topk_is_dominant(S, kept, b, t):
    """The top-k set is the unique set whose members all beat all non-members in (score desc, idx asc)."""
    kept = set(kept)
    out = [s for s in range(b, t + 1) if s not in kept]
    for u in kept:
        for v in out:
            su, sv = S[u - b], S[v - b]
            if not (su > sv or (su == sv and u < v)):
                return False
    return True


@pytest.mark.parametrize("k", [1, 3, 8, 40])
def test_topk_brute_force_tiny(k):
    """P1: brute force on tiny inputs, plus numpy lexsort and torch stable sort as library cross-checks."""
    rng = np.random.default_rng(10 + k)
    T, H_I, d_I = 40, 4, 64
    LNk = oracle.key_layernorm(_bf(rng.standard_normal((T, d_I))))
    rows = np.arange(T)
    q = _bf(rng.standard_normal((T, H_I, d_I)))
    w = _bf(rng.uniform(0, 0.5, (T, H_I)))
    cu = np.array([0, T], np.int32)
    idx, theta, keff = oracle.topk(rows, q, w, LNk, cu, k)
    for t in range(T):
        n = t + 1
        assert keff[t] == min(k, n)
        kept = [int(x) for x in idx[t] if x >= 0]
        assert kept == sorted(kept) and len(kept) == keff[t]
        S = oracle.index_scores(q[t], w[t], LNk, 0, t)
        assert _brute_topk_is_dominant(S, kept, 0, t)
        order = np.lexsort((np.arange(n), -S.astype(np.float64)))[: min(k, n)]
        assert sorted(order.tolist()) == kept
        tv, ti = torch.sort(torch.from_numpy(-S), stable=True)
        assert sorted(ti[: min(k, n)].tolist()) == kept


def test_topk_constructed_ties():
    """P2: equal scores resolve to the lower index, exactly."""
    T, H_I, d_I, k = 30, 4, 64, 5
    rng = np.random.default_rng(3)
    same = rng.standard_normal(d_I)
    k_I = _bf(np.tile(same, (T, 1)))                 # duplicated rows: all scores equal
    LNk = oracle.key_layernorm(k_I)
    q = _bf(rng.standard_normal((T, H_I, d_I)))
    w = _bf(rng.uniform(0, 1, (T, H_I)))
    idx, _, _ = oracle.topk(np.arange(T), q, w, LNk, np.array([0, T], np.int32), k)
    for t in range(k, T):
        assert list(idx[t]) == list(range(k))
    const = _bf(np.full((T, d_I), 0.75))              # LN of a constant row is 0, so S = +0
    LNc = oracle.key_layernorm(const)
    assert np.all(f32(LNc) == 0)
    idx, theta, _ = oracle.topk(np.arange(T), q, w, LNc, np.array([0, 10, T], np.int32), k)
    assert np.all(theta[np.arange(T) >= 10 + k] == 0)
    for t in range(10 + k, T):
        assert list(idx[t]) == list(range(10, 10 + k))


def test_topk_short_rows_keep_all_and_respect_documents():
    """P3: a row with at most k causal keys keeps them all (KC bullet 4); keys never cross documents."""
    cfg = tg.Config("mini", 11, [50, 7, 300, 1], topk=64, H=16, H_I=4, d_I=64)
    inp = tg.make_inputs(cfg)
    LNk = oracle.key_layernorm(inp["k_I"])
    cu = cfg.cu_seqlens
    rows = np.arange(cfg.T)
    idx, theta, keff = oracle.topk(rows, inp["q_I"], inp["w"], LNk, cu, cfg.topk)
    for t in rows:
        b = oracle.doc_begin(cu, t)
        n = t - b + 1
        kept = idx[t][: keff[t]]
        assert keff[t] == min(n, cfg.topk)
        assert kept.min() >= b and kept.max() <= t
        if n <= cfg.topk:
            assert list(kept) == list(range(b, t + 1)) and np.isnan(theta[t])


def test_topk_scale_invariance():
    """P8: doubling q_I or w leaves the index sets unchanged."""
    cfg = tg.get_config("tiny")
    inp = tg.make_inputs(cfg)
    LNk = oracle.key_layernorm(inp["k_I"])
    rows = np.arange(600, 1024, 7)
    a, _, _ = oracle.topk(rows, inp["q_I"][rows], inp["w"][rows], LNk, inp["cu_seqlens"], cfg.topk)
    b, _, _ = oracle.topk(rows, _bf(2 * f32(inp["q_I"][rows])), inp["w"][rows], LNk, inp["cu_seqlens"], cfg.topk)
    c, _, _ = oracle.topk(rows, inp["q_I"][rows], _bf(2 * f32(inp["w"][rows])), LNk, inp["cu_seqlens"], cfg.topk)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_near_tie_checker_flags_planted_mistake():
    """The index rule accepts the oracle's own rows and rejects a planted non-tie swap."""
    cfg = tg.get_config("tiny")
    inp = tg.make_inputs(cfg)
    LNk = oracle.key_layernorm(inp["k_I"])
    t = 900
    idx, theta, keff = oracle.topk([t], inp["q_I"][[t]], inp["w"][[t]], LNk, inp["cu_seqlens"], cfg.topk)
    row = idx[0].copy()
    assert check_index_row(row, idx[0], keff[0], 0, t, cfg.topk, inp["q_I"][t], inp["w"][t], LNk, theta[0]) is None
    S = oracle.index_scores(inp["q_I"][t], inp["w"][t], LNk, 0, t)
    kept = set(row.tolist())
    worst_out = min((s for s in range(t + 1) if s not in kept), key=lambda s: S[s])
    best_in = max(kept, key=lambda s: S[s])
    bad = np.array(sorted((kept - {best_in}) | {worst_out}), np.int32)
    assert check_index_row(bad, idx[0], keff[0], 0, t, cfg.topk, inp["q_I"][t], inp["w"][t], LNk, theta[0]) is not None


# ---------------------------------------------------------------- sparse MLA, V up-projection, gate

def _hand_case(case):
    H, T = 1, len(case["kv_rows"])
    kv = np.zeros((T, 576), np.float32)
    for r, entries in enumerate(case["kv_rows"]):
        for c, v in entries:
            kv[r, c] = v
    q = np.zeros((1, H, 576), np.float32)
    for c, v in case["q"]:
        q[0, 0, c] = v
    W = np.zeros((H, 512, 128), np.float32)
    for c, d, v in case["W"]:
        W[0, c, d] = v
    gate = np.array([[case["gate"]]], np.float32)
    idx = np.array([case["idx"]], np.int32)
    return _bf(kv), _bf(q), _bf(W), _bf(gate), idx


def test_hand_worked_mla_example():
    g = json.load(open(os.path.join(GOLDEN, "mla_hand.json")))
    for case in g["cases"]:
        kv, q, W, gate, idx = _hand_case(case)
        r = oracle.sparse_mla([len(case["idx"]) - 1], q, kv, idx, W, gate, case["scale"])
        assert np.allclose(r["o_pre"][0, 0, :2], case["o_expected"], atol=1e-11), case["name"]
        assert np.allclose(r["out"][0, 0, :2], case["out_expected"], atol=1e-11), case["name"]
        assert np.all(r["o_pre"][0, 0, 2:] == 0)
        assert abs(r["lse"][0, 0] - case["lse"]) < 1e-11


def test_softmax_rows_sum_to_one():
    """P5 on the tiny workload."""
    cfg = tg.get_config("tiny")
    inp = tg.make_inputs(cfg)
    rows = np.arange(0, 1024, 13)
    idx, theta, keff, mla = oracle.forward(cfg, inp, rows)
    assert np.abs(mla["psum"] - 1).max() <= 1e-12


def test_mla_closed_forms():
    """P6: one key -> its V row; zero query -> mean of the rows; zero gate -> half; block-identity W_UV -> slice."""
    cfg = tg.get_config("tiny")
    inp = tg.make_inputs(cfg)
    kv, W = inp["kv"], inp["W_UV"]
    H = cfg.H
    rows = np.array([0, 300, 1023])
    q = inp["q"][rows]
    gate = inp["gate"][rows]
    kvf, Wf = f32(kv).astype(np.float64), f32(W).astype(np.float64)
    # one key: first token of the document
    idx1 = np.full((3, 8), -1, np.int32)
    idx1[:, 0] = [0, 17, 1023]
    r = oracle.sparse_mla(rows, q, kv, idx1, W, gate, cfg.softmax_scale)
    for j, s in enumerate([0, 17, 1023]):
        want = np.einsum("c,hcd->hd", kvf[s, :512], Wf)
        assert np.abs(r["o_pre"][j] - want).max() < 1e-9 * np.abs(want).max()
    # zero query: uniform weights
    idx = np.stack([np.arange(0, 40), np.arange(100, 140), np.arange(900, 940)]).astype(np.int32)
    r0 = oracle.sparse_mla(rows, np.zeros_like(q), kv, idx, W, gate, cfg.softmax_scale)
    for j in range(3):
        want = np.einsum("c,hcd->hd", kvf[idx[j], :512].mean(0), Wf)
        assert np.abs(r0["o_pre"][j] - want).max() < 1e-9 * np.abs(want).max()
    # zero gate halves the output exactly
    rz = oracle.sparse_mla(rows, q, kv, idx, W, np.zeros_like(gate), cfg.softmax_scale)
    assert np.array_equal(rz["out"], rz["o_pre"] / 2)
    # block identity: W[h, c, d] = 1 when c == 128 * (h % 4) + d
    Wi = np.zeros((H, 512, 128), np.float32)
    for h in range(H):
        Wi[h, 128 * (h % 4) + np.arange(128), np.arange(128)] = 1
    ri = oracle.sparse_mla(rows, q, kv, idx, _bf(Wi), gate, cfg.softmax_scale)
    rI = oracle.sparse_mla(rows, q, kv, idx, _bf(np.tile(np.eye(512, 128, dtype=np.float32), (H, 1, 1))), gate,
                           cfg.softmax_scale)
    # o_lat rebuilt directly from its closed form: the block-identity run must return its slice
    qf = f32(q).astype(np.float64)
    for j in range(3):
        sel = idx[j]
        for h in range(H):
            l = cfg.softmax_scale * (kvf[sel] @ qf[j, h])
            p = np.exp(l - l.max()); p /= p.sum()
            o_lat = p @ kvf[sel, :512]
            b0 = 128 * (h % 4)
            assert np.abs(ri["o_pre"][j, h] - o_lat[b0:b0 + 128]).max() < 1e-12
            assert np.abs(rI["o_pre"][j, h] - o_lat[:128]).max() < 1e-12


def _torch_dense_reference(cfg, inp, rows):
    """Library cross-check: torch SDPA (float64, causal within the document) then W_UV and the gate."""
    out = []
    cu = inp["cu_seqlens"]
    kv = torch.from_numpy(f32(inp["kv"]).astype(np.float64))
    W = torch.from_numpy(f32(inp["W_UV"]).astype(np.float64))
    for t in rows:
        b = oracle.doc_begin(cu, t)
        q = torch.from_numpy(f32(inp["q"][t]).astype(np.float64))[:, None, :]   # [H,1,576]
        K = kv[b:t + 1][None].expand(cfg.H, -1, -1)
        V = kv[b:t + 1, :512][None].expand(cfg.H, -1, -1)
        o = torch.nn.functional.scaled_dot_product_attention(q, K, V, scale=cfg.softmax_scale)[:, 0]  # [H,512]
        o = torch.bmm(o[:, None, :], W)[:, 0]
        g = torch.from_numpy(f32(inp["gate"][t]).astype(np.float64))
        out.append((o * torch.sigmoid(g)[:, None]).numpy())
    return np.stack(out)


def test_dense_equivalence_tiny_shape():
    """P4 (KC bullet 4 with bullet 1): for T <= k the sparse path equals dense causal attention."""
    cfg = tg.Config("dense-tiny", 21, [256], topk=256, H=16, H_I=4, d_I=64, w_scale=0.5)
    inp = tg.make_inputs(cfg)
    rows = np.arange(cfg.T)
    idx, theta, keff, mla = oracle.forward(cfg, inp, rows)
    dense = oracle.dense_causal(rows, inp["q"], inp["kv"], inp["cu_seqlens"], inp["W_UV"], inp["gate"],
                                cfg.softmax_scale)
    assert np.abs(mla["out"] - dense).max() <= 1e-12 * np.abs(dense).max()
    sub = rows[::17]
    ref = _torch_dense_reference(cfg, inp, sub)
    assert np.abs(mla["out"][sub] - ref).max() <= 1e-10 * np.abs(ref).max()


def test_dense_equivalence_production_shape():
    """P4 at T = k = 2048 with 96 heads, on sampled rows (the dense reference is slow)."""
    cfg = tg.get_config("dense2048")
    keys = tg.key_side(cfg)
    rows = np.array([0, 1, 700, 2047])
    inp = dict(keys, cu_seqlens=cfg.cu_seqlens)
    qr = tg.query_rows(cfg, rows)
    full_q = np.zeros((cfg.T, cfg.H, 576), np.uint16)
    full_g = np.zeros((cfg.T, cfg.H), np.uint16)
    full_q[rows] = qr["q"].reshape(len(rows), cfg.H, 576)
    full_g[rows] = qr["gate"]
    LNk = oracle.key_layernorm(keys["k_I"])
    idx, theta, keff = oracle.topk(rows, qr["q_I"].reshape(len(rows), cfg.H_I, cfg.d_I), qr["w"], LNk,
                                   cfg.cu_seqlens, cfg.topk)
    assert list(keff) == [1, 2, 701, 2048]
    mla = oracle.sparse_mla(rows, full_q[rows], keys["kv"], idx, keys["W_UV"], full_g[rows], cfg.softmax_scale)
    dense = oracle.dense_causal(rows, full_q[rows], keys["kv"], cfg.cu_seqlens, keys["W_UV"], full_g[rows],
                                cfg.softmax_scale)
    assert np.abs(mla["out"] - dense).max() <= 1e-12 * np.abs(dense).max()
    inp["q"], inp["gate"] = full_q, full_g
    ref = _torch_dense_reference(cfg, inp, rows)
    assert np.abs(mla["out"] - ref).max() <= 1e-10 * np.abs(ref).max()


def test_packed_equals_per_document():
    """P7: a packed run equals the per-document runs, indices offset by the document start (KC: packed
    documents are contiguous)."""
    lens = [300, 40, 420]
    cfg = tg.Config("p7", 31, lens, topk=128, H=16, H_I=4, d_I=64, w_scale=0.5)
    inp = tg.make_inputs(cfg)
    rows = np.arange(cfg.T)
    idx, theta, keff, mla = oracle.forward(cfg, inp, rows)
    cu = cfg.cu_seqlens
    for d in range(len(lens)):
        b, e = int(cu[d]), int(cu[d + 1])
        sub = {k: (v[b:e] if k != "W_UV" else v) for k, v in inp.items() if k != "cu_seqlens"}
        sub["cu_seqlens"] = np.array([0, e - b], np.int32)
        c1 = tg.Config("p7d", 31, [e - b], topk=128, H=16, H_I=4, d_I=64)
        i1, th1, k1, m1 = oracle.forward(c1, sub, np.arange(e - b))
        shifted = np.where(i1 >= 0, i1 + b, -1)
        assert np.array_equal(idx[b:e], shifted)
        assert np.array_equal(mla["out_bf16"][b:e], m1["out_bf16"])


def test_float_timing_variant_matches_double():
    """The float-accumulated attention used only to time the CPU baseline computes the same outputs as
    the double reference, to float rounding."""
    cfg = tg.get_config("tiny")
    inp = tg.make_inputs(cfg)
    rows = np.arange(700, 1024, 41)
    idx, theta, keff, mla = oracle.forward(cfg, inp, rows)
    f = oracle.sparse_mla_f32(rows, inp["q"][rows], inp["kv"], idx, inp["W_UV"], inp["gate"][rows], cfg.softmax_scale)
    assert np.abs(f - mla["out"]).max() <= 1e-4 * np.abs(mla["out"]).max()


# ---------------------------------------------------------------- gate and sink variants (AD "Output gate + sink")

def _variant_inputs(seed=61, T=300, H=16, k=64):
    cfg = tg.Config("variant", seed, [T], topk=k, H=H, H_I=4, d_I=64, w_scale=0.5)
    inp = tg.make_inputs(cfg)
    rng = np.random.default_rng(seed)
    rows = np.array([0, 5, 63, 64, 150, 299])
    idx = np.full((len(rows), k), -1, np.int32)
    for j, t in enumerate(rows):
        n = min(k, t + 1)
        idx[j, :n] = np.sort(rng.choice(t + 1, n, replace=False))
    return cfg, inp, rows, idx


def test_sink_limits_and_mass():
    """A sink far below every logit changes nothing; far above, it takes all the weight (output 0, lse =
    sink); otherwise the keys' weights plus the sink's weight exp(sink - lse) sum to 1, and the lse is
    log(exp(lse without sink) + exp(sink))."""
    cfg, inp, rows, idx = _variant_inputs()
    q, g = inp["q"][rows], inp["gate"][rows]
    base = oracle.sparse_mla(rows, q, inp["kv"], idx, inp["W_UV"], g, cfg.softmax_scale)
    lo = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, inp["W_UV"], g, cfg.softmax_scale, sink=np.full(cfg.H, -1e4))
    assert np.array_equal(lo["out"], base["out"]) and np.array_equal(lo["lse"], base["lse"])
    hi = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, inp["W_UV"], g, cfg.softmax_scale, sink=np.full(cfg.H, 1e4))
    assert np.all(hi["out"] == 0) and np.all(hi["lse"] == 1e4)
    sink = np.random.default_rng(1).normal(0, 2, cfg.H)
    r = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, inp["W_UV"], g, cfg.softmax_scale, sink=sink)
    assert np.abs(r["psum"] + np.exp(sink[None, :] - r["lse"]) - 1).max() < 1e-12
    assert np.abs(r["lse"] - np.logaddexp(base["lse"], sink[None, :])).max() < 1e-12
    # the sink only rescales the keys' weights: o_pre = base o_pre * (sum of key weights)
    assert np.abs(r["o_pre"] - base["o_pre"] * r["psum"][..., None]).max() < 1e-12 * np.abs(base["o_pre"]).max()


def test_sink_one_key_is_logistic():
    """One selected key and a sink s: the key's weight is the logistic function of (l - s), so
    o_lat = sigma(l - s) * kv_row."""
    cfg, inp, rows, idx = _variant_inputs()
    idx1 = np.full((len(rows), 8), -1, np.int32)
    idx1[:, 0] = rows
    sink = np.linspace(-3, 3, cfg.H)
    r = oracle.sparse_mla_variant(rows, inp["q"][rows], inp["kv"], idx1, inp["W_UV"], inp["gate"][rows],
                                  cfg.softmax_scale, sink=sink)
    kvf = f32(inp["kv"]).astype(np.float64)
    Wf = f32(inp["W_UV"]).astype(np.float64)
    qf = f32(inp["q"][rows]).astype(np.float64)
    for j, t in enumerate(rows):
        for h in range(cfg.H):
            l = cfg.softmax_scale * (qf[j, h] @ kvf[t])
            wgt = 1.0 / (1.0 + math.exp(-(l - sink[h])))
            want = wgt * (kvf[t, :512] @ Wf[h])
            assert np.abs(r["o_pre"][j, h] - want).max() <= 1e-12 * max(np.abs(want).max(), 1e-300)


def test_gate_per_dim():
    """An elementwise gate equal to the per-head gate on every output gives the same outputs; with a
    block-identity W_UV each output is sigma(g[d]) times its own latent dim; g = 0 halves."""
    cfg, inp, rows, idx = _variant_inputs()
    q, g = inp["q"][rows], inp["gate"][rows]
    base = oracle.sparse_mla(rows, q, inp["kv"], idx, inp["W_UV"], g, cfg.softmax_scale)
    rep = np.repeat(g[:, :, None], 128, axis=2)
    r = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, inp["W_UV"], rep, cfg.softmax_scale, gate_per_dim=True)
    assert np.array_equal(r["out"], base["out"]) and np.array_equal(r["out_bf16"], base["out_bf16"])
    gd = tg.normal_bf16(7, 99, 0, len(rows) * cfg.H * 128, 1.0).reshape(len(rows), cfg.H, 128)
    Wi = np.zeros((cfg.H, 512, 128), np.float32)
    Wi[:, np.arange(128), np.arange(128)] = 1
    ri = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, _bf(Wi), gd, cfg.softmax_scale, gate_per_dim=True)
    sig = 1.0 / (1.0 + np.exp(-f32(gd).astype(np.float64)))
    assert np.abs(ri["out"] - ri["o_pre"] * sig).max() <= 1e-15 * np.abs(ri["o_pre"]).max()
    rz = oracle.sparse_mla_variant(rows, q, inp["kv"], idx, inp["W_UV"], np.zeros_like(gd), cfg.softmax_scale,
                                   gate_per_dim=True)
    assert np.array_equal(rz["out"], rz["o_pre"] / 2)


# ---------------------------------------------------------------- FP8 indexer (KC Implementation Limits, 2nd bullet)

def test_e4m3_decode_table():
    """All 256 E4M3 codes against the format's closed forms and torch's float8_e4m3fn (library
    cross-check): subnormals m*2^-9, normals (1+m/8)*2^(E-7), 448 the largest, S.1111.111 NaN."""
    codes = np.arange(256, dtype=np.uint8)
    mine = np.array([oracle.e4m3_decode(c) for c in codes])
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    same = (mine == ref) | (np.isnan(mine) & np.isnan(ref))
    assert same.all()
    assert [c for c in codes if np.isnan(mine[c])] == [0x7F, 0xFF]
    assert mine[0x01] == 2.0 ** -9 and mine[0x07] == 7 * 2.0 ** -9 and mine[0x08] == 2.0 ** -6
    assert mine[0x38] == 1.0 and mine[0x7E] == 448.0 and mine[0x80] == 0.0 and np.signbit(mine[0x80])
    assert np.nanmax(np.abs(mine)) == 448.0


def test_e4m3_encode_round_to_nearest_even():
    """Every finite code round-trips; every midpoint between neighbours goes to the neighbour with an
    even code, and the smallest step off a midpoint goes to the nearer one; negative values mirror;
    torch's conversion agrees on random values (library cross-check)."""
    pos = [c for c in range(0x7F)]  # 0x00 .. 0x7E: every nonnegative finite code, increasing in value
    vals = [oracle.e4m3_decode(c) for c in pos]
    assert all(a < b for a, b in zip(vals, vals[1:]))
    for c, v in zip(pos, vals):
        assert oracle.e4m3_encode(v) == c and oracle.e4m3_encode(-v) == (c | 0x80)
    for c in range(len(pos) - 1):
        lo, hi = vals[c], vals[c + 1]
        mid = (lo + hi) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even, (hex(c), mid)
        assert oracle.e4m3_encode(-mid) == (even | 0x80)
        step = (hi - lo) * 2.0 ** -12
        assert oracle.e4m3_encode(mid - step) == c and oracle.e4m3_encode(mid + step) == c + 1
    x = np.random.default_rng(3).uniform(-448, 448, 20000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ref, np.array([oracle.e4m3_encode(float(v)) for v in x]))


def test_fp8_scale_exponent_closed_forms():
    """The smallest e with amax * 2^-e <= 448."""
    cases = {448.0: 0, 450.0: 1, 224.0: -1, 225.0: 0, 1.0: -8, 1.75: -8, 1.875: -7, 3.5: -7, 2.0 ** -130: -138,
             0.0: 0, 896.0: 1, 897.0: 2}
    for amax, e in cases.items():
        assert oracle.fp8_scale_exponent(amax) == e, (amax, e)
        if amax > 0:
            assert amax * 2.0 ** -e <= 448.0 < amax * 2.0 ** -(e - 1)


def test_quantize_fp8_rows_bounds_and_torch():
    """Each row's codes times 2^e lie within half a code step of the bf16 values, the row maximum uses
    the top of the range, and the codes equal torch's E4M3 conversion of x * 2^-e."""
    x = tg.normal_bf16(12, 1, 0, 300 * 128, 1.0).reshape(300, 128)
    x[7] = 0
    x[8, :] = _bf(np.full(128, 2.0 ** -20))
    q8, e = oracle.quantize_fp8_rows(x)
    xf = f32(x).astype(np.float64)
    dec = np.vectorize(oracle.e4m3_decode)(q8) * np.ldexp(1.0, e)[:, None]
    for r in range(300):
        amax = np.abs(xf[r]).max()
        if amax == 0:
            assert e[r] == 0 and np.all(q8[r] == 0)
            continue
        assert 224.0 < amax * 2.0 ** -e[r] <= 448.0
        # half a step of E4M3 at each value's magnitude (subnormal step 2^-9), times 2^e
        mag = np.abs(xf[r]) * 2.0 ** -e[r]
        step = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 1e-300))) - 3))
        assert np.all(np.abs(dec[r] - xf[r]) <= step / 2 * 2.0 ** e[r] * (1 + 1e-12))
    scaled = torch.from_numpy((xf * np.ldexp(1.0, -e)[:, None]).astype(np.float32))
    assert np.array_equal(scaled.to(torch.float8_e4m3fn).view(torch.uint8).numpy(), q8)


def test_fp8_scores_equal_bf16_scores_when_exact():
    """When every q_I and LNk value is exactly representable in E4M3 after its row's scaling, the FP8
    indexer's scores equal the BF16 indexer's bit for bit (power-of-two scales commute with FP32
    rounding here), for every key."""
    rng = np.random.default_rng(13)
    H_I, d_I, T = 4, 64, 50
    grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 3, 4, 6], np.float32)
    def rows(n, width, top):
        v = rng.choice(grid, (n, width)) * rng.choice([-1, 1], (n, width))
        v[:, 0] = top                                    # fixes each row's maximum magnitude
        return v * np.ldexp(1.0, rng.integers(-3, 4, (n, 1))).astype(np.float32)
    LNk = _bf(rows(T, d_I, 7.0))
    q = _bf(rows(H_I, d_I, -5.0))
    w = _bf(rng.uniform(0, 1, H_I))
    k8, ek = oracle.quantize_fp8_rows(LNk)
    q8, eq = oracle.quantize_fp8_rows(q)
    assert np.array_equal(np.vectorize(oracle.e4m3_decode)(k8) * np.ldexp(1.0, ek)[:, None], f32(LNk))
    S8 = oracle.index_scores_fp8(q8, eq, w, k8, ek, 0, T - 1)
    S = oracle.index_scores(q, w, LNk, 0, T - 1)
    assert np.array_equal(S8, S)


def test_topk_fp8_brute_force_tiny():
    """FP8 top-k against a full sort of the FP8 scores by (score desc, index asc)."""
    rng = np.random.default_rng(14)
    T, H_I, d_I, k = 120, 64, 128, 17
    LNk = oracle.key_layernorm(_bf(rng.standard_normal((T, d_I))))
    k8, ek = oracle.quantize_fp8_rows(LNk)
    q = _bf(rng.standard_normal((T, H_I, d_I)))
    w = _bf(rng.uniform(0, 1 / 8, (T, H_I)))
    q8, eq = oracle.quantize_fp8_rows(q)
    rows = np.arange(T)
    idx, theta, keff = oracle.topk_fp8(rows, q8, eq, w, k8, ek, np.array([0, T], np.int32), k)
    agree = []
    for t in range(k, T):
        S = oracle.index_scores_fp8(q8[t], eq[t], w[t], k8, ek, 0, t)
        order = np.lexsort((np.arange(t + 1), -S.astype(np.float64)))[:k]
        assert sorted(order.tolist()) == idx[t][:k].tolist()
        assert theta[t] == S[order[-1]]
        b16 = oracle.topk([t], q[[t]], w[[t]], LNk, np.array([0, T], np.int32), k)[0][0]
        agree.append(len(set(b16.tolist()) & set(idx[t].tolist())) / k)
    assert np.mean(agree) > 0.8   # the FP8 selection stays close to the BF16 one


# ---------------------------------------------------------------- W_UK absorption (KC bullet 2; API MLA fields)

def test_q_absorb_matches_expanded_keys():
    """The absorbed latent query gives the same attention logits as the unabsorbed form with the
    per-head keys expanded: q_nope . (c_KV W_UK[h]) + q_pe . k_pe = q_lat . c_KV + q_pe . k_pe, for
    every head and key, computed here directly from the expanded keys."""
    rng = np.random.default_rng(31)
    n, H, T = 3, 8, 40
    q_nope = _bf(rng.standard_normal((n, H, 128)))
    q_pe = _bf(rng.standard_normal((n, H, 64)))
    W_UK = _bf(rng.standard_normal((H, 512, 128)) * 0.05)
    kv = _bf(rng.standard_normal((T, 576)))
    q, qf = oracle.q_absorb(q_nope, q_pe, W_UK, want_f64=True)
    assert np.array_equal(q[:, :, 512:], q_pe)
    Wf, kvf = f32(W_UK).astype(np.float64), f32(kv).astype(np.float64)
    k_nope = np.einsum("sc,hcd->hsd", kvf[:, :512], Wf)                    # expanded per-head keys
    expanded = np.einsum("nhd,hsd->nhs", f32(q_nope).astype(np.float64), k_nope) \
        + np.einsum("nhj,sj->nhs", f32(q_pe).astype(np.float64), kvf[:, 512:])
    absorbed = np.einsum("nhc,sc->nhs", qf, kvf[:, :512]) + np.einsum("nhj,sj->nhs", f32(q_pe).astype(np.float64),
                                                                      kvf[:, 512:])
    assert np.abs(absorbed - expanded).max() <= 1e-10 * np.abs(expanded).max()
    # the stored bf16 latent query is the double value rounded once to nearest
    y = f32(q[:, :, :512]).astype(np.float64)
    ulp = np.ldexp(1.0, np.frexp(np.abs(qf))[1] - 8)
    assert np.all(np.abs(y - qf) <= ulp / 2 + 1e-300)


def test_q_absorb_identity_weight():
    """W_UK[h, c, d] = 1 when c == d + 128*(h % 4): the latent query is q_nope shifted into block h % 4."""
    rng = np.random.default_rng(32)
    n, H = 2, 8
    q_nope = _bf(rng.standard_normal((n, H, 128)))
    q_pe = _bf(rng.standard_normal((n, H, 64)))
    W = np.zeros((H, 512, 128), np.float32)
    for h in range(H):
        W[h, 128 * (h % 4) + np.arange(128), np.arange(128)] = 1
    q = oracle.q_absorb(q_nope, q_pe, _bf(W))
    for h in range(H):
        b0 = 128 * (h % 4)
        assert np.array_equal(q[:, h, b0:b0 + 128], q_nope[:, h])
        rest = np.delete(np.arange(512), np.arange(b0, b0 + 128))
        assert np.all(f32(q[:, h, rest]) == 0)


# ---------------------------------------------------------------- o_proj (KC output-gate paragraph; API hidden_size)

def test_o_proj_against_library_matmul_and_selection():
    """o_proj equals a float64 library matrix product rounded once to bf16 (library cross-check), and a
    selection weight (W_o[n, k] = 1 for k = p(n)) returns the selected inputs exactly."""
    rng = np.random.default_rng(41)
    n, K, N = 5, 2048, 384
    x = _bf(rng.standard_normal((n, K)))
    W = _bf(rng.standard_normal((N, K)) * 0.02)
    y, yf = oracle.o_proj(x, W, want_f64=True)
    ref = f32(x).astype(np.float64) @ f32(W).astype(np.float64).T
    assert np.abs(yf - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.array_equal(y, bf(ref.astype(np.float32))) or np.abs(f32(y) - ref).max() <= np.abs(ref).max() * 2.0 ** -8
    perm = rng.permutation(K)[:N]
    S = np.zeros((N, K), np.float32)
    S[np.arange(N), perm] = 1
    assert np.array_equal(oracle.o_proj(x, _bf(S)), x[:, perm])


# ---------------------------------------------------------------- sparse MLA backward (KC: native-96-head backward)

def _bwd_case(seed, n, H, T, k):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, H, 576)) * 0.3
    kv = rng.standard_normal((T, 576))
    W = rng.standard_normal((H, 512, 128)) * 0.05
    gate = rng.standard_normal((n, H))
    dout = rng.standard_normal((n, H, 128))
    idx = np.full((n, k), -1, np.int32)
    for r in range(n):
        m = rng.integers(1, k + 1)
        idx[r, :m] = rng.integers(0, T, m)       # duplicates allowed
    idx[0, 1] = idx[0, 0]                       # a duplicate for sure
    idx[-1, 0] = T + 3                          # out of range: skipped
    return q, kv, idx, W, gate, dout


def test_backward_against_finite_differences():
    """Directional derivatives of L = sum(dout * out) by central differences of the oracle's own forward
    (double inputs) equal the backward's gradients, for q, kv, W_UV and the gate separately."""
    q, kv, idx, W, gate, dout = _bwd_case(51, 3, 4, 20, 7)
    scale = 1 / math.sqrt(192)
    g = oracle.sparse_mla_bwd(q, kv, idx, W, gate, scale, dout)

    def L(q_, kv_, W_, g_):
        return float((oracle.sparse_mla_f64in(q_, kv_, idx, W_, g_, scale)[0] * dout).sum())
    rng = np.random.default_rng(7)
    eps = 1e-6
    for name, x, grad in [("q", q, g["dq"]), ("kv", kv, g["dkv"]), ("W_UV", W, g["dW_UV"]), ("gate", gate, g["dgate"])]:
        v = rng.standard_normal(x.shape)
        args = {"q": q, "kv": kv, "W_UV": W, "gate": gate}
        plus, minus = dict(args), dict(args)
        plus[name], minus[name] = x + eps * v, x - eps * v
        fd = (L(plus["q"], plus["kv"], plus["W_UV"], plus["gate"]) - L(minus["q"], minus["kv"], minus["W_UV"],
                                                                      minus["gate"])) / (2 * eps)
        an = float((grad * v).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_backward_inner_product_identities():
    """Two closed forms of L = sum(dout * out) that the backward must satisfy at any size (the chain
    rule through W_UV and through the logits): for each head h,
      <dW_UV[h], W_UV[h]> = sum_r <dout[r,h], out[r,h]>,
    and over everything,
      sum_key <dkv[key], kv[key]> - sum_{r,h} <dq[r,h], q[r,h]> = sum_{r,h} <dout[r,h], out[r,h]>
    (the key part of dkv pairs with q as dq does; its value part gives do_lat . o_lat = dout . out).
    Duplicate and out-of-range indices included. The GPU test at T=131,072 checks these on the full
    gradients."""
    n, H, T, k = 6, 8, 40, 12
    q, kv, idx, W, gate, dout = _bwd_case(53, n, H, T, k)
    scale = 1 / math.sqrt(192)
    g = oracle.sparse_mla_bwd(q, kv, idx, W, gate, scale, dout)
    out = oracle.sparse_mla_f64in(q, kv, idx, W, gate, scale)[0]
    D = (dout * out).sum(axis=2)  # [n, H]
    lhs_w = (g["dW_UV"] * W).sum(axis=(1, 2))
    assert np.allclose(lhs_w, D.sum(axis=0), rtol=1e-10, atol=1e-12 * np.abs(D).sum())
    lhs = (g["dkv"] * kv).sum() - (g["dq"] * q).sum()
    assert abs(lhs - D.sum()) <= 1e-10 * (np.abs(g["dkv"] * kv).sum() + np.abs(g["dq"] * q).sum())
    # a planted mistake (the dkv row of one selected key halved) breaks the second form
    bad = g["dkv"].copy()
    bad[int(idx[2, 0])] *= 0.5
    assert abs((bad * kv).sum() - (g["dq"] * q).sum() - D.sum()) > 1e-6 * np.abs(D).sum()


@pytest.mark.parametrize("gate_per_dim,with_sink", [(True, False), (False, True), (True, True)])
def test_backward_variants_against_finite_differences(gate_per_dim, with_sink):
    """The gate and sink variants of the backward: directional derivatives of L = sum(dout * out) by
    central differences of the oracle's own variant forward (double inputs) equal the gradients, for
    q, kv, W_UV, the gate ([n,H,128] when per element) and the sink logits."""
    n, H, T, k = 3, 4, 20, 7
    q, kv, idx, W, gate, dout = _bwd_case(54, n, H, T, k)
    rng = np.random.default_rng(8)
    if gate_per_dim:
        gate = rng.standard_normal((n, H, 128))
    sink = rng.standard_normal(H) if with_sink else None
    scale = 1 / math.sqrt(192)
    g = oracle.sparse_mla_bwd(q, kv, idx, W, gate, scale, dout, gate_per_dim=gate_per_dim, sink=sink)
    assert g["dgate"].shape == gate.shape and (("dsink" in g) == with_sink)

    def L(q_, kv_, W_, g_, s_):
        return float((oracle.sparse_mla_f64in(q_, kv_, idx, W_, g_, scale, gate_per_dim, s_)[0] * dout).sum())
    eps = 1e-6
    args = {"q": q, "kv": kv, "W_UV": W, "gate": gate, "sink": sink}
    grads = [("q", g["dq"]), ("kv", g["dkv"]), ("W_UV", g["dW_UV"]), ("gate", g["dgate"])]
    if with_sink:
        grads.append(("sink", g["dsink"]))
    for name, grad in grads:
        v = rng.standard_normal(args[name].shape)
        plus, minus = dict(args), dict(args)
        plus[name], minus[name] = args[name] + eps * v, args[name] - eps * v
        fd = (L(plus["q"], plus["kv"], plus["W_UV"], plus["gate"], plus["sink"])
              - L(minus["q"], minus["kv"], minus["W_UV"], minus["gate"], minus["sink"])) / (2 * eps)
        an = float((grad * v).sum())
        assert abs(fd - an) <= 1e-6 * max(abs(an), 1e-3), (name, fd, an)


def test_backward_sink_against_torch_autograd():
    """Library cross-check of the sink and per-element gate: torch autograd in float64 on a dense
    formulation (the sink as one more softmax logit with a zero value row)."""
    n, H, T, k = 4, 8, 30, 9
    q, kv, idx, W, _, dout = _bwd_case(55, n, H, T, k)
    rng = np.random.default_rng(9)
    gate = rng.standard_normal((n, H, 128))
    sink = rng.standard_normal(H)
    scale = 1 / math.sqrt(192)
    g = oracle.sparse_mla_bwd(q, kv, idx, W, gate, scale, dout, gate_per_dim=True, sink=sink)
    tq = torch.tensor(q, requires_grad=True)
    tkv = torch.tensor(kv, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tg_ = torch.tensor(gate, requires_grad=True)
    ts = torch.tensor(sink, requires_grad=True)
    outs = []
    for r in range(n):
        sel = [int(s) for s in idx[r] if 0 <= s < T]
        K = tkv[sel]
        l = scale * torch.einsum("hi,mi->hm", tq[r], K)
        p = torch.softmax(torch.cat([l, ts[:, None]], dim=1), dim=1)[:, :-1]   # the sink takes its share
        o = torch.einsum("hc,hcd->hd", p @ K[:, :512], tW)
        outs.append(torch.sigmoid(tg_[r]) * o)
    (torch.stack(outs) * torch.tensor(dout)).sum().backward()
    for name, ref, got in [("dq", tq.grad, g["dq"]), ("dkv", tkv.grad, g["dkv"]), ("dW_UV", tW.grad, g["dW_UV"]),
                           ("dgate", tg_.grad, g["dgate"]), ("dsink", ts.grad, g["dsink"])]:
        ref = ref.numpy()
        assert np.abs(ref - got).max() <= 1e-12 * max(np.abs(ref).max(), 1e-30), name


def test_backward_against_torch_autograd():
    """Library cross-check: torch autograd in float64 on a dense gathered formulation of the same
    forward gives the same gradients."""
    n, H, T, k = 4, 8, 30, 9
    q, kv, idx, W, gate, dout = _bwd_case(52, n, H, T, k)
    scale = 1 / math.sqrt(192)
    g = oracle.sparse_mla_bwd(q, kv, idx, W, gate, scale, dout)
    tq = torch.tensor(q, requires_grad=True)
    tkv = torch.tensor(kv, requires_grad=True)
    tW = torch.tensor(W, requires_grad=True)
    tg_ = torch.tensor(gate, requires_grad=True)
    outs = []
    for r in range(n):
        sel = [int(s) for s in idx[r] if 0 <= s < T]
        K = tkv[sel]                                               # [m,576]
        l = scale * torch.einsum("hi,mi->hm", tq[r], K)
        p = torch.softmax(l, dim=1)
        ol = p @ K[:, :512]                                        # [H,512]
        o = torch.einsum("hc,hcd->hd", ol, tW)
        outs.append(torch.sigmoid(tg_[r])[:, None] * o)
    loss = (torch.stack(outs) * torch.tensor(dout)).sum()
    loss.backward()
    for name, ref, got in [("dq", tq.grad, g["dq"]), ("dkv", tkv.grad, g["dkv"]), ("dW_UV", tW.grad, g["dW_UV"]),
                           ("dgate", tg_.grad, g["dgate"])]:
        ref = ref.numpy()
        assert np.abs(ref - got).max() <= 1e-12 * max(np.abs(ref).max(), 1e-30), name
