"""Comparison rules shared by the oracle self-tests and the GPU parity tests.

Index rule: every row must hold exactly k_eff = min(k, n_t) distinct in-range causal indices followed
by -1; rows with n_t <= k must equal the full causal set; elsewhere each index s in the symmetric
difference with the oracle's row must be a near-tie of the oracle's k-th score theta:

    |S(s) - theta| <= 1e-3 * |theta|                       when theta != 0
    |S(s)|         <= 2 * gamma(d_I + H_I) * scale(s)      when theta == 0

S is the oracle's FP32 score. When theta is exactly zero the relative band is empty, and only an
FP32 rounding difference can legitimately separate the two sides: a dot product whose value is
within its own rounding error of zero may come out positive on one side and zero after the ReLU on
the other. The floor is the textbook bound on the difference of two FP32 evaluations of the same
score in any order: each lies within gamma(n) * scale(s) of the exact value, where
scale(s) = sum_h |w_h| sum_i |q_I[h,i] LNk[s,i]|, n = d_I + H_I terms deep and
gamma(n) = n u / (1 - n u), u = 2^-24. It applies to theta == 0 rows only.

Equal scores must resolve to the lower index: where the oracle's k-th score theta is shared by keys
inside and outside its set, the oracle keeps the lower ones. Swapped keys whose oracle score is
exactly theta are counted (``theta_swaps``: usually the oracle's k-th key itself, given up for a key
a rounding step away); tests with constructed exact ties check the tie rule directly
(``lower_index_rule_violations``).

Output rule: max |out - ref| <= 2e-2 * max |ref|.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_BAND = 1e-3
OUT_TOL = 2e-2


def gamma(n: int) -> float:
    u = 2.0 ** -24
    return n * u / (1 - n * u)


def new_stats() -> dict:
    """Counters filled by check_index_row: rows compared, rows whose sets differ, swapped indices,
    swaps that needed the theta == 0 floor, swapped keys scoring exactly theta, and the largest
    |S - theta| / |theta| among the swaps with theta != 0."""
    return {"rows": 0, "rows_swapped": 0, "swaps": 0, "floor_swaps": 0, "theta_swaps": 0, "worst_rel": 0.0}


def format_stats(st: dict) -> str:
    return (f"{st['rows']} rows, {st['rows_swapped']} with a swap, {st['swaps']} swapped indices "
            f"({st['floor_swaps']} at theta=0, {st['theta_swaps']} scoring exactly theta), "
            f"worst |S-theta|/|theta| {st['worst_rel']:.2e} (band {REL_BAND:.0e})")


def check_index_row(gpu_row, ora_row, keff, b, t, k, qI_row, w_row, LNk, theta, stats=None, score_fn=None,
                    scale_fn=None, dims=None):
    """Returns None if the GPU row passes the index rule, else a message. score_fn(qI_row, w_row, LNk, b, t)
    and scale_fn(...) give the oracle's scores and error scales of keys b..t (default: the BF16 indexer);
    dims = (H_I, d_I) when qI_row is not an array of that shape."""
    score_fn = score_fn or oracle.index_scores
    scale_fn = scale_fn or oracle.index_score_scale
    gpu_row = np.asarray(gpu_row)
    valid = gpu_row[:keff]
    if stats is not None:
        stats["rows"] += 1
    if np.any(gpu_row[keff:] != -1):
        return f"row {t}: entries after k_eff={keff} are not -1"
    if len(np.unique(valid)) != keff:
        return f"row {t}: duplicate indices"
    if valid.min(initial=b) < b or valid.max(initial=t) > t:
        return f"row {t}: index outside causal window [{b},{t}]"
    gs = set(valid.tolist())
    os_ = set(int(x) for x in ora_row[:keff])
    if gs == os_:
        return None
    if t - b + 1 <= k:
        return f"row {t}: short row must keep every causal key"
    diff = sorted(gs ^ os_)
    H_I, d_I = dims if dims is not None else np.asarray(qI_row).shape[-2:]
    S = score_fn(qI_row, w_row, LNk, b, t)
    th = float(theta)
    sc = scale_fn(qI_row, w_row, LNk, b, t) if th == 0.0 else None
    g = gamma(int(d_I) + int(H_I))
    if stats is not None:
        stats["rows_swapped"] += 1
        stats["swaps"] += len(diff)
    for s in diff:
        d = abs(float(S[s - b]) - th)
        if th != 0.0:
            if d > REL_BAND * abs(th):
                return (f"row {t}: index {s} (score {S[s - b]!r}) differs from oracle and is not a near-tie "
                        f"of theta={theta!r} (|S-theta|/|theta| = {d / abs(th):.3e})")
            if stats is not None:
                stats["worst_rel"] = max(stats["worst_rel"], d / abs(th))
        else:
            if d > 2 * g * sc[s - b]:
                return f"row {t}: index {s} (score {S[s - b]!r}) differs from oracle and theta is 0"
            if stats is not None:
                stats["floor_swaps"] += 1
        if stats is not None and d == 0.0:
            stats["theta_swaps"] += 1
    return None


def lower_index_rule_violations(idx_row, S, b, t):
    """Keys s < s2 with S(s) == S(s2), s2 kept and s dropped: each is a break of the lower-index tie
    rule. S: oracle scores of keys b..t; idx_row: the kept indices (-1 padded)."""
    kept = np.zeros(t - b + 1, bool)
    v = np.asarray(idx_row)
    kept[v[v >= 0] - b] = True
    bad = []
    order = np.lexsort((np.arange(t - b + 1), -S.astype(np.float64)))
    Ss = S[order]
    i = 0
    while i < len(order):
        j = i
        while j + 1 < len(order) and Ss[j + 1] == Ss[i]:
            j += 1
        if j > i:  # a group of equal scores, in ascending index order: kept ones must be a prefix
            grp = kept[order[i:j + 1]]
            first_drop = np.argmin(grp) if not grp.all() else len(grp)
            if grp[first_drop:].any():
                bad.append((int(order[i] + b), float(Ss[i])))
        i = j + 1
    return bad


def check_outputs(out, ref, tol=OUT_TOL):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref).max()
    m = np.abs(ref).max()
    return err <= tol * m, float(err), float(m)
