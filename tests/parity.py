"""Comparison rules shared by the oracle self-tests and the GPU parity tests.

Index rule: every row must hold exactly k_eff = min(k, n_t) distinct in-range causal indices followed
by -1; rows with n_t <= k must equal the full causal set; elsewhere each index in the symmetric
difference with the oracle's row must be a near-tie of the oracle's k-th score theta:
    |S(s) - theta| <= 1e-3 * |theta| + 4 * gamma * max(scale(s), scale(s_theta))
where S is the oracle's FP32 score, scale(s) = sum_h |w_h| sum_i |q_I[h,i] LNk[s,i]| and
gamma = (d_I + H_I) u / (1 - (d_I + H_I) u), u = 2^-24. The second term bounds the difference of two
FP32 evaluations of the same score in different orders; it only matters when theta is near 0.

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


def check_index_row(gpu_row, ora_row, keff, b, t, k, qI_row, w_row, LNk, theta):
    """Returns None if the GPU row passes the index rule, else a message."""
    gpu_row = np.asarray(gpu_row)
    valid = gpu_row[:keff]
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
    H_I, d_I = qI_row.shape
    S = oracle.index_scores(qI_row, w_row, LNk, b, t)
    sc = oracle.index_score_scale(qI_row, w_row, LNk, b, t)
    # index of the oracle's k-th key: its kept key with score theta and the largest index among them
    kept = np.array(sorted(os_))
    kth = kept[np.argmin(np.where(S[kept - b] == theta, -kept, np.inf))] if np.any(S[kept - b] == theta) else kept[0]
    g = gamma(d_I + H_I)
    for s in diff:
        band = REL_BAND * abs(float(theta)) + 4 * g * max(sc[s - b], sc[kth - b])
        if abs(float(S[s - b]) - float(theta)) > band:
            return f"row {t}: index {s} (score {S[s - b]!r}) differs from oracle and is not a near-tie of theta={theta!r}"
    return None


def check_outputs(out, ref, tol=OUT_TOL):
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    err = np.abs(out - ref).max()
    m = np.abs(ref).max()
    return err <= tol * m, float(err), float(m)
