"""Parity rule between the GPU ranking head and the CPU oracle.

Scores are compared with tau = 2e-3 * max|s| (max over the oracle scores that
were computed for the case), lse with an absolute 1e-3.  Indices must match
the oracle's top-K exactly except where the oracle scores of the differing
items lie within tau of the oracle's K-th score; inside the list, adjacent
entries may appear swapped only when their oracle scores differ by at most
tau.  Padding (id -1, score -inf) must match exactly.
"""
from __future__ import annotations

import numpy as np

SCORE_REL = 2e-3
LSE_ABS = 1e-3


def check_row(g_idx, g_sc, g_lse, o_idx, o_sc, o_lse, score_of, tau, where=""):
    """score_of(ids) -> oracle fp64 scores of those ids for this user."""
    K = len(o_idx)
    n_real = int((o_idx >= 0).sum())
    if not np.isfinite(o_lse):
        assert g_lse == o_lse, (where, g_lse, o_lse)
    else:
        assert abs(float(g_lse) - o_lse) <= LSE_ABS, (where, "lse", float(g_lse), o_lse)
    # padding exactly where the oracle pads
    assert (g_idx[n_real:] == -1).all() and np.isneginf(g_sc[n_real:]).all(), (where, "padding")
    gi = g_idx[:n_real].astype(np.int64)
    gs = g_sc[:n_real].astype(np.float64)
    assert (gi >= 0).all(), (where, "missing entries")
    assert np.unique(gi).size == n_real or _dups_allowed(o_idx[:n_real]), (where, "duplicate ids")
    assert (np.diff(gs) <= 0).all(), (where, "scores not descending")
    if n_real == 0:
        return
    so = score_of(gi)
    assert np.abs(gs - so).max() <= tau, (where, "score vs oracle at same id", np.abs(gs - so).max(), tau)
    assert np.abs(gs - o_sc[:n_real]).max() <= tau, (where, "score vs oracle rank", np.abs(gs - o_sc[:n_real]).max())
    s_k = o_sc[n_real - 1]
    diff = set(gi.tolist()) ^ set(o_idx[:n_real].tolist())
    if diff:
        ds = score_of(np.array(sorted(diff), dtype=np.int64))
        assert (np.abs(ds - s_k) <= tau).all(), (where, "set differs beyond tau", sorted(diff), ds, s_k, tau)
    inv = so[1:] > so[:-1]
    if inv.any():
        assert (so[1:][inv] - so[:-1][inv] <= tau).all(), (where, "order inversion beyond tau")


def _dups_allowed(o_idx):
    return np.unique(o_idx).size < o_idx.size


def check_dense(gpu, ref, tau=None, where=""):
    """gpu = (idx, scores, lse) host arrays for ALL users; ref = oracle.full(...) for ref['users']."""
    g_idx, g_sc, g_lse = gpu
    S = ref["S"]
    if tau is None:
        tau = SCORE_REL * np.abs(S).max()
    for r, b in enumerate(ref["users"]):
        check_row(g_idx[b], g_sc[b], g_lse[b], ref["idx"][r], ref["score"][r], ref["lse"][r],
                  lambda ids, r=r: S[r, ids], tau, where="%s user %d" % (where, b))
    return tau


def check_cand(gpu, ref, offsets, ids, tau=None, where=""):
    g_idx, g_sc, g_lse = gpu
    es = ref["entry_scores"]
    finite = es[np.isfinite(es)]
    if tau is None:
        tau = SCORE_REL * (np.abs(finite).max() if finite.size else 1.0)
    for r, b in enumerate(ref["users"]):
        lst = ids[offsets[b]:offsets[b + 1]]
        sc = es[offsets[b]:offsets[b + 1]]
        table = {}
        for i, s in zip(lst.tolist(), sc.tolist()):
            if np.isfinite(s):
                table[i] = s
        check_row(g_idx[b], g_sc[b], g_lse[b], ref["idx"][r], ref["score"][r], ref["lse"][r],
                  lambda q, t=table: np.array([t[int(x)] for x in q]), tau, where="%s user %d" % (where, b))
    return tau


# ---------------------------------------------------------------------------
# Catalog cross-entropy
# ---------------------------------------------------------------------------
# The GPU keeps G = w (softmax - target) in bf16 (rounded to nearest even,
# relative error <= 2^-9) and forms the softmax from fp32 scores and lse, each
# within the score tolerance tau of the exact value, so every entry of G is
# within c |A| of the exact one with c = 2^-9 + 2 tau and A = |G| + w P (the
# second term covers the label entry, whose G is w (p - 1)).  The products
# add at most depth * 2^-24 relative fp32 rounding on top (depth = the longest
# chain of fp32 additions into one output).  So, entrywise,
#   |dH_gpu - dH| <= (c + depth_H 2^-24) (A |E|)   and
#   |dE_gpu - dE| <= (c + depth_E 2^-24) (A^T |H|),
# loss and lse within the lse rule (loss scaled by w).
def check_ce(gpu, ref, E, H, widen, depth_h=1, depth_e=1, de_round=0.0, where=""):
    """gpu = (loss, lse, dH, dE or None) host arrays for the users in ref['users']
    (dE for the whole catalog); ref = oracle.ce(...); E, H = the raw inputs and
    widen = their exact fp64 conversion.  de_round: relative rounding of a dE
    stored in a narrower type (bf16: 2^-9 of a value that is itself within the
    bound, counted as 2^-8)."""
    loss, lse_g, dH, dE = gpu
    tau = SCORE_REL * np.abs(ref["S"]).max()
    w = ref["w"]
    assert np.abs(lse_g - ref["lse"]).max() <= LSE_ABS, (where, "lse", np.abs(lse_g - ref["lse"]).max())
    assert (np.abs(loss - ref["loss"]) <= w * 2 * LSE_ABS + 1e-6).all(), (where, "loss",
                                                                        np.abs(loss - ref["loss"]).max())
    c = 2.0 ** -9 + 2 * tau
    A = np.abs(ref["G"]) + w[:, None] * ref["P"]
    AE = np.zeros(dH.shape)
    for i0 in range(0, E.shape[0], 65536):  # A |E|, a block of catalog rows at a time
        AE += A[:, i0:i0 + 65536] @ np.abs(widen(E[i0:i0 + 65536]))
    tol_h = (c + depth_h * 2.0 ** -24) * AE + 1e-30
    err_h = np.abs(dH - ref["dH"])
    assert (err_h <= tol_h).all(), (where, "dH", err_h.max(), (err_h / tol_h).max())
    if dE is not None:
        tol_e = (c + depth_e * 2.0 ** -24 + de_round) * (A.T @ np.abs(widen(H))) + 1e-30
        err_e = np.abs(dE - ref["dE"])
        assert (err_e <= tol_e).all(), (where, "dE", err_e.max(), (err_e / tol_e).max())
