"""ctypes front end of the C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path.  It imports nothing
from the GPU package.

Every function takes host numpy arrays: bf16 inputs as uint16 bit patterns,
fp32 inputs as float32.  Results are fp64 scores / lse and int64 ids.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

BF16, F32 = 0, 1

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (fp64, OpenMP, no fast-math)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        lib = ctypes.CDLL(LIB)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.oracle_threads.restype = I32
        lib.oracle_scores.argtypes = [P, P, I32, I64, I64, P, I64, P]
        lib.oracle_pair_scores.argtypes = [P, P, I32, I64, P, P, I64, P]
        lib.oracle_lse.argtypes = [P, I64]
        lib.oracle_lse.restype = ctypes.c_double
        lib.oracle_topk_row.argtypes = [P, I64, I64, P, P]
        lib.oracle_full.argtypes = [P, P, I32, I64, I64, I64, P, I64, P, P, P, P]
        lib.oracle_full_masked.argtypes = [P, P, I32, I64, I64, I64, P, I64, P, I64, P, P, P, P]
        lib.oracle_cand.argtypes = [P, P, I32, I64, I64, I64, P, P, P, I64, P, P, P, P]
        lib.oracle_cand.restype = I64
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(X: np.ndarray) -> int:
    if X.dtype == np.uint16:
        return BF16
    if X.dtype == np.float32:
        return F32
    raise TypeError("oracle inputs are uint16 (bf16 bits) or float32, got %s" % X.dtype)


def _users(users, B: int) -> np.ndarray:
    if users is None:
        users = np.arange(B)
    u = np.ascontiguousarray(users, dtype=np.int64)
    if u.size and (u.min() < 0 or u.max() >= B):
        raise ValueError("user index out of range [0, %d)" % B)
    return u


def threads() -> int:
    return _load().oracle_threads()


def scores(H: np.ndarray, E: np.ndarray, users=None) -> np.ndarray:
    """fp64 score rows s[r][i] = h_{users[r]} . e_i for all items."""
    H, E = np.ascontiguousarray(H), np.ascontiguousarray(E)
    dt = _dtype_code(H)
    assert _dtype_code(E) == dt and H.shape[1] == E.shape[1]
    u = _users(users, H.shape[0])
    M, D = E.shape
    S = np.empty((u.size, M), dtype=np.float64)
    _load().oracle_scores(_ptr(H), _ptr(E), dt, D, M, _ptr(u), u.size, _ptr(S))
    return S


def pair_scores(H: np.ndarray, E: np.ndarray, users, items) -> np.ndarray:
    H, E = np.ascontiguousarray(H), np.ascontiguousarray(E)
    dt = _dtype_code(H)
    u = np.ascontiguousarray(users, dtype=np.int64)
    it = np.ascontiguousarray(items, dtype=np.int64)
    out = np.empty(u.size, dtype=np.float64)
    _load().oracle_pair_scores(_ptr(H), _ptr(E), dt, E.shape[1], _ptr(u), _ptr(it), u.size, _ptr(out))
    return out


def lse(s: np.ndarray) -> float:
    s = np.ascontiguousarray(s, dtype=np.float64)
    return _load().oracle_lse(_ptr(s), s.size)


def topk_row(s: np.ndarray, K: int) -> tuple[np.ndarray, np.ndarray]:
    s = np.ascontiguousarray(s, dtype=np.float64)
    idx = np.empty(K, dtype=np.int64)
    sc = np.empty(K, dtype=np.float64)
    _load().oracle_topk_row(_ptr(s), s.size, K, _ptr(idx), _ptr(sc))
    return idx, sc


def full(H: np.ndarray, E: np.ndarray, K: int, users=None):
    """Full-catalog head for the listed users.

    Returns dict(idx (nu,K) int64, score (nu,K) f64, lse (nu,) f64, S (nu,M) f64, users).
    """
    H, E = np.ascontiguousarray(H), np.ascontiguousarray(E)
    dt = _dtype_code(H)
    assert _dtype_code(E) == dt and H.shape[1] == E.shape[1]
    u = _users(users, H.shape[0])
    M, D = E.shape
    S = np.empty((u.size, M), dtype=np.float64)
    idx = np.empty((u.size, K), dtype=np.int64)
    sc = np.empty((u.size, K), dtype=np.float64)
    ls = np.empty(u.size, dtype=np.float64)
    _load().oracle_full(_ptr(H), _ptr(E), dt, D, M, K, _ptr(u), u.size, _ptr(S),
                        _ptr(idx), _ptr(sc), _ptr(ls))
    return dict(idx=idx, score=sc, lse=ls, S=S, users=u)


def full_masked(H: np.ndarray, E: np.ndarray, K: int, mask: np.ndarray, users=None):
    """Masked full-catalog head: item i takes part for user b only when bit i % 32
    of mask word [b][i // 32] (mask of shape (B, W)) or [i // 32] (shape (W,),
    one mask for all users) is set.  Same return value as full()."""
    H, E = np.ascontiguousarray(H), np.ascontiguousarray(E)
    dt = _dtype_code(H)
    assert _dtype_code(E) == dt and H.shape[1] == E.shape[1]
    u = _users(users, H.shape[0])
    M, D = E.shape
    mask = np.ascontiguousarray(mask, dtype=np.uint32)
    W = (M + 31) // 32
    if mask.ndim == 1:
        assert mask.size >= W
        stride = 0
    else:
        assert mask.shape[0] == H.shape[0] and mask.shape[1] >= W
        stride = mask.shape[1]
    S = np.empty((u.size, M), dtype=np.float64)
    idx = np.empty((u.size, K), dtype=np.int64)
    sc = np.empty((u.size, K), dtype=np.float64)
    ls = np.empty(u.size, dtype=np.float64)
    _load().oracle_full_masked(_ptr(H), _ptr(E), dt, D, M, K, _ptr(mask), stride, _ptr(u), u.size, _ptr(S),
                               _ptr(idx), _ptr(sc), _ptr(ls))
    return dict(idx=idx, score=sc, lse=ls, S=S, users=u)


def cand(H: np.ndarray, E: np.ndarray, offsets: np.ndarray, ids: np.ndarray, K: int, users=None):
    """Candidate-set head for the listed users.

    Returns dict(idx, score, lse, entry_scores (nnz,) f64 -- NaN where not
    computed or out of range --, n_bad, users).
    """
    H, E = np.ascontiguousarray(H), np.ascontiguousarray(E)
    dt = _dtype_code(H)
    off = np.ascontiguousarray(offsets, dtype=np.int64)
    idv = np.ascontiguousarray(ids, dtype=np.int32)
    B = off.size - 1
    u = _users(users, B)
    M, D = E.shape
    es = np.full(idv.size, np.nan, dtype=np.float64)
    idx = np.empty((u.size, K), dtype=np.int64)
    sc = np.empty((u.size, K), dtype=np.float64)
    ls = np.empty(u.size, dtype=np.float64)
    bad = _load().oracle_cand(_ptr(H), _ptr(E), dt, D, M, K, _ptr(off), _ptr(idv), _ptr(u), u.size,
                              _ptr(es), _ptr(idx), _ptr(sc), _ptr(ls))
    return dict(idx=idx, score=sc, lse=ls, entry_scores=es, n_bad=int(bad), users=u)


def widen(X: np.ndarray) -> np.ndarray:
    """Exact fp64 values of bf16 bit patterns (uint16) or float32 inputs."""
    if X.dtype == np.uint16:
        return (X.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    if X.dtype == np.float32:
        return X.astype(np.float64)
    raise TypeError("oracle inputs are uint16 (bf16 bits) or float32, got %s" % X.dtype)


def ce(H: np.ndarray, E: np.ndarray, labels: np.ndarray, weights=None, users=None, grads: bool = True):
    """Cross-entropy of the catalog softmax, reward-weighted per example.

    Follows the GenRec explainer page, "two objectives and reward-weighted
    ranking" section: the ranking objective is the cross-entropy of the
    softmax over the catalog, each example's loss multiplied by its scalar
    weight.  With s_bi = h_b . e_i (fp64, as scores()) and lse_b = ln sum_i
    exp(s_bi) (as lse()):
        loss_b = w_b (lse_b - s_{b, y_b})
        G[b][i] = w_b (exp(s_bi - lse_b) - [i == y_b])   (d loss_b / d s_bi)
        dH = G E,  dE = G^T H                               (chain rule through s = H E^T)
    An example whose label lies outside [0, M) is ignored: weight 0.
    users: rows to evaluate (default all); dE needs every user, so it is
    returned only when users is None.  Returns dict(loss, lse, users, S (the
    score rows), w (effective weights), and with grads: P (softmax rows), G,
    dH, and dE when users is None).
    """
    u = _users(users, H.shape[0])
    M = E.shape[0]
    S = scores(H, E, u)
    y = np.asarray(labels, dtype=np.int64)[u]
    w = np.ones(u.size) if weights is None else np.asarray(weights, dtype=np.float64)[u]
    valid = (y >= 0) & (y < M)
    w = np.where(valid, w, 0.0)
    lse_v = np.array([lse(S[r]) for r in range(u.size)])
    rows = np.arange(u.size)
    s_y = np.where(valid, S[rows, np.where(valid, y, 0)], 0.0)
    out = dict(loss=w * (lse_v - s_y), lse=lse_v, users=u, S=S, w=w)
    if grads:
        P = np.exp(S - lse_v[:, None])
        G = w[:, None] * P
        G[rows[valid], y[valid]] -= w[valid]
        out["P"] = P
        out["G"] = G
        # dH = G E, with E widened a block of rows at a time (memory only)
        dH = np.zeros((u.size, E.shape[1]))
        for i0 in range(0, M, 65536):
            dH += G[:, i0:i0 + 65536] @ widen(E[i0:i0 + 65536])
        out["dH"] = dH
        if users is None:
            out["dE"] = G.T @ widen(H)
    return out
