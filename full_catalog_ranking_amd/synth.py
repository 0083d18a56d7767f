"""Seeded synthetic inputs for the ranking head (user states H, item catalog E,
per-user candidate lists).

This module only draws inputs. It holds none of the ranking head's arithmetic
(no scores, no normaliser, no ranking), so both the GPU path and the CPU oracle
can consume what it produces without sharing any of the method's code.

Shapes follow the pages: a pooled user vector h of size D per user, batched as
H (B x D), and a catalog of M item embeddings stored row-major as E (M x D)
(GenRec concept page, the scoring formula s = E^T h and the two PyTorch demos,
which hold the catalog as an (M, D) tensor). Candidate sets are jagged
per-user lists (GenRec explainer page, top-K ranking over a separately given
candidate set; HSTU explainer page, ragged sequences).

Recipe (all host-side numpy; every array has its own counter-keyed stream so
that chunked / threaded generation is bit-identical to serial generation):

* ``H``: standard normal float32 draws (``N(0, 1)``), stream key (seed, 0).
  For the fp32 "tiny" workload the draws are scaled by float32(1/sqrt(D)).
* ``E``: row-chunks of ``ROW_CHUNK`` rows, chunk ``c`` drawn from stream key
  (seed, 1, c) as float32 standard normals, multiplied by a per-row float32
  scale ``norm_i / sqrt(D)``.  ``norm_i`` is the popularity norm of item i:
  item i has popularity rank r = i + 1, Zipf weight w_r = r**-1.1, and
  ``norm = 0.5 + 1.5 * (w_r - w_M) / (w_1 - w_M)``, a linear map of the weights
  onto [0.5, 2].  (Tiny workload: norm = 1, i.e. rows ~ N(0, I/D).)
* bf16 inputs are the float32 values rounded to nearest-even bfloat16; arrays
  are returned as uint16 bit patterns.
* Candidate lists: user b's list length is uniform on [lo, hi] (inclusive),
  drawn from stream (seed, 2, b); the ids are the first distinct values of an
  i.i.d. sequence drawn with probability proportional to the Zipf weights, from
  the same stream.  Keeping first occurrences of an i.i.d. weighted sequence is
  exactly successive weighted sampling without replacement, and the list keeps
  that sampled order.
* Clustered catalog (a robustness variant, ``make_dense(..., clusters=C)``):
  items stored grouped by category, see gen_E_clustered.
* Cross-entropy examples: user b's label (the engaged item) is one draw with
  probability proportional to the Zipf weights, from stream (seed, 3); its
  reward weight is uniform on [0.25, 2], from stream (seed, 4).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROW_CHUNK = 8192
ZIPF_S = 1.1


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(list(key)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def zipf_weights(M: int) -> np.ndarray:
    r = np.arange(1, M + 1, dtype=np.float64)
    return r ** (-ZIPF_S)


def zipf_norms(M: int) -> np.ndarray:
    """Popularity norms in [0.5, 2]: a linear map of the Zipf(1.1) weights."""
    w = zipf_weights(M)
    if M == 1:
        return np.full(1, 2.0)
    return 0.5 + 1.5 * (w - w[-1]) / (w[0] - w[-1])


def _threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def gen_H(B: int, D: int, seed: int, scale: float = 1.0) -> np.ndarray:
    z = _rng(seed, 0).standard_normal((B, D), dtype=np.float32)
    if scale != 1.0:
        z *= np.float32(scale)
    return z


def gen_E(M: int, D: int, seed: int, zipf: bool = True, permute: bool = False,
          bf16: bool = True, threads: int | None = None) -> np.ndarray:
    """Catalog rows (M x D): float32 normals scaled by norm_i / sqrt(D).

    Returns uint16 bf16 bits when ``bf16`` is set, float32 otherwise.
    ``permute`` assigns the popularity norms through a seeded permutation
    instead of by item index (robustness variant: popular items scattered).
    """
    if zipf:
        norms = zipf_norms(M)
        if permute:
            norms = norms[_rng(seed, 3).permutation(M)]
    else:
        norms = np.ones(M)
    scale = (norms / math.sqrt(D)).astype(np.float32)
    out = np.empty((M, D), dtype=np.uint16 if bf16 else np.float32)
    nchunk = (M + ROW_CHUNK - 1) // ROW_CHUNK

    def work(c: int) -> None:
        r0, r1 = c * ROW_CHUNK, min(M, (c + 1) * ROW_CHUNK)
        z = _rng(seed, 1, c).standard_normal((r1 - r0, D), dtype=np.float32)
        z *= scale[r0:r1, None]
        out[r0:r1] = f32_to_bf16_bits(z) if bf16 else z

    n = threads or _threads()
    if n == 1 or nchunk == 1:
        for c in range(nchunk):
            work(c)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, range(nchunk)))
    return out


def gen_E_clustered(M: int, D: int, seed: int, n_clusters: int, spread: float = 0.5, bf16: bool = True,
                    threads: int | None = None) -> np.ndarray:
    """A catalog stored grouped by category: item i belongs to cluster
    c = i * n_clusters // M (contiguous runs of ids), and
    E_i = (mu_c + spread * g_i) / sqrt(1 + spread^2) with the cluster centres
    mu_c (stream key (seed, 6)) and the item parts g_i (stream (seed, 7, chunk))
    both N(0, I/D).  A user's best items then come from the few clusters its
    vector favours: a handful of contiguous id ranges, unlike the exchangeable
    catalogs of gen_E.  Returns uint16 bf16 bits when ``bf16``, else float32.
    """
    s = np.float32(1.0 / math.sqrt(D))
    mu = _rng(seed, 6).standard_normal((n_clusters, D), dtype=np.float32) * s
    cl = (np.arange(M, dtype=np.int64) * n_clusters) // M
    a = np.float32(1.0 / math.sqrt(1.0 + spread * spread))
    out = np.empty((M, D), dtype=np.uint16 if bf16 else np.float32)
    nchunk = (M + ROW_CHUNK - 1) // ROW_CHUNK

    def work(c: int) -> None:
        r0, r1 = c * ROW_CHUNK, min(M, (c + 1) * ROW_CHUNK)
        z = _rng(seed, 7, c).standard_normal((r1 - r0, D), dtype=np.float32)
        z *= np.float32(spread) * s
        z += mu[cl[r0:r1]]
        z *= a
        out[r0:r1] = f32_to_bf16_bits(z) if bf16 else z

    n = threads or _threads()
    if n == 1 or nchunk == 1:
        for c in range(nchunk):
            work(c)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, range(nchunk)))
    return out


def gen_candidates(B: int, M: int, seed: int, lo: int, hi: int,
                   threads: int | None = None) -> tuple[np.ndarray, np.ndarray]:
    """Per-user jagged candidate lists in CSR form: (offsets int64[B+1], ids int32[nnz])."""
    w = zipf_weights(M)
    cdf = np.cumsum(w)
    cdf /= cdf[-1]
    lists: list[np.ndarray] = [None] * B  # type: ignore[list-item]

    def work(b: int) -> None:
        g = _rng(seed, 2, b)
        L = int(g.integers(lo, hi, endpoint=True))
        L = min(L, M)
        seen = np.zeros(0, dtype=np.int64)
        rounds = 0
        while seen.size < L:
            draw = np.searchsorted(cdf, g.random(max(2 * (L - seen.size), 64)), side="right")
            draw = np.minimum(draw, M - 1)
            # first occurrences, in draw order, of ids not drawn before
            _, first = np.unique(draw, return_index=True)
            first.sort()
            cand = draw[first]
            cand = cand[~np.isin(cand, seen)]
            seen = np.concatenate([seen, cand])
            rounds += 1
            if rounds > 64 and seen.size < L:
                # lists close to the catalog size: finish with the unseen ids
                # in index order (never reached by the benchmark shapes)
                rest = np.setdiff1d(np.arange(M), seen)
                seen = np.concatenate([seen, rest])
        lists[b] = seen[:L].astype(np.int32)

    n = threads or _threads()
    if n == 1 or B < 8:
        for b in range(B):
            work(b)
    else:
        with ThreadPoolExecutor(n) as ex:
            list(ex.map(work, range(B)))
    lens = np.array([x.size for x in lists], dtype=np.int64)
    offsets = np.zeros(B + 1, dtype=np.int64)
    np.cumsum(lens, out=offsets[1:])
    ids = np.concatenate(lists) if B else np.zeros(0, dtype=np.int32)
    return offsets, ids.astype(np.int32)


def gen_labels(B: int, M: int, seed: int) -> np.ndarray:
    """One engaged item per example (int32 [B]), Zipf-weighted by popularity rank."""
    cdf = np.cumsum(zipf_weights(M))
    cdf /= cdf[-1]
    y = np.searchsorted(cdf, _rng(seed, 3).random(B), side="right")
    return np.minimum(y, M - 1).astype(np.int32)


def gen_weights(B: int, seed: int) -> np.ndarray:
    """Per-example reward weights (float32 [B]), uniform on [0.25, 2]."""
    return _rng(seed, 4).uniform(0.25, 2.0, B).astype(np.float32)


# ---------------------------------------------------------------------------
# Named workloads.  Sizes follow the five benchmark shapes of this project:
# a 4-user fp32 toy with planted items, a single-user GEMV, a 256-user batch,
# a 1,024-user x 1,000,000-item compute-bound catalog, and 4,096 users with
# jagged Zipf-weighted candidate lists over a 1,000,000-item catalog.
# ---------------------------------------------------------------------------
WORKLOADS = {
    "tiny":  dict(B=4, D=256, M=5000, K=10, dtype="f32"),
    "gemv":  dict(B=1, D=2048, M=5000, K=100, dtype="bf16"),
    "batch": dict(B=256, D=2048, M=100_000, K=100, dtype="bf16"),
    # the batch shape with fp32 inputs (the fp32 matrix-core path)
    "batch_f32": dict(B=256, D=2048, M=100_000, K=100, dtype="f32"),
    "large": dict(B=1024, D=4096, M=1_000_000, K=500, dtype="bf16"),
    "cand":  dict(B=4096, D=2048, M=1_000_000, K=100, dtype="bf16", lo=100, hi=3000),
    # one user against an 8 GB catalog: sustained catalog streaming at B = 1
    "gemv_big": dict(B=1, D=4096, M=1_000_000, K=100, dtype="bf16"),
    # beam steps: R requests of width x width continuation scores -> the best `width`
    "beam128": dict(R=256, N=128 * 128, K=128, kind="beam"),
    "beam512": dict(R=64, N=512 * 512, K=512, kind="beam"),
    # reward-weighted catalog cross-entropy, forward + backward, at the large shape
    "ce": dict(B=1024, D=4096, M=1_000_000, K=0, dtype="bf16", kind="ce"),
}

TINY_PLANT_ITEM = 17


def make_tiny(seed: int = 0, B: int = 4, D: int = 256, M: int = 5000,
              plant: int = TINY_PLANT_ITEM) -> dict:
    """fp32 toy: H, E ~ N(0, I/D); user u's planted row plant+u is 2 * h_u."""
    s = np.float32(1.0 / math.sqrt(D))
    H = gen_H(B, D, seed, scale=float(s))
    E = gen_E(M, D, seed, zipf=False, bf16=False)
    for u in range(B):
        if plant + u < M:
            E[plant + u] = np.float32(2.0) * H[u]
    return dict(H=H, E=E, B=B, D=D, M=M, dtype="f32")


def make_dense(B: int, D: int, M: int, seed: int = 0, permute: bool = False,
               bf16: bool = True, clusters: int = 0) -> dict:
    """H ~ N(0, 1); E rows N(0, I/D) scaled by Zipf-ranked popularity norms
    (with ``clusters``: the clustered catalog of gen_E_clustered instead)."""
    H = gen_H(B, D, seed)
    if clusters:
        E = gen_E_clustered(M, D, seed, clusters, bf16=bf16)
    else:
        E = gen_E(M, D, seed, zipf=True, permute=permute, bf16=bf16)
    if bf16:
        H = f32_to_bf16_bits(H)
    return dict(H=H, E=E, B=B, D=D, M=M, dtype="bf16" if bf16 else "f32")


def gen_scores(R: int, N: int, seed: int, decimals: int | None = None) -> np.ndarray:
    """Beam-step scores (R x N float32): a per-row offset (the beam's running
    log-probability) plus N(0, 1) continuation scores; with `decimals` the
    values are rounded, which makes exact ties frequent."""
    z = _rng(seed, 4).standard_normal((R, N), dtype=np.float32)
    z += _rng(seed, 5).standard_normal((R, 1), dtype=np.float32) * np.float32(3.0)
    if decimals is not None:
        z = np.round(z, decimals).astype(np.float32)
    return z


def make_workload(name: str, seed: int = 0, **over) -> dict:
    cfg = dict(WORKLOADS[name])
    cfg.update(over)
    if cfg.get("kind") == "beam":
        return dict(scores=gen_scores(cfg["R"], cfg["N"], seed), R=cfg["R"], N=cfg["N"], K=cfg["K"], kind="beam")
    if name == "tiny":
        d = make_tiny(seed, B=cfg["B"], D=cfg["D"], M=cfg["M"])
    else:
        d = make_dense(cfg["B"], cfg["D"], cfg["M"], seed, bf16=cfg["dtype"] == "bf16",
                       clusters=cfg.get("clusters", 0))
    d["K"] = cfg["K"]
    if name == "cand":
        d["offsets"], d["ids"] = gen_candidates(cfg["B"], cfg["M"], seed, cfg["lo"], cfg["hi"])
    if cfg.get("kind") == "ce":
        d["labels"] = gen_labels(cfg["B"], cfg["M"], seed)
        d["weights"] = gen_weights(cfg["B"], seed)
        d["kind"] = "ce"
    return d
