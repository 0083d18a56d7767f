"""Seeded input generator: determinism, distributions and structure."""
import math

import numpy as np
import torch

from full_catalog_ranking_amd import synth


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(100_000) * np.exp(rng.uniform(-20, 20, 100_000))).astype(np.float32)
    x[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]  # exact halfway cases
    ours = synth.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = synth.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_catalog_chunked_generation_is_thread_independent():
    a = synth.gen_E(3 * synth.ROW_CHUNK + 77, 64, seed=4, threads=1)
    b = synth.gen_E(3 * synth.ROW_CHUNK + 77, 64, seed=4, threads=5)
    assert np.array_equal(a, b)
    c = synth.gen_E(3 * synth.ROW_CHUNK + 77, 64, seed=5, threads=5)
    assert not np.array_equal(a, c)


def test_zipf_norms():
    n = synth.zipf_norms(1_000_000)
    assert n[0] == 2.0 and abs(n[-1] - 0.5) < 1e-15
    assert (np.diff(n) <= 0).all()
    assert (n > 0.6).sum() == 11  # only a handful of items stand out
    assert 0.5 < n.mean() < 0.51


def test_catalog_row_norms_follow_popularity():
    D, M = 2048, 20000
    E = synth.bf16_bits_to_f32(synth.gen_E(M, D, seed=0)).astype(np.float64)
    norms = np.linalg.norm(E, axis=1)
    target = synth.zipf_norms(M)
    # ||g|| for g ~ N(0, I/D) concentrates at 1 with std ~ 1/sqrt(2D)
    assert np.abs(norms / target - 1).max() < 8 / math.sqrt(2 * D)
    H = synth.bf16_bits_to_f32(synth.make_dense(4, D, 10, seed=0)["H"])
    assert abs(H.std() - 1) < 0.02


def test_candidate_lists_structure():
    off, ids = synth.gen_candidates(64, 1_000_000, seed=0, lo=100, hi=3000)
    lens = np.diff(off)
    assert off[0] == 0 and off[-1] == ids.size
    assert lens.min() >= 100 and lens.max() <= 3000
    assert ids.min() >= 0 and ids.max() < 1_000_000
    for b in range(64):
        lst = ids[off[b]:off[b + 1]]
        assert np.unique(lst).size == lst.size  # without replacement
    # Zipf weighting: the most popular item appears in (nearly) every list
    assert (ids == 0).sum() >= 60
    off2, ids2 = synth.gen_candidates(64, 1_000_000, seed=0, lo=100, hi=3000, threads=1)
    assert np.array_equal(off, off2) and np.array_equal(ids, ids2)


def test_tiny_workload_recipe():
    d = synth.make_workload("tiny")
    assert d["H"].dtype == np.float32 and d["E"].shape == (5000, 256)
    for u in range(4):
        assert np.array_equal(d["E"][17 + u], 2 * d["H"][u])
    assert abs(d["E"][1000:].std() * math.sqrt(256) - 1) < 0.01


def test_beam_scores_seeded_and_shaped():
    a = synth.gen_scores(3, 1000, seed=4)
    b = synth.gen_scores(3, 1000, seed=4)
    assert a.dtype == np.float32 and a.shape == (3, 1000) and np.array_equal(a, b)
    t = synth.gen_scores(2, 5000, seed=4, decimals=1)
    assert np.unique(t[0]).size < 500   # rounding makes ties common
    w = synth.make_workload("beam128")
    assert w["scores"].shape == (256, 16384) and w["K"] == 128


def test_clustered_catalog():
    """Contiguous clusters: rows of one cluster share its centre (their mean
    pairwise inner product is the centre's share, 1 / 1.25), rows of different
    clusters do not; threaded generation equals serial generation."""
    M, D, C = 12_000, 128, 6
    E = synth.gen_E_clustered(M, D, 3, C, bf16=False)
    assert np.array_equal(E, synth.gen_E_clustered(M, D, 3, C, bf16=False, threads=1))
    assert abs(float((E * E).sum(1).mean()) - 1.0) < 0.02
    same = float((E[:1000] * E[1000:2000]).sum(1).mean())
    assert abs(same - 0.8) < 0.1  # rows 0..1999 are cluster 0 (M / C = 2,000 rows a cluster)
    other = float((E[:1000] * E[M // C:M // C + 1000]).sum(1).mean())
    assert abs(other) < 0.2
    bits = synth.gen_E_clustered(M, D, 3, C)
    assert np.array_equal(bits, synth.f32_to_bf16_bits(E))
