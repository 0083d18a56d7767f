"""GPU parity: the HIP ranking head (through the C ABI) against the CPU oracle
on seeded synthetic inputs, element by element under the rule in parity.py."""
import math

import numpy as np
import pytest

from full_catalog_ranking_amd import synth
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from full_catalog_ranking_amd import genrec
    genrec.lib()  # fails loudly if the HIP library is missing
    return torch.device("cuda:0")


def to_dev(a, dev):
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def run_dense(d, K, dev):
    from full_catalog_ranking_amd import genrec
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    print("  dense B=%d D=%d M=%d K=%d %s plan=%s" % (d["B"], d["D"], d["M"], K, H.dtype,
                                                     genrec.describe_plan(d["B"], d["D"], d["M"], K, H.dtype)),
          flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, E, K)
    torch.cuda.synchronize()
    out = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    del H, E
    return out


def run_cand(d, K, dev, repeats=0):
    """One call (outputs, device error counts); with repeats, that many more
    calls on the same device inputs, each of whose outputs must equal the
    first call's bit for bit (the selection's result does not depend on the
    order in which threads arrive, so a difference is a race)."""
    from full_catalog_ranking_amd import genrec
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    off = torch.from_numpy(d["offsets"]).to(dev)
    ids = torch.from_numpy(d["ids"]).to(dev)
    print("  cand B=%d D=%d M=%d nnz=%d K=%d" % (d["B"], d["D"], d["M"], d["ids"].size, K), flush=True)
    idx, sc, ls, ws = genrec.score_candidates_topk(H, E, off, ids, K)
    errs = genrec.device_errors(ws)
    out = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    for r in range(repeats):
        idx2, sc2, ls2, _ = genrec.score_candidates_topk(H, E, off, ids, K)
        again = idx2.cpu().numpy(), sc2.cpu().numpy(), ls2.cpu().numpy()
        for name, x, y in zip(("idx", "score", "lse"), out, again):
            bad = np.flatnonzero(~((x == y) | (np.isnan(x) & np.isnan(y))).reshape(x.shape[0], -1).all(axis=1))
            assert bad.size == 0, ("repeat %d differs in %s for users" % (r + 1, name), bad[:8].tolist())
    return out, errs


# ---------------------------------------------------------------------------
# The five benchmark workloads
# ---------------------------------------------------------------------------
def test_tiny_fp32_planted(dev, oracle_mod):
    d = synth.make_workload("tiny")
    K = d["K"]
    g = run_dense(d, K, dev)
    ref = oracle_mod.full(d["H"], d["E"], K)
    parity.check_dense(g, ref, where="tiny")
    assert (g[0][:, 0] == synth.TINY_PLANT_ITEM + np.arange(4)).all()


def test_gemv_b1(dev, oracle_mod):
    d = synth.make_workload("gemv")
    g = run_dense(d, d["K"], dev)
    ref = oracle_mod.full(d["H"], d["E"], d["K"])
    parity.check_dense(g, ref, where="gemv")


def test_batch_b256_all_users(dev, oracle_mod):
    d = synth.make_workload("batch")
    g = run_dense(d, d["K"], dev)
    ref = oracle_mod.full(d["H"], d["E"], d["K"])
    parity.check_dense(g, ref, where="batch")


@pytest.fixture(scope="module")
def large_run(dev):
    """The full-size large workload (1,024 x 1e6 x 4,096, K 500) and one call's
    host outputs, shared by the tests below."""
    d = synth.make_workload("large")
    return d, run_dense(d, d["K"], dev)


def test_large_b1024_sampled_users(dev, oracle_mod, large_run):
    """40 users against the oracle: ten in each of the four 256-user tiles, at
    tile positions that cover every wave's user columns (64 per wave tile, two
    32-wide blocks each); their top-K items come from every one of the eight
    XCD groups of catalog chunks."""
    from full_catalog_ranking_amd import genrec
    d, g = large_run
    offs = [0, 31, 32, 63, 64, 100, 127, 160, 200, 255]
    users = [256 * t + o for t in range(4) for o in offs]
    ref = oracle_mod.full(d["H"], d["E"], d["K"], users=users)
    parity.check_dense(g, ref, where="large")
    # chunk c of the main pass runs on XCD group c // (P / 8); every group's
    # catalog range holds some of the checked users' top-K items
    P = genrec.describe_plan(d["B"], d["D"], d["M"], d["K"], torch.bfloat16)["P"]
    assert P % 8 == 0
    base, rem = divmod(-(-d["M"] // 256), P)  # chunk c = tiles [c base + min(c, rem), ...)
    starts = np.array([c * base + min(c, rem) for c in range(P)])
    chunk_of = np.searchsorted(starts, ref["idx"].ravel() // 256, side="right") - 1
    groups = set((chunk_of // (P // 8)).tolist())
    assert groups == set(range(8)), groups
    # every user: lse and scores are finite and descending, ids distinct and in range
    idx, sc, ls = g
    assert np.isfinite(ls).all() and (idx >= 0).all() and (idx < d["M"]).all()
    assert (np.diff(sc, axis=1) <= 0).all()
    assert all(np.unique(r).size == d["K"] for r in idx[::37])


def _widen_bf16(bits):
    """bf16 bit patterns -> float32, exactly (the bf16 value is the top half)."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def test_large_b1024_all_users(dev, large_run):
    """Every one of the 1,024 users of the full-size call, by properties that
    need no oracle row (the oracle's full sort of 1e9 scores is out of reach):
    (1) the score returned with each id is the fp64 dot product of that user's
    and item's bf16 rows, within the parity rule's tau; (2) no item outside a
    user's list scores above the list's K-th score by more than tau; (3) the
    lse is the log-sum-exp of all M scores, within the parity rule's bound.
    (2) and (3) take the scores from a float32 library product of the widened
    rows, chunk by chunk (its rounding, ~1e-5 relative at D = 4,096, is far
    inside tau)."""
    _check_all_users(large_run[0], large_run[1], dev)


def test_large_masked_b1024_all_users(dev, large_run):
    """The masked head at the full large shape (one global mask allowing 90% of
    the items): every user's list holds allowed items only, and the checks of
    test_large_b1024_all_users hold over the allowed items."""
    from full_catalog_ranking_amd import genrec
    d = large_run[0]
    allowed = np.random.default_rng(91).random(d["M"]) < 0.9
    mask = torch.from_numpy(_pack_mask(allowed).view(np.int32)).to(dev)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    print("  masked full size B=%d M=%d K=%d" % (d["B"], d["M"], d["K"]), flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, E, d["K"], mask=mask)
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    del H, E, idx, sc, ls
    torch.cuda.empty_cache()
    assert allowed[g[0].astype(np.int64)].all()
    _check_all_users(d, g, dev, allowed)


def _check_all_users(d, g, dev, allowed=None):
    """The properties above for every user (over the allowed items only when a
    mask is given)."""
    idx, sc, ls = g
    B, M, K = d["B"], d["M"], d["K"]
    assert idx.shape == (B, K) and (idx >= 0).all() and np.isfinite(sc).all()
    Hf = _widen_bf16(d["H"])
    tau = parity.SCORE_REL * float(np.abs(sc).max())
    worst = 0.0
    for b in range(B):
        s64 = _widen_bf16(d["E"][idx[b]]).astype(np.float64) @ Hf[b].astype(np.float64)
        worst = max(worst, float(np.abs(s64 - sc[b].astype(np.float64)).max()))
    assert worst <= tau, ("returned scores vs fp64 rescoring", worst, tau)
    prev = (torch.backends.cuda.matmul.allow_tf32, torch.get_float32_matmul_precision())
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.set_float32_matmul_precision("highest")
    try:
        Ht = torch.from_numpy(Hf).to(dev).t().contiguous()  # [D][B]: no transposed operand view
        thr = torch.from_numpy(sc[:, K - 1].astype(np.float32) + np.float32(tau)).to(dev)
        lse = torch.full((B,), -math.inf, dtype=torch.float64, device=dev)
        keys = []
        step = 65536
        for r0 in range(0, M, step):
            r1 = min(M, r0 + step)
            St = to_dev(d["E"][r0:r1], dev).float() @ Ht  # [items][B] fp32
            if allowed is not None:
                St[torch.from_numpy(~allowed[r0:r1]).to(dev)] = -math.inf
            lse = torch.logaddexp(lse, torch.logsumexp(St.double(), dim=0))
            nz = torch.nonzero(St > thr[None, :]).cpu().numpy().astype(np.int64)  # (item, user)
            keys.append(nz[:, 1] * M + nz[:, 0] + r0)
            del St
        lse = lse.cpu().numpy()
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev[0]
        torch.set_float32_matmul_precision(prev[1])
    above = np.concatenate(keys)
    listed = (np.arange(B, dtype=np.int64)[:, None] * M + idx.astype(np.int64)).ravel()
    missing = above[~np.isin(above, listed)]
    assert missing.size == 0, ("items above the K-th score + tau not listed", (missing // M)[:8], (missing % M)[:8])
    err = np.abs(lse - ls.astype(np.float64))
    assert err.max() <= parity.LSE_ABS, ("lse", int(err.argmax()), float(err.max()))


@pytest.mark.parametrize("B,D,M,K", [
    (600, 64, 700_000, 10),   # MFMA path, > 512 users: 256-thread threshold, 22,016-item sample
    (1, 64, 700_000, 50),     # VALU path, one user: 1024-thread threshold, same sample size
])
def test_threshold_full_capacity(dev, oracle_mod, B, D, M, K):
    """Samples above 16,384 items take the threshold kernel's 32,768-key build."""
    from full_catalog_ranking_amd import genrec
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    assert plan["sample"] == 1 and 16384 < plan["n_sample"] <= 32768
    d = synth.make_dense(B, D, M, seed=B + K)
    g = run_dense(d, K, dev)
    users = sorted({0, min(1, B - 1), B // 2, B - 1})
    ref = oracle_mod.full(d["H"], d["E"], K, users=users)
    parity.check_dense(g, ref, where="threshold capacity %s" % ((B, D, M, K),))


def test_candidates_b4096(dev, oracle_mod):
    # lists of up to 3,000 entries take the selection's multi-pass route
    # (more keys than its LDS gather holds); the repeats guard the barriers
    # between its passes
    d = synth.make_workload("cand")
    g, errs = run_cand(d, d["K"], dev, repeats=3)
    assert errs == (0, 0)
    ref = oracle_mod.cand(d["H"], d["E"], d["offsets"], d["ids"], d["K"])
    parity.check_cand(g, ref, d["offsets"], d["ids"], where="cand")


# ---------------------------------------------------------------------------
# Ragged shapes and edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,D,M,K", [
    (3, 96, 70000, 50),       # a small batch on the matrix cores, sampled pre-pass
    (8, 2048, 4097, 100),     # B = 8: one user tile 97% empty
    (2, 8, 300, 20),          # smallest D: one k-step, all of it k tail
    (300, 200, 70001, 37),    # two user tiles (ragged), sampled pass, ragged item tail, k tail (D % 32 != 0)
    (9, 64, 50, 64),          # K > M: padding; smallest MFMA batch
    (17, 128, 3000, 1),       # K = 1
    (33, 256, 3000, 1024),    # K = KMAX
    (513, 512, 20000, 100),   # three user tiles, no sampling
])
def test_mfma_ragged(dev, oracle_mod, B, D, M, K):
    d = synth.make_dense(B, D, M, seed=B + M)
    g = run_dense(d, K, dev)
    users = sorted(set([0, 1, B // 2, B - 1] + list(range(0, B, max(1, B // 12)))))
    ref = oracle_mod.full(d["H"], d["E"], K, users=users)
    parity.check_dense(g, ref, where="mfma %s" % ((B, D, M, K),))


@pytest.mark.parametrize("D,split", [(512, True), (72, False)])
def test_fast_threshold_rescue(dev, oracle_mod, D, split):
    """A user whose sampled catalog tile (the first window's) holds 40 scaled
    copies of its own vector: the fast threshold (a high-ranked sampled score) lets fewer
    than K catalog items through for that user, the merge flags it, and the
    rescue pass must still give the exact result -- with the K-th sampled
    score when the sample is bit-identical to the main pass (D = 72: no
    reduction split), with every score when the sample was a split reduction
    (D = 512: two splits of eight k-steps); every other user keeps its
    first-pass result."""
    from full_catalog_ranking_amd import genrec
    B, M, K = 16, 131072, 100
    d = synth.make_dense(B, D, M, seed=11)
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    assert plan["path"] == "mfma" and plan["fast"] == 1 and plan["r_fast"] < 40 < K
    assert (plan["sample_splits"] > 1) == split and plan["safe_exact"] == (not split)
    h = synth.bf16_bits_to_f32(d["H"][3])
    E = d["E"].copy()
    row0 = plan["first_sampled_tile"] * 256
    assert 0 <= row0 < plan["stride"] * 256
    for i in range(40):
        E[row0 + i] = synth.f32_to_bf16_bits((h * np.float32(0.05 + 0.001 * i)).astype(np.float32))
    H, Ed = to_dev(d["H"], dev), to_dev(E, dev)
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
    print("  rescue B=%d D=%d M=%d K=%d plan=%s" % (B, D, M, K, plan), flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, Ed, K, workspace=ws)
    n_rescued = genrec.rescued_users(ws)
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    ref = oracle_mod.full(d["H"], E, K)
    parity.check_dense(g, ref, where="rescue")
    assert set(g[0][3, :40].tolist()) == set(range(row0, row0 + 40))
    # user 3 at least; users whose vectors lean towards user 3's can find the
    # planted rows among their own top sampled scores and be rescued as well
    # (every user's result is exact: checked above)
    assert 1 <= n_rescued <= B
    # a second call on the same workspace without the planted rows: no rescue
    idx, sc, ls = genrec.score_lse_topk(H, to_dev(d["E"], dev), K, workspace=ws)
    assert genrec.rescued_users(ws) == 0
    parity.check_dense((idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()),
                       oracle_mod.full(d["H"], d["E"], K, users=[0, 3, 15]), where="no rescue")


def test_periodic_catalog_is_not_sampled_in_step(dev, oracle_mod):
    """Every 32nd catalog tile (tiles 0, 32, 64, ...) holds rows of 4x the norm,
    so they hold every user's highest scores -- a catalog stored in a periodic
    order.  A sample of the first tile of every 32-tile window would be exactly
    those tiles, and its fast threshold would let fewer than K items through
    for every user (all of them rescued).  The sample takes a hashed position
    inside each window, so at most one or two of its 13 tiles are such tiles:
    the threshold is representative for nearly every user (the 14th-largest
    score of one sampled 4x tile leaves fewer than K items for a few percent
    of users, which the rescue pass handles), and the results match the
    oracle."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 256, 128, 100_000, 100
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    assert plan["path"] == "mfma" and plan["fast"] == 1 and plan["stride"] == 32
    d = synth.make_dense(B, D, M, seed=12)
    E = synth.bf16_bits_to_f32(d["E"])
    for t in range(0, M // 256, 32):
        E[t * 256:(t + 1) * 256] *= np.float32(4.0)
    Eb = synth.f32_to_bf16_bits(E)
    H, Ed = to_dev(d["H"], dev), to_dev(Eb, dev)
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
    print("  periodic catalog B=%d D=%d M=%d K=%d plan=%s" % (B, D, M, K, plan), flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, Ed, K, workspace=ws)
    n_rescued = genrec.rescued_users(ws)
    print("  rescued users: %d of %d" % (n_rescued, B), flush=True)
    assert n_rescued < B // 8
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    users = [0, 1, 77, 128, 255]
    parity.check_dense(g, oracle_mod.full(d["H"], Eb, K, users=users), where="periodic catalog")


def _pack_mask(allowed):
    M = allowed.shape[-1]
    W = (M + 31) // 32
    pad = np.zeros(allowed.shape[:-1] + (W * 32,), dtype=bool)
    pad[..., :M] = allowed
    bits = pad.reshape(allowed.shape[:-1] + (W, 32)).astype(np.uint64)
    return (bits << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)


@pytest.mark.parametrize("case,B,D,M,K,per_user,bf16", [
    ("global 90%, sampled fast path", 256, 512, 100_000, 100, False, True),
    ("per-user densities incl. none and < K, ragged, k tail", 300, 200, 70_001, 37, True, True),
    ("per-user, VALU path with sample", 3, 96, 70_000, 50, True, True),
    ("global 2% (< K allowed), unsampled MFMA", 17, 128, 3000, 64, False, True),
    ("per-user incl. none and < K, fused one-launch path (fp32)", 3, 64, 5000, 40, True, False),
])
def test_masked_head(dev, oracle_mod, case, B, D, M, K, per_user, bf16):
    from full_catalog_ranking_amd import genrec
    d = synth.make_dense(B, D, M, seed=B + D, bf16=bf16)
    rng = np.random.default_rng(B * 31 + M)
    if per_user:
        dens = np.concatenate([[0.0, 1e-4, 1.0], rng.uniform(0.005, 1.0, max(0, B - 3))])[:B]
        allowed = rng.random((B, M)) < dens[:, None]
    else:
        allowed = np.broadcast_to(rng.random(M) < (0.9 if M > 10_000 else 0.02), (B, M))
    words = _pack_mask(allowed if per_user else allowed[0])
    mask = torch.from_numpy(words.view(np.int32)).to(dev)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    print("  masked %s B=%d D=%d M=%d K=%d" % (case, B, D, M, K), flush=True)
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
    idx, sc, ls = genrec.score_lse_topk(H, E, K, workspace=ws, mask=mask)
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    users = sorted(set([0, 1, 2, B - 1] + list(range(0, B, max(1, B // 10)))))
    if not bf16:
        assert genrec.describe_plan(B, D, M, K, H.dtype)["fused"] == 1
    ref = oracle_mod.full_masked(d["H"], d["E"], K, words, users=users)
    parity.check_dense(g, ref, where="masked %s" % case)
    for b in range(B):  # every returned item is allowed, every padded slot is (-1, -inf)
        ids = g[0][b]
        assert allowed[b][ids[ids >= 0]].all()
        assert (np.isneginf(g[1][b][ids < 0])).all()
    if not per_user and M > 10_000:
        assert genrec.rescued_users(ws) == 0


def test_masked_all_allowed_equals_unmasked(dev):
    from full_catalog_ranking_amd import genrec
    d = synth.make_dense(40, 256, 70_000, seed=8)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    words = _pack_mask(np.ones(70_000, dtype=bool))
    a = genrec.score_lse_topk(H, E, 30)
    b = genrec.score_lse_topk(H, E, 30, mask=torch.from_numpy(words.view(np.int32)).to(dev))
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,D,M,K,bf16", [
    (1, 96, 70000, 50, True),    # VALU path (B = 1) with the sampled pre-pass
    (1, 8, 1, 5, True),          # M = 1, K > M
    (1, 64, 70000, 50, False),   # fp32 VALU path with the sampled pre-pass
    (20, 256, 1500, 10, False),  # fp32 with many users (one launch)
    (2, 4, 333, 333, False),     # K = M, smallest fp32 D
])
def test_stream_ragged(dev, oracle_mod, B, D, M, K, bf16):
    d = synth.make_dense(B, D, M, seed=B * 7 + M, bf16=bf16)
    g = run_dense(d, K, dev)
    ref = oracle_mod.full(d["H"], d["E"], K)
    parity.check_dense(g, ref, where="stream %s" % ((B, D, M, K, bf16),))


def test_permuted_popularity_batch(dev, oracle_mod):
    d = synth.make_dense(256, 1024, 100_000, seed=3, permute=True)
    g = run_dense(d, 100, dev)
    ref = oracle_mod.full(d["H"], d["E"], 100, users=list(range(0, 256, 5)))
    parity.check_dense(g, ref, where="permuted")


def test_exact_ties_break_by_lower_id(dev):
    # rows 10, 500, 2000 and 4999 identical: equal scores for every user
    for B in (1, 2, 64):  # fused one-launch path, MFMA paths
        d = synth.make_dense(B, 256, 5000, seed=11)
        E = d["E"].copy()
        H = synth.bf16_bits_to_f32(d["H"])
        # make the tied rows the best items: a large multiple of each user's sign pattern is not
        # shared across users, so use a row aligned with the mean user vector
        big = synth.f32_to_bf16_bits(np.sign(H.mean(0)).astype(np.float32) * 0.25)
        for r in (4999, 2000, 500, 10):
            E[r] = big
        g = run_dense(dict(d, E=E), 8, dev)
        idx, sc = g[0], g[1]
        for b in range(B):
            pos = {int(i): j for j, i in enumerate(idx[b])}
            tied = [r for r in (10, 500, 2000, 4999) if r in pos]
            # the tied ids that made the list are the lowest of the group, in increasing id order
            assert tied == [10, 500, 2000, 4999][:len(tied)]
            assert [pos[r] for r in tied] == sorted(pos[r] for r in tied)
            assert len(set(float(sc[b][pos[r]]) for r in tied)) <= 1


def test_all_equal_scores(dev):
    # B = 1: the fused path, its fast selection (1,000 keys at the threshold)
    # and its radix fallback (3,000 keys at the threshold); then the MFMA path
    for B, M in ((1, 1000), (1, 3000), (3, 1000), (40, 1000)):
        H = synth.f32_to_bf16_bits(np.ones((B, 64), dtype=np.float32))
        E = np.zeros((M, 64), dtype=np.uint16)
        g = run_dense(dict(H=H, E=E, B=B, D=64, M=M), 20, dev)
        idx, sc, ls = g
        assert (idx == np.arange(20)).all() and (sc == 0).all()
        assert np.allclose(ls, math.log(M), atol=1e-4)


@pytest.mark.parametrize("kind", ["integer scores", "all equal"])
def test_sampled_threshold_ties(dev, oracle_mod, kind):
    """The sampled threshold pass under exact ties.  Integer-valued scores
    put a few hundred sampled keys, many of them equal, at or above the bound
    from the group maxima (ranked directly); equal scores put all 6,400 there,
    more than are ranked directly (the narrowing passes).  Either way the
    result is the exact top-K."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 40, 64, 200_000, 20
    rng = np.random.default_rng(31)
    if kind == "all equal":
        H, E = np.ones((B, D), np.float32), np.zeros((M, D), np.float32)
    else:
        H = rng.integers(-1, 2, (B, D)).astype(np.float32)
        E = rng.integers(-1, 2, (M, D)).astype(np.float32)
    d = dict(H=synth.f32_to_bf16_bits(H), E=synth.f32_to_bf16_bits(E), B=B, D=D, M=M)
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    assert plan["sample"] == 1 and plan["n_sample"] == 6400
    g = run_dense(d, K, dev)
    ref = oracle_mod.full(d["H"], d["E"], K)
    parity.check_dense(g, ref, where="threshold ties, %s" % kind)


def test_deterministic(dev):
    d = synth.make_dense(64, 512, 70_000, seed=5)
    a = run_dense(d, 50, dev)
    b = run_dense(d, 50, dev)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_candidate_edge_cases(dev, oracle_mod):
    B, D, M, K = 6, 128, 4000, 10
    d = synth.make_dense(B, D, M, seed=2)
    lists = [
        np.array([], dtype=np.int32),                      # empty
        np.array([5, 7, 3999], dtype=np.int32),            # shorter than K
        np.array([12, 12, 40, 12], dtype=np.int32),        # duplicates
        np.arange(0, 4000, 3, dtype=np.int32),             # long, several pieces
        np.array([1, -3, 4000, 2, 9999], dtype=np.int32),  # out-of-range ids
        np.array([77], dtype=np.int32),
    ]
    offsets = np.zeros(B + 1, dtype=np.int64)
    offsets[1:] = np.cumsum([len(x) for x in lists])
    ids = np.concatenate(lists)
    dd = dict(d, offsets=offsets, ids=ids)
    g, errs = run_cand(dd, K, dev)
    assert errs == (3, 0)
    ref = oracle_mod.cand(d["H"], d["E"], offsets, ids, K)
    assert ref["n_bad"] == 3
    parity.check_cand(g, ref, offsets, ids, where="cand-edge")
    assert g[2][0] == -math.inf and (g[0][0] == -1).all()
    assert list(g[0][2][:4]) in ([12, 12, 12, 40], [40, 12, 12, 12], [12, 12, 40, 12], [12, 40, 12, 12])


@pytest.mark.parametrize("B,M,lo,hi,seed", [
    (600, 20_000, 400, 800, 21),   # more than 16,384 items reach the minimum count: the threshold rises
    (300, 5_000, 50, 400, 22),     # every listed popular item is hot, the tail is gathered
])
def test_candidates_hot_head(dev, oracle_mod, B, M, lo, hi, seed):
    """Zipf-weighted lists over a small catalog: the most-listed rows are scored
    densely on the matrix cores and looked up, the rest gathered; duplicates
    and out-of-range ids keep their meaning, and two runs agree bit for bit."""
    d = synth.make_dense(B, 64, M, seed=seed)
    off, ids = synth.gen_candidates(B, M, seed, lo, hi)
    ids = ids.copy()
    ids[5] = ids[4]        # a duplicate inside user 0's list
    ids[17] = -3           # out of range, skipped and counted
    ids[40] = M + 7
    d["offsets"], d["ids"] = off, ids
    g, errs = run_cand(d, 50, dev)
    assert errs == (2, 0)
    ref = oracle_mod.cand(d["H"], d["E"], off, ids, 50)
    parity.check_cand(g, ref, off, ids, where="hot head %s" % ((B, M),))
    g2, _ = run_cand(d, 50, dev)
    for x, y in zip(g, g2):
        assert np.array_equal(x, y)


def test_hot_counts_exact(dev):
    """The hot head's per-item list counts (every 16th entry of the id array,
    in-range ids only) equal a host count id for id, under a Zipf head whose
    popular ids recur many times in one wave's samples; the count threshold
    and the number of hot rows follow the plan's rule from those counts."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 600, 64, 20_000, 50
    d = synth.make_dense(B, D, M, seed=23)
    off, ids = synth.gen_candidates(B, M, 23, 400, 800)
    ids = ids.copy()
    ids[16] = -5          # a sampled entry out of range: not counted
    ids[32] = M + 1
    plan = genrec.describe_cand_plan(B, D, M, ids.size, K, torch.bfloat16)
    assert plan["hot"] == 1 and plan["sample_every"] == 16
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    _, _, _, ws = genrec.score_candidates_topk(H, E, torch.from_numpy(off).to(dev), torch.from_numpy(ids).to(dev), K)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    cnt = w[plan["off_counts"]:plan["off_counts"] + 4 * M].view(np.int32)
    s = ids[::16].astype(np.int64)
    s = s[(s >= 0) & (s < M)]
    expect = np.bincount(s, minlength=M)
    assert np.array_equal(cnt, expect), np.flatnonzero(cnt != expect)[:8]
    c, n_hot = w[plan["off_meta"]:plan["off_meta"] + 8].view(np.int32)
    if n_hot > 0:
        # c: the smallest count >= c_min that leaves at most t_max rows hot
        assert c >= plan["c_min"] and n_hot == int((expect >= c).sum()) <= plan["t_max"]
        assert c == plan["c_min"] or int((expect >= c - 1).sum()) > plan["t_max"]


@pytest.mark.parametrize("B,D,M,lo,hi,seed", [
    (100, 264, 50, 42, 50, 54098347),  # every item hot; D % 32 = 8
    (300, 72, 3000, 50, 400, 61),      # part of the catalog hot; D % 32 = 8
])
def test_candidates_hot_rows_k_tail_stale_workspace(dev, oracle_mod, B, D, M, lo, hi, seed):
    """The hot rows are gathered into the workspace; with D not a multiple of
    the 32-deep k-step the last k-step of a row reaches into the next staged
    row, which past the live rows is whatever the workspace held.  Filled with
    0xFF bytes (NaN as bf16 and as fp32) before the call, it must not reach any
    score (found by the randomized sweep: a stale NaN row poisoned the last
    hot row's scores)."""
    from full_catalog_ranking_amd import genrec
    K = 100
    d = synth.make_dense(B, D, M, seed=seed)
    off, ids = synth.gen_candidates(B, M, seed, lo, hi)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    ws = torch.full((genrec.cand_workspace_bytes(B, D, M, ids.size, K, H.dtype),), 255, dtype=torch.uint8, device=dev)
    print("  cand stale workspace B=%d D=%d M=%d nnz=%d" % (B, D, M, ids.size), flush=True)
    idx, sc, ls, ws = genrec.score_candidates_topk(H, E, torch.from_numpy(off).to(dev), torch.from_numpy(ids).to(dev),
                                                   K, workspace=ws)
    assert genrec.device_errors(ws) == (0, 0)
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    ref = oracle_mod.cand(d["H"], d["E"], off, ids, K)
    parity.check_cand(g, ref, off, ids, where="stale workspace %s" % ((B, D, M),))


def test_candidate_malformed_offsets(dev):
    B, D, M, K = 4, 64, 100, 5
    d = synth.make_dense(B, D, M, seed=9)
    ids = np.arange(40, dtype=np.int32) % M
    offsets = np.array([0, 10, 5, 30, 40], dtype=np.int64)  # user 1 runs backwards; user 2 overlaps user 0
    g, errs = run_cand(dict(d, offsets=offsets, ids=ids), K, dev)
    assert errs[1] == 2
    assert (g[0][1] == -1).all() and (g[0][2] == -1).all()
    assert (g[0][0] >= 0).all() and (g[0][3] >= 0).all()


def test_candidates_equal_full_catalog(dev, oracle_mod):
    """Every list = the whole catalog: the candidate path gives the dense
    path's answer.  The two sum the dot products in different orders (VALU
    gather vs MFMA tiles), so scores agree to fp32 rounding, not bit for bit."""
    B, D, M, K = 5, 256, 3000, 40
    d = synth.make_dense(B, D, M, seed=21)
    offsets = np.arange(B + 1, dtype=np.int64) * M
    ids = np.tile(np.arange(M, dtype=np.int32), B)
    gc, errs = run_cand(dict(d, offsets=offsets, ids=ids), K, dev)
    gd = run_dense(d, K, dev)
    assert errs == (0, 0)
    ref = oracle_mod.full(d["H"], d["E"], K)
    parity.check_dense(gc, ref, where="candidates = catalog")
    parity.check_dense(gd, ref, where="dense")
    assert np.allclose(gc[1], gd[1], rtol=0, atol=1e-5)
    assert np.allclose(gc[2], gd[2], atol=1e-5)


# ---------------------------------------------------------------------------
# Batched top-K of dense score rows (beam step)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("R,N,K,decimals,ld_pad", [
    (7, 128 * 128, 128, None, 0),     # width-128 beam step
    (3, 512 * 512, 512, None, 0),     # width-512 beam step (bitonic final sort)
    (4, 5000, 1024, 1, 3),            # many exact ties, K = KMAX, padded row stride
    (5, 100, 128, None, 0),           # K > N: padding
    (2, 6144, 200, 2, 0),             # exactly the LDS gather size, ties
    (1, 1, 1, None, 0),
    (2, 100_000, 50, 2, 5),           # seven chunks merged, ties across chunks
    (3, 16_385, 100, None, 0),        # a one-column last chunk
    (2, 16_384, 1024, 1, 0),          # K = KMAX over four chunks, heavy ties
    (2, 20_000, 512, 0, 0),           # a handful of distinct scores: ties decided by column
    (2, 300_000, 1024, 2, 0),
    # register-resident selection (>= 512 segment blocks of 16,384 columns)
    (40, 13 * 16_384, 512, None, 0),
    (33, 16 * 16_384 + 5, 256, 0, 3),  # whole-number scores: hundreds share a score; a 5-column last segment
    (520, 2 * 16_384, 1024, 2, 0),    # K = KMAX, the row merge's 2,048 keys
    # one block per row (N <= 16,384, K <= 256): threshold from the threads' maxima
    (64, 16_384, 256, None, 7),       # K = 256, padded row stride
    (9, 16_384, 100, 0, 0),           # whole-number scores: thousands at the threshold -> bit selection
    (11, 300, 256, 1, 0),             # fewer columns than threads; K > N / 2, ties
    (6, 4_097, 1, None, 0),           # K = 1
    # one block per row, 256 < K <= 512: the bound from 1,024 group maxima
    (8, 16_384, 512, None, 0),        # K = 512
    (3, 9_000, 400, None, 0),         # a short row: groups with empty slots
    (5, 16_384, 300, 0, 0),           # whole-number scores: thousands at the bound -> bit selection
    (24, 22 * 16_384, 300, None, 0),  # 528 segment blocks, K = 300
    # where the filter route does not apply: rows too short for 3 K keys at the
    # sampled bound, rows too long for its list
    (256, 17_000, 512, None, 0),      # two segments a row: register-resident selection
    (4, 5_000_000, 20, 1, 0),         # 306 segments a row, ties
])
def test_topk_rows(dev, oracle_mod, R, N, K, decimals, ld_pad):
    from full_catalog_ranking_amd import genrec
    s = synth.gen_scores(R, N, seed=R * 7 + N, decimals=decimals)
    full = np.zeros((R, N + ld_pad), dtype=np.float32)
    full[:, :N] = s
    t = torch.from_numpy(full).to(dev)[:, :N]
    print("  topk_rows R=%d N=%d K=%d ties=%s" % (R, N, K, decimals), flush=True)
    idx, val = genrec.topk_rows(t, K)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(R):
        ri, rv = oracle_mod.topk_row(s[r].astype(np.float64), K)
        assert np.array_equal(idx[r], ri), r   # exact: same fp32 values, same (score, column) order
        assert np.array_equal(val[r], rv.astype(np.float32)), r


@pytest.mark.parametrize("N,K", [(512 * 512, 512), (512 * 512, 100), (40_000, 7)])
def test_topk_rows_filter_fallbacks(dev, oracle_mod, N, K):
    """The filter route (rows longer than 16,384 columns, K <= 512) per row:
    the keys at or above a bound taken from 256 sampled runs of 64 columns are
    listed and ranked; a row whose list is shorter than K (a sample that
    misses the row's top: here every unsampled column holds -1,000) or longer
    than the list (all scores equal) is ranked from the whole row.  Rows of
    both kinds, ascending and descending rows and an unordered one share one
    call; every row is exact against the oracle."""
    from full_catalog_ranking_amd import genrec
    assert genrec.lib().genrec_topk_rows_workspace(5, N, K) == \
        -(-5 * 8192 * 8 // 256) * 256 + 256 + 5 * 256  # the filter route's workspace
    rng = np.random.default_rng(N + K)
    s = np.empty((5, N), dtype=np.float32)
    s[0] = -1000.0
    rs = N // 256
    for q in range(256):  # the sampled runs
        s[0, q * rs:q * rs + 64] = rng.random(64, dtype=np.float32)
    s[1] = 0.25
    s[2] = np.arange(N, dtype=np.float32) / N
    s[3] = s[2, ::-1]
    s[4] = rng.standard_normal(N, dtype=np.float32)
    print("  topk_rows filter fallbacks N=%d K=%d" % (N, K), flush=True)
    idx, val = genrec.topk_rows(torch.from_numpy(s).to(dev), K)
    idx, val = idx.cpu().numpy(), val.cpu().numpy()
    for r in range(5):
        ri, rv = oracle_mod.topk_row(s[r].astype(np.float64), K)
        assert np.array_equal(idx[r], ri), r
        assert np.array_equal(val[r], rv.astype(np.float32)), r


def test_binding_rejects_bad_buffers(dev, oracle_mod):
    """Caller-provided outputs, workspaces and inputs of the wrong shape, dtype,
    device or layout are refused before anything is launched; a valid call
    afterwards is unaffected."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 3, 64, 500, 7
    d = synth.make_dense(B, D, M, seed=41)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    i32, f32 = torch.int32, torch.float32
    good = (torch.empty((B, K), dtype=i32, device=dev), torch.empty((B, K), dtype=f32, device=dev),
            torch.empty((B,), dtype=f32, device=dev))
    with pytest.raises(ValueError):
        genrec.score_lse_topk(H, E, K, out=(good[0][:, :K - 1], good[1], good[2]))
    with pytest.raises(TypeError):
        genrec.score_lse_topk(H, E, K, out=(good[1], good[1], good[2]))
    with pytest.raises(ValueError):
        genrec.score_lse_topk(H, E, K, out=(torch.empty((K, B), dtype=i32, device=dev).t(), good[1], good[2]))
    with pytest.raises(ValueError):
        genrec.score_lse_topk(H, E, K, out=(good[0], good[1], torch.empty((B,), dtype=f32)))
    need = genrec.workspace_bytes(B, D, M, K, H.dtype)
    with pytest.raises(ValueError):
        genrec.score_lse_topk(H, E, K, workspace=torch.empty(need - 1, dtype=torch.uint8, device=dev))
    with pytest.raises(ValueError):
        genrec.score_lse_topk(H, E.cpu(), K)
    scores = torch.randn(4, 100, device=dev)
    with pytest.raises(ValueError):
        genrec.topk_rows(scores, 5, out=(torch.empty((4, 4), dtype=i32, device=dev),
                                         torch.empty((4, 5), dtype=f32, device=dev)))
    labels = torch.zeros(B, dtype=torch.int64, device=dev)
    with pytest.raises(TypeError):
        genrec.ce_forward(H, E, labels)
    idx, sc, ls = genrec.score_lse_topk(H, E, K, out=good)
    torch.cuda.synchronize()
    ref = oracle_mod.full(d["H"], d["E"], K)
    parity.check_dense((idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()), ref, where="after refusals")


def test_concurrent_calls_on_two_streams(dev, oracle_mod):
    """The library keeps no state between calls: two full-catalog calls and a
    candidate call, each with its own workspace, run on two streams at once
    (no ordering between them) and each matches the oracle."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 70, 128, 20_000, 20
    d1 = synth.make_dense(B, D, M, seed=51)
    d2 = synth.make_dense(B + 9, D, M, seed=52)
    off, ids = synth.gen_candidates(B, M, 53, 50, 400)
    H1, E1 = to_dev(d1["H"], dev), to_dev(d1["E"], dev)
    H2, E2 = to_dev(d2["H"], dev), to_dev(d2["E"], dev)
    offd, idsd = torch.from_numpy(off).to(dev), torch.from_numpy(ids).to(dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            r1 = genrec.score_lse_topk(H1, E1, K)
            rc = genrec.score_candidates_topk(H1, E1, offd, idsd, K)[:3]
        with torch.cuda.stream(s2):
            r2 = genrec.score_lse_topk(H2, E2, K)
        torch.cuda.synchronize()
        outs.append([tuple(x.cpu().numpy() for x in r) for r in (r1, r2, rc)])
    ref1 = oracle_mod.full(d1["H"], d1["E"], K)
    ref2 = oracle_mod.full(d2["H"], d2["E"], K)
    refc = oracle_mod.cand(d1["H"], d1["E"], off, ids, K)
    for g1, g2, gc in outs:
        parity.check_dense(g1, ref1, where="stream 1")
        parity.check_dense(g2, ref2, where="stream 2")
        parity.check_cand(gc, refc, off, ids, where="stream 1 candidates")
    for rep in outs[1:]:
        for a, b in zip(rep, outs[0]):
            for x, y in zip(a, b):
                assert np.array_equal(x, y)


def test_poisoned_workspaces_and_outputs(dev, oracle_mod):
    """Every entry point on workspaces and outputs filled with 0xFF bytes (NaN
    as bf16 / fp32, -1 as int32) before the call: no result may depend on
    memory the call has not written.  Shapes with a k tail (D % 32 != 0),
    ragged tiles and the sample / rescue passes."""
    from full_catalog_ranking_amd import genrec

    def poison(n):
        return torch.full((n,), 255, dtype=torch.uint8, device=dev)

    def outs(B, K):
        o = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
             torch.empty((B,), dtype=torch.float32, device=dev))
        for t in o:
            t.view(torch.uint8).fill_(255)
        return o

    # dense: MFMA with sample, fast threshold and rescue; VALU (B = 1); masked
    for B, D, M, K, mask in [(70, 200, 70_000, 40, False), (1, 136, 40_000, 30, False), (33, 72, 9_000, 25, True),
                             (1, 136, 7_000, 30, True), (1, 2048, 5_000, 100, False)]:
        d = synth.make_dense(B, D, M, seed=B + D)
        H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
        ws = poison(genrec.workspace_bytes(B, D, M, K, H.dtype))
        print("  poisoned dense B=%d D=%d M=%d K=%d mask=%s" % (B, D, M, K, mask), flush=True)
        if mask:
            allowed = np.random.default_rng(D).random(M) < 0.5
            W = (M + 31) // 32
            pad = np.zeros(W * 32, dtype=bool)
            pad[:M] = allowed
            words = (pad.reshape(W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
            g = genrec.score_lse_topk(H, E, K, workspace=ws, out=outs(B, K),
                                      mask=torch.from_numpy(words.view(np.int32)).to(dev))
            ref = oracle_mod.full_masked(d["H"], d["E"], K, words)
        else:
            g = genrec.score_lse_topk(H, E, K, workspace=ws, out=outs(B, K))
            ref = oracle_mod.full(d["H"], d["E"], K)
        parity.check_dense(tuple(x.cpu().numpy() for x in g), ref, where="poisoned dense %s" % ((B, D, M),))
    # candidate lists with a hot head and gathered rows
    B, D, M, K = 150, 104, 4000, 30
    d = synth.make_dense(B, D, M, seed=77)
    off, ids = synth.gen_candidates(B, M, 77, 20, 300)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    print("  poisoned cand B=%d D=%d M=%d nnz=%d" % (B, D, M, ids.size), flush=True)
    ws = poison(genrec.cand_workspace_bytes(B, D, M, ids.size, K, H.dtype))
    g = genrec.score_candidates_topk(H, E, torch.from_numpy(off).to(dev), torch.from_numpy(ids).to(dev), K,
                                     workspace=ws, out=outs(B, K))[:3]
    parity.check_cand(tuple(x.cpu().numpy() for x in g), oracle_mod.cand(d["H"], d["E"], off, ids, K), off, ids,
                      where="poisoned cand")
    # batched top-K rows of several chunks (histogram narrowing), of a few
    # segments (register-resident selection, a 3-column last segment), and
    # filtered (list parts and their counts in the workspace)
    for R, N, K in [(5, 50_000, 600), (520, 2 * 16_384 + 3, 600), (5, 50_000, 200), (40, 13 * 16_384 + 3, 200)]:
        S = synth.gen_scores(R, N, seed=78, decimals=3)
        need = genrec.lib().genrec_topk_rows_workspace(R, N, K)
        o = outs(R, K)[:2]
        print("  poisoned topk_rows R=%d N=%d K=%d" % (R, N, K), flush=True)
        idx, val = genrec.topk_rows(torch.from_numpy(S).to(dev), K, out=o, workspace=poison(max(need, 1)))
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        for r in range(R):
            ri, rv = oracle_mod.topk_row(S[r].astype(np.float64), K)
            assert np.array_equal(idx[r], ri) and np.array_equal(val[r], rv.astype(np.float32))


# ---------------------------------------------------------------------------
# The fused one-launch path (VALU path, no sample, catalogs up to 8,192 items)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,D,M,K,bf16", [
    (1, 64, 8192, 1024, True),    # largest catalog, K = KMAX (wave sorts and rank merge)
    (300, 32, 2000, 64, False),   # many users, several blocks each
    (5, 256, 257, 300, False),    # K > M: padding; 8 keys per thread
    (2, 12, 4097, 7, False),      # ragged: 32 keys per thread, a one-item last block
    (1, 2048, 4096, 1, True),     # K = 1, 16 keys per thread
])
def test_fused_small_catalog(dev, oracle_mod, B, D, M, K, bf16):
    from full_catalog_ranking_amd import genrec
    dt = torch.bfloat16 if bf16 else torch.float32
    assert genrec.describe_plan(B, D, M, K, dt)["fused"] == 1
    d = synth.make_dense(B, D, M, seed=B * 13 + M, bf16=bf16)
    g = run_dense(d, K, dev)
    users = sorted(set([0, B - 1] + list(range(0, B, max(1, B // 16)))))
    ref = oracle_mod.full(d["H"], d["E"], K, users=users)
    parity.check_dense(g, ref, where="fused %s" % ((B, D, M, K, bf16),))


def test_fused_workspace_contents_do_not_matter(dev, oracle_mod):
    """The per-user arrival words of the fused path live in the workspace: any
    earlier contents -- zeros, 0xFF, random bytes, a previous call of another
    shape, or the same call again -- give the same results."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 3, 128, 6000, 50
    d = synth.make_dense(B, D, M, seed=61, bf16=False)
    d2 = synth.make_dense(7, D, 300, seed=62, bf16=False)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    H2, E2 = to_dev(d2["H"], dev), to_dev(d2["E"], dev)
    need = max(genrec.workspace_bytes(B, D, M, K, H.dtype), genrec.workspace_bytes(7, D, 300, 9, H.dtype))
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    ref = oracle_mod.full(d["H"], d["E"], K)
    first = None
    rng = np.random.default_rng(63)
    for fill in ("zeros", "ff", "random", "other call", "again"):
        if fill == "zeros":
            ws.zero_()
        elif fill == "ff":
            ws.fill_(255)
        elif fill == "random":
            ws.copy_(torch.from_numpy(rng.integers(0, 256, need, dtype=np.uint8)).to(dev))
        elif fill == "other call":
            genrec.score_lse_topk(H2, E2, 9, workspace=ws)
        print("  fused workspace %s" % fill, flush=True)
        g = tuple(x.cpu().numpy() for x in genrec.score_lse_topk(H, E, K, workspace=ws))
        parity.check_dense(g, ref, where="fused ws %s" % fill)
        if first is None:
            first = g
        for x, y in zip(g, first):
            assert np.array_equal(x, y)


def test_fused_two_streams(dev, oracle_mod):
    """Fused calls on two streams at once, each with its own workspace."""
    from full_catalog_ranking_amd import genrec
    d1 = synth.make_dense(1, 2048, 5000, seed=71)
    d2 = synth.make_dense(4, 256, 5000, seed=72, bf16=False)
    H1, E1 = to_dev(d1["H"], dev), to_dev(d1["E"], dev)
    H2, E2 = to_dev(d2["H"], dev), to_dev(d2["E"], dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(3):
        with torch.cuda.stream(s1):
            r1 = genrec.score_lse_topk(H1, E1, 100)
        with torch.cuda.stream(s2):
            r2 = genrec.score_lse_topk(H2, E2, 10)
        torch.cuda.synchronize()
        outs.append([tuple(x.cpu().numpy() for x in r) for r in (r1, r2)])
    ref1 = oracle_mod.full(d1["H"], d1["E"], 100)
    ref2 = oracle_mod.full(d2["H"], d2["E"], 10)
    for g1, g2 in outs:
        parity.check_dense(g1, ref1, where="fused stream 1")
        parity.check_dense(g2, ref2, where="fused stream 2")
    for rep in outs[1:]:
        for a, b in zip(rep, outs[0]):
            for x, y in zip(a, b):
                assert np.array_equal(x, y)


# ---------------------------------------------------------------------------
# fp32 inputs on the matrix cores (v_mfma_f32_32x32x2_f32): batches of two or
# more users over catalogs past the one-launch size
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("B,D,M,K", [
    (256, 2048, 100_000, 100),   # the batch shape: sample, fast threshold
    (300, 200, 70_001, 37),      # two user tiles (ragged), k tail (200 % 16 = 8), sampled pass
    (3, 12, 9000, 20),           # one k-step, all of it k tail; no sample
    (40, 64, 20_000, 1024),      # K = KMAX
])
def test_fp32_matrix_cores(dev, oracle_mod, B, D, M, K):
    from full_catalog_ranking_amd import genrec
    assert genrec.describe_plan(B, D, M, K, torch.float32)["path"] == "mfma"
    d = synth.make_dense(B, D, M, seed=B + M + 1, bf16=False)
    g = run_dense(d, K, dev)
    users = sorted(set([0, 1, B // 2, B - 1] + list(range(0, B, max(1, B // 10)))))
    ref = oracle_mod.full(d["H"], d["E"], K, users=users)
    parity.check_dense(g, ref, where="fp32 mfma %s" % ((B, D, M, K),))


def test_fp32_matrix_cores_masked(dev, oracle_mod):
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 70, 96, 30_000, 25
    d = synth.make_dense(B, D, M, seed=77, bf16=False)
    rng = np.random.default_rng(78)
    allowed = rng.random((B, M)) < rng.uniform(0.001, 1.0, B)[:, None]
    words = _pack_mask(allowed)
    mask = torch.from_numpy(words.view(np.int32)).to(dev)
    H, E = to_dev(d["H"], dev), to_dev(d["E"], dev)
    print("  fp32 mfma masked B=%d D=%d M=%d K=%d" % (B, D, M, K), flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, E, K, mask=mask)
    g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    users = list(range(0, B, 7)) + [B - 1]
    ref = oracle_mod.full_masked(d["H"], d["E"], K, words, users=users)
    parity.check_dense(g, ref, where="fp32 mfma masked")
