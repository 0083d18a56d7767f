"""Seeded sweep of random shapes through every entry point against the CPU
oracle (under the rules in parity.py): dense bf16 / fp32, masked, candidate
lists, batched top-K rows and the cross-entropy.  Each case draws its kind
and sizes from one seeded generator, within the supported shapes and sizes
the oracle finishes in about a second."""
import os

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


def _td(a, dev):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev) if a.dtype == np.uint16 \
        else torch.from_numpy(a).to(dev)


# Size distributions of the two families: "common" shapes, and "edge" shapes
# at tile, chunk and capacity boundaries (M = 256k +- 1, 65,536 +- 1, K = 255 /
# 256 / 257 / 1,024, lists longer than the small merge build's 2,048-key gather,
# cross-entropy catalogs at the 65,536-row chunk boundary).
SIZES = {
    "common": dict(
        dense_B=[1, 2, 3, 8, 40, 256, 300, 513], dense_D=lambda rng: int(rng.integers(1, 65)) * 8,
        dense_M=[1, 7, 300, 4097, 20000, 70001], dense_K=[1, 10, 64, 100, 257, 500, 1024],
        cand_B=[1, 5, 64, 100, 300], cand_D=lambda rng: int(rng.integers(1, 65)) * 8, cand_M=[50, 3000, 50000],
        cand_lo=lambda rng: int(rng.integers(0, 50)), cand_span=lambda rng: int(rng.integers(0, 600)),
        cand_K=[1, 10, 100, 300],
        topk_R=[1, 3, 64, 100], topk_N=[1, 5, 4096, 4097, 30000, 300000],
        ce_B=[1, 7, 64, 300], ce_D=lambda rng: int(rng.integers(1, 65)) * 8, ce_M=[1, 70, 5000, 70000]),
    "edge": dict(
        dense_B=[1, 2, 255, 256, 257, 511, 1025], dense_D=lambda rng: int(rng.choice([8, 16, 24, 32, 40, 264, 520])),
        dense_M=[255, 256, 257, 8191, 8193, 65535, 65537, 131073, 262147], dense_K=[1, 255, 256, 257, 1000, 1024],
        cand_B=[1, 63, 64, 65, 257], cand_D=lambda rng: int(rng.choice([8, 24, 72, 264])), cand_M=[300, 20000, 300000],
        cand_lo=lambda rng: int(rng.choice([0, 1000, 2000])), cand_span=lambda rng: int(rng.choice([0, 100, 3000, 9000])),
        cand_K=[1, 100, 1000, 1024],
        topk_R=[1, 7, 65], topk_N=[1, 1023, 1024, 1025, 4095, 4096, 4097, 12289, 65537, 200000],
        ce_B=[1, 33, 257], ce_D=lambda rng: int(rng.choice([8, 40, 264])), ce_M=[1, 255, 65535, 65536, 65537, 131073]),
}


@pytest.mark.parametrize("family,case", [("common", c) for c in range(16)] + [("edge", c) for c in range(12)])
def test_random_shapes(dev, oracle_mod, family, case):
    from full_catalog_ranking_amd import genrec
    oracle = oracle_mod
    sz = SIZES[family]
    # GENREC_SWEEP_SEED draws another set of cases (the suite's own: 20261203)
    base = int(os.environ.get("GENREC_SWEEP_SEED", "20261203"))
    rng = np.random.default_rng([base, case] + ([7] if family == "edge" else []))
    td = lambda a: _td(a, dev)

    def pick_users(B):
        return sorted(set([0, B - 1] + list(rng.integers(0, B, min(B, 6)))))

    kind = rng.choice(["dense", "dense", "masked", "cand", "topk", "ce"])
    if kind in ("dense", "masked"):
        bf16 = bool(rng.random() < 0.8)
        B = int(rng.choice(sz["dense_B"]))
        D = sz["dense_D"](rng)
        M = int(rng.choice(sz["dense_M"]))
        if B * M * D > 3e9:  # keep the oracle's work to about a second
            M = max(1, int(3e9 // (B * D)))
        K = int(min(1024, rng.choice(sz["dense_K"])))
        seed = int(rng.integers(0, 1 << 30))
        print("case %s %d %s B=%d D=%d M=%d K=%d bf16=%s seed=%d" % (family, case, kind, B, D, M, K, bf16, seed), flush=True)
        d = synth.make_dense(B, D, M, seed=seed, bf16=bf16)
        H, E = td(d["H"]), td(d["E"])
        users = pick_users(B)
        if kind == "masked":
            per_user = bool(rng.random() < 0.5)
            dens = rng.uniform(0.0, 1.0, B if per_user else 1)
            allowed = rng.random((B if per_user else 1, M)) < dens[:, None]
            W = (M + 31) // 32
            pad = np.zeros((allowed.shape[0], W * 32), dtype=bool)
            pad[:, :M] = allowed
            bits = pad.reshape(allowed.shape[0], W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)
            words = bits.sum(axis=-1).astype(np.uint32)
            words = words if per_user else words[0]
            mask = torch.from_numpy(np.ascontiguousarray(words).view(np.int32)).to(dev)
            idx, sc, ls = genrec.score_lse_topk(H, E, K, mask=mask)
            ref = oracle.full_masked(d["H"], d["E"], K, words, users=users)
        else:
            idx, sc, ls = genrec.score_lse_topk(H, E, K)
            ref = oracle.full(d["H"], d["E"], K, users=users)
        g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
        parity.check_dense(g, ref, where="sweep %s %d" % (family, case))
    elif kind == "cand":
        B = int(rng.choice(sz["cand_B"]))
        D = sz["cand_D"](rng)
        M = int(rng.choice(sz["cand_M"]))
        lo = sz["cand_lo"](rng)
        hi = lo + sz["cand_span"](rng)
        hi = min(hi, M)
        lo = min(lo, hi)
        K = int(min(1024, rng.choice(sz["cand_K"])))
        seed = int(rng.integers(0, 1 << 30))
        print("case %s %d cand B=%d D=%d M=%d lists=[%d,%d] K=%d seed=%d" % (family, case, B, D, M, lo, hi, K, seed), flush=True)
        d = synth.make_dense(B, D, M, seed=seed)
        off, ids = synth.gen_candidates(B, M, seed, lo, hi)
        H, E = td(d["H"]), td(d["E"])
        idx, sc, ls, ws = genrec.score_candidates_topk(H, E, torch.from_numpy(off).to(dev),
                                                       torch.from_numpy(ids).to(dev), K)
        assert genrec.device_errors(ws) == (0, 0)
        g = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
        ref = oracle.cand(d["H"], d["E"], off, ids, K)
        parity.check_cand(g, ref, off, ids, where="sweep %s %d" % (family, case))
    elif kind == "topk":
        R = int(rng.choice(sz["topk_R"]))
        N = int(rng.choice(sz["topk_N"]))
        K = int(min(1024, rng.choice([1, 8, 128, 257, 512, 1024])))
        dec = [None, 2][int(rng.integers(0, 2))]
        seed = int(rng.integers(0, 1 << 30))
        print("case %s %d topk R=%d N=%d K=%d dec=%s seed=%d" % (family, case, R, N, K, dec, seed), flush=True)
        s = synth.gen_scores(R, N, seed=seed, decimals=dec)
        idx, val = genrec.topk_rows(torch.from_numpy(s).to(dev), K)
        idx, val = idx.cpu().numpy(), val.cpu().numpy()
        for r in range(R):
            ri, rv = oracle.topk_row(s[r].astype(np.float64), K)
            assert np.array_equal(idx[r], ri), ("topk idx", r)
            assert np.array_equal(val[r], rv.astype(np.float32)), ("topk val", r)
    else:
        B = int(rng.choice(sz["ce_B"]))
        D = sz["ce_D"](rng)
        M = int(rng.choice(sz["ce_M"]))
        if B * M * D > 2e9:
            M = max(1, int(2e9 // (B * D)))
        seed = int(rng.integers(0, 1 << 30))
        weighted = bool(rng.random() < 0.7)
        print("case %s %d ce B=%d D=%d M=%d weighted=%s seed=%d" % (family, case, B, D, M, weighted, seed), flush=True)
        d = synth.make_dense(B, D, M, seed=seed)
        labels = synth.gen_labels(B, M, seed)
        w = synth.gen_weights(B, seed) if weighted else None
        H, E = td(d["H"]), td(d["E"])
        lab = torch.from_numpy(labels).to(dev)
        wt = torch.from_numpy(w).to(dev) if weighted else None
        loss, lse, _ = genrec.ce_forward(H, E, lab, wt)
        dH, dE = genrec.ce_backward(H, E, lab, lse, wt)
        torch.cuda.synchronize()
        g = (loss.cpu().numpy(), lse.cpu().numpy(), dH.cpu().numpy(), dE.cpu().numpy())
        ref = oracle.ce(d["H"], d["E"], labels, w)
        plan = genrec.describe_ce_plan(B, D, M)  # the products' addition depths, from the library
        parity.check_ce(g, ref, d["E"], d["H"], oracle.widen, plan["depth_h"], plan["depth_e"],
                        where="sweep %s %d" % (family, case))
