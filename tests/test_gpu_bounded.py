"""GPU parity of the bounded candidate regions: pieces of a fixed number of
keys, and the exact rescue (counting passes that narrow a user's bound on its
ranking keys, then a collect pass) for users whose pieces overflowed or who
were left short of K.  GENREC_KEY_BUDGET=0 makes every sampled matrix-core
plan use bounded regions, so small shapes reach every branch; each case is
checked against the oracle and against the same call with regions of every
item (the scores come from the same kernel, so the outputs must be equal bit
for bit)."""
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


def run(H, E, K, budget, monkeypatch, mask=None, ovf=None):
    """One call under the given key budget (and overflow-region size, None:
    the default): (outputs on the host, plan, rescued users)."""
    from full_catalog_ranking_amd import genrec
    monkeypatch.setenv("GENREC_KEY_BUDGET", str(budget))
    if ovf is None:  # the default size, whatever the process environment says
        monkeypatch.delenv("GENREC_OVERFLOW_KEYS", raising=False)
    else:
        monkeypatch.setenv("GENREC_OVERFLOW_KEYS", str(ovf))
    B, D, M = H.shape[0], H.shape[1], E.shape[0]
    plan = genrec.describe_plan(B, D, M, K, H.dtype)
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=H.device)
    ws.fill_(255)  # nothing may depend on bytes the call did not write
    print("  B=%d D=%d M=%d K=%d budget=%d bounded=%d cap=%d ccol=%d" %
          (B, D, M, K, budget, plan["bounded"], plan["cap"], plan["ccol"]), flush=True)
    idx, sc, ls = genrec.score_lse_topk(H, E, K, workspace=ws, mask=mask)
    n_rescued = genrec.rescued_users(ws)
    out = idx.cpu().numpy(), sc.cpu().numpy(), ls.cpu().numpy()
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    monkeypatch.delenv("GENREC_OVERFLOW_KEYS", raising=False)
    return out, plan, n_rescued


def bounded_vs_full(Hb, Eb, K, dev, monkeypatch, mask=None, ovf=None):
    H, E = to_dev(Hb, dev), to_dev(Eb, dev)
    g, plan, n_resc = run(H, E, K, 0, monkeypatch, mask, ovf)
    assert plan["bounded"] == 1 and (ovf is None or plan["ovf_cap"] == ovf)
    f, fplan, _ = run(H, E, K, 1 << 50, monkeypatch, mask)
    assert fplan["bounded"] == 0
    for name, x, y in zip(("idx", "score", "lse"), g, f):
        assert np.array_equal(x, y), ("bounded and full regions differ in", name)
    return g, plan, n_resc


def plant_unsampled(E, B, D, M, K, dtype, n_tiles, scale, monkeypatch):
    """Scales n_tiles catalog tiles of the first sample window other than the
    sampled one (the fast threshold then comes from ordinary items, and a
    large share of the scaled ones pass it, all in the first chunks' pieces);
    returns the scaled rows' range and the bounded plan."""
    from full_catalog_ranking_amd import genrec
    monkeypatch.setenv("GENREC_KEY_BUDGET", "0")
    plan = genrec.describe_plan(B, D, M, K, dtype)
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    assert plan["bounded"] == 1 and plan["stride"] > n_tiles
    f = plan["first_sampled_tile"]
    tiles = [t for t in range(plan["stride"]) if t != f][:n_tiles]
    for t in tiles:
        E[t * 256:(t + 1) * 256] *= np.float32(scale)
    return plan


def test_bounded_exchangeable(dev, oracle_mod, monkeypatch):
    """Zipf-normed catalog, ragged users and a k tail: no piece overflows."""
    B, D, M, K = 300, 136, 140_001, 100
    d = synth.make_dense(B, D, M, seed=41)
    g, plan, n_resc = bounded_vs_full(d["H"], d["E"], K, dev, monkeypatch)
    assert n_resc == 0
    users = [0, 1, 150, 255, 256, 299]
    parity.check_dense(g, oracle_mod.full(d["H"], d["E"], K, users=users), where="bounded exchangeable")


@pytest.mark.parametrize("n_tiles,ovf", [(12, None), (31, None), (12, 0), (31, 0)])
def test_bounded_clustered_overflow(dev, oracle_mod, monkeypatch, n_tiles, ovf):
    """Catalog tiles of 20 times the norm that the sample skips: they hold
    every user's top K, and pieces of the first chunks fill for nearly every
    user.  With the overflow regions (default size) the extra keys land there
    and no user is rescued.  Without them (size 0) every such user is rescued:
    with 12 scaled tiles the keys past the fast threshold fit the collect
    region (one collect pass); with 31 they do not (counting passes first)."""
    B, D, M, K = 260, 64, 150_000, 200
    d = synth.make_dense(B, D, M, seed=42)
    E = synth.bf16_bits_to_f32(d["E"])
    plant_unsampled(E, B, D, M, K, torch.bfloat16, n_tiles, 20.0, monkeypatch)
    Eb = synth.f32_to_bf16_bits(E)
    g, plan, n_resc = bounded_vs_full(d["H"], Eb, K, dev, monkeypatch, ovf=ovf)
    print("  rescued users: %d of %d (cap %d, overflow %d)" % (n_resc, B, plan["cap"], plan["ovf_cap"]), flush=True)
    if ovf == 0:
        assert n_resc > B // 2
    else:
        assert n_resc == 0
    users = [0, 7, 100, 255, 256, 259]
    parity.check_dense(g, oracle_mod.full(d["H"], Eb, K, users=users), where="bounded clustered")


@pytest.mark.parametrize("clusters", [150, 1500])
def test_bounded_clustered_catalog(dev, oracle_mod, monkeypatch, clusters):
    """A catalog stored grouped by category (contiguous runs of 1,000 or 100
    similar items): every user's best items sit in a few id ranges, so the
    first chunks' pieces can overflow and the sample can miss a user's best
    clusters.  Exact either way, equal to regions of every item."""
    B, D, M, K = 260, 64, 150_000, 200
    d = synth.make_dense(B, D, M, seed=46, clusters=clusters)
    g, plan, n_resc = bounded_vs_full(d["H"], d["E"], K, dev, monkeypatch)
    print("  clustered catalog (%d clusters): rescued users %d of %d" % (clusters, n_resc, B), flush=True)
    users = [0, 9, 128, 255, 256, 259]
    parity.check_dense(g, oracle_mod.full(d["H"], d["E"], K, users=users), where="clustered %d" % clusters)


@pytest.mark.parametrize("kind", ["integer scores", "all equal"])
def test_bounded_ties(dev, oracle_mod, monkeypatch, kind):
    """Exact ties at the K-th score: with equal scores every item passes the
    threshold and the counting passes narrow down to the ids (lowest first)."""
    B, D, M, K = 40, 64, 200_000, 20
    rng = np.random.default_rng(31)
    if kind == "all equal":
        H, E = np.ones((B, D), np.float32), np.zeros((M, D), np.float32)
    else:
        H = rng.integers(-1, 2, (B, D)).astype(np.float32)
        E = rng.integers(-1, 2, (M, D)).astype(np.float32)
    Hb, Eb = synth.f32_to_bf16_bits(H), synth.f32_to_bf16_bits(E)
    g, plan, n_resc = bounded_vs_full(Hb, Eb, K, dev, monkeypatch)
    if kind == "all equal":
        assert n_resc == B
        assert (g[0] == np.arange(K)).all() and (g[1] == 0).all()
    parity.check_dense(g, oracle_mod.full(Hb, Eb, K), where="bounded ties, %s" % kind)


def test_bounded_short_user_rescue(dev, oracle_mod, monkeypatch):
    """A user whose sampled tile holds 40 scaled copies of its vector: the fast
    threshold lets fewer than K items through, and the rescue starts from the
    K-th sampled score."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 16, 72, 131072, 100
    d = synth.make_dense(B, D, M, seed=11)
    monkeypatch.setenv("GENREC_KEY_BUDGET", "0")
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    assert plan["fast"] == 1 and plan["safe_exact"] == 1 and plan["bounded"] == 1
    h = synth.bf16_bits_to_f32(d["H"][3])
    E = d["E"].copy()
    row0 = plan["first_sampled_tile"] * 256
    for i in range(40):
        E[row0 + i] = synth.f32_to_bf16_bits((h * np.float32(0.05 + 0.001 * i)).astype(np.float32))
    g, _, n_resc = bounded_vs_full(d["H"], E, K, dev, monkeypatch)
    assert n_resc >= 1
    assert set(g[0][3, :40].tolist()) == set(range(row0, row0 + 40))
    parity.check_dense(g, oracle_mod.full(d["H"], E, K), where="bounded short rescue")


def test_bounded_short_user_split_sample(dev, oracle_mod, monkeypatch):
    """As above with a split-reduction sample (no safe threshold): the rescue
    starts from every finite score."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 16, 512, 131072, 100
    d = synth.make_dense(B, D, M, seed=11)
    monkeypatch.setenv("GENREC_KEY_BUDGET", "0")
    plan = genrec.describe_plan(B, D, M, K, torch.bfloat16)
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    assert plan["sample_splits"] > 1 and plan["safe_exact"] == 0 and plan["bounded"] == 1
    h = synth.bf16_bits_to_f32(d["H"][3])
    E = d["E"].copy()
    row0 = plan["first_sampled_tile"] * 256
    for i in range(40):
        E[row0 + i] = synth.f32_to_bf16_bits((h * np.float32(0.05 + 0.001 * i)).astype(np.float32))
    g, _, n_resc = bounded_vs_full(d["H"], E, K, dev, monkeypatch)
    assert n_resc >= 1
    parity.check_dense(g, oracle_mod.full(d["H"], E, K, users=[0, 3, 8, 15]), where="bounded split rescue")


@pytest.mark.parametrize("ovf", [None, 0])
def test_bounded_masked_clustered(dev, oracle_mod, monkeypatch, ovf):
    """The masked head over bounded regions: per-user masks (one user with
    none allowed, one with fewer than K) on scaled tiles the sample skips;
    with and without the overflow regions."""
    B, D, M, K = 70, 96, 300_000, 50
    d = synth.make_dense(B, D, M, seed=43)
    E = synth.bf16_bits_to_f32(d["E"])
    plant_unsampled(E, B, D, M, K, torch.bfloat16, 20, 20.0, monkeypatch)
    Eb = synth.f32_to_bf16_bits(E)
    rng = np.random.default_rng(44)
    dens = np.concatenate([[0.0, 2e-4, 1.0], rng.uniform(0.05, 1.0, B - 3)])
    allowed = rng.random((B, M)) < dens[:, None]
    W = (M + 31) // 32
    pad = np.zeros((B, W * 32), dtype=bool)
    pad[:, :M] = allowed
    words = (pad.reshape(B, W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(axis=-1).astype(np.uint32)
    mask = torch.from_numpy(words.view(np.int32)).to(dev)
    g, plan, n_resc = bounded_vs_full(d["H"], Eb, K, dev, monkeypatch, mask=mask, ovf=ovf)
    assert n_resc > 0 or ovf is None
    users = [0, 1, 2, 3, 35, 69]
    parity.check_dense(g, oracle_mod.full_masked(d["H"], Eb, K, words, users=users), where="bounded masked")
    for b in range(B):
        ids = g[0][b]
        assert allowed[b][ids[ids >= 0]].all()


@pytest.mark.parametrize("ovf", [None, 0])
def test_bounded_fp32_matrix_cores(dev, oracle_mod, monkeypatch, ovf):
    """fp32 operands on the matrix cores, bounded regions, scaled tiles the
    sample skips; with and without the overflow regions."""
    B, D, M, K = 40, 48, 300_000, 30
    d = synth.make_dense(B, D, M, seed=45, bf16=False)
    E = d["E"].copy()
    plant_unsampled(E, B, D, M, K, torch.float32, 20, 20.0, monkeypatch)
    g, plan, n_resc = bounded_vs_full(d["H"], E, K, dev, monkeypatch, ovf=ovf)
    assert plan["path"] == "mfma" and (n_resc > 0 or ovf is None)
    parity.check_dense(g, oracle_mod.full(d["H"], E, K, users=[0, 13, 39]), where="bounded fp32")


def test_bounded_graph_replays(dev, monkeypatch):
    """A captured bounded call whose users are rescued, replayed four times
    with eager work in between: every replay equals the eager call."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 260, 64, 150_000, 200
    d = synth.make_dense(B, D, M, seed=42)
    E = synth.bf16_bits_to_f32(d["E"])
    plant_unsampled(E, B, D, M, K, torch.bfloat16, 31, 20.0, monkeypatch)
    H, Ed = to_dev(d["H"], dev), to_dev(synth.f32_to_bf16_bits(E), dev)
    monkeypatch.setenv("GENREC_KEY_BUDGET", "0")
    monkeypatch.setenv("GENREC_OVERFLOW_KEYS", "0")  # the rescue's launches do the work
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
    out = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B,), dtype=torch.float32, device=dev))
    eager = [t.clone() for t in genrec.score_lse_topk(H, Ed, K, workspace=ws, out=out)]
    assert genrec.rescued_users(ws) > 0
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        genrec.score_lse_topk(H, Ed, K, workspace=ws, out=out)
    torch.cuda.synchronize()
    junk = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for t in out:
            t.fill_(7)  # a fill kernel, outside the graph
        (junk * 2).sum().item()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for x, y in zip(out, eager):
            assert torch.equal(x, y), "replay %d" % rep
    del g
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    monkeypatch.delenv("GENREC_OVERFLOW_KEYS")
