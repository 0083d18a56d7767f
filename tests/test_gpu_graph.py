"""HIP-graph capture of the library's calls: the compute entry points only
launch kernels on the caller's stream (no allocation, no copy, no memset,
no synchronisation), so a call captured once and replayed gives, on every
replay, the eager call's results bit for bit -- checked over several replays
with eager work and synchronisations in between."""
import numpy as np
import pytest

from full_catalog_ranking_amd import synth

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
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _check_replays(call, dev, other):
    """call() returns its output tensors (only library launches happen in it);
    `other` is unrelated eager work."""
    ref = [o.clone() for o in call()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = call()
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            o.fill_(7)  # a fill kernel, outside the graph
        other()
        torch.cuda.synchronize()
        g.replay()
        other()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), "replay %d differs" % rep
    del g


def _dense_case(B, D, M, K, dev, seed, mask=None):
    from full_catalog_ranking_amd import genrec
    d = synth.make_dense(B, D, M, seed=seed)
    H, E = _td(d["H"], dev), _td(d["E"], dev)
    ws = torch.empty(genrec.workspace_bytes(B, D, M, K, H.dtype), dtype=torch.uint8, device=dev)
    out = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B,), dtype=torch.float32, device=dev))
    return H, E, ws, out


@pytest.mark.parametrize("B,D,M,K,seed", [
    (1, 2048, 5000, 100, 1),     # VALU path, no sample
    (64, 128, 100_000, 20, 2),   # MFMA path: sample pass, threshold, fast threshold, rescue pass
    (300, 64, 20_000, 1024, 3),  # K = KMAX: rank merges, the default merge build
])
def test_dense_graph_replays(dev, B, D, M, K, seed):
    from full_catalog_ranking_amd import genrec
    H, E, ws, out = _dense_case(B, D, M, K, dev, seed)
    H2, E2, ws2, out2 = _dense_case(3, 64, 700, 5, dev, seed + 100)
    print("  graph dense B=%d D=%d M=%d K=%d plan=%s" % (B, D, M, K, genrec.describe_plan(B, D, M, K, H.dtype)),
          flush=True)
    _check_replays(lambda: genrec.score_lse_topk(H, E, K, workspace=ws, out=out), dev,
                   lambda: genrec.score_lse_topk(H2, E2, 5, workspace=ws2, out=out2))


def test_masked_graph_replays(dev):
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 40, 96, 70_000, 30
    H, E, ws, out = _dense_case(B, D, M, K, dev, 4)
    allowed = np.random.default_rng(4).random(M) < 0.6
    W = (M + 31) // 32
    pad = np.zeros(W * 32, dtype=bool)
    pad[:M] = allowed
    words = (pad.reshape(W, 32).astype(np.uint64) << np.arange(32, dtype=np.uint64)).sum(axis=1).astype(np.uint32)
    mask = torch.from_numpy(words.view(np.int32)).to(dev)
    print("  graph masked B=%d D=%d M=%d K=%d" % (B, D, M, K), flush=True)
    _check_replays(lambda: genrec.score_lse_topk(H, E, K, workspace=ws, out=out, mask=mask), dev,
                   lambda: torch.cumsum(H.float(), 0))


def test_candidate_graph_replays(dev):
    """Hot head (eight selection kernels, the dense hot scores), list pass and merge."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 300, 64, 5000, 50
    d = synth.make_dense(B, D, M, seed=5)
    off, ids = synth.gen_candidates(B, M, 5, 50, 400)
    H, E = _td(d["H"], dev), _td(d["E"], dev)
    offd, idsd = torch.from_numpy(off).to(dev), torch.from_numpy(ids).to(dev)
    ws = torch.empty(genrec.cand_workspace_bytes(B, D, M, ids.size, K, H.dtype), dtype=torch.uint8, device=dev)
    out = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B,), dtype=torch.float32, device=dev))
    print("  graph cand B=%d D=%d M=%d nnz=%d" % (B, D, M, ids.size), flush=True)
    _check_replays(lambda: genrec.score_candidates_topk(H, E, offd, idsd, K, workspace=ws, out=out)[:3], dev,
                   lambda: torch.cumsum(E.float(), 0))


def test_topk_rows_and_ce_graph_replays(dev):
    from full_catalog_ranking_amd import genrec
    # the filter route (two shapes), histogram chunks (K > 512), then
    # register-resident segments (256 x 2 segment blocks)
    for R, N, K in [(64, 40_000, 128), (64, 8 * 16_384, 128), (64, 40_000, 600), (256, 17_000, 512)]:
        S = torch.from_numpy(synth.gen_scores(R, N, seed=6, decimals=2)).to(dev)
        need = genrec.lib().genrec_topk_rows_workspace(R, N, K)
        tws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        tout = (torch.empty((R, K), dtype=torch.int32, device=dev),
                torch.empty((R, K), dtype=torch.float32, device=dev))
        print("  graph topk_rows R=%d N=%d K=%d" % (R, N, K), flush=True)
        _check_replays(lambda: genrec.topk_rows(S, K, out=tout, workspace=tws), dev, lambda: torch.cumsum(S, 1))

    B, D, M = 70, 64, 70_000  # two catalog chunks in the backward
    d = synth.make_dense(B, D, M, seed=7)
    H, E = _td(d["H"], dev), _td(d["E"], dev)
    lab = torch.from_numpy(synth.gen_labels(B, M, 7)).to(dev)
    w = torch.from_numpy(synth.gen_weights(B, 7)).to(dev)
    L = genrec.lib()
    wsf = torch.empty(L.genrec_ce_forward_workspace(B, D, M), dtype=torch.uint8, device=dev)
    wsb = torch.empty(L.genrec_ce_backward_workspace(B, D, M), dtype=torch.uint8, device=dev)
    dH = torch.empty((B, D), dtype=torch.float32, device=dev)
    dE = torch.empty((M, D), dtype=torch.float32, device=dev)

    def ce_step():
        loss, lse, _ = genrec.ce_forward(H, E, lab, w, workspace=wsf)
        genrec.ce_backward(H, E, lab, lse, w, workspace=wsb, out=(dH, dE))
        return loss, lse, dH, dE
    print("  graph ce B=%d D=%d M=%d" % (B, D, M), flush=True)
    _check_replays(ce_step, dev, lambda: torch.cumsum(H.float(), 0))


def test_fused_graph_replays_share_workspace_with_eager_calls(dev):
    """The fused path's captured call replays correctly while eager fused calls
    of another shape (each with its own ticket) use the same workspace between
    the replays."""
    from full_catalog_ranking_amd import genrec
    B, D, M, K = 4, 256, 5000, 10
    d = synth.make_dense(B, D, M, seed=8, bf16=False)
    d2 = synth.make_dense(1, D, 3000, seed=9, bf16=False)
    H, E = _td(d["H"], dev), _td(d["E"], dev)
    H2, E2 = _td(d2["H"], dev), _td(d2["E"], dev)
    ws = torch.empty(max(genrec.workspace_bytes(B, D, M, K, H.dtype), genrec.workspace_bytes(1, D, 3000, 20, H.dtype)),
                     dtype=torch.uint8, device=dev)
    out = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
           torch.empty((B,), dtype=torch.float32, device=dev))
    assert genrec.describe_plan(B, D, M, K, H.dtype)["fused"] == 1
    print("  graph fused B=%d D=%d M=%d K=%d" % (B, D, M, K), flush=True)
    _check_replays(lambda: genrec.score_lse_topk(H, E, K, workspace=ws, out=out), dev,
                   lambda: genrec.score_lse_topk(H2, E2, 20, workspace=ws))
