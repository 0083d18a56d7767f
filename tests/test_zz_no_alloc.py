"""The allocation-free entry point (genrec_score_lse_topk_noalloc, through
the C ABI): on the library's per-GPU scratch it gives exactly the results of
genrec_score_lse_topk on a caller workspace, on two calls in a row -- the
second with a smaller input, on the scratch the first one left behind --
and both match the oracle."""
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
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    return torch.from_numpy(a).to(dev)


def _outs(B, K, dev):
    o = (torch.empty((B, K), dtype=torch.int32, device=dev), torch.empty((B, K), dtype=torch.float32, device=dev),
         torch.empty((B,), dtype=torch.float32, device=dev))
    for t in o:
        t.view(torch.uint8).fill_(255)
    return o


def test_noalloc_matches_workspace_entry_point(dev, oracle_mod):
    from full_catalog_ranking_amd import genrec
    # first a matrix-core call with the sampled threshold pass, then a smaller
    # one-launch call on the scratch the first left behind, then the first again
    cases = [(40, 256, 70_000, 50, True), (1, 2048, 5000, 100, True), (40, 256, 70_000, 50, True)]
    for B, D, M, K, bf16 in cases:
        dt = torch.bfloat16 if bf16 else torch.float32
        assert genrec.workspace_bytes(B, D, M, K, dt) <= genrec.NOALLOC_SCRATCH_BYTES
        d = synth.make_dense(B, D, M, seed=B + M, bf16=bf16)
        H, E = _td(d["H"], dev), _td(d["E"], dev)
        print("  noalloc B=%d D=%d M=%d K=%d plan=%s" % (B, D, M, K, genrec.describe_plan(B, D, M, K, dt)), flush=True)
        got = genrec.score_lse_topk_noalloc(H, E, K, out=_outs(B, K, dev))
        ws = torch.full((genrec.workspace_bytes(B, D, M, K, dt),), 255, dtype=torch.uint8, device=dev)
        ref = genrec.score_lse_topk(H, E, K, workspace=ws, out=_outs(B, K, dev))
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
        users = sorted({0, B // 2, B - 1})
        o = oracle_mod.full(d["H"], d["E"], K, users=users)
        parity.check_dense(tuple(x.cpu().numpy() for x in got), o, where="noalloc %s" % ((B, D, M, K),))
