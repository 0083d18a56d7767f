"""GPU parity of the catalog cross-entropy (forward and backward, through the C
ABI) against the CPU oracle, under the rule in parity.check_ce."""
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


def _bf16(a, dev):
    return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)


def run_ce(d, labels, weights, dev, backward=True, de_dtype=None):
    from full_catalog_ranking_amd import genrec
    B, D, M = d["B"], d["D"], d["M"]
    print("  ce B=%d D=%d M=%d weights=%s" % (B, D, M, weights is not None), flush=True)
    H, E = _bf16(d["H"], dev), _bf16(d["E"], dev)
    lab = torch.from_numpy(labels).to(dev)
    w = torch.from_numpy(weights).to(dev) if weights is not None else None
    loss, lse, ws = genrec.ce_forward(H, E, lab, w)
    errs = genrec.device_errors(ws)
    out = [loss.cpu().numpy(), lse.cpu().numpy(), None, None]
    if backward:
        dH, dE = genrec.ce_backward(H, E, lab, lse, w, de_dtype=de_dtype or torch.float32)
        torch.cuda.synchronize()
        out[2] = dH.cpu().numpy()
        out[3] = dE.float().cpu().numpy()
        del dH, dE
    del H, E
    return out, errs


def _depths(B, D, M):
    """Longest fp32 addition chains of the two products, from the library's own
    plan (see parity.check_ce)."""
    from full_catalog_ranking_amd import genrec
    p = genrec.describe_ce_plan(B, D, M)
    return p["depth_h"], p["depth_e"]


@pytest.mark.parametrize("B,D,M,seed,bad,weighted", [
    (3, 64, 1000, 1, False, True),        # one user tile, four item tiles
    (300, 200, 5000, 2, True, True),      # two user tiles, k tail (D % 32 = 8), ragged item tile, bad labels
    (40, 96, 140_000, 3, False, True),    # three catalog chunks, the last partial
    (513, 256, 3000, 4, False, False),    # three user tiles, B % 32 != 0, no weights
    (8, 8, 70, 5, False, True),           # smallest D, catalog below one tile
])
def test_ce_parity(dev, oracle_mod, B, D, M, seed, bad, weighted):
    d = synth.make_dense(B, D, M, seed=seed)
    labels = synth.gen_labels(B, M, seed)
    w = synth.gen_weights(B, seed) if weighted else None
    if bad:
        labels[1], labels[-1] = -1, M  # outside [0, M): ignored and counted
    g, errs = run_ce(d, labels, w, dev)
    assert errs == ((2, 0) if bad else (0, 0))
    ref = oracle_mod.ce(d["H"], d["E"], labels, w)
    dh_depth, de_depth = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, de_depth, where="ce %s" % ((B, D, M),))
    if bad:
        assert g[0][1] == 0.0 and g[0][-1] == 0.0
        assert np.abs(g[2][1]).max() == 0.0 and np.abs(g[2][-1]).max() == 0.0


def test_ce_bf16_grad_catalog(dev, oracle_mod):
    """dE stored in bf16: the same bound plus the rounding of the stored value."""
    B, D, M = 300, 200, 5000
    d = synth.make_dense(B, D, M, seed=11)
    labels = synth.gen_labels(B, M, 11)
    w = synth.gen_weights(B, 11)
    g, errs = run_ce(d, labels, w, dev, de_dtype=torch.bfloat16)
    assert errs == (0, 0)
    ref = oracle_mod.ce(d["H"], d["E"], labels, w)
    dh_depth, de_depth = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, de_depth, de_round=2.0 ** -8,
                    where="ce bf16 dE")


def test_ce_wide_rows(dev, oracle_mod):
    """D = 4096 (the benchmark width: 16 column tiles of the dE product) over two
    catalog chunks."""
    B, D, M = 256, 4096, 70_000
    d = synth.make_dense(B, D, M, seed=7)
    labels = synth.gen_labels(B, M, 7)
    w = synth.gen_weights(B, 7)
    g, errs = run_ce(d, labels, w, dev)
    assert errs == (0, 0)
    ref = oracle_mod.ce(d["H"], d["E"], labels, w)
    dh_depth, de_depth = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, de_depth, where="ce wide")


def test_ce_wide_d_smaller_chunks(dev, oracle_mod):
    """D = 16,384: the backward's chunk shrinks to 32,768 catalog rows (each
    blocked operand under 1 GiB), two chunks here."""
    from full_catalog_ranking_amd import genrec
    B, D, M = 8, 16384, 36_000
    assert genrec.lib().genrec_ce_backward_workspace(B, D, M) < (1 << 30) + (64 << 20)
    d = synth.make_dense(B, D, M, seed=13)
    labels = synth.gen_labels(B, M, 13)
    w = synth.gen_weights(B, 13)
    g, errs = run_ce(d, labels, w, dev)
    assert errs == (0, 0)
    ref = oracle_mod.ce(d["H"], d["E"], labels, w)
    dh_depth, de_depth = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, de_depth, where="ce wide D")


def test_ce_full_size_sampled_users(dev, oracle_mod):
    """The benchmark shape (1,024 x 1e6 x 4,096): loss, lse and dH rows of
    sampled users against the oracle; dE over the whole catalog sums to about
    zero per column (the rows of G sum to zero) and is finite."""
    from full_catalog_ranking_amd import genrec
    d = synth.make_workload("ce")
    B, D, M = d["B"], d["D"], d["M"]
    H, E = _bf16(d["H"], dev), _bf16(d["E"], dev)
    lab = torch.from_numpy(d["labels"]).to(dev)
    w = torch.from_numpy(d["weights"]).to(dev)
    print("  ce full size", flush=True)
    loss, lse, ws = genrec.ce_forward(H, E, lab, w)
    dH, dE = genrec.ce_backward(H, E, lab, lse, w)
    torch.cuda.synchronize()
    assert genrec.device_errors(ws) == (0, 0)
    col = dE.sum(dim=0, dtype=torch.float64).cpu().numpy()
    finite = bool(torch.isfinite(dE).all())
    users = [0, 1, 255, 256, 511, 512, 800, 1023]  # every 256-user tile, both halves of a wave's users
    g = (loss.cpu().numpy()[users], lse.cpu().numpy()[users], dH.cpu().numpy()[users], None)
    del dE, dH, H, E
    torch.cuda.empty_cache()
    assert finite
    ref = oracle_mod.ce(d["H"], d["E"], d["labels"], d["weights"], users=users)
    dh_depth, _ = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, where="ce full size")
    # sum_i dE[i] = sum_b h_b sum_i G[b][i] = 0; |sum_i G_gpu[b][i]| <= c sum_i A[b][i] <= 3 c w_b
    tau = parity.SCORE_REL * np.abs(ref["S"]).max()
    c = 2.0 ** -9 + 2 * tau + (-(-B // 32) * 32) * 2.0 ** -24
    bound = 3 * c * (d["weights"].astype(np.float64)[:, None] * np.abs(oracle_mod.widen(d["H"]))).sum(axis=0)
    assert (np.abs(col) <= bound).all(), (np.abs(col).max(), bound.min())


def check_ce_by_definition(d, loss, lse, dH, dE, dh_depth, de_depth, step=65536):
    """Every user and every catalog row of a cross-entropy call, against the
    definitions (G = w (softmax - onehot), dH = G E, dE = G^T H, loss =
    w (lse - s_label)) recomputed from a float32 library product of the
    widened bf16 rows, chunk by chunk, on the device the outputs live on.  The
    bounds are the parity rule's (parity.check_ce): lse within LSE_ABS, loss
    within 2 w LSE_ABS, each gradient element within (c + depth 2^-24) times
    the same product of the absolute values, c = 2^-9 + 2 tau.  The float32
    reference's own rounding (about 1e-5 relative at these depths) is far
    inside c.  Labels must lie in [0, M)."""
    B, D, M = d["B"], d["D"], d["M"]
    dv = dH.device
    assert ((d["labels"] >= 0) & (d["labels"] < M)).all()
    prev = (torch.backends.cuda.matmul.allow_tf32, torch.get_float32_matmul_precision())
    torch.backends.cuda.matmul.allow_tf32 = False
    torch.set_float32_matmul_precision("highest")
    try:
        Hf = _bf16(d["H"], dv).float()
        Ht = Hf.t().contiguous()  # [D][B]: no transposed operand view
        aH = Hf.abs()
        wd = torch.from_numpy(d["weights"].astype(np.float64)).to(dv)
        lab = torch.from_numpy(d["labels"].astype(np.int64)).to(dv)
        lse_r = torch.full((B,), -math.inf, dtype=torch.float64, device=dv)
        smax = 0.0
        for r0 in range(0, M, step):  # pass 1: lse and the largest |score|
            St = _bf16(d["E"][r0:r0 + step], dv).float() @ Ht
            lse_r = torch.logaddexp(lse_r, torch.logsumexp(St.double(), dim=0))
            smax = max(smax, float(St.abs().max()))
            del St
        s_lab = (_bf16(d["E"][d["labels"]], dv).double() * Hf.double()).sum(dim=1)
        loss_r = wd * (lse_r - s_lab)
        err = (lse.double() - lse_r).abs()
        assert float(err.max()) <= parity.LSE_ABS, ("lse", int(err.argmax()), float(err.max()))
        err = (loss.double() - loss_r).abs()
        assert bool((err <= wd * 2 * parity.LSE_ABS + 1e-6).all()), ("loss", int(err.argmax()), float(err.max()))
        c = 2.0 ** -9 + 2 * parity.SCORE_REL * smax
        dH_r = torch.zeros((B, D), dtype=torch.float64, device=dv)
        AE = torch.zeros((B, D), dtype=torch.float64, device=dv)
        worst_e = 0.0
        for r0 in range(0, M, step):  # pass 2: G and A of the chunk, its dE rows, its share of dH
            r1 = min(M, r0 + step)
            Ec = _bf16(d["E"][r0:r1], dv).float()
            Pt = torch.exp((Ec @ Ht).double() - lse_r[None, :])  # [items][B]
            Gt = wd[None, :] * Pt
            hit = (lab >= r0) & (lab < r1)
            ub = torch.nonzero(hit).flatten()
            Gt[lab[ub] - r0, ub] -= wd[ub]
            At = Gt.abs() + wd[None, :] * Pt
            Gt32, At32 = Gt.float(), At.float()
            del Pt, Gt, At
            tol_e = (c + de_depth * 2.0 ** -24) * (At32 @ aH) + 1e-30
            err_e = (dE[r0:r1].float() - Gt32 @ Hf).abs()
            ratio = float((err_e / tol_e).max())
            assert ratio <= 1.0, ("dE", r0, float(err_e.max()), ratio)
            worst_e = max(worst_e, ratio)
            del tol_e, err_e
            dH_r += (Gt32.t().contiguous() @ Ec).double()
            AE += (At32.t().contiguous() @ Ec.abs()).double()
            del Ec, Gt32, At32
        tol_h = (c + dh_depth * 2.0 ** -24) * AE + 1e-30
        ratio_h = float(((dH.double() - dH_r).abs() / tol_h).max())
        assert ratio_h <= 1.0, ("dH", ratio_h)
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev[0]
        torch.set_float32_matmul_precision(prev[1])
    return worst_e, ratio_h


def test_ce_full_size_all_users(dev):
    """The benchmark shape (1,024 x 1e6 x 4,096): loss and lse of every user,
    dH of every user and dE of every catalog row, each against the gradients'
    definitions under the parity rule's bounds (check_ce_by_definition; the
    oracle checks sampled users of this shape in the test above)."""
    from full_catalog_ranking_amd import genrec
    d = synth.make_workload("ce")
    B, D, M = d["B"], d["D"], d["M"]
    H, E = _bf16(d["H"], dev), _bf16(d["E"], dev)
    lab = torch.from_numpy(d["labels"]).to(dev)
    w = torch.from_numpy(d["weights"]).to(dev)
    print("  ce full size, every user and row", flush=True)
    loss, lse, ws = genrec.ce_forward(H, E, lab, w)
    dH, dE = genrec.ce_backward(H, E, lab, lse, w)
    torch.cuda.synchronize()
    assert genrec.device_errors(ws) == (0, 0)
    del H, E
    torch.cuda.empty_cache()
    dh_depth, de_depth = _depths(B, D, M)
    worst_e, worst_h = check_ce_by_definition(d, loss, lse, dH, dE, dh_depth, de_depth)
    print("  largest error / bound: dE %.3g, dH %.3g" % (worst_e, worst_h), flush=True)


def test_ce_poisoned_workspaces_and_outputs(dev, oracle_mod):
    """Forward and backward on workspaces and outputs filled with 0xFF bytes
    (NaN) before the calls; two catalog chunks and a k tail (D % 32 = 8)."""
    from full_catalog_ranking_amd import genrec
    B, D, M = 70, 40, 70_000
    d = synth.make_dense(B, D, M, seed=19)
    labels = synth.gen_labels(B, M, 19)
    w = synth.gen_weights(B, 19)
    H, E = _bf16(d["H"], dev), _bf16(d["E"], dev)
    lab, wt = torch.from_numpy(labels).to(dev), torch.from_numpy(w).to(dev)
    L = genrec.lib()
    wsf = torch.full((L.genrec_ce_forward_workspace(B, D, M),), 255, dtype=torch.uint8, device=dev)
    wsb = torch.full((L.genrec_ce_backward_workspace(B, D, M),), 255, dtype=torch.uint8, device=dev)
    dH = torch.full((B, D), float("nan"), dtype=torch.float32, device=dev)
    dE = torch.full((M, D), float("nan"), dtype=torch.float32, device=dev)
    print("  ce poisoned B=%d D=%d M=%d" % (B, D, M), flush=True)
    loss, lse, _ = genrec.ce_forward(H, E, lab, wt, workspace=wsf)
    genrec.ce_backward(H, E, lab, lse, wt, workspace=wsb, out=(dH, dE))
    torch.cuda.synchronize()
    assert genrec.device_errors(wsf) == (0, 0)
    g = (loss.cpu().numpy(), lse.cpu().numpy(), dH.cpu().numpy(), dE.cpu().numpy())
    ref = oracle_mod.ce(d["H"], d["E"], labels, w)
    dh_depth, de_depth = _depths(B, D, M)
    parity.check_ce(g, ref, d["E"], d["H"], oracle_mod.widen, dh_depth, de_depth, where="ce poisoned")
