"""C ABI of libgenrec.so on the host: exported symbols, argument validation
and workspace planning.  No call here reaches a kernel launch."""
import ctypes
import os
import re

import pytest

from full_catalog_ranking_amd import genrec

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, -1, -2, -3, -4


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(genrec.LIB_PATH):
        pytest.skip("libgenrec.so not built")
    return genrec.lib()


def header_functions():
    src = open(os.path.join(ROOT, "include", "genrec.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(genrec_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_function_is_exported(L):
    names = header_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(genrec.EXPORTED)


def test_status_strings(L):
    assert genrec.status_string(OK) == "GENREC_OK"
    assert genrec.status_string(UNSUPPORTED) == "GENREC_ERR_UNSUPPORTED"
    assert L.genrec_version() == 10000


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced on these paths


def call_dense(L, H=FAKE, E=FAKE, dtype=0, B=4, D=64, M=100, K=10, oi=FAKE, os_=FAKE, ol=FAKE,
               ws=FAKE, wsb=0):
    return L.genrec_score_lse_topk(H, E, dtype, B, D, M, K, oi, os_, ol, ws, wsb, None)


def test_dense_argument_errors(L):
    assert call_dense(L, H=None) == INVALID
    assert call_dense(L, E=None) == INVALID
    assert call_dense(L, oi=None) == INVALID
    assert call_dense(L, dtype=7) == INVALID
    assert call_dense(L, B=0) == INVALID
    assert call_dense(L, D=-8) == INVALID
    assert call_dense(L, M=0) == INVALID
    assert call_dense(L, K=0) == INVALID
    assert call_dense(L, K=1025) == UNSUPPORTED
    assert call_dense(L, D=12) == UNSUPPORTED            # bf16 needs D % 8 == 0
    assert call_dense(L, dtype=1, D=12) != UNSUPPORTED   # fp32 needs D % 4 == 0 ...
    assert call_dense(L, dtype=1, D=6) == UNSUPPORTED
    assert call_dense(L, M=1 << 31) == UNSUPPORTED
    assert call_dense(L, H=FAKE + 8) == INVALID          # misaligned
    assert call_dense(L, ws=None, wsb=1 << 40) == WORKSPACE
    need = L.genrec_score_lse_topk_workspace(4, 64, 100, 10, 0)
    assert need > 0
    assert call_dense(L, wsb=need - 1) == WORKSPACE
    assert call_dense(L, ws=FAKE + 16, wsb=need) == INVALID  # workspace must be 256-byte aligned


def test_candidate_argument_errors(L):
    f = L.genrec_score_candidates_topk
    assert f(FAKE, FAKE, 0, None, FAKE, 4, 64, 100, 10, 5, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, 0, FAKE, None, 4, 64, 100, 10, 5, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 4, 64, 100, -1, 5, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 4, 64, 100, 10, 0, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == INVALID
    need = L.genrec_score_candidates_topk_workspace(4, 64, 100, 10, 5, 0)
    assert need > 0
    assert f(FAKE, FAKE, 0, FAKE, FAKE, 4, 64, 100, 10, 5, FAKE, FAKE, FAKE, FAKE, need - 1, None) == WORKSPACE
    assert L.genrec_get_device_errors(None, None, None, None) == INVALID
    assert L.genrec_get_rescued_users(None, None, None) == INVALID
    t = L.genrec_topk_rows
    assert t(None, 2, 100, 100, 5, FAKE, FAKE, None, 0, None) == INVALID       # no scores
    assert t(FAKE, 0, 100, 100, 5, FAKE, FAKE, None, 0, None) == INVALID       # R = 0
    assert t(FAKE, 2, 100, 99, 5, FAKE, FAKE, None, 0, None) == INVALID        # ld < N
    assert t(FAKE, 2, 100, 100, 0, FAKE, FAKE, None, 0, None) == INVALID       # K = 0
    assert t(FAKE, 2, 100, 100, 2000, FAKE, FAKE, None, 0, None) == UNSUPPORTED  # K > KMAX
    # rows of up to 16,384 columns with K <= 512: one block per row, no workspace
    assert L.genrec_topk_rows_workspace(8, 4096, 128) == 0
    assert L.genrec_topk_rows_workspace(8, 16384, 128) == 0
    assert L.genrec_topk_rows_workspace(8, 16384, 256) == 0
    assert L.genrec_topk_rows_workspace(8, 4096, 257) == 0
    assert L.genrec_topk_rows_workspace(8, 16384, 512) == 0
    # histogram narrowing for larger K: one pass up to 4,096 columns; longer rows
    # need the chunk results' workspace
    assert L.genrec_topk_rows_workspace(8, 4096, 513) == 0
    assert L.genrec_topk_rows_workspace(8, 16384, 600) == 8 * 4 * 600 * 8
    need = L.genrec_topk_rows_workspace(8, 512 * 512, 600)
    assert need > 0 and need % (8 * 8 * 600) == 0 and need // (8 * 8 * 600) * 600 <= 6144
    assert t(FAKE, 8, 512 * 512, 512 * 512, 600, FAKE, FAKE, None, 0, None) == WORKSPACE

    # the filter route (rows of more than 16,384 columns, K <= 512, when about
    # 3 K keys reaching the sampled bound stay within half of the 8,192-key
    # list): per row the list, then the bounds and the counts of its 64 parts
    def filt(R):
        return -(-R * 8192 * 8 // 256) * 256 + -(-R * 4 // 256) * 256 + -(-R * 64 * 4 // 256) * 256
    for R, N, K in ((8, 512 * 512, 512), (64, 512 * 512, 512), (8, 64 * 16384, 128), (1, 16385, 100),
                    (256, 2 * 16384, 512), (1, 4_000_000, 1)):
        assert L.genrec_topk_rows_workspace(R, N, K) == filt(R), (R, N, K)
    assert t(FAKE, 8, 512 * 512, 512 * 512, 512, FAKE, FAKE, None, 0, None) == WORKSPACE
    # register-resident selection: rows of >= 2 segments of 16,384 columns whose
    # K keys fit the 8,192-key row merge, with >= 512 segment blocks in all,
    # where the filter route does not apply: K > 512, too short a row for 3 K
    # keys at the sampled bound (N < ~36 K), or too long for the list (N > ~4e6)
    assert L.genrec_topk_rows_workspace(520, 2 * 16384, 1024) == 520 * 2 * 1024 * 8
    assert L.genrec_topk_rows_workspace(256, 17_000, 512) == 256 * 2 * 512 * 8
    assert L.genrec_topk_rows_workspace(8, 5_000_000, 20) == 8 * 306 * 20 * 8
    assert L.genrec_topk_rows_workspace(1, 4_200_000, 1) == 1026 * 8  # one row: 1,026 histogram chunks
    m = L.genrec_score_lse_topk_masked
    ws = L.genrec_score_lse_topk_workspace(4, 64, 100, 10, 0)
    assert m(FAKE, FAKE, 0, 4, 64, 100, 10, None, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == INVALID   # no mask
    assert m(FAKE, FAKE, 0, 4, 64, 100, 10, FAKE, 3, FAKE, FAKE, FAKE, FAKE, ws, None) == INVALID   # stride < 4 words
    assert m(FAKE, FAKE, 0, 4, 64, 100, 10, FAKE, -1, FAKE, FAKE, FAKE, FAKE, ws, None) == INVALID


def test_workspace_queries(L):
    assert L.genrec_score_lse_topk_workspace(0, 64, 100, 10, 0) == 0
    assert L.genrec_score_lse_topk_workspace(4, 64, 100, 2000, 0) == 0
    big = L.genrec_score_lse_topk_workspace(1024, 4096, 1_000_000, 500, 0)
    # bounded candidate regions: 1,024 users x 64 chunks x 4 lane groups x 64
    # keys of 8 bytes and 20 bytes of record each, per user an overflow region
    # of 16,384 keys (and its record), the 16,128-item sample (4 bytes a
    # score), per-user histograms of 4,096 counts, collect regions of 5,120
    # keys and room to gather the rescued users' rows (4,096 bf16 each)
    parts = (1024 * 256 * (64 * 8 + 20) + 1024 * (16384 * 8 + 20) + 1024 * 16128 * 4 + 1024 * 4096 * 4
             + 1024 * 5120 * 8 + 1024 * 4096 * 2)
    assert parts <= big <= parts * 1.02 and big <= 0.5e9
    # 4,096 users over a catalog of 10 million items: plannable, under 1.5 GB
    # (regions of every item would take 328 GB; the overflow regions, 16,384
    # keys a user, take 0.54 GB of it)
    huge = L.genrec_score_lse_topk_workspace(4096, 2048, 10_000_000, 100, 0)
    assert 0 < huge < 1.5e9
    # shapes whose regions of every item fit the key budget keep them
    mid = L.genrec_score_lse_topk_workspace(256, 2048, 100_000, 100, 0)
    assert 256 * 100_096 * 8 <= mid <= 256 * 100_096 * 8 * 1.3
    # fp32: no hot head; 8 bytes per list entry dominate
    c = L.genrec_score_candidates_topk_workspace(4096, 2048, 1_000_000, 6_400_000, 100, 1)
    assert 6_400_000 * 8 <= c <= 6_400_000 * 8 * 1.5
    # bf16 adds the hot head: per-item counts and hot index (2 x 4 bytes per catalog item),
    # 16,384 gathered rows of 2 D bytes and their dense scores for every user
    hot = 2 * 4 * 1_000_000 + 16384 * 2048 * 2 + 4096 * 16384 * 4
    cb = L.genrec_score_candidates_topk_workspace(4096, 2048, 1_000_000, 6_400_000, 100, 0)
    assert c + hot <= cb <= c + hot * 1.01
    # few users: no hot head
    assert (L.genrec_score_candidates_topk_workspace(8, 2048, 1_000_000, 20_000, 100, 0)
            == L.genrec_score_candidates_topk_workspace(8, 2048, 1_000_000, 20_000, 100, 1))


def test_key_budget(L, monkeypatch):
    """Bounded regions past the key budget (GENREC_KEY_BUDGET overrides it):
    pieces of 8 times the expected count (at least 64 keys), a collect region
    of 8 K + 1,024 keys rounded to 256; below the budget, regions of every
    item; plans without a sampled fast threshold never bound their regions."""
    import torch
    p = genrec.describe_plan(1024, 4096, 1_000_000, 500, torch.bfloat16)
    assert p["bounded"] == 1 and p["cap"] == 64 and p["ccol"] == 5120 and p["ovf_cap"] == 16384
    p = genrec.describe_plan(4096, 2048, 10_000_000, 1024, torch.bfloat16)
    # 4 K / (4 P) = 64 expected per piece (P = 16), times 8
    assert p["bounded"] == 1 and p["P"] == 16 and p["cap"] == 512 and p["ccol"] == 9216 and p["ovf_cap"] == 18432
    assert genrec.describe_plan(256, 2048, 100_000, 100, torch.bfloat16)["bounded"] == 0
    monkeypatch.setenv("GENREC_KEY_BUDGET", "0")
    p = genrec.describe_plan(256, 2048, 100_000, 100, torch.bfloat16)
    assert p["bounded"] == 1 and p["cap"] == 64
    w0 = genrec.workspace_bytes(256, 2048, 100_000, 100, torch.bfloat16)
    assert genrec.describe_plan(4, 64, 50_000, 10, torch.bfloat16)["bounded"] == 0  # no sample
    assert genrec.describe_plan(1, 2048, 1_000_000, 100, torch.bfloat16)["bounded"] == 0  # one user: VALU path
    monkeypatch.setenv("GENREC_KEY_BUDGET", str(1 << 50))
    assert genrec.describe_plan(1024, 4096, 1_000_000, 500, torch.bfloat16)["bounded"] == 0
    for junk in ("not a number", "-1", " 5", "5x", ""):  # ignored: the default budget
        monkeypatch.setenv("GENREC_KEY_BUDGET", junk)
        assert genrec.describe_plan(1024, 4096, 1_000_000, 500, torch.bfloat16)["bounded"] == 1
    monkeypatch.delenv("GENREC_KEY_BUDGET")
    assert genrec.workspace_bytes(256, 2048, 100_000, 100, torch.bfloat16) > w0


def test_overflow_keys(L, monkeypatch):
    """GENREC_OVERFLOW_KEYS sets each user's overflow region in the bounded
    layout (0: none; unparsable: the default max(16,384, 2 ccol)); the
    workspace follows it by B x 8 bytes per key; regions of every item have
    none."""
    import torch
    shape = (1024, 4096, 1_000_000, 500)
    base = genrec.workspace_bytes(*shape, torch.bfloat16)
    assert genrec.describe_plan(*shape, torch.bfloat16)["ovf_cap"] == 16384
    monkeypatch.setenv("GENREC_OVERFLOW_KEYS", "0")
    assert genrec.describe_plan(*shape, torch.bfloat16)["ovf_cap"] == 0
    assert genrec.workspace_bytes(*shape, torch.bfloat16) == base - 1024 * 16384 * 8
    monkeypatch.setenv("GENREC_OVERFLOW_KEYS", "1000")
    assert genrec.describe_plan(*shape, torch.bfloat16)["ovf_cap"] == 1000
    monkeypatch.setenv("GENREC_OVERFLOW_KEYS", "-5")  # unparsable as a count: the default
    assert genrec.describe_plan(*shape, torch.bfloat16)["ovf_cap"] == 16384
    monkeypatch.setenv("GENREC_KEY_BUDGET", str(1 << 50))
    p = genrec.describe_plan(*shape, torch.bfloat16)
    assert p["bounded"] == 0 and p["ovf_cap"] == 0


def test_plan_selection(L):
    import torch
    p = genrec.describe_plan(1024, 4096, 1_000_000, 500, torch.bfloat16)
    assert p["path"] == "mfma" and p["sample"] == 1 and p["UT"] == 4 and p["P"] == 64
    # MFMA path: ~32 M / (4 K) = 16,000 sampled items suffice for a fast
    # threshold of rank >= 32: every 62nd of the 3906 full tiles (63 tiles);
    # fast threshold rank ceil(4 K n_sample / M)
    assert p["stride"] == 62 and p["n_sample"] == 63 * 256
    assert p["fast"] == 1 and p["r_fast"] == -(-4 * 500 * 63 * 256 // 1_000_000) >= 32
    p = genrec.describe_plan(256, 2048, 100_000, 100, torch.bfloat16)
    assert p["path"] == "mfma" and p["sample"] == 1 and p["P"] == 256
    assert p["fast"] == 1 and p["r_fast"] == -(-4 * 100 * p["n_sample"] // 100_000)
    # the VALU path keeps the K-th sampled score (no rescue pass)
    p = genrec.describe_plan(1, 96, 70_000, 50, torch.bfloat16)
    assert p["path"] == "stream" and p["sample"] == 1 and p["fast"] == 0
    # ... and the largest sample: every 32nd full tile, at most 128 tiles
    p = genrec.describe_plan(1, 4096, 1_000_000, 100, torch.bfloat16)
    assert p["stride"] == 32 and p["n_sample"] == 123 * 256
    # small bf16 batches go to the matrix cores (E read once, not once per user)
    assert genrec.describe_plan(2, 96, 70_000, 50, torch.bfloat16)["path"] == "mfma"
    # fp32 batches too, past the one-launch catalog size; one fp32 user streams
    assert genrec.describe_plan(8, 4096, 1_000_000, 100, torch.float32)["path"] == "mfma"
    assert genrec.describe_plan(256, 2048, 100_000, 100, torch.float32)["path"] == "mfma"
    assert genrec.describe_plan(1, 4096, 1_000_000, 100, torch.float32)["path"] == "stream"
    assert genrec.describe_plan(300, 256, 8192, 10, torch.float32)["fused"] == 1
    p = genrec.describe_plan(1, 2048, 5000, 100, torch.bfloat16)
    assert p["path"] == "stream" and p["sample"] == 0
    p = genrec.describe_plan(4, 256, 5000, 10, torch.float32)
    assert p["path"] == "stream"
    p = genrec.describe_plan(9, 64, 50, 64, torch.bfloat16)
    assert p["path"] == "mfma" and p["sample"] == 0
    with pytest.raises(genrec.GenrecError):
        genrec.describe_plan(4, 12, 100, 10, torch.bfloat16)


def test_merge_build_selection(L):
    import torch
    # 4 K = 2,000 expected candidates and 64 x 4 pieces per user: the small build
    assert genrec.describe_plan(1024, 4096, 1_000_000, 500, torch.bfloat16)["merge_small"] == 1
    # K = 1,024: ~4,096 candidates expected
    assert genrec.describe_plan(1024, 4096, 1_000_000, 1024, torch.bfloat16)["merge_small"] == 0
    # 256 chunks x 4 lane groups = 1,024 pieces per user
    assert genrec.describe_plan(256, 2048, 100_000, 100, torch.bfloat16)["merge_small"] == 0
    # no sample: every item is a candidate
    assert genrec.describe_plan(1, 2048, 5000, 100, torch.bfloat16)["merge_small"] == 0
    assert genrec.describe_plan(9, 64, 1500, 64, torch.bfloat16)["merge_small"] == 1


def test_ce_validation_and_workspace(L):
    """Cross-entropy entry points: argument errors come back before any launch."""
    f, b = L.genrec_ce_forward, L.genrec_ce_backward
    wf = L.genrec_ce_forward_workspace(300, 64, 5000)
    wb = L.genrec_ce_backward_workspace(300, 64, 5000)
    assert wf > 0 and wb > 0
    assert L.genrec_ce_forward_workspace(0, 64, 5000) == 0
    assert f(FAKE, FAKE, 0, 64, 5000, FAKE, None, FAKE, FAKE, FAKE, wf, None) == INVALID        # B = 0
    assert f(FAKE, FAKE, 300, 60, 5000, FAKE, None, FAKE, FAKE, FAKE, wf, None) == UNSUPPORTED  # D % 8
    assert f(FAKE, FAKE, 300, 64, 5000, None, None, FAKE, FAKE, FAKE, wf, None) == INVALID      # no labels
    assert f(FAKE, FAKE, 300, 64, 5000, FAKE, None, FAKE, FAKE, FAKE, wf - 1, None) == WORKSPACE
    assert b(FAKE, FAKE, 300, 64, 5000, FAKE, None, FAKE, FAKE, FAKE, 0, FAKE, wb - 1, None) == WORKSPACE
    assert b(FAKE, FAKE, 300, 64, 5000, FAKE, None, FAKE, FAKE, FAKE, 7, FAKE, wb, None) == INVALID  # dE dtype
    assert b(FAKE, FAKE, 300, 64, 5000, FAKE, None, None, FAKE, FAKE, 1, FAKE, wb, None) == INVALID  # no lse
    # backward workspace at the benchmark shape: H^T, one chunk's E^T and G in two
    # layouts (65,536 rows), 8 partial dH buffers
    big = L.genrec_ce_backward_workspace(1024, 4096, 1_000_000)
    parts = 2 * 4096 * 1024 + 2 * 4096 * 65536 + 2 * 2 * 1024 * 65536 + 4 * 8 * 1024 * 4096
    assert parts <= big <= parts + 1_000_000


def test_ce_chunk_bounds(L):
    """Wide rows shrink the backward's catalog chunk; past 2^21 users it is refused."""
    w_small = L.genrec_ce_backward_workspace(8, 65536, 100_000)
    # one chunk of 8,192 rows: E^T 65,536 x 8,192 bf16 = 1 GiB dominates
    assert (1 << 30) <= w_small <= (1 << 30) + (64 << 20)
    assert L.genrec_ce_backward_workspace(3_000_000, 8, 1000) == 0
    assert L.genrec_ce_forward_workspace(3_000_000, 8, 1000) > 0
    FAKE = 1 << 20
    assert L.genrec_ce_backward(FAKE, FAKE, 3_000_000, 8, 1000, FAKE, None, FAKE, FAKE, FAKE, 1, FAKE,
                                1 << 40, None) == UNSUPPORTED


def test_plans_at_the_largest_supported_sizes(L):
    """Workspace and plan arithmetic at the edge of the supported shapes stays
    in 64-bit range and consistent (no launch)."""
    import torch
    M = (1 << 31) - 1
    # dense: bounded candidate regions (regions of every item would take
    # B x 256 ceil(M / 256) keys of 8 bytes: 68.7 GB)
    w = L.genrec_score_lse_topk_workspace(4, 8, M, 1024, 0)
    p = genrec.describe_plan(4, 8, M, 1024, torch.bfloat16)
    assert p["workspace"] == w and p["path"] == "mfma" and p["sample"] == 1 and p["bounded"] == 1
    assert 0 < w < 4 * ((M + 255) // 256 * 256) * 8 // 100
    assert L.genrec_score_lse_topk_workspace(1, 16384, M, 1, 1) >= M * 8   # fp32, VALU path
    assert L.genrec_score_lse_topk_workspace(4, 65536, 100, 10, 0) > 0     # GENREC_DMAX
    assert L.genrec_score_lse_topk_workspace(4, 65544, 100, 10, 0) == 0    # D past the maximum
    # candidates: 8 bytes per entry plus the hot head's per-item arrays
    nnz = (1 << 33) + 5
    c = L.genrec_score_candidates_topk_workspace(4096, 2048, M, nnz, 100, 0)
    assert c >= nnz * 8 + 2 * 4 * M
    # cross-entropy: the chunk shrinks so that each blocked operand stays under 1 GiB
    assert L.genrec_ce_backward_workspace(1 << 21, 8, M) > 0
    assert L.genrec_ce_backward_workspace((1 << 21) + 1, 8, M) == 0


def test_ce_plan_query(L):
    """The backward's plan as the library reports it: consistent with its
    workspace query, and the addition depths follow from chunking and splits."""
    for B, D, M in ((1024, 4096, 1_000_000), (3, 64, 1000), (8, 16384, 36_000), (300, 200, 5000)):
        p = genrec.describe_ce_plan(B, D, M)
        assert p["workspace"] == L.genrec_ce_backward_workspace(B, D, M)
        assert p["Mcp"] % 256 == 0 and p["Mcp"] >= p["chunk"] and p["n_chunks"] == -(-M // p["chunk"])
        assert p["Bp"] == -(-B // 32) * 32 and p["splits"] in (1, 2, 4, 8)
        assert p["depth_h"] == p["Mcp"] // p["splits"] + p["n_chunks"] + p["splits"]
        assert p["depth_e"] == p["Bp"]
    buf = ctypes.create_string_buffer(64)
    assert L.genrec_describe_ce_plan(0, 64, 100, buf, 64) == INVALID
    assert L.genrec_describe_ce_plan(4, 64, 100, None, 64) == INVALID
    assert L.genrec_describe_ce_plan(4, 64, 1 << 31, buf, 64) == UNSUPPORTED


def test_noalloc_rejects_shapes_beyond_its_scratch(L):
    """The allocation-free entry point refuses a call whose workspace exceeds
    its fixed scratch before touching the device (argument errors first)."""
    f = L.genrec_score_lse_topk_noalloc
    big = (1024, 4096, 1_000_000, 500)
    assert L.genrec_score_lse_topk_workspace(*big, 0) > genrec.NOALLOC_SCRATCH_BYTES
    assert f(FAKE, FAKE, 0, *big, FAKE, FAKE, FAKE, None) == -5
    assert genrec.status_string(-5) == "GENREC_ERR_TOO_LARGE"
    assert f(None, FAKE, 0, *big, FAKE, FAKE, FAKE, None) == INVALID
    assert f(FAKE, FAKE, 0, 4, 64, 100, 0, FAKE, FAKE, FAKE, None) == INVALID
    small = (1, 2048, 5000, 100)
    assert L.genrec_score_lse_topk_workspace(*small, 0) <= genrec.NOALLOC_SCRATCH_BYTES
