"""Python binding of libgenrec.so (ctypes): argument marshalling only.

PyTorch supplies device memory and the current HIP stream; every step of the
ranking head runs in the library's HIP kernels.  If the library is missing
or cannot be loaded this module raises -- there is no fallback path.
"""
from __future__ import annotations

import contextlib
import ctypes
import json
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgenrec.so")

GENREC_BF16, GENREC_F32 = 0, 1
KMAX = 1024
NOALLOC_SCRATCH_BYTES = 64 << 20  # GENREC_NOALLOC_SCRATCH_BYTES

EXPORTED = (
    "genrec_score_lse_topk_workspace",
    "genrec_score_lse_topk",
    "genrec_score_lse_topk_noalloc",
    "genrec_score_lse_topk_masked",
    "genrec_score_lse_topk_masked_profiled",
    "genrec_score_candidates_topk_workspace",
    "genrec_score_candidates_topk",
    "genrec_get_device_errors",
    "genrec_get_rescued_users",
    "genrec_topk_rows",
    "genrec_topk_rows_workspace",
    "genrec_describe_plan",
    "genrec_describe_ce_plan",
    "genrec_describe_cand_plan",
    "genrec_status_string",
    "genrec_version",
    "genrec_profiler_create",
    "genrec_profiler_destroy",
    "genrec_profiler_reset",
    "genrec_profiler_summary",
    "genrec_score_lse_topk_profiled",
    "genrec_score_candidates_topk_profiled",
    "genrec_ce_forward_workspace",
    "genrec_ce_forward",
    "genrec_ce_forward_profiled",
    "genrec_ce_backward_workspace",
    "genrec_ce_backward",
    "genrec_ce_backward_profiled",
)
# must list GENREC_NUM_KERNEL_KINDS names: the summary fills that many slots
KERNEL_KINDS = ("sample_score", "threshold", "main_score", "merge", "cand_plan", "rescue", "hot_select",
                "hot_score", "ce_small", "transpose", "grad_tiles", "grad_E", "grad_H")


class GenrecError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__("%s failed: %s (%d)" % (where, status_string(status), status))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libgenrec.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libgenrec.so is not built (%s); run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
        L.genrec_score_lse_topk_workspace.argtypes = [I, I, I64, I, I]
        L.genrec_score_lse_topk_workspace.restype = SZ
        L.genrec_score_lse_topk.argtypes = [P, P, I, I, I, I64, I, P, P, P, P, SZ, P]
        L.genrec_score_lse_topk.restype = I
        L.genrec_score_lse_topk_noalloc.argtypes = [P, P, I, I, I, I64, I, P, P, P, P]
        L.genrec_score_lse_topk_noalloc.restype = I
        L.genrec_score_candidates_topk_workspace.argtypes = [I, I, I64, I64, I, I]
        L.genrec_score_candidates_topk_workspace.restype = SZ
        L.genrec_score_candidates_topk.argtypes = [P, P, I, P, P, I, I, I64, I64, I, P, P, P, P, SZ, P]
        L.genrec_score_candidates_topk.restype = I
        L.genrec_get_device_errors.argtypes = [P, P, P, P]
        L.genrec_get_device_errors.restype = I
        L.genrec_topk_rows.argtypes = [P, I, I64, I64, I, P, P, P, SZ, P]
        L.genrec_topk_rows.restype = I
        L.genrec_topk_rows_workspace.argtypes = [I, I64, I]
        L.genrec_topk_rows_workspace.restype = SZ
        L.genrec_get_rescued_users.argtypes = [P, P, P]
        L.genrec_get_rescued_users.restype = I
        L.genrec_describe_plan.argtypes = [I, I, I64, I, I, ctypes.c_char_p, SZ]
        L.genrec_describe_plan.restype = I
        L.genrec_describe_ce_plan.argtypes = [I, I, I64, ctypes.c_char_p, SZ]
        L.genrec_describe_ce_plan.restype = I
        L.genrec_describe_cand_plan.argtypes = [I, I, I64, I64, I, I, ctypes.c_char_p, SZ]
        L.genrec_describe_cand_plan.restype = I
        L.genrec_status_string.argtypes = [I]
        L.genrec_status_string.restype = ctypes.c_char_p
        L.genrec_version.restype = I
        L.genrec_profiler_create.argtypes = [I]
        L.genrec_profiler_create.restype = P
        L.genrec_profiler_destroy.argtypes = [P]
        L.genrec_profiler_reset.argtypes = [P]
        L.genrec_profiler_reset.restype = I
        L.genrec_profiler_summary.argtypes = [P, P, P]
        L.genrec_profiler_summary.restype = I
        L.genrec_score_lse_topk_profiled.argtypes = L.genrec_score_lse_topk.argtypes + [P]
        L.genrec_score_lse_topk_profiled.restype = I
        L.genrec_score_lse_topk_masked.argtypes = [P, P, I, I, I, I64, I, P, I64, P, P, P, P, SZ, P]
        L.genrec_score_lse_topk_masked.restype = I
        L.genrec_score_lse_topk_masked_profiled.argtypes = L.genrec_score_lse_topk_masked.argtypes + [P]
        L.genrec_score_lse_topk_masked_profiled.restype = I
        L.genrec_score_candidates_topk_profiled.argtypes = L.genrec_score_candidates_topk.argtypes + [P]
        L.genrec_score_candidates_topk_profiled.restype = I
        L.genrec_ce_forward_workspace.argtypes = [I, I, I64]
        L.genrec_ce_forward_workspace.restype = SZ
        L.genrec_ce_backward_workspace.argtypes = [I, I, I64]
        L.genrec_ce_backward_workspace.restype = SZ
        L.genrec_ce_forward.argtypes = [P, P, I, I, I64, P, P, P, P, P, SZ, P]
        L.genrec_ce_forward.restype = I
        L.genrec_ce_forward_profiled.argtypes = L.genrec_ce_forward.argtypes + [P]
        L.genrec_ce_forward_profiled.restype = I
        L.genrec_ce_backward.argtypes = [P, P, I, I, I64, P, P, P, P, P, I, P, SZ, P]
        L.genrec_ce_backward.restype = I
        L.genrec_ce_backward_profiled.argtypes = L.genrec_ce_backward.argtypes + [P]
        L.genrec_ce_backward_profiled.restype = I
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().genrec_status_string(int(status)).decode()


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GENREC_BF16
    if t == torch.float32:
        return GENREC_F32
    raise TypeError("H and E must be bfloat16 or float32, got %s" % t)


def workspace_bytes(B: int, D: int, M: int, K: int, dtype: torch.dtype) -> int:
    return int(lib().genrec_score_lse_topk_workspace(B, D, M, K, dtype_code(dtype)))


def cand_workspace_bytes(B: int, D: int, M: int, nnz: int, K: int, dtype: torch.dtype) -> int:
    return int(lib().genrec_score_candidates_topk_workspace(B, D, M, nnz, K, dtype_code(dtype)))


def describe_plan(B: int, D: int, M: int, K: int, dtype: torch.dtype) -> dict:
    buf = ctypes.create_string_buffer(512)
    st = lib().genrec_describe_plan(B, D, M, K, dtype_code(dtype), buf, 512)
    if st != 0:
        raise GenrecError(st, "genrec_describe_plan")
    return json.loads(buf.value.decode())


def describe_cand_plan(B: int, D: int, M: int, nnz: int, K: int, dtype: torch.dtype) -> dict:
    """The candidate path's plan: the hot head and where its per-item counts
    and result sit in the workspace."""
    buf = ctypes.create_string_buffer(512)
    st = lib().genrec_describe_cand_plan(B, D, M, nnz, K, dtype_code(dtype), buf, 512)
    if st != 0:
        raise GenrecError(st, "genrec_describe_cand_plan")
    return json.loads(buf.value.decode())


def describe_ce_plan(B: int, D: int, M: int) -> dict:
    """The cross-entropy backward's plan: chunking, splits and the longest
    fp32 addition chains of its two gradient products (depth_h, depth_e)."""
    buf = ctypes.create_string_buffer(512)
    st = lib().genrec_describe_ce_plan(B, D, M, buf, 512)
    if st != 0:
        raise GenrecError(st, "genrec_describe_ce_plan")
    return json.loads(buf.value.decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream_handle(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _on_device(device: torch.device):
    """The library launches on the current device: make it the inputs' device
    for the call (a no-op when it already is)."""
    if device.index is None or device.index == torch.cuda.current_device():
        return contextlib.nullcontext()
    return torch.cuda.device(device)


def _check_inputs(H: torch.Tensor, E: torch.Tensor):
    if not (H.is_cuda and E.is_cuda):
        raise ValueError("H and E must be device tensors")
    if E.device != H.device:
        raise ValueError("H and E must be on one device")
    if H.dim() != 2 or E.dim() != 2 or H.shape[1] != E.shape[1]:
        raise ValueError("H must be (B, D) and E (M, D), got %s and %s" % (tuple(H.shape), tuple(E.shape)))
    if H.dtype != E.dtype:
        raise ValueError("H and E must share a dtype")
    if not (H.is_contiguous() and E.is_contiguous()):
        raise ValueError("H and E must be contiguous")


def _check_tensor(t: torch.Tensor, name: str, device, dtype=None, shape=None):
    """A caller-provided tensor the kernels read or write: on `device`,
    contiguous, and of the given dtype and shape when those are given."""
    if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != device:
        raise ValueError("%s must be a tensor on %s" % (name, device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))


def _check_workspace(ws: torch.Tensor, device, need: int):
    _check_tensor(ws, "workspace", device)
    if ws.numel() * ws.element_size() < need:
        raise ValueError("workspace holds %d bytes, %d needed" % (ws.numel() * ws.element_size(), need))


def _check_outs(out, B: int, K: int, device):
    if len(out) != 3:
        raise ValueError("out = (idx int32 [B, K], scores float32 [B, K], lse float32 [B])")
    _check_tensor(out[0], "out idx", device, torch.int32, (B, K))
    _check_tensor(out[1], "out scores", device, torch.float32, (B, K))
    _check_tensor(out[2], "out lse", device, torch.float32, (B,))


# Testing aid: with GENREC_POISON=1 in the environment, every workspace and
# output this module allocates starts filled with 0xFF bytes (NaN as bf16 and
# fp32, -1 as int32) instead of whatever the allocator hands back, so that a
# kernel reading memory the call has not written shows up as a wrong result.
_POISON = os.environ.get("GENREC_POISON") == "1"


def _empty(shape, dtype, device):
    t = torch.empty(shape, dtype=dtype, device=device)
    if _POISON and t.numel():
        t.view(torch.uint8).fill_(255)
    return t


def _outputs(B: int, K: int, device):
    idx = _empty((B, K), torch.int32, device)
    sc = _empty((B, K), torch.float32, device)
    ls = _empty((B,), torch.float32, device)
    return idx, sc, ls


class Profiler:
    """HIP-event timing of every kernel the profiled calls launch."""

    def __init__(self, max_launches: int = 4096):
        self.h = lib().genrec_profiler_create(max_launches)
        if not self.h:
            raise RuntimeError("genrec_profiler_create failed")

    def reset(self):
        lib().genrec_profiler_reset(self.h)

    def summary(self) -> dict:
        """{kind: (launches, total_ms)} -- synchronises on the last recorded event."""
        counts = (ctypes.c_int * len(KERNEL_KINDS))()
        ms = (ctypes.c_double * len(KERNEL_KINDS))()
        st = lib().genrec_profiler_summary(self.h, counts, ms)
        if st != 0:
            raise GenrecError(st, "genrec_profiler_summary")
        return {k: (counts[i], ms[i]) for i, k in enumerate(KERNEL_KINDS) if counts[i]}

    def __del__(self):
        try:
            if self.h:
                lib().genrec_profiler_destroy(self.h)
                self.h = None
        except Exception:
            pass


def score_lse_topk(H: torch.Tensor, E: torch.Tensor, K: int, workspace: torch.Tensor | None = None,
                   out=None, profiler: Profiler | None = None, mask: torch.Tensor | None = None):
    """Full-catalog ranking head: returns (idx int32 [B,K], scores f32 [B,K], lse f32 [B]).

    mask (optional): int32/uint32 device tensor of item-mask words, shape (W,) for one
    mask shared by all users or (B, W) per user, W >= ceil(M/32); bit i % 32 of word
    i // 32 set = item i takes part."""
    _check_inputs(H, E)
    B, D = H.shape
    M = E.shape[0]
    if mask is not None:
        if mask.dtype not in (torch.int32, torch.uint32):
            raise TypeError("mask must be a contiguous int32/uint32 device tensor")
        _check_tensor(mask, "mask", H.device)
        W = (M + 31) // 32
        if mask.dim() == 1:
            if mask.numel() < W:
                raise ValueError("mask needs ceil(M/32) words")
            stride = 0
        elif mask.dim() == 2 and mask.shape[0] == B and mask.shape[1] >= W:
            stride = mask.shape[1]
        else:
            raise ValueError("mask must be (W,) or (B, W) with W >= ceil(M/32)")
    need = workspace_bytes(B, D, M, K, H.dtype)
    if need == 0:
        raise GenrecError(lib().genrec_score_lse_topk(None, None, dtype_code(H.dtype), B, D, M, K,
                                                      None, None, None, None, 0, None),
                          "genrec_score_lse_topk")
    if workspace is None:
        workspace = _empty(need, torch.uint8, H.device)
    _check_workspace(workspace, H.device, need)
    if out is not None:
        _check_outs(out, B, K, H.device)
    idx, sc, ls = out if out is not None else _outputs(B, K, H.device)
    tail = (_ptr(idx), _ptr(sc), _ptr(ls), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_handle(H.device))
    head = (_ptr(H), _ptr(E), dtype_code(H.dtype), B, D, M, K)
    if mask is None:
        name = "genrec_score_lse_topk"
        args = head + tail
    else:
        name = "genrec_score_lse_topk_masked"
        args = head + (_ptr(mask), stride) + tail
    with _on_device(H.device):
        if profiler is None:
            st = getattr(lib(), name)(*args)
        else:
            st = getattr(lib(), name + "_profiled")(*args, profiler.h)
    if st != 0:
        raise GenrecError(st, name)
    return idx, sc, ls


def score_lse_topk_noalloc(H: torch.Tensor, E: torch.Tensor, K: int, out):
    """genrec_score_lse_topk_noalloc: the full-catalog head on the library's
    fixed per-GPU scratch (no workspace); out = (idx int32 [B,K], scores f32
    [B,K], lse f32 [B]) provided by the caller."""
    _check_inputs(H, E)
    B, D = H.shape
    M = E.shape[0]
    _check_outs(out, B, K, H.device)
    idx, sc, ls = out
    with _on_device(H.device):
        st = lib().genrec_score_lse_topk_noalloc(_ptr(H), _ptr(E), dtype_code(H.dtype), B, D, M, K, _ptr(idx),
                                                 _ptr(sc), _ptr(ls), _stream_handle(H.device))
    if st != 0:
        raise GenrecError(st, "genrec_score_lse_topk_noalloc")
    return idx, sc, ls


def score_candidates_topk(H: torch.Tensor, E: torch.Tensor, offsets: torch.Tensor, ids: torch.Tensor,
                          K: int, workspace: torch.Tensor | None = None, out=None,
                          profiler: Profiler | None = None):
    """Candidate-set ranking head over CSR lists (offsets int64 [B+1], ids int32 [nnz])."""
    _check_inputs(H, E)
    if offsets.dtype != torch.int64 or ids.dtype != torch.int32:
        raise TypeError("offsets must be int64 and ids int32")
    _check_tensor(offsets, "offsets", H.device)
    _check_tensor(ids, "ids", H.device)
    B, D = H.shape
    M = E.shape[0]
    if offsets.numel() != B + 1:
        raise ValueError("offsets must hold B+1 entries")
    nnz = ids.numel()
    need = cand_workspace_bytes(B, D, M, nnz, K, H.dtype)
    if need == 0:
        raise GenrecError(lib().genrec_score_candidates_topk(None, None, dtype_code(H.dtype), None, None, B, D,
                                                             M, nnz, K, None, None, None, None, 0, None),
                          "genrec_score_candidates_topk")
    if workspace is None:
        workspace = _empty(need, torch.uint8, H.device)
    _check_workspace(workspace, H.device, need)
    if out is not None:
        _check_outs(out, B, K, H.device)
    idx, sc, ls = out if out is not None else _outputs(B, K, H.device)
    args = (_ptr(H), _ptr(E), dtype_code(H.dtype), _ptr(offsets), _ptr(ids) if nnz else None, B, D, M, nnz, K,
            _ptr(idx), _ptr(sc), _ptr(ls), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_handle(H.device))
    with _on_device(H.device):
        if profiler is None:
            st = lib().genrec_score_candidates_topk(*args)
        else:
            st = lib().genrec_score_candidates_topk_profiled(*args, profiler.h)
    if st != 0:
        raise GenrecError(st, "genrec_score_candidates_topk")
    return idx, sc, ls, workspace


def _check_ce(H: torch.Tensor, E: torch.Tensor, labels: torch.Tensor, weights):
    _check_inputs(H, E)
    if H.dtype != torch.bfloat16:
        raise TypeError("the cross-entropy entry points take bfloat16 H and E")
    B = H.shape[0]
    _check_tensor(labels, "labels", H.device, torch.int32, (B,))
    if weights is not None:
        _check_tensor(weights, "weights", H.device, torch.float32, (B,))


def ce_forward(H: torch.Tensor, E: torch.Tensor, labels: torch.Tensor, weights: torch.Tensor | None = None,
               workspace: torch.Tensor | None = None, profiler: Profiler | None = None):
    """Catalog cross-entropy forward: (loss f32 [B], lse f32 [B], workspace).

    loss_b = w_b (lse_b - h_b . e_{y_b}); an out-of-range label gives loss 0
    and is counted (device_errors(workspace)[0])."""
    _check_ce(H, E, labels, weights)
    B, D = H.shape
    M = E.shape[0]
    need = lib().genrec_ce_forward_workspace(B, D, M)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, H.device)
    _check_workspace(workspace, H.device, need)
    loss = _empty((B,), torch.float32, H.device)
    lse = _empty((B,), torch.float32, H.device)
    args = (_ptr(H), _ptr(E), B, D, M, _ptr(labels), _ptr(weights), _ptr(loss), _ptr(lse), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream_handle(H.device))
    with _on_device(H.device):
        if profiler is None:
            st = lib().genrec_ce_forward(*args)
        else:
            st = lib().genrec_ce_forward_profiled(*args, profiler.h)
    if st != 0:
        raise GenrecError(st, "genrec_ce_forward")
    return loss, lse, workspace


def ce_backward(H: torch.Tensor, E: torch.Tensor, labels: torch.Tensor, lse: torch.Tensor,
                weights: torch.Tensor | None = None, workspace: torch.Tensor | None = None, out=None,
                profiler: Profiler | None = None, de_dtype: torch.dtype = torch.float32):
    """Gradients of sum_b loss_b: (dH f32 [B, D], dE [M, D] in de_dtype (float32 or
    bfloat16)); lse from ce_forward."""
    _check_ce(H, E, labels, weights)
    B, D = H.shape
    M = E.shape[0]
    _check_tensor(lse, "lse", H.device, torch.float32, (B,))
    need = lib().genrec_ce_backward_workspace(B, D, M)
    if workspace is None:
        workspace = _empty(max(need, 1), torch.uint8, H.device)
    _check_workspace(workspace, H.device, need)
    if de_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("de_dtype must be float32 or bfloat16")
    if out is None:
        dH = _empty((B, D), torch.float32, H.device)
        dE = _empty((M, D), de_dtype, H.device)
    else:
        dH, dE = out
        _check_tensor(dH, "out dH", H.device, torch.float32, (B, D))
        _check_tensor(dE, "out dE", H.device, de_dtype, (M, D))
    args = (_ptr(H), _ptr(E), B, D, M, _ptr(labels), _ptr(weights), _ptr(lse), _ptr(dH), _ptr(dE),
            dtype_code(de_dtype), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream_handle(H.device))
    with _on_device(H.device):
        if profiler is None:
            st = lib().genrec_ce_backward(*args)
        else:
            st = lib().genrec_ce_backward_profiled(*args, profiler.h)
    if st != 0:
        raise GenrecError(st, "genrec_ce_backward")
    return dH, dE


def device_errors(workspace: torch.Tensor) -> tuple[int, int]:
    """(skipped out-of-range ids, users with malformed offsets) of the last candidate call."""
    _check_tensor(workspace, "workspace", workspace.device)
    a, b = ctypes.c_int64(0), ctypes.c_int64(0)
    st = lib().genrec_get_device_errors(_ptr(workspace), _stream_handle(workspace.device),
                                        ctypes.byref(a), ctypes.byref(b))
    if st != 0:
        raise GenrecError(st, "genrec_get_device_errors")
    return a.value, b.value


def rescued_users(workspace: torch.Tensor) -> int:
    """Users of the last full-catalog call on this workspace that needed the rescue pass."""
    _check_tensor(workspace, "workspace", workspace.device)
    n = ctypes.c_int64(0)
    st = lib().genrec_get_rescued_users(_ptr(workspace), _stream_handle(workspace.device), ctypes.byref(n))
    if st != 0:
        raise GenrecError(st, "genrec_get_rescued_users")
    return n.value


def topk_rows(scores: torch.Tensor, K: int, out=None, workspace: torch.Tensor | None = None):
    """Batched top-K of fp32 score rows [R, N] (row stride may exceed N):
    returns (idx int32 [R, K], values f32 [R, K]), score descending, ties by column."""
    if scores.dtype != torch.float32 or not scores.is_cuda or scores.dim() != 2 or scores.stride(1) != 1:
        raise TypeError("scores must be a float32 device tensor [R, N] with unit column stride")
    R, N = scores.shape
    if scores.stride(0) < N:
        raise ValueError("scores rows must not overlap (row stride >= N)")
    if out is None:
        idx = _empty((R, K), torch.int32, scores.device)
        val = _empty((R, K), torch.float32, scores.device)
    else:
        idx, val = out
        _check_tensor(idx, "out idx", scores.device, torch.int32, (R, K))
        _check_tensor(val, "out values", scores.device, torch.float32, (R, K))
    need = int(lib().genrec_topk_rows_workspace(R, N, K))
    if need and workspace is None:
        workspace = _empty(need, torch.uint8, scores.device)
    if workspace is not None:
        _check_workspace(workspace, scores.device, need)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    with _on_device(scores.device):
        st = lib().genrec_topk_rows(_ptr(scores), R, N, scores.stride(0), K, _ptr(idx), _ptr(val),
                                    _ptr(workspace), wsb, _stream_handle(scores.device))
    if st != 0:
        raise GenrecError(st, "genrec_topk_rows")
    return idx, val
