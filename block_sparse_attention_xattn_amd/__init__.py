"""Python binding of libxattn.so (XAttention-style block-sparse prefill attention
on MI355X / gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI
declared in include/xattn.h. PyTorch supplies device memory and the current
stream. If the library is missing the import fails loudly; there is no
fallback.

Functions take contiguous CUDA (HIP) tensors: q (B, Hq, M, C), k and v
(B, Hkv, Mk, C), all bfloat16 or all float32. Mk > M is a chunked prefill (the
queries are the last M of the Mk tokens; Mk - M a multiple of the block), and
neither length needs to be a multiple of the block or the stride.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python block_sparse_attention_xattn_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)

XATTN_BF16 = 0
XATTN_F32 = 1
ABI_VERSION = 5
MAX_HEADS = 256

EXPORTS = (
    "xattn_abi_version", "xattn_status_string", "xattn_last_error", "xattn_workspace_bytes",
    "xattn_score_workspace_bytes", "xattn_select_workspace_bytes", "xattn_attn_workspace_bytes",
    "xattn_prefill_workspace_bytes", "xattn_score", "xattn_select", "bsa_fwd",
    "dense_fwd", "xattn_prefill", "xattn_prefill_noalloc",
)


ANTIDIAGONAL = 0
DIAGONAL = 1
DUSA1 = 2

SELECT_ROW = 0
SELECT_GLOBAL = 1
SELECT_GQA_UNION = 2

# xattn_flags
SELECT_IN_SCORE = 1

_SELECTIONS = {"row": SELECT_ROW, "global": SELECT_GLOBAL, "gqa_union": SELECT_GQA_UNION}


class Problem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "Hq", "Hkv", "M", "C", "block", "stride", "causal", "dtype", "pattern", "selection",
                 "Mk", "flags")]


_P = ctypes.POINTER(Problem)
_vp = ctypes.c_void_p
_f = ctypes.c_float
_lib.xattn_abi_version.restype = ctypes.c_int32
_lib.xattn_status_string.restype = ctypes.c_char_p
_lib.xattn_status_string.argtypes = [ctypes.c_int]
_lib.xattn_last_error.restype = ctypes.c_char_p
_lib.xattn_workspace_bytes.restype = ctypes.c_size_t
_lib.xattn_workspace_bytes.argtypes = [_P]
_lib.xattn_score_workspace_bytes.restype = ctypes.c_size_t
_lib.xattn_score_workspace_bytes.argtypes = [_P]
_lib.xattn_select_workspace_bytes.restype = ctypes.c_size_t
_lib.xattn_select_workspace_bytes.argtypes = [_P]
_lib.xattn_attn_workspace_bytes.restype = ctypes.c_size_t
_lib.xattn_attn_workspace_bytes.argtypes = [_P]
_lib.xattn_prefill_workspace_bytes.restype = ctypes.c_size_t
_lib.xattn_prefill_workspace_bytes.argtypes = [_P]
_lib.xattn_score.restype = ctypes.c_int
_lib.xattn_score.argtypes = [_P, _vp, _vp, _f, _vp, _vp, ctypes.c_size_t, _vp]
_lib.xattn_select.restype = ctypes.c_int
_lib.xattn_select.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.bsa_fwd.restype = ctypes.c_int
_lib.bsa_fwd.argtypes = [_P, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _vp, ctypes.c_size_t, _vp]
_lib.dense_fwd.restype = ctypes.c_int
_lib.dense_fwd.argtypes = [_P, _vp, _vp, _vp, _f, _vp, _vp, _vp]
_lib.xattn_prefill_noalloc.restype = ctypes.c_int
_lib.xattn_prefill_noalloc.argtypes = [_P, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
_lib.xattn_prefill.restype = ctypes.c_int
_lib.xattn_prefill.argtypes = [_P, _vp, _vp, _vp, _vp, _f, _f, _vp, _vp, _vp, _vp, _vp,
                               ctypes.c_size_t, _vp, _vp, _vp]

if _lib.xattn_abi_version() != ABI_VERSION:
    raise ImportError("libxattn.so ABI version mismatch")


class XAttnError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        msg = _lib.xattn_status_string(status).decode()
        detail = _lib.xattn_last_error().decode()
        super().__init__(f"xattn status {status} ({msg}): {detail}")


def _check(status: int):
    if status != 0:
        raise XAttnError(status)


def _selection(sel) -> int:
    return _SELECTIONS[sel] if isinstance(sel, str) else int(sel)


def problem(B, Hq, Hkv, M, C, block, stride, causal, dtype, pattern=ANTIDIAGONAL,
            selection=SELECT_ROW, Mk=0, flags=0) -> Problem:
    """C struct for the given sizes; dtype is torch.bfloat16/torch.float32 or 0/1;
    selection is an xattn_selection value or "row" / "global" / "gqa_union";
    Mk is the key length (0: M; the queries are the last M of Mk tokens);
    flags OR-s xattn_flags (SELECT_IN_SCORE)."""
    if isinstance(dtype, torch.dtype):
        dtype = {torch.bfloat16: XATTN_BF16, torch.float32: XATTN_F32}.get(dtype, 99)
    return Problem(B, Hq, Hkv, M, C, block, stride, int(bool(causal)), dtype, pattern,
                   _selection(selection), Mk, flags)


def _problem_of(q, k, block, stride, causal, pattern=ANTIDIAGONAL, selection=SELECT_ROW, v=None,
                flags=0) -> Problem:
    """Sizes from q (B, Hq, M, C), k (B, Hkv, Mk, C) and, if given, v (k's shape)."""
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q and k must be 4-D (B, H, M, C)")
    B, Hq, M, C = q.shape
    if k.shape[0] != B or k.shape[3] != C:
        raise ValueError(f"k {tuple(k.shape)} does not match q {tuple(q.shape)} in batch or head dim")
    if v is not None and v.shape != k.shape:
        raise ValueError(f"v {tuple(v.shape)} must have k's shape {tuple(k.shape)}")
    return problem(B, Hq, k.shape[1], M, C, block, stride, causal, q.dtype, pattern, selection,
                   Mk=k.shape[2], flags=flags)


def _expect(t, name, shape, dtype, device):
    """Raise unless tensor t (if given) has this shape, dtype and device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} of shape {tuple(shape)}, got {t.dtype} {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _cdiv(a, b):
    return -(-a // b)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on a GPU device")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(dev):
    return torch.cuda.current_stream(dev).cuda_stream


def _same(q, *ts):
    # (that they sit on a GPU is checked when their pointers are taken, after
    # every shape check and before any launch)
    for t in ts:
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share dtype and device")


def _blocks(q, k, block):
    """(B, Hq, NBq, NBk) of the block tensors for q and k."""
    return (q.shape[0], q.shape[1], _cdiv(q.shape[2], block), _cdiv(k.shape[2], block))


def total_workspace_bytes(p: Problem) -> int:
    """Workspace bytes that serve every entry point (xattn_workspace_bytes)."""
    return int(_lib.xattn_workspace_bytes(ctypes.byref(p)))


def workspace_bytes(p: Problem) -> int:
    """Workspace bytes of xattn_score."""
    return int(_lib.xattn_score_workspace_bytes(ctypes.byref(p)))


def select_workspace_bytes(p: Problem) -> int:
    """Workspace bytes of xattn_select."""
    return int(_lib.xattn_select_workspace_bytes(ctypes.byref(p)))


def attn_workspace_bytes(p: Problem) -> int:
    """Workspace bytes of bsa_fwd."""
    return int(_lib.xattn_attn_workspace_bytes(ctypes.byref(p)))


def prefill_workspace_bytes(p: Problem) -> int:
    """Workspace bytes of xattn_prefill."""
    return int(_lib.xattn_prefill_workspace_bytes(ctypes.byref(p)))


def xattn_score(q, k, block, stride, score_scale, causal=True, block_scores=None, ws=None,
                pattern=ANTIDIAGONAL):
    """Block scores (B, Hq, NBq, NBk) float32."""
    _same(q, k)
    p = _problem_of(q, k, block, stride, causal, pattern)
    shp = _blocks(q, k, block)
    _expect(block_scores, "block_scores", shp, torch.float32, q.device)
    if block_scores is None:
        block_scores = torch.empty(shp, dtype=torch.float32, device=q.device)
    need = workspace_bytes(p)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check(_lib.xattn_score(ctypes.byref(p), _ptr(q), _ptr(k), float(score_scale), _ptr(block_scores),
                            _ptr(ws), ws.numel() * ws.element_size(), _stream(q.device)))
    return block_scores


def _tau_host(tau, hq):
    t = torch.as_tensor(tau, dtype=torch.float32).reshape(-1)
    if t.numel() == 1:
        t = t.expand(hq)
    if t.numel() != hq:
        raise ValueError(f"tau must have 1 or Hq={hq} entries")
    return t.cpu().contiguous()


def xattn_select(block_scores, tau, block, stride, causal=True, Hkv=None, C=128, dtype=torch.bfloat16,
                 want_mask=True, mask=None, kv_idx=None, kv_cnt=None, selection=SELECT_ROW):
    """(mask u8 or None, kv_idx int32, kv_cnt int32) for block scores (B, Hq, NBq, NBk);
    NBk > NBq means the queries are the last NBq blocks of the NBk-block sequence."""
    if block_scores.dim() != 4 or block_scores.dtype != torch.float32:
        raise ValueError("block_scores must be float32 (B, Hq, NBq, NBk)")
    B, Hq, nbq, nbk = block_scores.shape
    p = problem(B, Hq, Hkv or Hq, nbq * block, C, block, stride, causal, dtype, selection=selection,
                Mk=nbk * block)
    dev = block_scores.device
    _expect(mask, "mask", (B, Hq, nbq, nbk), torch.uint8, dev)
    _expect(kv_idx, "kv_idx", (B, Hq, nbq, nbk), torch.int32, dev)
    _expect(kv_cnt, "kv_cnt", (B, Hq, nbq), torch.int32, dev)
    if mask is None and want_mask:
        mask = torch.empty((B, Hq, nbq, nbk), dtype=torch.uint8, device=dev)
    if kv_idx is None:
        kv_idx = torch.empty((B, Hq, nbq, nbk), dtype=torch.int32, device=dev)
    if kv_cnt is None:
        kv_cnt = torch.empty((B, Hq, nbq), dtype=torch.int32, device=dev)
    tau_h = _tau_host(tau, Hq)
    need = select_workspace_bytes(p)
    ws = torch.empty(need, dtype=torch.uint8, device=dev) if need else None
    _check(_lib.xattn_select(ctypes.byref(p), _ptr(block_scores), tau_h.data_ptr(), _ptr(mask),
                             _ptr(kv_idx), _ptr(kv_cnt), _ptr(ws), need, _stream(dev)))
    return mask, kv_idx, kv_cnt


def bsa_fwd(q, k, v, kv_idx, kv_cnt, block, sm_scale, causal=True, out=None, want_lse=False, ws=None,
            selection=SELECT_ROW):
    """Block-sparse attention: (out, lse or None). selection=SELECT_GQA_UNION
    declares lists shared by sibling heads (any lists stay correct)."""
    _same(q, k, v)
    p = _problem_of(q, k, block, 0, causal, selection=selection, v=v)
    B, Hq, nbq, nbk = _blocks(q, k, block)
    _expect(kv_idx, "kv_idx", (B, Hq, nbq, nbk), torch.int32, q.device)
    _expect(kv_cnt, "kv_cnt", (B, Hq, nbq), torch.int32, q.device)
    _expect(out, "out", q.shape, q.dtype, q.device)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    if ws is None:
        ws = torch.empty(max(attn_workspace_bytes(p), 4), dtype=torch.uint8, device=q.device)
    _check(_lib.bsa_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(kv_idx), _ptr(kv_cnt),
                        float(sm_scale), _ptr(out), _ptr(lse), _ptr(ws), ws.numel() * ws.element_size(),
                        _stream(q.device)))
    return out, lse


def dense_fwd(q, k, v, block, sm_scale, causal=True, out=None, want_lse=False):
    """Dense attention (every candidate block): (out, lse or None)."""
    _same(q, k, v)
    p = _problem_of(q, k, block, 0, causal, v=v)
    _expect(out, "out", q.shape, q.dtype, q.device)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device) if want_lse else None
    _check(_lib.dense_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), float(sm_scale), _ptr(out),
                          _ptr(lse), _stream(q.device)))
    return out, lse


class PrefillBuffers:
    """Reusable device buffers for xattn_prefill (allocated once per shape).

    ``key`` records what the buffers were sized for; xattn_prefill refuses
    inputs or arguments that differ from it. want_scores=False leaves the block
    scores unwritten (not allowed with global selection). select_in_score asks
    for normalisation and selection inside the scoring launch
    (XATTN_SELECT_IN_SCORE)."""

    def __init__(self, q, k, block, stride, causal=True, want_mask=True, want_lse=False,
                 pattern=ANTIDIAGONAL, selection=SELECT_ROW, want_scores=True, want_ws=True,
                 select_in_score=False):
        p = _problem_of(q, k, block, stride, causal, pattern, selection,
                        flags=SELECT_IN_SCORE if select_in_score else 0)
        B, Hq, M, C = q.shape
        nbq, nbk = _cdiv(M, block), _cdiv(k.shape[2], block)
        dev = q.device
        self.problem = p
        self.key = _prefill_key(q, k, block, stride, causal, pattern, selection, select_in_score)
        self.block_scores = (torch.empty((B, Hq, nbq, nbk), dtype=torch.float32, device=dev)
                             if want_scores else None)
        self.mask = torch.empty((B, Hq, nbq, nbk), dtype=torch.uint8, device=dev) if want_mask else None
        self.kv_idx = torch.empty((B, Hq, nbq, nbk), dtype=torch.int32, device=dev)
        self.kv_cnt = torch.empty((B, Hq, nbq), dtype=torch.int32, device=dev)
        self.ws = (torch.empty(max(total_workspace_bytes(p), 4), dtype=torch.uint8, device=dev)
                   if want_ws else None)
        self.out = torch.empty_like(q)
        self.lse = torch.empty((B, Hq, M), dtype=torch.float32, device=dev) if want_lse else None


def _prefill_key(q, k, block, stride, causal, pattern, selection, select_in_score=False):
    return (tuple(q.shape), tuple(k.shape), q.dtype, str(q.device), int(block), int(stride),
            bool(causal), int(pattern), _selection(selection), bool(select_in_score))


def xattn_prefill(q, k, v, tau, block, stride, score_scale, sm_scale, causal=True, buffers=None,
                  pattern=ANTIDIAGONAL, selection=SELECT_ROW, want_scores=True, select_in_score=False):
    """All three stages in one call. Returns the PrefillBuffers holding the results
    (block_scores is None when want_scores is False). select_in_score: normalise
    and select inside the scoring launch (same results, one launch fewer; slower
    on MI355X, see XATTN_SELECT_IN_SCORE)."""
    _same(q, k, v)
    _problem_of(q, k, block, stride, causal, pattern, selection, v=v)
    key = _prefill_key(q, k, block, stride, causal, pattern, selection, select_in_score)
    if buffers is not None and buffers.key != key:
        raise ValueError(f"buffers were made for other inputs or arguments: {buffers.key} != {key}")
    bufs = buffers or PrefillBuffers(q, k, block, stride, causal, pattern=pattern, selection=selection,
                                     want_scores=want_scores, select_in_score=select_in_score)
    tau_h = _tau_host(tau, q.shape[1])
    b = bufs
    _check(_lib.xattn_prefill(ctypes.byref(b.problem), _ptr(q), _ptr(k), _ptr(v), tau_h.data_ptr(),
                              float(score_scale), float(sm_scale), _ptr(b.block_scores), _ptr(b.mask),
                              _ptr(b.kv_idx), _ptr(b.kv_cnt), _ptr(b.ws),
                              b.ws.numel(), _ptr(b.out), _ptr(b.lse), _stream(q.device)))
    return b


NOALLOC_SCRATCH_BYTES = 64 << 20


def xattn_prefill_noalloc(q, k, v, tau, block, stride, score_scale, sm_scale, causal=True, buffers=None,
                          pattern=ANTIDIAGONAL, selection=SELECT_ROW, want_scores=True, select_in_score=False):
    """xattn_prefill on the library's own per-GPU scratch (no workspace), for
    callers that cannot allocate device memory. Pass ``buffers`` (a
    PrefillBuffers, e.g. made with want_ws=False) to allocate nothing here
    either. Calls that overlap on one GPU share the scratch and race."""
    _same(q, k, v)
    _problem_of(q, k, block, stride, causal, pattern, selection, v=v)
    if buffers is not None and buffers.key != _prefill_key(q, k, block, stride, causal, pattern, selection,
                                                          select_in_score):
        raise ValueError("buffers were made for other inputs or arguments")
    bufs = buffers or PrefillBuffers(q, k, block, stride, causal, pattern=pattern, selection=selection,
                                     want_scores=want_scores, want_ws=False, select_in_score=select_in_score)
    tau_h = _tau_host(tau, q.shape[1])
    b = bufs
    _check(_lib.xattn_prefill_noalloc(ctypes.byref(b.problem), _ptr(q), _ptr(k), _ptr(v), tau_h.data_ptr(),
                                      float(score_scale), float(sm_scale), _ptr(b.block_scores), _ptr(b.mask),
                                      _ptr(b.kv_idx), _ptr(b.kv_cnt), _ptr(b.out), _ptr(b.lse),
                                      _stream(q.device)))
    return b


# The pages' names for the stages, as aliases.
score = xattn_score
select = xattn_select
prefill = xattn_prefill
