"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before anything is enqueued
(no device pointer is touched on these paths)."""
import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xattn.h")


@pytest.fixture(scope="module")
def xa():
    import block_sparse_attention_xattn_amd as x
    return x


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))


def test_every_declared_symbol_is_exported(xa):
    names = _declared()
    assert {"xattn_score", "xattn_select", "bsa_fwd", "dense_fwd", "xattn_prefill"} <= set(names)
    for n in names:
        assert hasattr(xa._lib, n), n
    assert set(xa.EXPORTS) == set(names)


def test_version_and_strings(xa):
    assert xa._lib.xattn_abi_version() == 3
    for s in range(8):
        assert xa._lib.xattn_status_string(s)
    assert xa._lib.xattn_status_string(99) == b"unknown status"


def _p(xa, **kw):
    base = dict(B=1, Hq=4, Hkv=2, M=1024, C=128, block=128, stride=8, causal=1, dtype=0, pattern=0,
                selection=0, Mk=0)
    base.update(kw)
    return xa.Problem(*[base[k] for k in ("B", "Hq", "Hkv", "M", "C", "block", "stride", "causal", "dtype",
                                          "pattern", "selection", "Mk")])


FAKE = 0x1000  # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), 2), (dict(Mk=1000), 2), (dict(Mk=1100), 2), (dict(stride=3), 2), (dict(C=96), 5),
    (dict(block=32, stride=4), 5), (dict(stride=128), 5), (dict(stride=1), 5),
    (dict(dtype=7), 3), (dict(causal=2), 4), (dict(Hq=512, Hkv=1), 5), (dict(B=0), 2),
    (dict(M=4096 * 128 * 2), 5), (dict(pattern=2), 4), (dict(pattern=-1), 4),
    (dict(selection=3), 4), (dict(selection=-1), 4), (dict(Mk=4096 * 128 + 128), 5),
    # empty problems are errors, not silent no-ops
    (dict(M=0), 2), (dict(Hq=0), 2), (dict(Hkv=0), 2), (dict(C=0), 2), (dict(block=0), 2),
    (dict(stride=0), 2), (dict(M=-5), 2),
])
def test_score_rejects_bad_problems(xa, kw, status):
    p = _p(xa, **kw)
    rc = xa._lib.xattn_score(ctypes.byref(p), FAKE, FAKE, 0.01, FAKE, FAKE, 1 << 40, None)
    assert rc == status, xa._lib.xattn_last_error()
    assert xa._lib.xattn_last_error()


def test_ragged_and_chunked_problems_validate(xa):
    # lengths off the block and stride grid, and queries that are the last M of
    # Mk tokens, are valid; the workspace follows NBq x NBk
    for kw, nbq, nbk in ((dict(M=1000), 8, 8), (dict(M=1000, Mk=1256), 8, 10),
                         (dict(M=1, Mk=129), 1, 2), (dict(M=128, Mk=4096 * 128), 1, 4096)):
        p = _p(xa, **kw)
        assert xa.workspace_bytes(p) == 4 * nbq * nbk * 16 * 4, kw
        assert xa.attn_workspace_bytes(p) == 1024


def test_workspace_bytes(xa):
    p = _p(xa)
    assert xa.workspace_bytes(p) == 1 * 4 * 8 * 128 * 4
    assert xa.workspace_bytes(_p(xa, Hkv=3)) == 0
    assert xa.attn_workspace_bytes(p) == 1024
    assert xa.attn_workspace_bytes(_p(xa, Hkv=3)) == 0
    # attention ignores the stride
    assert xa.attn_workspace_bytes(_p(xa, stride=0)) == 1024
    # score partials, then the queues at the next 256-byte boundary
    assert xa.prefill_workspace_bytes(p) == 1 * 4 * 8 * 128 * 4 + 1024
    odd = _p(xa, B=1, Hq=1, Hkv=1, M=192, block=64, stride=32, C=64)   # 3 * 6 * 4 = 72 bytes
    assert xa.workspace_bytes(odd) == 72
    assert xa.prefill_workspace_bytes(odd) == 256 + 1024
    assert xa.prefill_workspace_bytes(_p(xa, stride=0)) == 0
    # selection scratch: none per row or for the GQA union; per head a 64-byte
    # state, a 4096-bucket histogram (8 + 4 bytes each) and NB words for global
    assert xa.select_workspace_bytes(p) == 0
    assert xa.select_workspace_bytes(_p(xa, selection=2)) == 0
    g = _p(xa, selection=1)
    assert xa.select_workspace_bytes(g) == 4 * (64 + 4096 * 12 + 4 * 8)
    sel_end = 16384 + 4 * (64 + 4096 * 12 + 4 * 8)
    assert xa.prefill_workspace_bytes(g) == (sel_end + 255) // 256 * 256 + 1024


def test_null_and_workspace_errors(xa):
    p = _p(xa)
    L = xa._lib
    assert L.xattn_score(None, FAKE, FAKE, 0.01, FAKE, FAKE, 1 << 40, None) == 1
    assert L.xattn_score(ctypes.byref(p), None, FAKE, 0.01, FAKE, FAKE, 1 << 40, None) == 1
    assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, 0.01, FAKE, FAKE, 16, None) == 6
    assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, 0.01, FAKE, None, 1 << 40, None) == 6
    assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, -1.0, FAKE, FAKE, 1 << 40, None) == 4
    assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, math.inf, FAKE, FAKE, 1 << 40, None) == 4
    assert L.bsa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, None, FAKE, 0.1, FAKE, None, FAKE, 1024, None) == 1
    assert L.bsa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.0, FAKE, None, FAKE, 1024, None) == 4
    assert L.bsa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, None, 1024, None) == 6
    assert L.bsa_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 0.1, FAKE, None, FAKE, 1023, None) == 6
    assert L.dense_fwd(ctypes.byref(p), FAKE, FAKE, None, 0.1, FAKE, None, None) == 1
    assert L.dense_fwd(ctypes.byref(_p(xa, C=32)), FAKE, FAKE, FAKE, 0.1, FAKE, None, None) == 5


def test_select_rejects_bad_tau(xa):
    p = _p(xa)
    L = xa._lib
    for bad in ([0.9, 0.9, 1.5, 0.9], [0.9, -0.1, 0.9, 0.9], [0.9, 0.9, 0.9, float("nan")]):
        arr = (ctypes.c_float * 4)(*bad)
        assert L.xattn_select(ctypes.byref(p), FAKE, arr, None, FAKE, FAKE, None, 0, None) == 4
    arr = (ctypes.c_float * 4)(0.9, 0.9, 0.9, 0.9)
    assert L.xattn_select(ctypes.byref(p), FAKE, None, None, FAKE, FAKE, None, 0, None) == 1
    assert L.xattn_select(ctypes.byref(p), None, arr, None, FAKE, FAKE, None, 0, None) == 1
    # global selection needs its scratch
    g = _p(xa, selection=1)
    need = xa.select_workspace_bytes(g)
    assert L.xattn_select(ctypes.byref(g), FAKE, arr, None, FAKE, FAKE, None, 0, None) == 6
    assert L.xattn_select(ctypes.byref(g), FAKE, arr, None, FAKE, FAKE, FAKE, need - 1, None) == 6
    assert L.xattn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, arr, 0.01, 0.1, FAKE, None, FAKE, FAKE,
                           FAKE, 16, FAKE, None, None) == 6
    # the score partials alone are too little: the attention queues follow them
    assert L.xattn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, arr, 0.01, 0.1, FAKE, None, FAKE, FAKE,
                           FAKE, xa.workspace_bytes(p), FAKE, None, None) == 6


def test_attention_ignores_stride(xa):
    # stride is a scoring parameter; attention validates without it
    p = _p(xa, stride=0)
    L = xa._lib
    assert L.dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, 0.0, FAKE, None, None) == 4
    assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, 0.01, FAKE, FAKE, 1 << 40, None) == 2
