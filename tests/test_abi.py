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
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
    return sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))


def test_every_declared_symbol_is_exported(xa):
    names = _declared()
    # the boundary's calls: workspace size, the three stages, the dense
    # baseline, the fused prefill and the housekeeping queries
    assert {"xattn_workspace_bytes", "xattn_score", "xattn_select", "bsa_fwd", "dense_fwd", "xattn_prefill",
            "xattn_status_string", "xattn_abi_version"} <= set(names)
    for n in names:
        assert hasattr(xa._lib, n), n
    assert set(xa.EXPORTS) == set(names)


def test_version_and_strings(xa):
    assert xa._lib.xattn_abi_version() == 5
    for s in range(8):
        assert xa._lib.xattn_status_string(s)
    assert xa._lib.xattn_status_string(99) == b"unknown status"


def _p(xa, **kw):
    base = dict(B=1, Hq=4, Hkv=2, M=1024, C=128, block=128, stride=8, causal=1, dtype=0, pattern=0,
                selection=0, Mk=0, flags=0)
    base.update(kw)
    return xa.Problem(*[base[k] for k in ("B", "Hq", "Hkv", "M", "C", "block", "stride", "causal", "dtype",
                                          "pattern", "selection", "Mk", "flags")])


FAKE = 0x1000  # never dereferenced: validation fails first


@pytest.mark.parametrize("kw,status", [
    (dict(Hkv=3), 2), (dict(Mk=1000), 2), (dict(Mk=1100), 2), (dict(stride=3), 2), (dict(C=96), 5),
    (dict(block=32, stride=4), 5), (dict(stride=128), 5), (dict(stride=1), 5),
    (dict(dtype=7), 3), (dict(causal=2), 4), (dict(Hq=512, Hkv=1), 5), (dict(B=0), 2),
    (dict(M=4096 * 128 * 2), 5), (dict(pattern=3), 4), (dict(pattern=-1), 4),
    # DuSA1 scoring: bf16 only, lengths multiples of the stride
    (dict(pattern=2, dtype=1), 5), (dict(pattern=2, M=1004), 2), (dict(pattern=2, M=1024, Mk=1540), 2),
    (dict(selection=3), 4), (dict(selection=-1), 4), (dict(Mk=4096 * 128 + 128), 5),
    # only xattn_flags bits
    (dict(flags=2), 4), (dict(flags=-1), 4),
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
    # selection inside the scoring launch adds one arrival counter per
    # (b, h, 256-row query tile) before the queues, where it applies
    assert xa.prefill_workspace_bytes(_p(xa, flags=1)) == 1 * 4 * 8 * 128 * 4 + 256 + 1024
    assert xa.prefill_workspace_bytes(_p(xa, flags=1, M=1004)) == xa.prefill_workspace_bytes(_p(xa, M=1004))
    assert xa.prefill_workspace_bytes(_p(xa, flags=1, dtype=1)) == xa.prefill_workspace_bytes(_p(xa, dtype=1))
    assert xa.prefill_workspace_bytes(_p(xa, flags=1, selection=1)) == xa.prefill_workspace_bytes(g := _p(xa, selection=1))
    assert xa.prefill_workspace_bytes(_p(xa, flags=1, B=2, Hq=8, M=8192)) == \
        xa.prefill_workspace_bytes(_p(xa, B=2, Hq=8, M=8192)) + 256
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


def test_one_workspace_size_serves_every_entry_point(xa):
    for kw in (dict(), dict(selection=1), dict(selection=2), dict(M=1000, Mk=1256), dict(stride=16),
               dict(dtype=1, M=512)):
        p = _p(xa, **kw)
        total = xa.total_workspace_bytes(p)
        assert total == xa.prefill_workspace_bytes(p) > 0
        assert total >= max(xa.workspace_bytes(p), xa.select_workspace_bytes(p), xa.attn_workspace_bytes(p))
    assert xa.total_workspace_bytes(_p(xa, Hkv=3)) == 0


def test_f32_envelope(xa):
    # the scalar fp32 kernels take at most 16384 key tokens; bf16 has no such limit
    L = xa._lib
    ok = _p(xa, dtype=1, M=16384)
    big = _p(xa, dtype=1, M=16384 + 128)
    chunk = _p(xa, dtype=1, M=128, Mk=16384 + 128)
    assert xa.workspace_bytes(ok) > 0
    for p in (big, chunk):
        assert xa.workspace_bytes(p) == 0
        assert L.xattn_score(ctypes.byref(p), FAKE, FAKE, 0.01, FAKE, FAKE, 1 << 40, None) == 5
        assert L.dense_fwd(ctypes.byref(p), FAKE, FAKE, FAKE, 0.1, FAKE, None, None) == 5
        assert b"16384" in L.xattn_last_error()
    assert xa.workspace_bytes(_p(xa, dtype=0, M=16384 + 128)) > 0


def test_prefill_block_scores_optional_except_global(xa):
    L = xa._lib
    arr = (ctypes.c_float * 4)(0.9, 0.9, 0.9, 0.9)
    g = _p(xa, selection=1)
    need = xa.total_workspace_bytes(g)
    assert L.xattn_prefill(ctypes.byref(g), FAKE, FAKE, FAKE, arr, 0.01, 0.1, None, None, FAKE, FAKE,
                           FAKE, need, FAKE, None, None) == 1
    assert b"global" in L.xattn_last_error()
    # per-row selection: a NULL block_scores passes validation (the workspace
    # check, which comes later, is what fails here)
    p = _p(xa)
    assert L.xattn_prefill(ctypes.byref(p), FAKE, FAKE, FAKE, arr, 0.01, 0.1, None, None, FAKE, FAKE,
                           FAKE, 16, FAKE, None, None) == 6


# ---------------------------------------------------------------- the binding's own checks
# Shapes, dtypes and devices are checked in Python before any pointer is taken
# or any launch is made; CPU tensors reach the device check last.

def _t(*shape, dtype=None):
    import torch
    return torch.zeros(shape, dtype=dtype or torch.bfloat16)


def test_binding_rejects_mismatched_tensors_before_launch(xa):
    import torch
    q, k, v = _t(1, 4, 256, 128), _t(1, 2, 256, 128), _t(1, 2, 256, 128)
    i32, f32, u8 = torch.int32, torch.float32, torch.uint8
    with pytest.raises(ValueError, match="v "):
        xa.bsa_fwd(q, k, _t(1, 2, 255, 128), _t(1, 4, 2, 2, dtype=i32), _t(1, 4, 2, dtype=i32), 128, 0.1)
    with pytest.raises(ValueError, match="v "):
        xa.dense_fwd(q, k, _t(1, 1, 256, 128), 128, 0.1)
    with pytest.raises(ValueError, match="kv_idx"):
        xa.bsa_fwd(q, k, v, _t(1, 4, 2, 3, dtype=i32), _t(1, 4, 2, dtype=i32), 128, 0.1)
    with pytest.raises(ValueError, match="kv_idx"):
        xa.bsa_fwd(q, k, v, _t(1, 4, 2, 2, dtype=torch.int64), _t(1, 4, 2, dtype=i32), 128, 0.1)
    with pytest.raises(ValueError, match="kv_cnt"):
        xa.bsa_fwd(q, k, v, _t(1, 4, 2, 2, dtype=i32), _t(1, 4, 3, dtype=i32), 128, 0.1)
    with pytest.raises(ValueError, match="out"):
        xa.bsa_fwd(q, k, v, _t(1, 4, 2, 2, dtype=i32), _t(1, 4, 2, dtype=i32), 128, 0.1,
                   out=_t(1, 4, 256, 64))
    with pytest.raises(ValueError, match="k "):
        xa.xattn_score(q, _t(1, 2, 256, 64), 128, 8, 0.01)
    with pytest.raises(ValueError, match="block_scores"):
        xa.xattn_score(q, k, 128, 8, 0.01, block_scores=_t(1, 4, 2, 2, dtype=torch.float64))
    with pytest.raises(ValueError, match="block_scores"):
        xa.xattn_select(_t(1, 4, 2, 2), [0.9], 128, 8)
    with pytest.raises(ValueError, match="kv_cnt"):
        xa.xattn_select(_t(1, 4, 2, 2, dtype=f32), [0.9], 128, 8, kv_cnt=_t(1, 4, 2, dtype=torch.int16))
    with pytest.raises(ValueError, match="mask"):
        xa.xattn_select(_t(1, 4, 2, 2, dtype=f32), [0.9], 128, 8, mask=_t(1, 4, 2, 2, dtype=torch.bool))
    with pytest.raises(ValueError, match="dtype"):
        xa.dense_fwd(q, k.float(), v, 128, 0.1)
    # well-formed CPU tensors reach the device check, still before any launch
    with pytest.raises(ValueError, match="GPU"):
        xa.dense_fwd(q, k, v, 128, 0.1)
    with pytest.raises(ValueError, match="GPU"):
        xa.bsa_fwd(q, k, v, _t(1, 4, 2, 2, dtype=i32), _t(1, 4, 2, dtype=i32), 128, 0.1)
    del u8


def test_prefill_buffers_refuse_other_inputs(xa):
    q, k, v = _t(1, 4, 256, 128), _t(1, 2, 256, 128), _t(1, 2, 256, 128)
    bufs = xa.PrefillBuffers(q, k, 128, 8, True)
    assert bufs.key[0] == (1, 4, 256, 128)
    q2, k2, v2 = _t(1, 4, 384, 128), _t(1, 2, 384, 128), _t(1, 2, 384, 128)
    with pytest.raises(ValueError, match="buffers"):
        xa.xattn_prefill(q2, k2, v2, 0.9, 128, 8, 0.01, 0.1, True, buffers=bufs)
    for kw in (dict(stride=16), dict(causal=False), dict(selection="global"), dict(pattern=1)):
        args = dict(stride=8, causal=True)
        args.update({x: y for x, y in kw.items() if x in args})
        extra = {x: y for x, y in kw.items() if x not in args}
        with pytest.raises(ValueError, match="buffers"):
            xa.xattn_prefill(q, k, v, 0.9, 128, args["stride"], 0.01, 0.1, args["causal"], buffers=bufs,
                             **extra)
    with pytest.raises(ValueError, match="v "):
        xa.xattn_prefill(q, k, _t(1, 2, 128, 128), 0.9, 128, 8, 0.01, 0.1, True, buffers=bufs)
    with pytest.raises(ValueError, match="GPU"):
        xa.xattn_prefill(q, k, v, 0.9, 128, 8, 0.01, 0.1, True, buffers=bufs)
    nos = xa.PrefillBuffers(q, k, 128, 8, True, want_scores=False)
    assert nos.block_scores is None


def test_noalloc_rejects_oversized_problems_on_the_host(xa):
    # 32 heads at 32K tokens need 128 MiB of scratch, past the 64 MiB the
    # no-allocation entry point holds: refused before the device is touched
    L = xa._lib
    arr = (ctypes.c_float * 32)(*([0.9] * 32))
    p = _p(xa, Hq=32, Hkv=8, M=32768)
    assert xa.total_workspace_bytes(p) > xa.NOALLOC_SCRATCH_BYTES == 64 << 20
    rc = L.xattn_prefill_noalloc(ctypes.byref(p), FAKE, FAKE, FAKE, arr, 0.01, 0.1, FAKE, None, FAKE, FAKE,
                                 FAKE, None, None)
    assert rc == 6
    assert b"scratch" in L.xattn_last_error()
    assert L.xattn_prefill_noalloc(ctypes.byref(_p(xa, C=96)), FAKE, FAKE, FAKE, arr, 0.01, 0.1, FAKE, None,
                                   FAKE, FAKE, FAKE, None, None) == 5


def test_peaks_library_exports_its_header():
    # the peak-rate microbenchmarks live in a library of their own
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_xattn_amd", "libxattn_peaks.so"))
    text = open(os.path.join(ROOT, "include", "xattn_peaks.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)
    names = sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))
    assert names == ["xattn_peak_copy", "xattn_peak_mfma", "xattn_peak_mfma_waves_per_block"]
    for n in names:
        assert hasattr(lib, n), n
    assert lib.xattn_peak_mfma_waves_per_block() == 8
    # bad arguments are refused on the host (hipErrorInvalidValue), nothing launched
    lib.xattn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    assert lib.xattn_peak_copy(None, None, 16, None) != 0
    assert lib.xattn_peak_copy(FAKE, FAKE, 15, None) != 0
    lib.xattn_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    assert lib.xattn_peak_mfma(0, 10, FAKE, None, None) != 0


def test_dusa1_workspace(xa):
    # per (phase, strided row) log-sum-exps (B*Hq*M floats, 256-byte aligned),
    # then room for the block scores; the attention workspace follows in prefill
    p = _p(xa, pattern=2)
    lse = 1 * 4 * 1024 * 4
    assert xa.workspace_bytes(p) == (lse + 255) // 256 * 256 + 1 * 4 * 8 * 8 * 4
    assert xa.total_workspace_bytes(p) == (xa.workspace_bytes(p) + 255) // 256 * 256 + 1024


def test_validation_layer_under_address_sanitizer():
    # api.hip's host code and a driver of every refused path, built with
    # AddressSanitizer on the host side (device code unchanged); no GPU needed
    import importlib.util
    import shutil
    import subprocess
    if not shutil.which(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")):
        pytest.skip("hipcc not available")
    spec = importlib.util.spec_from_file_location(
        "_xattn_build", os.path.join(ROOT, "block_sparse_attention_xattn_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build_asan_check()
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0")
    res = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all validation paths refused as expected" in res.stdout
    assert "AddressSanitizer" not in res.stderr


def test_debug_library_exports_its_header():
    # the debug build exports one more entry point, declared in xattn_debug.h;
    # the release library does not
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_xattn_amd", "libxattn_debug.so"))
    text = open(os.path.join(ROOT, "include", "xattn_debug.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)
    names = sorted(set(re.findall(r"\b(\w+)\s*\([^;{]*\)\s*;", text)))
    assert names == ["xattn_debug_violations"]
    assert hasattr(lib, "xattn_debug_violations")
    for n in _declared():
        assert hasattr(lib, n), n
    import block_sparse_attention_xattn_amd as xa
    assert not hasattr(xa._lib, "xattn_debug_violations")
    lib.xattn_debug_violations.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32]
    assert lib.xattn_debug_violations(None, 8, 0) == 4
