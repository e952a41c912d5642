"""The debug build (libxattn_debug.so, -DXATTN_DEBUG=1): the kernels' bounds
checks at every indexing site stay at zero failures over layers that reach each
kernel and mode (per-row, global and GQA-union selection, selection inside the
scoring launch; antidiagonal and DuSA1 scoring; single, sibling and row-pair attention; ragged and chunked
lengths; dense attention), and the debug build's outputs equal the release
build's bitwise (the checks only count, they change no value)."""
import ctypes
import os

import pytest
import torch

import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEBUG_LIB = os.path.join(ROOT, "block_sparse_attention_xattn_amd", "libxattn_debug.so")
CATEGORIES = ["score store", "selection state", "K/V rows", "LDS slot / list entry", "work item", "DuSA1 index",
              "unused", "unused"]


@pytest.fixture(scope="module")
def libs():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(DEBUG_LIB):
        pytest.fail(f"{DEBUG_LIB} is missing: build with block_sparse_attention_xattn_amd/build.py")
    import block_sparse_attention_xattn_amd as xa
    dbg = ctypes.CDLL(DEBUG_LIB)
    vp, f = ctypes.c_void_p, ctypes.c_float
    P = ctypes.POINTER(xa.Problem)
    dbg.xattn_prefill.restype = ctypes.c_int
    dbg.xattn_prefill.argtypes = [P, vp, vp, vp, vp, f, f, vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp]
    dbg.dense_fwd.restype = ctypes.c_int
    dbg.dense_fwd.argtypes = [P, vp, vp, vp, f, vp, vp, vp]
    dbg.xattn_debug_violations.restype = ctypes.c_int
    dbg.xattn_debug_violations.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32, ctypes.c_int32]
    return xa, dbg


def _violations(dbg, reset=True):
    out = (ctypes.c_uint32 * 8)()
    assert dbg.xattn_debug_violations(out, 8, int(reset)) == 0
    return list(out)


CASES = [
    # name, workload overrides, prefill keywords
    ("llama32k-rows", dict(M=4096, Hq=8, Hkv=2), {}),
    ("llama128k-pairs", dict(M=131072, Hq=2, Hkv=1), {}),
    ("video-nc-pairs", dict(M=76800, Hq=1, Hkv=1), {}),
    ("llama8k-global", dict(M=4096, Hq=4, Hkv=2), dict(selection="global")),
    ("llama8k-gqa-union", dict(M=4096, Hq=4, Hkv=2), dict(selection="gqa_union")),
    ("llama32k-dusa1", dict(M=4096, Hq=4, Hkv=1), dict(pattern=2)),
    ("llama32k-select-in-score", dict(M=4096, Hq=8, Hkv=2), dict(select_in_score=True)),
    ("ragged-3000", dict(M=3000, Hq=4, Hkv=2), {}),
]


@pytest.mark.parametrize("name,over,kw", CASES, ids=[c[0] for c in CASES])
def test_debug_build_checks_clean_and_bitwise_equal(libs, name, over, kw):
    xa, dbg = libs
    base = "video" if name.startswith("video") else ("llama128k" if "128k" in name else "llama32k")
    w = wl.WORKLOADS[base].scaled(**over)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    if kw.get("pattern") == 2:
        sscale = smscale
    print(f"[debug] {name}: M={w.M} Hq={w.Hq} Hkv={w.Hkv} {kw}", flush=True)
    ref = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal, **kw)
    bufs = xa.PrefillBuffers(x["q"], x["k"], w.block, w.stride, w.causal, **kw)
    tau = torch.as_tensor(x["tau"], dtype=torch.float32).cpu().contiguous()
    _violations(dbg)  # start from zero
    rc = dbg.xattn_prefill(ctypes.byref(bufs.problem), x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                           tau.data_ptr(), sscale, smscale, bufs.block_scores.data_ptr(), bufs.mask.data_ptr(),
                           bufs.kv_idx.data_ptr(), bufs.kv_cnt.data_ptr(), bufs.ws.data_ptr(), bufs.ws.numel(),
                           bufs.out.data_ptr(), None, torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    dense_ref = dense_dbg = None
    if not kw:
        dense_ref, _ = xa.dense_fwd(x["q"], x["k"], x["v"], w.block, smscale, w.causal)
        dense_dbg = torch.empty_like(x["q"])
        assert dbg.dense_fwd(ctypes.byref(bufs.problem), x["q"].data_ptr(), x["k"].data_ptr(), x["v"].data_ptr(),
                             smscale, dense_dbg.data_ptr(), None, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    v = _violations(dbg)
    print(f"[debug] {name}: failed checks per category {dict(zip(CATEGORIES, v))}", flush=True)
    assert sum(v) == 0, dict(zip(CATEGORIES, v))
    assert torch.equal(ref.block_scores, bufs.block_scores)
    assert torch.equal(ref.mask, bufs.mask)
    assert torch.equal(ref.kv_cnt, bufs.kv_cnt)
    valid = torch.arange(ref.kv_idx.shape[-1], device=DEV) < ref.kv_cnt[..., None]
    assert torch.equal(ref.kv_idx[valid], bufs.kv_idx[valid])
    assert torch.equal(ref.out, bufs.out)
    if dense_ref is not None:
        assert torch.equal(dense_ref, dense_dbg)
