"""xattn_prefill_noalloc, the entry point for callers that cannot allocate:
through the C ABI it must give what xattn_prefill gives on a caller
workspace, call after call on its shared per-GPU scratch (the second call
smaller than the first, so stale scratch contents from the first are present),
and refuse problems whose scratch need exceeds its fixed size."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check_index, check_mask, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _same_results(ref, got):
    assert torch.equal(ref.block_scores, got.block_scores)
    assert torch.equal(ref.mask, got.mask)
    assert torch.equal(ref.kv_cnt, got.kv_cnt)
    valid = torch.arange(ref.kv_idx.shape[-1], device=DEV) < ref.kv_cnt[..., None]
    assert torch.equal(ref.kv_idx[valid], got.kv_idx[valid])
    assert torch.equal(ref.out, got.out)


@pytest.mark.parametrize("selection", ["row", "global"])
def test_noalloc_equals_prefill_on_two_calls(xa, selection):
    layers = [wl.WORKLOADS["llama8k"].scaled(M=8192, Hq=8, Hkv=2),     # 8 MiB of scratch... then
              wl.WORKLOADS["llama32k"].scaled(M=2048, Hq=4, Hkv=1)]    # a smaller layer on stale scratch
    for w in layers:
        print(f"[noalloc] {selection} M={w.M} Hq={w.Hq} S={w.stride}", flush=True)
        x = wl.make_inputs(w, device=DEV)
        sscale, smscale = wl.default_scales(w)
        args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
        p = xa.problem(w.B, w.Hq, w.Hkv, w.M, w.C, w.block, w.stride, w.causal, x["q"].dtype,
                       selection=selection)
        assert 0 < xa.total_workspace_bytes(p) <= xa.NOALLOC_SCRATCH_BYTES
        ref = xa.xattn_prefill(*args, selection=selection)
        bufs = xa.PrefillBuffers(x["q"], x["k"], w.block, w.stride, w.causal, selection=selection, want_ws=False)
        assert bufs.ws is None
        got = xa.xattn_prefill_noalloc(*args, selection=selection, buffers=bufs)
        torch.cuda.synchronize()
        _same_results(ref, got)
        # and against the oracle: selection on the GPU's scores, attention with the GPU's mask
        g_sc = f64(got.block_scores)
        tau = x["tau"].numpy().astype(np.float64)
        m = got.mask.cpu().numpy()
        if selection == "row":
            check_mask(f"noalloc M={w.M}", m, oracle.select(g_sc, tau, w.causal), g_sc, tau, w.causal, 1e-5)
        check_index(m, got.kv_idx.cpu().numpy(), got.kv_cnt.cpu().numpy())
        q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
        ref_out, _ = oracle.attend(q, k, v, m, w.block, smscale, w.causal, heads=[0, w.Hq - 1])
        err = max(np.abs(f64(got.out[:, h]) - ref_out[:, h]).max() for h in (0, w.Hq - 1))
        assert err <= 2e-2, err
        del x, ref, got, bufs


def test_noalloc_without_block_scores_and_repeat(xa):
    # the optional block-score output, then the same call again: bitwise equal
    w = wl.WORKLOADS["video"].scaled(M=2560, Hq=2, Hkv=2)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    ref = xa.xattn_prefill(*args)
    a = xa.xattn_prefill_noalloc(*args, want_scores=False)
    b = xa.xattn_prefill_noalloc(*args, want_scores=False)
    torch.cuda.synchronize()
    for got in (a, b):
        assert got.block_scores is None
        assert torch.equal(ref.mask, got.mask)
        assert torch.equal(ref.kv_cnt, got.kv_cnt)
        assert torch.equal(ref.out, got.out)


def test_noalloc_refuses_oversized_problems(xa):
    # the full 32K layer needs 128 MiB of score partials: refused before any launch
    w = wl.WORKLOADS["llama32k"]
    p = xa.problem(w.B, w.Hq, w.Hkv, w.M, w.C, w.block, w.stride, w.causal, torch.bfloat16)
    assert xa.total_workspace_bytes(p) > xa.NOALLOC_SCRATCH_BYTES
    q = torch.empty((1, w.Hq, w.M, w.C), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((1, w.Hkv, w.M, w.C), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(xa.XAttnError, match="scratch"):
        xa.xattn_prefill_noalloc(q, k, k, 0.9, w.block, w.stride, 0.01, 0.1, True)
