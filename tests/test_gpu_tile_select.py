"""Selection inside the scoring launch (XATTN_SELECT_IN_SCORE: xattn_prefill
with per-row or GQA-union selection, bf16 with complete stride groups): the
workgroup that stores a query tile's last partials normalises and selects the
tile's query-block rows.

Checked bitwise against the staged calls (xattn_score, then xattn_select, then
bsa_fwd) over every block/stride ratio r the kernels take, both head sizes,
causal and non-causal, chunked prefill, a last query tile with an odd number of
rows, thresholds that keep nothing or everything, GQA-union lists, the optional
outputs left out, two calls in a row on one set of buffers, and a partial last
stride group (where the option does not apply and xattn_prefill runs the
separate selection launch); and against the
oracle: block scores element by element, the selection on the GPU's own scores
(XAttention AI summary, "Approach"; FlexPrefill rebuttal, "R Q3").
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check_index, check_mask, f64, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _inputs(B, Hq, Hkv, M, Mk, C, seed):
    # sink- and local-heavy rows (the llama-like generator) so the selections
    # are neither empty nor full
    w = wl.WORKLOADS["llama8k"].scaled(B=B, Hq=Hq, Hkv=Hkv, M=Mk, C=C, seed=seed)
    x = wl.make_inputs(w)
    q = x["q"][:, :, Mk - M:].contiguous()
    return q, x["k"], x["v"]


CASES = [
    # id, B, Hq, Hkv, M, Mk, C, block, stride, causal, tau
    ("r16-causal", 1, 4, 2, 4096, 4096, 128, 128, 8, True, "mixed"),
    ("r16-odd-last-tile", 1, 2, 1, 2688, 2688, 128, 128, 8, True, "mixed"),     # 21 query blocks: 16 + 5
    ("r8-causal", 1, 4, 1, 2048, 2048, 128, 128, 16, True, "mixed"),
    ("r4-noncausal", 1, 2, 2, 2048, 2048, 128, 128, 32, False, "mixed"),
    ("r2-causal", 1, 2, 1, 1536, 1536, 128, 128, 64, True, "mixed"),
    ("r32-causal", 1, 2, 1, 2048, 2048, 128, 128, 4, True, "mixed"),
    ("c64-r16", 2, 2, 1, 2048, 2048, 64, 64, 4, True, "mixed"),
    ("c64-r8-noncausal", 1, 2, 2, 1536, 1536, 64, 128, 16, False, "mixed"),
    ("chunk-causal", 2, 4, 2, 1024, 3072, 128, 128, 8, True, "mixed"),
    ("chunk-noncausal", 1, 2, 1, 1280, 2560, 128, 128, 16, False, "mixed"),
    ("tau0", 1, 2, 1, 2048, 2048, 128, 128, 8, True, "zero"),
    ("tau1", 1, 2, 1, 2048, 2048, 128, 128, 8, True, "one"),
    ("long-rows", 1, 2, 1, 40960, 40960, 128, 128, 16, True, "mixed"),          # 320 key blocks: long row form
]


def _tau(kind, Hq):
    if kind == "zero":
        return torch.zeros(Hq)
    if kind == "one":
        return torch.ones(Hq)
    return torch.tensor([0.9, 0.95, 0.8, 0.99, 0.5, 0.9, 0.97, 0.85][:Hq] * (Hq // 8 + 1))[:Hq]


def _staged(xa, q, k, v, tau, block, stride, sscale, smscale, causal, selection):
    sc = xa.xattn_score(q, k, block, stride, sscale, causal)
    mk, idx, cnt = xa.xattn_select(sc, tau, block, stride, causal, Hkv=k.shape[1], C=q.shape[-1],
                                   dtype=q.dtype, selection=selection)
    out, _ = xa.bsa_fwd(q, k, v, idx, cnt, block, smscale, causal, selection=selection)
    return sc, mk, idx, cnt, out


def _equal_lists(idx_a, idx_b, cnt):
    valid = torch.arange(idx_a.shape[-1], device=idx_a.device) < cnt[..., None]
    return torch.equal(idx_a[valid], idx_b[valid])


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_tile_select_equals_staged_calls_and_oracle(xa, case):
    name, B, Hq, Hkv, M, Mk, C, block, stride, causal, tau_kind = case
    print(f"[tile-select] {name}", flush=True)
    q, k, v = _inputs(B, Hq, Hkv, M, Mk, C, seed=11 + M + Mk + stride)
    tau = _tau(tau_kind, Hq)
    sscale, smscale = 1.0 / (stride * math.sqrt(C)), 1.0 / math.sqrt(C)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    got = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, causal, select_in_score=True)
    sc, mk, idx, cnt, out = _staged(xa, qd, kd, vd, tau, block, stride, sscale, smscale, causal, xa.SELECT_ROW)
    torch.cuda.synchronize()
    assert torch.equal(got.block_scores, sc)
    assert torch.equal(got.mask, mk)
    assert torch.equal(got.kv_cnt, cnt)
    assert _equal_lists(got.kv_idx, idx, cnt)
    assert torch.equal(got.out, out)
    if tau_kind == "zero":   # only the diagonal block
        assert (cnt == 1).all()
    if tau_kind == "one" and causal and M == Mk:
        assert torch.equal(cnt[0, 0].cpu(), torch.arange(1, cnt.shape[-1] + 1, dtype=torch.int32))
    # the oracle: scores element by element, the selection on these scores
    if M * Mk <= 4096 * 4096:
        g = f64(sc)
        ref = oracle.block_scores(f64(q), f64(k), block, stride, sscale, causal)
        bad = np.abs(g - ref) > score_tol(ref)
        assert not bad.any(), (np.argwhere(bad)[:5], np.abs(g - ref).max())
    g = f64(sc)
    t64 = tau.numpy().astype(np.float64)
    check_mask(f"tile-select {name}", got.mask.cpu().numpy(), oracle.select(g, t64, causal), g, t64, causal, 1e-5,
               qoff=(Mk - M) // block)
    check_index(got.mask.cpu().numpy(), got.kv_idx.cpu().numpy(), got.kv_cnt.cpu().numpy())


def test_tile_select_gqa_union_and_optional_outputs(xa):
    B, Hq, Hkv, M, C, block, stride = 1, 8, 2, 4096, 128, 128, 8
    q, k, v = _inputs(B, Hq, Hkv, M, M, C, seed=5)
    tau = _tau("mixed", Hq)
    sscale, smscale = 1.0 / (stride * math.sqrt(C)), 1.0 / math.sqrt(C)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    got = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, True, selection=xa.SELECT_GQA_UNION,
                           select_in_score=True)
    sc, mk, idx, cnt, out = _staged(xa, qd, kd, vd, tau, block, stride, sscale, smscale, True,
                                    xa.SELECT_GQA_UNION)
    torch.cuda.synchronize()
    assert torch.equal(got.block_scores, sc) and torch.equal(got.mask, mk) and torch.equal(got.kv_cnt, cnt)
    assert _equal_lists(got.kv_idx, idx, cnt) and torch.equal(got.out, out)
    # no block scores and no mask: the same lists and output
    bufs = xa.PrefillBuffers(qd, kd, block, stride, True, want_mask=False, want_scores=False,
                             selection=xa.SELECT_GQA_UNION, select_in_score=True)
    lean = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, True, buffers=bufs,
                            selection=xa.SELECT_GQA_UNION, select_in_score=True)
    torch.cuda.synchronize()
    assert lean.block_scores is None and lean.mask is None
    assert torch.equal(lean.kv_cnt, cnt) and _equal_lists(lean.kv_idx, idx, cnt)
    assert torch.equal(lean.out, out)


def test_tile_select_twice_on_one_buffer_set(xa):
    # the arrival counters are cleared by every call: a second call on the same
    # buffers (other inputs) matches the staged path again
    B, Hq, Hkv, M, C, block, stride = 1, 4, 1, 4096, 128, 128, 16
    sscale, smscale = 1.0 / (stride * math.sqrt(C)), 1.0 / math.sqrt(C)
    bufs = None
    for seed in (1, 2):
        q, k, v = _inputs(B, Hq, Hkv, M, M, C, seed=seed)
        qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
        tau = _tau("mixed", Hq)
        if bufs is None:
            bufs = xa.PrefillBuffers(qd, kd, block, stride, True, select_in_score=True)
        got = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, True, buffers=bufs,
                               select_in_score=True)
        sc, mk, idx, cnt, out = _staged(xa, qd, kd, vd, tau, block, stride, sscale, smscale, True, xa.SELECT_ROW)
        torch.cuda.synchronize()
        assert torch.equal(got.block_scores, sc) and torch.equal(got.mask, mk)
        assert torch.equal(got.kv_cnt, cnt) and _equal_lists(got.kv_idx, idx, cnt)
        assert torch.equal(got.out, out)


def test_partial_stride_group_takes_the_staged_path(xa):
    # 3000 tokens at stride 8: the last stride group is partial, so the option
    # does not apply: xattn_prefill scores with the register-staged kernel and
    # selects in a separate launch; the results still equal the staged calls
    B, Hq, Hkv, M, C, block, stride = 1, 2, 1, 3000, 128, 128, 8
    q, k, v = _inputs(B, Hq, Hkv, M, M, C, seed=9)
    tau = _tau("mixed", Hq)
    sscale, smscale = 1.0 / (stride * math.sqrt(C)), 1.0 / math.sqrt(C)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    got = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, True, select_in_score=True)
    sc, mk, idx, cnt, out = _staged(xa, qd, kd, vd, tau, block, stride, sscale, smscale, True, xa.SELECT_ROW)
    torch.cuda.synchronize()
    assert torch.equal(got.block_scores, sc) and torch.equal(got.mask, mk)
    assert torch.equal(got.kv_cnt, cnt) and _equal_lists(got.kv_idx, idx, cnt)
    assert torch.equal(got.out, out)


def test_tile_select_replays_from_a_hip_graph(xa):
    # the arrival counters and the attention queues are zeroed by a kernel, so
    # the one-launch form can be captured; every replay, with eager work and
    # synchronisations in between, equals the eager call
    w = wl.WORKLOADS["llama32k"].scaled(M=4096, Hq=8, Hkv=2)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    ref = xa.xattn_prefill(*args, select_in_score=True)
    bufs = xa.PrefillBuffers(x["q"], x["k"], w.block, w.stride, w.causal, select_in_score=True)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        xa.xattn_prefill(*args, buffers=bufs, select_in_score=True)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.xattn_prefill(*args, buffers=bufs, select_in_score=True)
    torch.cuda.synchronize()
    valid = torch.arange(ref.kv_idx.shape[-1], device=DEV) < ref.kv_cnt[..., None]
    for _ in range(3):
        for t, fill in ((bufs.out, 0.0), (bufs.block_scores, -1.0), (bufs.mask, 7), (bufs.kv_cnt, -3)):
            t.fill_(fill)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ref.block_scores, bufs.block_scores)
        assert torch.equal(ref.mask, bufs.mask)
        assert torch.equal(ref.kv_cnt, bufs.kv_cnt)
        assert torch.equal(ref.kv_idx[valid], bufs.kv_idx[valid])
        assert torch.equal(ref.out, bufs.out)


def test_tile_select_without_a_workspace(xa):
    # the entry point that allocates nothing, with the option: two calls on the
    # shared scratch, the second smaller, each equal to the default path
    for w in (wl.WORKLOADS["llama8k"].scaled(M=8192, Hq=8, Hkv=2), wl.WORKLOADS["llama32k"].scaled(M=2048, Hq=4, Hkv=1)):
        print(f"[tile-select noalloc] M={w.M} Hq={w.Hq}", flush=True)
        x = wl.make_inputs(w, device=DEV)
        sscale, smscale = wl.default_scales(w)
        args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
        ref = xa.xattn_prefill(*args)
        got = xa.xattn_prefill_noalloc(*args, select_in_score=True)
        torch.cuda.synchronize()
        assert torch.equal(ref.block_scores, got.block_scores) and torch.equal(ref.mask, got.mask)
        assert torch.equal(ref.kv_cnt, got.kv_cnt) and _equal_lists(ref.kv_idx, got.kv_idx, ref.kv_cnt)
        assert torch.equal(ref.out, got.out)
