"""GPU parity for ragged lengths (not multiples of the stride or the block) and
chunked prefill (the queries are the last Mq of Mk tokens), stage by stage and
end to end, through the C ABI. Tolerances as in the other parity tests:
block scores |g - o| <= 1e-4 |o| + 1e-7; bf16 outputs max-abs 2e-2, fp32 1e-3;
masks identical except blocks within 1e-5 of a row's cut (on the GPU's scores).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import check_index, check_mask, f64, near_tau_blocks, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype
CASES = [
    (1, 2, 1, 1000, 1000, 128, 128, 8, True, torch.bfloat16),     # partial last block
    (1, 2, 2, 1001, 1001, 64, 64, 8, True, torch.bfloat16),       # partial stride group
    (1, 2, 1, 1003, 1003, 128, 128, 16, False, torch.bfloat16),
    (1, 4, 2, 512, 2048, 128, 128, 8, True, torch.bfloat16),      # chunk, aligned
    (1, 2, 1, 700, 1468, 128, 128, 16, True, torch.bfloat16),     # chunk, ragged both
    (1, 2, 1, 6952, 9000, 128, 128, 8, True, torch.bfloat16),     # trapezoid of score tiles
    (1, 3, 1, 1000, 1768, 128, 128, 8, True, torch.bfloat16),     # odd group, chunk, ragged
    (1, 1, 1, 300, 556, 64, 64, 8, True, torch.float32),
    (1, 1, 1, 77, 77, 64, 64, 8, False, torch.float32),
]


def _ids(c):
    return f"{c[3]}of{c[4]}-C{c[5]}-b{c[6]}-s{c[7]}-{'c' if c[8] else 'n'}-{str(c[9])[-4:]}"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _inputs(case, seed):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    g = torch.Generator().manual_seed(seed)
    # a few strong key columns so the selection is not uniform
    k = torch.randn((B, Hkv, Mk, C), generator=g)
    k[:, :, ::97] *= 3.0
    q = torch.randn((B, Hq, Mq, C), generator=g)
    v = torch.randn((B, Hkv, Mk, C), generator=g)
    return q.to(dtype), k.to(dtype), v.to(dtype)


def _tol(dtype):
    return 2e-2 if dtype == torch.bfloat16 else 1e-3


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_scores_ragged_chunked(xa, case):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    q, k, _ = _inputs(case, 1)
    ss = 1.0 / (stride * math.sqrt(C))
    sc = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, ss, causal)
    torch.cuda.synchronize()
    ref = oracle.block_scores(f64(q), f64(k), block, stride, ss, causal)
    got = f64(sc)
    assert got.shape == ref.shape
    bad = np.abs(got - ref) > score_tol(ref)
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(got - ref).max())
    np.testing.assert_allclose(got.sum(axis=-1), 1.0, rtol=1e-4)


def _check_rows(mask_gpu, scores_gpu, tau, causal, qoff):
    ref = oracle.select(scores_gpu, tau, causal)
    check_mask(f"ragged/chunked select qoff={qoff}", mask_gpu, ref, scores_gpu, tau, causal, 1e-5, qoff=qoff)


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_select_ragged_chunked(xa, case):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    q, k, _ = _inputs(case, 2)
    ss = 1.0 / (stride * math.sqrt(C))
    sc = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, ss, causal)
    tau = np.array([0.9, 0.6, 0.95, 0.8][:Hq], dtype=np.float32)
    mk, idx, cnt = xa.xattn_select(sc, tau, block, stride, causal, Hkv=Hkv, C=C, dtype=dtype)
    torch.cuda.synchronize()
    s64 = f64(sc)
    nbq, nbk = s64.shape[-2:]
    m = mk.cpu().numpy()
    _check_rows(m, s64, tau.astype(np.float64), causal, nbk - nbq)
    check_index(m, idx.cpu().numpy(), cnt.cpu().numpy())
    # every row holds its diagonal block I + (NBk - NBq)
    assert m[..., np.arange(nbq), np.arange(nbq) + nbk - nbq].all()


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_attention_ragged_chunked(xa, case):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    q, k, v = _inputs(case, 3)
    nbq, nbk = -(-Mq // block), -(-Mk // block)
    qoff = nbk - nbq
    rng = np.random.default_rng(Mq + Mk)
    mask = (rng.random((B, Hq, nbq, nbk)) < 0.35).astype(np.uint8)
    mask[..., np.arange(nbq), np.arange(nbq) + qoff] = 1
    if causal:
        mask *= np.tril(np.ones((nbq, nbk), dtype=np.uint8), k=qoff)
    idx, cnt = oracle.mask_to_index(mask)
    sm = 1.0 / math.sqrt(C)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    out, lse = xa.bsa_fwd(qd, kd, vd, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV),
                          block, sm, causal, want_lse=True)
    dout, dlse = xa.dense_fwd(qd, kd, vd, block, sm, causal, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attend(f64(q), f64(k), f64(v), mask, block, sm, causal)
    assert np.abs(f64(out) - ref).max() <= _tol(dtype)
    assert np.abs(f64(lse) - ref_lse).max() <= 2e-3
    dref, dref_lse = oracle.dense(f64(q), f64(k), f64(v), block, sm, causal)
    assert np.abs(f64(dout) - dref).max() <= _tol(dtype)
    assert np.abs(f64(dlse) - dref_lse).max() <= 2e-3


@pytest.mark.parametrize("selection", ["row", "global", "gqa_union"])
@pytest.mark.parametrize("case", [CASES[1], CASES[4], CASES[7]], ids=_ids)
def test_prefill_ragged_chunked_end_to_end(xa, case, selection):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    q, k, v = _inputs(case, 4)
    ss, sm = 1.0 / (stride * math.sqrt(C)), 1.0 / math.sqrt(C)
    tau = np.array([0.9, 0.7][:Hq], dtype=np.float32)
    bufs = xa.xattn_prefill(q.to(DEV), k.to(DEV), v.to(DEV), tau, block, stride, ss, sm, causal,
                            selection=selection)
    torch.cuda.synchronize()
    q64, k64, v64 = f64(q), f64(k), f64(v)
    ref_sc = oracle.block_scores(q64, k64, block, stride, ss, causal)
    got_sc = f64(bufs.block_scores)
    assert (np.abs(got_sc - ref_sc) <= score_tol(ref_sc)).all()
    m = bufs.mask.cpu().numpy()
    nbq, nbk = got_sc.shape[-2:]
    if selection == "row":
        _check_rows(m, got_sc, tau.astype(np.float64), causal, nbk - nbq)
    elif selection == "gqa_union":
        # siblings share one list, which holds each sibling's own row selection
        # (up to blocks near that sibling's cut)
        np.testing.assert_array_equal(m, oracle.gqa_union(m, Hkv))
        rows = oracle.select(got_sc, tau.astype(np.float64), causal)
        for h, i, J in zip(*np.nonzero(rows[0].astype(bool) & ~m[0].astype(bool))):
            assert int(J) in near_tau_blocks(got_sc[0, h, i], i + nbk - nbq, float(tau[h]), causal, 1e-5)
    else:
        for h in range(Hq):
            assert global_cut_ok_chunk(m[0, h].astype(bool), got_sc[0, h], float(tau[h]), causal)
    check_index(m, bufs.kv_idx.cpu().numpy(), bufs.kv_cnt.cpu().numpy())
    ref_out, _ = oracle.attend(q64, k64, v64, m, block, sm, causal)
    assert np.abs(f64(bufs.out) - ref_out).max() <= _tol(dtype)


def global_cut_ok_chunk(keep, scores, tau, causal, rel=1e-8):
    """global_cut_ok for a rectangular (NBq, NBk) block matrix."""
    nbq, nbk = scores.shape
    qoff = nbk - nbq
    rows, cols = [], []
    for i in range(nbq):
        n = i + qoff + 1 if causal else nbk
        rows.extend([i] * n)
        cols.extend(range(n))
    rows, cols = np.asarray(rows), np.asarray(cols)
    flat = scores[rows, cols].astype(np.float64)
    diag = np.zeros((nbq, nbk), dtype=bool)
    diag[np.arange(nbq), np.arange(nbq) + qoff] = True
    order = np.lexsort((np.arange(flat.size), -flat))
    csum = np.concatenate([[0.0], np.cumsum(flat[order])])
    thr, eps = tau * csum[-1], rel * csum[-1] + 1e-12
    k_or = int(np.argmax(csum >= thr))
    for kk in range(max(0, k_or - 4), min(flat.size, k_or + 4) + 1):
        if csum[kk] >= thr - eps and (kk == 0 or csum[kk - 1] < thr + eps):
            want = diag.copy()
            want[rows[order[:kk]], cols[order[:kk]]] = True
            if (want == keep).all():
                return True
    return False


@pytest.mark.parametrize("case", [CASES[0], CASES[4], CASES[7]], ids=_ids)
def test_ragged_outputs_stay_inside_buffers(xa, case):
    # every output and the workspace sit between guard regions that must stay
    # untouched (a store past the last query row would land in the tail guard)
    import ctypes
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, dtype = case
    q, k, v = _inputs(case, 5)
    nbq, nbk = -(-Mq // block), -(-Mk // block)
    guard = 8192

    def guarded(n, dt, fill):
        t = torch.full((n + 2 * guard,), fill, dtype=dt, device=DEV)
        return t, t[guard:guard + n]

    sc_all, sc = guarded(B * Hq * nbq * nbk, torch.float32, -7.0)
    mk_all, mk = guarded(B * Hq * nbq * nbk, torch.uint8, 0xAB)
    ix_all, ix = guarded(B * Hq * nbq * nbk, torch.int32, -5)
    ct_all, ct = guarded(B * Hq * nbq, torch.int32, -5)
    out_all, out = guarded(B * Hq * Mq * C, dtype, 3.0)
    lse_all, lse = guarded(B * Hq * Mq, torch.float32, -7.0)
    p = xa.problem(B, Hq, Hkv, Mq, C, block, stride, causal, dtype, Mk=Mk)
    ws_all, ws = guarded(xa.prefill_workspace_bytes(p), torch.uint8, 0x5A)
    tau = torch.full((Hq,), 0.9)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    st = torch.cuda.current_stream().cuda_stream
    rc = xa._lib.xattn_prefill(ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), tau.data_ptr(),
                               1 / (stride * math.sqrt(C)), 1 / math.sqrt(C), sc.data_ptr(), mk.data_ptr(),
                               ix.data_ptr(), ct.data_ptr(), ws.data_ptr(), ws.numel(), out.data_ptr(),
                               lse.data_ptr(), st)
    assert rc == 0, xa._lib.xattn_last_error()
    torch.cuda.synchronize()
    for full, fill in ((sc_all, -7.0), (mk_all, 0xAB), (ix_all, -5), (ct_all, -5), (out_all, 3.0),
                       (lse_all, -7.0), (ws_all, 0x5A)):
        assert (full[:guard] == fill).all() and (full[-guard:] == fill).all()
    assert torch.isfinite(out.float()).all()


@pytest.mark.parametrize("mk,chunk_blocks", [(131149, 0), (262221, 512)])
def test_paired_rows_long_ragged_sampled(xa, mk, chunk_blocks):
    # long rows run two neighbouring query blocks per workgroup over the union
    # of their lists; an odd number of query blocks leaves the last pair with
    # an empty slot. Sampled rows (incl. the last) against the oracle.
    import workloads as wl
    w = wl.WORKLOADS["llama128k"].scaled(M=mk, Hq=2, Hkv=1)
    x = wl.make_inputs(w, device=DEV)
    off = 128 * chunk_blocks
    q = x["q"][:, :, off:].contiguous()
    k, v = x["k"], x["v"]
    mq = mk - off
    nbq, nbk = -(-mq // 128), -(-mk // 128)
    assert nbq >= 1024 and nbq % 2 == 1
    print(f"[paired] Mq={mq} Mk={mk} NBq={nbq}", flush=True)
    ss, sm = wl.default_scales(w)
    bufs = xa.xattn_prefill(q, k, v, x["tau"], 128, w.stride, ss, sm, True)
    torch.cuda.synchronize()
    kh, vh = f64(k[0, 0]), f64(v[0, 0])
    for h, big_i in ((0, 0), (1, nbq // 2), (0, nbq - 2), (1, nbq - 1)):
        qh = f64(q[0, h])
        ref = oracle.block_score_row(qh, kh, big_i, 128, w.stride, ss, True)
        got = f64(bufs.block_scores[0, h, big_i])
        assert (np.abs(got - ref) <= score_tol(ref)).all(), (h, big_i)
        keep = bufs.mask[0, h, big_i].cpu().numpy().astype(bool)
        o_ref, l_ref = oracle.attend_row(qh, kh, vh, keep, big_i, 128, sm, True)
        o_got = f64(bufs.out[0, h, big_i * 128:big_i * 128 + o_ref.shape[0]])
        err = np.abs(o_got - o_ref).max()
        assert err <= 2e-2, (h, big_i, err)
        print(f"[paired] h={h} I={big_i} kept={int(keep.sum())} err={err:.2e}", flush=True)
