"""GPU parity of the selection variants through the C ABI: global (flattened
per-head) selection, the GQA union, and attention over GQA-union lists (two
sibling heads per workgroup).

Acceptance for global selection (floating point decides the cut): on the
GPU's own float32 block scores, the GPU keeps order[:k] plus the diagonal
blocks, where order is the oracle's candidate order (score descending, (I, J)
row-major) and k is a cut whose prefix mass reaches tau * T while the prefix
one shorter stays below it, both within 1e-8 * T (the GPU sums fixed-point
masses, the oracle float64 prefixes). Scores that are exact binary fractions
must give the oracle's mask bit for bit. The GQA union must equal the union of
the GPU's own per-row masks exactly.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check_index, f64, near_tau_blocks, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _candidates(nb, causal):
    rows, cols = [], []
    for i in range(nb):
        n = i + 1 if causal else nb
        rows.extend([i] * n)
        cols.extend(range(n))
    return np.asarray(rows), np.asarray(cols)


def global_cut_ok(keep: np.ndarray, scores: np.ndarray, tau: float, causal: bool, rel: float = 1e-8):
    """True if ``keep`` (NB, NB) is a valid global selection of ``scores``."""
    nb = scores.shape[0]
    rows, cols = _candidates(nb, causal)
    flat = scores[rows, cols].astype(np.float64)
    n = flat.size
    diag = np.zeros((nb, nb), dtype=bool)
    diag[np.arange(nb), np.arange(nb)] = True
    if tau >= 1.0:
        want = np.zeros((nb, nb), dtype=bool)
        want[rows, cols] = True
        return bool((want == keep).all())
    order = np.lexsort((np.arange(n), -flat))
    csum = np.concatenate([[0.0], np.cumsum(flat[order])])
    thr = tau * csum[-1]
    eps = rel * csum[-1] + 1e-12
    k_or = int(np.argmax(csum >= thr))
    for k in range(max(0, k_or - 4), min(n, k_or + 4) + 1):
        if csum[k] >= thr - eps and (k == 0 or csum[k - 1] < thr + eps):
            want = diag.copy()
            want[rows[order[:k]], cols[order[:k]]] = True
            if (want == keep).all():
                return True
    return False


CASES = [
    ("tiny", {}),
    ("llama8k", dict(M=4096, Hq=4, Hkv=2)),
    ("video", dict(M=2560, Hq=2, Hkv=2)),
]


@pytest.mark.parametrize("name,over", CASES)
def test_global_select_on_gpu_scores(xa, name, over):
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, _ = wl.default_scales(w)
    qd, kd = x["q"].to(DEV), x["k"].to(DEV)
    sc = xa.xattn_score(qd, kd, w.block, w.stride, sscale, w.causal)
    hq = w.Hq
    for taus in ([0.9] * hq, [0.0, 1.0] * (hq // 2) if hq > 1 else [0.5], [0.5] * hq, [0.99] * hq):
        mk, idx, cnt = xa.xattn_select(sc, taus, w.block, w.stride, w.causal, Hkv=w.Hkv, C=w.C,
                                       dtype=qd.dtype, selection="global")
        torch.cuda.synchronize()
        s64 = f64(sc)
        m = mk.cpu().numpy().astype(bool)
        for b in range(w.B):
            for h in range(hq):
                assert global_cut_ok(m[b, h], s64[b, h], float(taus[h]), w.causal), (name, b, h, taus[h])
        check_index(mk.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy())


@pytest.mark.parametrize("causal", [True, False])
def test_global_select_exact_on_binary_fraction_scores(xa, causal):
    # scores on a 1/64 grid: sums are exact in both the fixed-point GPU sums and
    # the oracle's float64 prefixes, so the masks must agree bit for bit,
    # including the many ties at the cut (broken by (I, J) row-major)
    rng = np.random.default_rng(11 if causal else 12)
    B, Hq, nb = 1, 3, 24
    sc = np.floor(rng.random((B, Hq, nb, nb)) ** 3 * 8) / 64
    if causal:
        sc = np.tril(sc)
    scd = torch.from_numpy(sc.astype(np.float32)).to(DEV)
    for t in (0.3, 0.6, 0.75, 0.9, 0.97):
        tau = float(np.float32(t))   # the value the library receives
        mk, idx, cnt = xa.xattn_select(scd, [tau] * Hq, 128, 8, causal, Hkv=Hq, selection="global")
        torch.cuda.synchronize()
        want = oracle.select(sc, [tau] * Hq, causal, mode="global")
        np.testing.assert_array_equal(mk.cpu().numpy(), want, err_msg=f"tau={tau}")
        check_index(mk.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy())


@pytest.mark.parametrize("name,over", CASES)
def test_gqa_union_is_union_of_gpu_rows(xa, name, over):
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, _ = wl.default_scales(w)
    qd, kd = x["q"].to(DEV), x["k"].to(DEV)
    sc = xa.xattn_score(qd, kd, w.block, w.stride, sscale, w.causal)
    row = xa.xattn_select(sc, x["tau"], w.block, w.stride, w.causal, Hkv=w.Hkv, C=w.C, dtype=qd.dtype)
    uni = xa.xattn_select(sc, x["tau"], w.block, w.stride, w.causal, Hkv=w.Hkv, C=w.C, dtype=qd.dtype,
                          selection="gqa_union")
    torch.cuda.synchronize()
    want = oracle.gqa_union(row[0].cpu().numpy(), w.Hkv)
    np.testing.assert_array_equal(uni[0].cpu().numpy(), want)
    check_index(want, uni[1].cpu().numpy(), uni[2].cpu().numpy())


@pytest.mark.parametrize("Hq,Hkv,M,C,causal", [(4, 2, 1024, 128, True), (8, 2, 768, 128, False),
                                               (4, 1, 512, 64, True)])
def test_bsa_over_gqa_union_lists(xa, Hq, Hkv, M, C, causal):
    # random per-head masks, united per KV group; the sibling-pair kernel must
    # match the oracle and the one-head-per-workgroup kernel
    block = 128
    nb = M // block
    g = torch.Generator().manual_seed(Hq * 100 + M)
    q = torch.randn((1, Hq, M, C), generator=g).to(torch.bfloat16)
    k = torch.randn((1, Hkv, M, C), generator=g).to(torch.bfloat16)
    v = torch.randn((1, Hkv, M, C), generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(M + Hq)
    mk = (rng.random((1, Hq, nb, nb)) < 0.3).astype(np.uint8)
    mk[..., np.arange(nb), np.arange(nb)] = 1
    if causal:
        mk = np.tril(mk)
    uni = oracle.gqa_union(mk, Hkv)
    sm = 1 / np.sqrt(C)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    for m, sel in ((uni, "gqa_union"), (mk, "gqa_union"), (uni, "row")):
        idx, cnt = oracle.mask_to_index(m)
        out, lse = xa.bsa_fwd(qd, kd, vd, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV),
                              block, sm, causal, want_lse=True, selection=xa._selection(sel))
        torch.cuda.synchronize()
        ref, ref_lse = oracle.attend(f64(q), f64(k), f64(v), m, block, sm, causal)
        err = np.abs(f64(out) - ref).max()
        assert err <= 2e-2, (sel, err)
        assert np.abs(f64(lse) - ref_lse).max() <= 2e-3
    # per-head lists through the sibling-pair kernel equal the per-head kernel
    idx, cnt = oracle.mask_to_index(mk)
    a, _ = xa.bsa_fwd(qd, kd, vd, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV), block, sm,
                      causal, selection=xa.SELECT_GQA_UNION)
    b, _ = xa.bsa_fwd(qd, kd, vd, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV), block, sm,
                      causal, selection=xa.SELECT_ROW)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("selection", ["global", "gqa_union"])
@pytest.mark.parametrize("name,over", [("llama8k", dict(M=4096, Hq=4, Hkv=2)), ("tiny", {})])
def test_prefill_selection_end_to_end(xa, selection, name, over):
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    bufs = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, w.causal,
                            selection=selection)
    torch.cuda.synchronize()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    ref_sc = oracle.block_scores(q, k, w.block, w.stride, sscale, w.causal)
    got_sc = f64(bufs.block_scores)
    assert (np.abs(got_sc - ref_sc) <= score_tol(ref_sc)).all()
    m = bufs.mask.cpu().numpy()
    tau = x["tau"].numpy().astype(np.float64)
    if selection == "global":
        for h in range(w.Hq):
            assert global_cut_ok(m[0, h].astype(bool), got_sc[0, h], float(tau[h]), w.causal), h
    else:
        row = oracle.select(got_sc, tau, w.causal)
        uni = oracle.gqa_union(row, w.Hkv)
        # identical except blocks near some sibling's cut on these scores
        G = w.Hq // w.Hkv
        for h, big_i, J in zip(*np.nonzero(m[0] != uni[0])):
            sib = range((h // G) * G, (h // G + 1) * G)
            ok = set().union(*[near_tau_blocks(got_sc[0, s2, big_i], big_i, float(tau[s2]), w.causal, 1e-5)
                               for s2 in sib])
            assert int(J) in ok, (h, big_i, J)
    check_index(m, bufs.kv_idx.cpu().numpy(), bufs.kv_cnt.cpu().numpy())
    ref_out, _ = oracle.attend(q, k, v, m, w.block, smscale, w.causal)
    err = np.abs(f64(bufs.out) - ref_out).max()
    assert err <= (2e-2 if w.dtype == "bf16" else 1e-3), err


def test_global_select_fullsize_128k(xa):
    # the bench-sized layer: the whole prefill with global selection, checked on
    # the GPU's own scores for three heads (about 525K candidates each)
    w = wl.WORKLOADS["llama128k"]
    print(f"[selection] global prefill {w.name}", flush=True)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal,
                            selection="global")
    torch.cuda.synchronize()
    tau = x["tau"].numpy().astype(np.float64)
    for h in (0, w.Hq // 2, w.Hq - 1):
        s64 = f64(bufs.block_scores[0, h])
        keep = bufs.mask[0, h].cpu().numpy().astype(bool)
        assert global_cut_ok(keep, s64, float(tau[h]), w.causal), h
        cnt = bufs.kv_cnt[0, h].cpu().numpy()
        np.testing.assert_array_equal(cnt, keep.sum(axis=1))
        print(f"[selection] h={h} tau={tau[h]:.2f} kept={int(cnt.sum())}", flush=True)
    del bufs, x
    torch.cuda.empty_cache()
