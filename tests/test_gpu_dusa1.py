"""GPU parity of the DuSA1 multi-stride scoring variant (pattern 2) against the
CPU oracle: block scores element by element, the selection on the GPU's own
scores, the whole prefill end to end, and sampled rows of the full 32K layer.

Reading (DuSA rebuttal, "Response to Q2", DuSA1): the S phases of the
(S, M/S, C) reshape are softmaxed on their own; a block scores the phases'
summed mass over its S * r rows divided by S * r. The score temperature is the
attention scale 1/sqrt(C), a phase logit being one dot product. Tolerances as
in the other parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check_index, check_mask, f64, near_tau_blocks, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(torch.bfloat16)


SCORE_CASES = [
    # B, Hq, Hkv, Mq, Mk, C, block, stride, causal
    (1, 4, 1, 2048, 2048, 128, 128, 8, True),     # r = 16
    (1, 2, 2, 1280, 1280, 128, 128, 16, False),   # r = 8, non-causal
    (1, 2, 1, 1024, 1024, 64, 64, 8, True),       # C = 64, r = 8
    (1, 2, 1, 512, 512, 64, 64, 32, True),        # r = 2
    (1, 2, 1, 512, 512, 128, 128, 32, False),     # r = 4
    (1, 2, 2, 768, 768, 128, 64, 4, True),        # r = 16, 64-token blocks
    (1, 2, 1, 1000, 1000, 128, 128, 8, True),     # partial last block (M a multiple of S only)
    (2, 2, 1, 512, 1536, 128, 128, 8, True),      # chunked: the last 512 queries of 1536 tokens
    (1, 1, 1, 4104, 4104, 128, 128, 8, False),    # a partial last tile of strided rows and keys
]


def _ids(c):
    return "-".join(map(str, c))


@pytest.mark.parametrize("case", SCORE_CASES, ids=_ids)
def test_dusa1_scores_match_oracle(xa, case):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal = case
    q = _rand((B, Hq, Mq, C), 500 + Mq)
    k = _rand((B, Hkv, Mk, C), 501 + Mk)
    sscale = 1.0 / math.sqrt(C)
    got = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, sscale, causal, pattern=xa.DUSA1)
    torch.cuda.synchronize()
    ref = oracle.block_scores(f64(q), f64(k), block, stride, sscale, causal, pattern="dusa1")
    g = f64(got)
    assert (g >= 0).all()
    viol = np.abs(g - ref) > score_tol(ref)
    assert not viol.any(), (np.argwhere(viol)[:5], np.abs(g - ref).max())
    np.testing.assert_allclose(g.sum(-1), 1.0, rtol=1e-4)
    # the variant really differs from the two single-softmax patterns here
    diag = oracle.block_scores(f64(q), f64(k), block, stride, sscale / stride, causal, pattern="diagonal")
    assert np.abs(diag - ref).max() > 1e-4


E2E = [("llama32k", dict(M=2048, Hq=8, Hkv=2)), ("llama128k", dict(M=4096, Hq=4, Hkv=1)),
       ("video", dict(M=2560, Hq=2, Hkv=2))]


@pytest.mark.parametrize("name,over", E2E, ids=[c[0] for c in E2E])
def test_dusa1_prefill_end_to_end(xa, name, over):
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, smscale = 1.0 / math.sqrt(w.C), 1.0 / math.sqrt(w.C)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    bufs = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, w.causal, pattern=xa.DUSA1)
    sc = xa.xattn_score(qd, kd, w.block, w.stride, sscale, w.causal, pattern=xa.DUSA1)
    nos = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, w.causal, pattern=xa.DUSA1,
                           want_scores=False)
    torch.cuda.synchronize()
    assert torch.equal(bufs.block_scores, sc)
    assert torch.equal(nos.mask, bufs.mask) and torch.equal(nos.out, bufs.out)
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    tau = x["tau"].numpy().astype(np.float64)
    ref_sc = oracle.block_scores(q, k, w.block, w.stride, sscale, w.causal, pattern="dusa1")
    g_sc = f64(bufs.block_scores)
    assert not (np.abs(g_sc - ref_sc) > score_tol(ref_sc)).any()
    g_mask = bufs.mask.cpu().numpy()
    check_mask(f"dusa1 {name} select on GPU scores", g_mask, oracle.select(g_sc, tau, w.causal), g_sc, tau,
               w.causal, 1e-5)
    band = 1e-5 + 1e-4 + w.nb * 1e-7
    check_mask(f"dusa1 {name} end to end", g_mask, oracle.select(ref_sc, tau, w.causal), ref_sc, tau, w.causal, band)
    check_index(g_mask, bufs.kv_idx.cpu().numpy(), bufs.kv_cnt.cpu().numpy())
    ref_out, _ = oracle.attend(q, k, v, g_mask, w.block, smscale, w.causal)
    err = np.abs(f64(bufs.out) - ref_out).max()
    assert err <= 2e-2, err
    print(f"[dusa1] {name}: density={oracle.density(g_mask, w.causal):.3f} max_abs_err={err:.2e}", flush=True)


def test_dusa1_fullsize_sampled_rows(xa):
    # the full 32K layer (32 query / 8 KV heads, stride 8): 32 rows over every KV group
    w = wl.WORKLOADS["llama32k"]
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = 1.0 / math.sqrt(w.C), 1.0 / math.sqrt(w.C)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal,
                            pattern=xa.DUSA1)
    torch.cuda.synchronize()
    tau = x["tau"].numpy().astype(np.float64)
    G = w.Hq // w.Hkv
    n_near = 0
    rows = [(g * G + (t % G), int((t + 0.5 + g / w.Hkv) * w.nb / 4) % w.nb)
            for g in range(w.Hkv) for t in range(4)]
    for g in range(w.Hkv):
        kh, vh = f64(x["k"][0, g]), f64(x["v"][0, g])
        for h, big_i in [r for r in rows if r[0] // G == g]:
            qh = f64(x["q"][0, h])
            ref = oracle.block_score_row(qh, kh, big_i, w.block, w.stride, sscale, w.causal, pattern="dusa1")
            got = f64(bufs.block_scores[0, h, big_i])
            bad = np.abs(got - ref) > score_tol(ref)
            assert not bad.any(), (h, big_i, np.nonzero(bad)[0][:5], np.abs(got - ref).max())
            gmask = bufs.mask[0, h, big_i].cpu().numpy().astype(bool)
            diff = np.nonzero(oracle.select_row(got, big_i, float(tau[h]), w.causal) != gmask)[0]
            ok = near_tau_blocks(got, big_i, float(tau[h]), w.causal, 1e-5)
            assert all(int(j) in ok for j in diff), (h, big_i, diff[:5])
            diff = np.nonzero(oracle.select_row(ref, big_i, float(tau[h]), w.causal) != gmask)[0]
            ok = near_tau_blocks(ref, big_i, float(tau[h]), w.causal, 1e-5 + 1e-4 + w.nb * 1e-7)
            assert all(int(j) in ok for j in diff), (h, big_i, diff[:5])
            n_near += len(diff)
            o_ref, _ = oracle.attend_row(qh, kh, vh, gmask, big_i, w.block, smscale, w.causal)
            err = np.abs(f64(bufs.out[0, h, big_i * w.block:(big_i + 1) * w.block]) - o_ref).max()
            assert err <= 2e-2, (h, big_i, err)
            print(f"[dusa1-full] h={h} I={big_i} kept={int(gmask.sum())} err={err:.2e}", flush=True)
    print(f"[mask] dusa1 llama32k: {len(rows)} sampled rows, {n_near} near-tau differences end to end", flush=True)
    assert n_near <= 4
