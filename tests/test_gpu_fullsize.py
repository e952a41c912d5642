"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: the whole layer runs through xattn_prefill on the GPU; the oracle then
recomputes sampled query-block rows one by one (block scores, the selection on
its own scores and on the GPU's scores, and attention with the GPU's mask).

Rows are sampled evenly over I, across heads with different per-head
densities, including the first and last rows. Tolerances as in the small
parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import f64, near_tau_blocks, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = ["llama8k", "llama32k", "llama128k", "llama256k", "video"]


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _sample_rows(w, n_rows):
    nb = w.nb
    rng = np.random.default_rng(1234 + w.seed)
    heads = rng.choice(w.Hq, size=n_rows, replace=True)
    rows = np.unique(np.concatenate([[0, nb - 1], np.linspace(0, nb - 1, n_rows - 2).round()]).astype(int))
    return list(zip(heads[: len(rows)].tolist(), rows.tolist()))


@pytest.mark.parametrize("name", CASES)
def test_fullsize_sampled_rows(xa, name):
    w = wl.WORKLOADS[name]
    print(f"[fullsize] {name}: M={w.M} Hq={w.Hq} Hkv={w.Hkv} S={w.stride}", flush=True)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    torch.cuda.synchronize()
    tau = x["tau"].numpy().astype(np.float64)
    G = w.Hq // w.Hkv
    n_rows = 6 if w.M >= 131072 else 10
    kv_cache = {}
    for h, big_i in _sample_rows(w, n_rows):
        g = h // G
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (f64(x["k"][0, g]), f64(x["v"][0, g]))
        kh, vh = kv_cache[g]
        qh = f64(x["q"][0, h])
        ref = oracle.block_score_row(qh, kh, big_i, w.block, w.stride, sscale, w.causal)
        got = bufs.block_scores[0, h, big_i].double().cpu().numpy()
        bad = np.abs(got - ref) > score_tol(ref)
        assert not bad.any(), (name, h, big_i, np.nonzero(bad)[0][:5], np.abs(got - ref).max())
        gmask = bufs.mask[0, h, big_i].cpu().numpy().astype(bool)
        # selection on the GPU's own scores: identical up to near-tau blocks
        same = oracle.select_row(got, big_i, float(tau[h]), w.causal)
        diff = np.nonzero(same != gmask)[0]
        ok = near_tau_blocks(got, big_i, float(tau[h]), w.causal, 1e-5)
        assert all(int(j) in ok for j in diff), (name, h, big_i, diff[:5])
        # end to end against the oracle's own scores
        mine = oracle.select_row(ref, big_i, float(tau[h]), w.causal)
        diff = np.nonzero(mine != gmask)[0]
        ok = near_tau_blocks(ref, big_i, float(tau[h]), w.causal, 1e-5 + 1e-4 + w.nb * 1e-7)
        assert all(int(j) in ok for j in diff), (name, h, big_i, diff[:5])
        cnt = int(bufs.kv_cnt[0, h, big_i])
        idx = bufs.kv_idx[0, h, big_i, :cnt].cpu().numpy()
        np.testing.assert_array_equal(idx, np.nonzero(gmask)[0])
        # attention with the GPU's mask
        o_ref, l_ref = oracle.attend_row(qh, kh, vh, gmask, big_i, w.block, smscale, w.causal)
        o_got = f64(bufs.out[0, h, big_i * w.block:(big_i + 1) * w.block])
        err = np.abs(o_got - o_ref).max()
        assert err <= 2e-2, (name, h, big_i, err)
        print(f"[fullsize] {name} h={h} I={big_i} kept={cnt} max_abs_err={err:.2e}", flush=True)
    del bufs, x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("causal", [True, False])
def test_max_block_count_sampled_rows(xa, causal):
    # The largest layer the interface takes: 4096 key blocks (64-token blocks
    # over 262144 tokens). Row 4095 has 4096 candidates, which fills the
    # selection's per-row state and the attention's cached block list exactly.
    w = wl.WORKLOADS["llama256k"].scaled(Hq=2 if causal else 1, Hkv=1, block=64, stride=8, causal=causal)
    assert w.nb == 4096
    print(f"[maxblocks] causal={causal} M={w.M} block={w.block} S={w.stride}", flush=True)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    torch.cuda.synchronize()
    tau = x["tau"].numpy().astype(np.float64)
    kh, vh = f64(x["k"][0, 0]), f64(x["v"][0, 0])
    for h, big_i in ((0, 0), (w.Hq - 1, 2047), (0, 4094), (w.Hq - 1, 4095)):
        qh = f64(x["q"][0, h])
        ref = oracle.block_score_row(qh, kh, big_i, w.block, w.stride, sscale, w.causal)
        got = f64(bufs.block_scores[0, h, big_i])
        bad = np.abs(got - ref) > score_tol(ref)
        assert not bad.any(), (h, big_i, np.nonzero(bad)[0][:5], np.abs(got - ref).max())
        gmask = bufs.mask[0, h, big_i].cpu().numpy().astype(bool)
        same = oracle.select_row(got, big_i, float(tau[h]), w.causal)
        diff = np.nonzero(same != gmask)[0]
        ok = near_tau_blocks(got, big_i, float(tau[h]), w.causal, 1e-5)
        assert all(int(j) in ok for j in diff), (h, big_i, diff[:5])
        cnt = int(bufs.kv_cnt[0, h, big_i])
        np.testing.assert_array_equal(bufs.kv_idx[0, h, big_i, :cnt].cpu().numpy(), np.nonzero(gmask)[0])
        o_ref, _ = oracle.attend_row(qh, kh, vh, gmask, big_i, w.block, smscale, w.causal)
        o_got = f64(bufs.out[0, h, big_i * w.block:(big_i + 1) * w.block])
        err = np.abs(o_got - o_ref).max()
        assert err <= 2e-2, (h, big_i, err)
        print(f"[maxblocks] h={h} I={big_i} kept={cnt} max_abs_err={err:.2e}", flush=True)
    del bufs, x
    torch.cuda.empty_cache()
