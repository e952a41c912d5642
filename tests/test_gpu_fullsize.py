"""GPU parity at the full workload sizes, in the launch configuration bench.py
times: the whole layer runs through xattn_prefill on the GPU; the oracle then
recomputes sampled query-block rows one by one (block scores, the selection on
its own scores and on the GPU's scores, and attention with the GPU's mask).

At least 32 rows per layer are sampled, evenly over I and over every KV
group, always including each group's densest head and the first and last
rows. A second test checks the selection of every row of each layer: the
oracle's minimal sets on the GPU's own block scores against the GPU's mask.
Tolerances as in the small parity tests; the count of allowed near-tau mask
differences is printed and capped.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests.gpu_util import check_mask, f64, near_tau_blocks, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
CASES = ["llama8k", "llama32k", "llama128k", "llama256k", "video"]


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _sample_rows(w, kv_cnt, n_rows=32):
    """(head, query block) rows to recompute: at least ``n_rows``, spread over
    every KV group. Each group's densest head (most kept blocks, read from the
    GPU's counts) is always among them; the group's other heads are drawn
    without replacement. Query blocks are spaced evenly over the layer with a
    per-group offset, and the first and last blocks are included."""
    nb = w.nb
    G = w.Hq // w.Hkv
    rng = np.random.default_rng(1234 + w.seed)
    per_group = -(-n_rows // w.Hkv)
    dens = kv_cnt.sum(axis=-1)                                  # (Hq,)
    out = []
    for g in range(w.Hkv):
        heads = list(range(g * G, (g + 1) * G))
        top = max(heads, key=lambda h: dens[h])
        rest = [h for h in rng.permutation(heads).tolist() if h != top]
        order = [top] + rest
        pos = (np.arange(per_group) + (g + 0.5) / w.Hkv) * nb / per_group
        for t in range(per_group):
            out.append((order[t % len(order)], int(min(nb - 1, pos[t]))))
    out[0] = (out[0][0], 0)
    out[-1] = (out[-1][0], nb - 1)
    return sorted(set(out))


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
    kv_cnt = bufs.kv_cnt[0].cpu().numpy()
    rows = _sample_rows(w, kv_cnt)
    assert len(rows) >= 32 and {h // G for h, _ in rows} == set(range(w.Hkv))
    n_near_self = n_near_e2e = 0
    kv_cache = {}
    q_cache = {}
    for h, big_i in rows:
        g = h // G
        if g not in kv_cache:
            kv_cache.clear()
            kv_cache[g] = (f64(x["k"][0, g]), f64(x["v"][0, g]))
        kh, vh = kv_cache[g]
        if h not in q_cache:
            q_cache.clear()
            q_cache[h] = f64(x["q"][0, h])
        qh = q_cache[h]
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
        n_near_self += len(diff)
        # end to end against the oracle's own scores
        mine = oracle.select_row(ref, big_i, float(tau[h]), w.causal)
        diff = np.nonzero(mine != gmask)[0]
        ok = near_tau_blocks(ref, big_i, float(tau[h]), w.causal, 1e-5 + 1e-4 + w.nb * 1e-7)
        assert all(int(j) in ok for j in diff), (name, h, big_i, diff[:5])
        n_near_e2e += len(diff)
        cnt = int(bufs.kv_cnt[0, h, big_i])
        idx = bufs.kv_idx[0, h, big_i, :cnt].cpu().numpy()
        np.testing.assert_array_equal(idx, np.nonzero(gmask)[0])
        # attention with the GPU's mask
        o_ref, l_ref = oracle.attend_row(qh, kh, vh, gmask, big_i, w.block, smscale, w.causal)
        o_got = f64(bufs.out[0, h, big_i * w.block:(big_i + 1) * w.block])
        err = np.abs(o_got - o_ref).max()
        assert err <= 2e-2, (name, h, big_i, err)
        print(f"[fullsize] {name} h={h} I={big_i} kept={cnt} max_abs_err={err:.2e}", flush=True)
    print(f"[mask] {name} sampled rows: {len(rows)} rows; near-tau differences: {n_near_self} against the "
          f"oracle's selection on the GPU's scores, {n_near_e2e} end to end", flush=True)
    assert n_near_e2e <= max(2, len(rows) // 8)
    del bufs, x
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", CASES)
def test_fullsize_whole_layer_selection(xa, name):
    # Every row of the full layer: the oracle's minimal sets, computed on the
    # GPU's own block scores, against the GPU's mask (identical up to blocks
    # whose cumulative mass lies within 1e-5 of tau); and the kept-block lists
    # against the mask.
    w = wl.WORKLOADS[name]
    print(f"[wholelayer] {name}: M={w.M} Hq={w.Hq}", flush=True)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    torch.cuda.synchronize()
    tau = x["tau"].numpy().astype(np.float64)
    del x
    g_sc = f64(bufs.block_scores)
    g_mask = bufs.mask.cpu().numpy()
    kv_idx, kv_cnt = bufs.kv_idx.cpu().numpy(), bufs.kv_cnt.cpu().numpy()
    del bufs
    torch.cuda.empty_cache()
    ref = oracle.select(g_sc, tau, w.causal)
    check_mask(f"{name} whole layer, oracle selection on the GPU's scores", g_mask, ref, g_sc, tau, w.causal,
               1e-5, cap_frac=0.001)
    nb = w.nb
    assert g_mask[..., np.arange(nb), np.arange(nb)].all()
    np.testing.assert_array_equal(kv_cnt, g_mask.astype(bool).sum(-1))
    valid = np.arange(nb)[None, None, None, :] < kv_cnt[..., None]
    cols = np.broadcast_to(np.arange(nb), g_mask.shape)
    np.testing.assert_array_equal(kv_idx[valid], cols[g_mask.astype(bool)])


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
