"""Seeded random problems across the whole interface: ragged and chunked lengths,
both head sizes and block sizes, every block/stride ratio, GQA group sizes
1-4 and 8, batch 1-2, causal and not, the three scoring patterns, the three
selection modes, selection inside the scoring launch, bf16 and fp32.

Each problem runs xattn_prefill and the staged calls (xattn_score, then
xattn_select, then bsa_fwd), which must agree bit for bit (and so must the
one-launch form where it applies); then the oracle: block scores element by
element (XAttention AI summary, "Approach"; "DuSA ..." rebuttal, "Response to
Q2"), the per-row selection on the GPU's own scores (FlexPrefill rebuttal,
"R Q3"), and attention with the GPU's mask (XAttention arXiv abstract), at the
same tolerances as the other parity tests.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import check_index, check_mask, f64, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_CASES = 96


def _case(seed, group=None):
    rng = np.random.default_rng(1000 + seed)
    C = int(rng.choice([64, 128]))
    block = int(rng.choice([64, 128]))
    r = int(rng.choice([2, 4, 8, 16, 32]))
    stride = block // r
    hkv = int(rng.choice([1, 2]))
    hq = hkv * int(rng.integers(1, 5))
    if group is not None:
        hq = hkv * group
    B = int(rng.choice([1, 1, 2]))
    causal = bool(rng.random() < 0.7)
    pattern = str(rng.choice(["antidiagonal", "antidiagonal", "antidiagonal", "diagonal", "dusa1"]))
    dtype = "f32" if (pattern != "dusa1" and rng.random() < 0.15) else "bf16"
    selection = str(rng.choice(["row", "row", "row", "global", "gqa_union"]))
    nbq = int(rng.integers(1, 11))
    M = nbq * block - int(rng.integers(0, block))          # a ragged last block
    Mk = M + block * int(rng.choice([0, 0, 1, 3]))          # chunked prefill
    if pattern == "dusa1":                                   # lengths multiples of the stride
        M, Mk = M - M % stride or stride, Mk - Mk % stride or stride
        Mk = max(Mk, M)
        Mk = M + ((Mk - M) // block) * block
    tau = rng.choice([0.5, 0.8, 0.9, 0.95, 0.99, 1.0], size=hq).astype(np.float32)
    return dict(C=C, block=block, stride=stride, Hkv=hkv, Hq=hq, B=B, causal=causal, pattern=pattern,
                dtype=dtype, selection=selection, M=M, Mk=Mk, tau=tau, seed=seed)


# and eight with GQA groups of 8 (sibling pairs of four per KV head)
CASES = [_case(i) for i in range(N_CASES)] + [_case(i, group=8) for i in range(N_CASES, N_CASES + 8)]


def _ids(c):
    return (f"{c['seed']}-{c['dtype']}-{c['pattern'][:4]}-{c['selection']}-B{c['B']}h{c['Hq']}g{c['Hkv']}-"
            f"M{c['M']}k{c['Mk']}-C{c['C']}b{c['block']}s{c['stride']}{'c' if c['causal'] else 'n'}")


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _inputs(c):
    # sink- and local-heavy rows, so the selections are neither empty nor full
    g = torch.Generator().manual_seed(77 + c["seed"])
    B, Hq, Hkv, M, Mk, C = c["B"], c["Hq"], c["Hkv"], c["M"], c["Mk"], c["C"]
    q = torch.randn((B, Hq, M, C), generator=g) / math.sqrt(C)
    k = torch.randn((B, Hkv, Mk, C), generator=g) / math.sqrt(C)
    v = torch.randn((B, Hkv, Mk, C), generator=g)
    q[..., 0] += 2.0
    k[:, :, :4, 0] += 6.0
    walk = torch.cumsum(torch.randn((B, Hkv, Mk, C), generator=g) / C, dim=2)
    k += walk
    q += walk[:, :, Mk - M:].repeat_interleave(Hq // Hkv, dim=1)
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    return q.to(dt), k.to(dt), v.to(dt)


def _equal(a, b):
    assert torch.equal(a.block_scores, b.block_scores)
    assert torch.equal(a.mask, b.mask)
    assert torch.equal(a.kv_cnt, b.kv_cnt)
    valid = torch.arange(a.kv_idx.shape[-1], device=DEV) < a.kv_cnt[..., None]
    assert torch.equal(a.kv_idx[valid], b.kv_idx[valid])
    assert torch.equal(a.out, b.out)


class _Staged:
    pass


@pytest.mark.parametrize("c", CASES, ids=[_ids(c) for c in CASES])
def test_random_problem(xa, c):
    print(f"[random] {_ids(c)}", flush=True)
    q, k, v = _inputs(c)
    pat = {"antidiagonal": xa.ANTIDIAGONAL, "diagonal": xa.DIAGONAL, "dusa1": xa.DUSA1}[c["pattern"]]
    block, stride, causal, C = c["block"], c["stride"], c["causal"], c["C"]
    smscale = 1.0 / math.sqrt(C)
    sscale = smscale if c["pattern"] == "dusa1" else smscale / stride
    tau = torch.from_numpy(c["tau"])
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sel = c["selection"]
    got = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, causal, pattern=pat, selection=sel)
    # the staged calls
    st = _Staged()
    st.block_scores = xa.xattn_score(qd, kd, block, stride, sscale, causal, pattern=pat)
    st.mask, st.kv_idx, st.kv_cnt = xa.xattn_select(st.block_scores, tau, block, stride, causal, Hkv=c["Hkv"], C=C,
                                                    dtype=qd.dtype, selection=sel)
    st.out, _ = xa.bsa_fwd(qd, kd, vd, st.kv_idx, st.kv_cnt, block, smscale, causal, selection=sel)
    torch.cuda.synchronize()
    _equal(got, st)
    if sel != "global":
        one = xa.xattn_prefill(qd, kd, vd, tau, block, stride, sscale, smscale, causal, pattern=pat, selection=sel,
                               select_in_score=True)
        torch.cuda.synchronize()
        _equal(got, one)
    # the oracle
    q64, k64, v64 = f64(q), f64(k), f64(v)
    ref_sc = oracle.block_scores(q64, k64, block, stride, sscale, causal, pattern=c["pattern"])
    g_sc = f64(got.block_scores)
    bad = np.abs(g_sc - ref_sc) > score_tol(ref_sc)
    assert not bad.any(), (np.argwhere(bad)[:5], np.abs(g_sc - ref_sc).max())
    g_mask = got.mask.cpu().numpy()
    t64 = c["tau"].astype(np.float64)
    qoff = (c["Mk"] - c["M"]) // block
    if sel == "row":
        check_mask(f"random {c['seed']}", g_mask, oracle.select(g_sc, t64, causal), g_sc, t64, causal, 1e-5, qoff=qoff)
    else:
        # every diagonal block kept; with GQA union the siblings share their lists
        nbq = g_mask.shape[2]
        assert (g_mask[..., np.arange(nbq), np.arange(nbq) + qoff] == 1).all()
        if sel == "gqa_union":
            G = c["Hq"] // c["Hkv"]
            grp = g_mask.reshape(c["B"], c["Hkv"], G, nbq, -1)
            assert (grp == grp[:, :, :1]).all()
    check_index(g_mask, got.kv_idx.cpu().numpy(), got.kv_cnt.cpu().numpy())
    ref_out, _ = oracle.attend(q64, k64, v64, g_mask, block, smscale, causal)
    err = np.abs(f64(got.out) - ref_out).max()
    tol = 2e-2 if c["dtype"] == "bf16" else 1e-3
    print(f"[random] {c['seed']}: density {g_mask.mean():.3f}, max_abs_err {err:.2e}", flush=True)
    assert err <= tol, err
