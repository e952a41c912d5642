"""Large logits: queries scaled by powers of two (exact in bf16 and fp32) so
that the scaled logits reach hundreds in log2 units, where the softmaxes of
both stages are nearly one-hot, the attention's running maximum is raised on
many tiles and most exponentials underflow to zero.

Checked against the oracle as in the other parity tests, with each tolerance
widened by what fp32 accumulation of the logits can shift at that magnitude.
A logit summing n exact bf16 products in fp32 is off by at most
n * 2^-24 * (sum of the products' magnitudes). A strided scoring logit sums
S * C products over S query/key pairs (C products with DuSA1), an attention
logit C products over one pair, so the magnitude sum is at most S (or 1)
times P, the largest sum_c |q_c k_c| over query/key pairs. An error d (after
the scale, natural units) in every logit moves a softmax weight, and so a
block score, by at most 2d relative (numerator and normaliser). It moves an
attention output by at most 2d times max |v|, and its log-sum-exp by d.
Block scores follow the XAttention AI summary, "Approach", and the "DuSA ..."
rebuttal, "Response to Q2"; attention the XAttention arXiv abstract.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import check_index, check_mask, f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    # (pattern, C, block, stride, causal, Hq, Hkv, M, Mk, dtype, alpha)
    ("antidiagonal", 128, 128, 8, True, 4, 2, 1000, 1000, "bf16", 16.0),
    ("antidiagonal", 128, 128, 8, True, 4, 2, 1000, 1000, "bf16", 128.0),
    ("antidiagonal", 64, 64, 4, False, 2, 1, 700, 700, "bf16", 64.0),
    ("antidiagonal", 128, 128, 16, True, 2, 1, 900, 1156, "bf16", -64.0),
    ("antidiagonal", 64, 64, 8, True, 2, 2, 640, 640, "f32", 128.0),
    ("diagonal", 128, 128, 8, True, 2, 1, 1024, 1024, "bf16", 64.0),
    ("dusa1", 128, 128, 8, True, 2, 1, 1024, 1024, "bf16", 64.0),
]


def _ids(c):
    return f"{c[0][:4]}-C{c[1]}b{c[2]}s{c[3]}{'c' if c[4] else 'n'}-h{c[5]}g{c[6]}-M{c[7]}k{c[8]}-{c[9]}-x{c[10]:g}"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _inputs(Hq, Hkv, M, Mk, C, dt, alpha, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn((1, Hq, M, C), generator=g) / math.sqrt(C)
    k = torch.randn((1, Hkv, Mk, C), generator=g) / math.sqrt(C)
    v = torch.randn((1, Hkv, Mk, C), generator=g)
    q[..., 0] += 2.0
    k[:, :, :4, 0] += 6.0
    walk = torch.cumsum(torch.randn((1, Hkv, Mk, C), generator=g) / C, dim=2)
    k += walk
    q += walk[:, :, Mk - M:].repeat_interleave(Hq // Hkv, dim=1)
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    return q * alpha, k, v   # a power of two: exact in either type


def _pair_abs(q64, k64, G):
    """P: the largest sum_c |q_c k_c| over heads and (query, key) pairs"""
    out = 0.0
    for h in range(q64.shape[1]):
        aq, ak = np.abs(q64[0, h]), np.abs(k64[0, h // G])
        out = max(out, float((aq @ ak.T).max()))
    return out


@pytest.mark.parametrize("case", CASES, ids=[_ids(c) for c in CASES])
def test_large_logits(xa, case):
    pattern, C, block, stride, causal, Hq, Hkv, M, Mk, dts, alpha = case
    print(f"[range] {_ids(case)}", flush=True)
    dt = torch.bfloat16 if dts == "bf16" else torch.float32
    q, k, v = _inputs(Hq, Hkv, M, Mk, C, dt, alpha, 4242 + int(abs(alpha)))
    pat = {"antidiagonal": xa.ANTIDIAGONAL, "diagonal": xa.DIAGONAL, "dusa1": xa.DUSA1}[pattern]
    smscale = 1.0 / math.sqrt(C)
    sscale = smscale if pattern == "dusa1" else smscale / stride
    tau = np.array([0.9, 0.95, 0.99, 0.8][:Hq], dtype=np.float32)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    bufs = xa.PrefillBuffers(qd, kd, block, stride, causal, want_lse=True, pattern=pat)
    got = xa.xattn_prefill(qd, kd, vd, torch.from_numpy(tau), block, stride, sscale, smscale, causal,
                           buffers=bufs, pattern=pat)
    torch.cuda.synchronize()
    out = got.out.float()
    assert torch.isfinite(out).all() and torch.isfinite(got.lse).all()

    q64, k64, v64 = f64(q), f64(k), f64(v)
    G = Hq // Hkv
    # the derived fp32-accumulation allowances on top of the usual tolerances
    P = _pair_abs(q64, k64, G)
    u = 2.0 ** -24
    n_sc, pairs_sc = (C, 1) if pattern == "dusa1" else (stride * C, stride)
    d_sc = sscale * n_sc * u * pairs_sc * P     # scoring logit error, natural units
    d_at = smscale * C * u * P                  # attention logit error, natural units
    rel = 1e-4 + 2.0 * d_sc
    ref_sc = oracle.block_scores(q64, k64, block, stride, sscale, causal, pattern=pattern)
    g_sc = f64(got.block_scores)
    err = np.abs(g_sc - ref_sc)
    bad = err > rel * np.abs(ref_sc) + 1e-7
    print(f"[range] P {P:.1f}, score rel tol {rel:.2e}, "
          f"max rel err {(err / (np.abs(ref_sc) + 1e-30)).max() if (ref_sc > 1e-3).any() else 0:.2e}", flush=True)
    assert not bad.any(), (np.argwhere(bad)[:5], err.max())
    # selection on the GPU's own scores
    g_mask = got.mask.cpu().numpy()
    qoff = (Mk - M) // block
    t64 = tau.astype(np.float64)
    check_mask(f"range {_ids(case)}", g_mask, oracle.select(g_sc, t64, causal), g_sc, t64, causal, 1e-5, qoff=qoff)
    check_index(g_mask, got.kv_idx.cpu().numpy(), got.kv_cnt.cpu().numpy())
    # attention with the GPU's mask, and dense attention
    ref_out, ref_lse = oracle.attend(q64, k64, v64, g_mask, block, smscale, causal)
    vmax = float(np.abs(v64).max())
    tol = (2e-2 if dts == "bf16" else 1e-3) + 2.0 * d_at * vmax
    e_out = np.abs(f64(got.out) - ref_out).max()
    e_lse = np.abs(f64(got.lse) - ref_lse).max()
    print(f"[range] density {g_mask.mean():.3f}, out err {e_out:.2e} (tol {tol:.2e}), lse err {e_lse:.2e}",
          flush=True)
    assert e_out <= tol, e_out
    assert e_lse <= 1e-3 * max(1.0, float(np.abs(ref_lse).max())) + d_at, e_lse
    dense, _ = xa.dense_fwd(qd, kd, vd, block, smscale, causal)
    torch.cuda.synchronize()
    full = np.ones_like(g_mask)
    ref_d, _ = oracle.attend(q64, k64, v64, full, block, smscale, causal)
    e_d = np.abs(f64(dense) - ref_d).max()
    print(f"[range] dense out err {e_d:.2e}", flush=True)
    assert e_d <= tol, e_d
