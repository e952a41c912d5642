"""GPU parity of the scoring launches that run persistent workgroups (at least
two 256 x 256 strided tiles per resident workgroup, and a contraction of at
least eight 32-element chunks): each workgroup walks several tiles and fetches
the next tile's first chunks while it finishes the current one. Shapes cover
the smallest contraction the form takes (eight chunks: S*C = 256), head sizes
64 and 128, non-causal problems, chunked prefill (the trapezoid of tiles) and
the diagonal pattern. Sampled rows, first and last query blocks included, are
recomputed by the oracle; block scores must agree to |g - o| <= 1e-4 |o| + 1e-7
and each row must sum to 1.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import f64, score_tol

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# B, Hq, Hkv, Mq, Mk, C, block, stride, causal, pattern; each has >= 512 tiles
CASES = [
    (1, 16, 4, 8192, 8192, 64, 64, 4, True, "antidiagonal"),      # 576 tiles, 8 chunks
    (1, 8, 2, 8192, 8192, 64, 64, 4, False, "antidiagonal"),      # 512 tiles
    (1, 16, 16, 4096, 4096, 128, 64, 2, True, "antidiagonal"),    # 576 tiles, 8 chunks, r = 32
    (1, 32, 8, 8192, 32768, 128, 128, 8, True, "antidiagonal"),   # chunked: 1856 tiles
    (1, 16, 4, 16384, 16384, 128, 128, 8, True, "diagonal"),      # 576 tiles
    (2, 8, 2, 8192, 8192, 64, 64, 4, True, "antidiagonal"),       # two batch entries: 576 tiles
]


def _ids(c):
    return f"B{c[0]}-h{c[1]}-{c[3]}of{c[4]}-C{c[5]}-b{c[6]}-s{c[7]}-{'c' if c[8] else 'n'}-{c[9]}"


@pytest.fixture(scope="module")
def xa():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_attention_xattn_amd as x
    return x


def _tiles(B, Hq, Mq, Mk, stride, causal, tile=256):
    rq, rk = Mq // stride, Mk // stride
    tq, tk = -(-rq // tile), -(-rk // tile)
    c0 = -(-((Mk - Mq) // stride) // tile)
    pairs = sum(min(tk, t + c0 + 1) for t in range(tq)) if causal else tq * tk
    return B * Hq * pairs


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_persistent_scoring_sampled_rows(xa, case):
    B, Hq, Hkv, Mq, Mk, C, block, stride, causal, pattern = case
    assert _tiles(B, Hq, Mq, Mk, stride, causal) >= 512 and stride * C // 32 >= 8
    print(f"[persistent] {_ids(case)}", flush=True)
    g = torch.Generator().manual_seed(Mq + Mk + C + stride)
    k = torch.randn((B, Hkv, Mk, C), generator=g)
    k[:, :, ::61] *= 3.0   # a few strong key columns
    q = torch.randn((B, Hq, Mq, C), generator=g)
    q, k = q.to(torch.bfloat16), k.to(torch.bfloat16)
    pat = {"antidiagonal": xa.ANTIDIAGONAL, "diagonal": xa.DIAGONAL}[pattern]
    ss = 1.0 / (stride * math.sqrt(C))
    sc = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, ss, causal, pattern=pat)
    torch.cuda.synchronize()
    got_all = f64(sc)
    nbq = Mq // block
    np.testing.assert_allclose(got_all.sum(axis=-1), 1.0, rtol=1e-4)
    rng = np.random.default_rng(7)
    rows = {(0, 0, 0), (B - 1, Hq - 1, nbq - 1)}
    rows |= {(int(b), int(h), int(i)) for b, h, i in
             zip(rng.integers(0, B, 10), rng.integers(0, Hq, 10), rng.integers(0, nbq, 10))}
    G = Hq // Hkv
    for b, h, big_i in sorted(rows):
        ref = oracle.block_score_row(f64(q[b, h]), f64(k[b, h // G]), big_i, block, stride, ss, causal,
                                     pattern=pattern)
        got = got_all[b, h, big_i]
        bad = np.abs(got - ref) > score_tol(ref)
        assert not bad.any(), (b, h, big_i, np.nonzero(bad)[0][:5], np.abs(got - ref).max())
    print(f"[persistent] {_ids(case)}: {len(rows)} rows within tolerance", flush=True)
