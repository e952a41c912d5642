"""Pins for the CPU oracle: each check rests on something other than the oracle.

* brute force over the full attention matrix (antidiagonal tile sums);
* a hand-worked example stored under tests/golden/;
* the stride-1 closed form (textbook per-block attention mass via scipy softmax);
* exhaustive subset enumeration for the minimal set, per row and over a
  whole head's flattened block matrix (global selection);
* torch's scaled_dot_product_attention (CPU, float64) with an element mask;
* invariants: non-negative scores, rows summing to 1, tau=1 keeps every
  candidate and equals dense attention, monotonicity in tau, diagonal kept.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            rows[key] = np.array([float(x) for x in vals])
    return rows


# ----------------------------------------------------------------- scoring

@pytest.mark.parametrize("stride,m,c", [(2, 16, 3), (4, 32, 5), (8, 64, 2), (1, 8, 4)])
def test_strided_logits_equal_bruteforce_antidiagonal(stride, m, c):
    rng = _rng(stride)
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    full = q @ k.T
    r = m // stride
    brute = np.zeros((r, r))
    for i in range(r):
        for j in range(r):
            # walk the tile's antidiagonal from its lower-left to its upper-right corner
            for a in range(stride):
                brute[i, j] += full[i * stride + stride - 1 - a, j * stride + a]
    got = oracle.strided_logits(q, k, stride, 1.0, causal=False)
    np.testing.assert_allclose(got, brute, rtol=1e-12, atol=1e-12)


def test_strided_logits_are_not_the_diagonal_sums():
    # A dropped reversal would give the main-diagonal tile sums instead.
    rng = _rng(7)
    q = rng.standard_normal((32, 4))
    k = rng.standard_normal((32, 4))
    full = q @ k.T
    s = 4
    diag = np.array([[sum(full[i * s + a, j * s + a] for a in range(s)) for j in range(8)]
                     for i in range(8)])
    got = oracle.strided_logits(q, k, s, 1.0, causal=False)
    assert np.abs(got - diag).max() > 1e-3


def test_strided_logits_causal_mask_and_scale():
    rng = _rng(3)
    q = rng.standard_normal((32, 4))
    k = rng.standard_normal((32, 4))
    a = oracle.strided_logits(q, k, 4, 0.25, causal=True)
    b = oracle.strided_logits(q, k, 4, 1.0, causal=False)
    r = 8
    for i in range(r):
        for j in range(r):
            if j > i:
                assert a[i, j] == -np.inf
            else:
                assert a[i, j] == pytest.approx(0.25 * b[i, j], rel=1e-14)


def test_golden_hand_example():
    g = _read_golden("antidiag_hand_example.txt")
    q = np.array([[1.0], [2.0], [3.0], [4.0]])
    k = np.array([[1.0], [1.0], [2.0], [2.0]])
    a = oracle.strided_logits(q, k, 2, 1.0, causal=False)
    np.testing.assert_array_equal(a.reshape(-1), g["strided_scores"])
    sc = oracle.block_scores(q[None, None], k[None, None], 2, 2, 1.0, causal=True)[0, 0]
    np.testing.assert_allclose(sc[0], g["block_scores_row0"], rtol=1e-15, atol=0)
    np.testing.assert_allclose(sc[1], g["block_scores_row1"], rtol=1e-14, atol=0)
    m9 = oracle.select(sc[None, None], [0.9], causal=True)[0, 0, 1]
    np.testing.assert_array_equal(m9, g["mask_row1_tau0.9"])
    m99 = oracle.select(sc[None, None], [0.9995], causal=True)[0, 0, 1]
    np.testing.assert_array_equal(m99, g["mask_row1_tau0.9995"])


@pytest.mark.parametrize("causal", [True, False])
def test_stride_one_equals_textbook_block_attention_mass(causal):
    # With S=1 each strided cell is a single logit, so the block score is the
    # per-block attention mass averaged over the block's query rows.
    rng = _rng(11)
    m, c, block = 64, 8, 16
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    scale = 0.7
    logits = scale * (q @ k.T)
    if causal:
        logits = np.where(np.tril(np.ones((m, m), dtype=bool)), logits, -np.inf)
    p = scipy.special.softmax(logits, axis=1)
    nb = m // block
    expect = np.zeros((nb, nb))
    for big_i in range(nb):
        for big_j in range(nb):
            expect[big_i, big_j] = p[big_i * block:(big_i + 1) * block,
                                     big_j * block:(big_j + 1) * block].sum() / block
    got = oracle.block_scores(q[None, None], k[None, None], block, 1, scale, causal)[0, 0]
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("stride,r", [(2, 2), (2, 4), (4, 2), (4, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_block_scores_bruteforce_composition(stride, r, causal):
    # The whole scoring stage at S > 1 and r > 1, built from the token-level
    # logit matrix with plain loops: every strided cell walks its S x S tile's
    # antidiagonal (query row descending while the key column ascends), each
    # strided query row is softmaxed over its strided keys (j <= i when causal),
    # and every r x r tile of probabilities is summed and divided by r.
    rng = _rng(100 + 10 * stride + r)
    block = stride * r
    nb, c = 3, 5
    m = nb * block
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    scale = 0.37
    big_r = m // stride
    cell = [[0.0] * big_r for _ in range(big_r)]
    for i in range(big_r):
        for j in range(big_r):
            tot = 0.0
            for a in range(stride):
                tot += float(q[i * stride + stride - 1 - a] @ k[j * stride + a])
            cell[i][j] = scale * tot
    expect = np.zeros((nb, nb))
    for i in range(big_r):
        keys = range(i + 1) if causal else range(big_r)
        top = max(cell[i][j] for j in keys)
        z = sum(math.exp(cell[i][j] - top) for j in keys)
        for j in keys:
            expect[i // r, j // r] += math.exp(cell[i][j] - top) / z / r
    got = oracle.block_scores(q[None, None], k[None, None], block, stride, scale, causal)[0, 0]
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-15)
    # the other score temperatures (the literal sum, and attention on the
    # reshaped rows) only rescale the cells
    for temp in (1.0, 1.0 / math.sqrt(stride)):
        exp2 = np.zeros((nb, nb))
        for i in range(big_r):
            keys = range(i + 1) if causal else range(big_r)
            vals = [temp * cell[i][j] / scale for j in keys]
            top = max(vals)
            z = sum(math.exp(x - top) for x in vals)
            for j, x in zip(keys, vals):
                exp2[i // r, j // r] += math.exp(x - top) / z / r
        got2 = oracle.block_scores(q[None, None], k[None, None], block, stride, temp, causal)[0, 0]
        np.testing.assert_allclose(got2, exp2, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_block_score_invariants(causal):
    rng = _rng(5)
    q = rng.standard_normal((1, 4, 256, 16))
    k = rng.standard_normal((1, 2, 256, 16))
    sc = oracle.block_scores(q, k, 32, 4, 0.3, causal)
    assert (sc >= 0).all()
    np.testing.assert_allclose(sc.sum(axis=-1), 1.0, rtol=1e-12)
    if causal:
        nb = sc.shape[-1]
        upper = np.triu(np.ones((nb, nb), dtype=bool), k=1)
        assert (sc[..., upper] == 0).all()


def test_block_scores_gqa_reads_shared_kv_head():
    rng = _rng(9)
    q = rng.standard_normal((1, 4, 128, 8))
    k = rng.standard_normal((1, 2, 128, 8))
    sc = oracle.block_scores(q, k, 32, 4, 0.5, True)
    # repeat-KV MHA must give the same scores
    k_rep = np.repeat(k, 2, axis=1)
    sc2 = oracle.block_scores(q, k_rep, 32, 4, 0.5, True)
    np.testing.assert_array_equal(sc, sc2)
    # and head 1 must differ from using KV head 1 instead of 0
    wrong = oracle.block_scores(q[:, 1:2], k[:, 1:2], 32, 4, 0.5, True)
    assert np.abs(wrong[0, 0] - sc[0, 1]).max() > 1e-6


# --------------------------------------------------------------- selection

def test_minimal_set_matches_exhaustive_search():
    rng = _rng(21)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        cand = rng.dirichlet(np.full(n, 0.5))
        if trial % 5 == 0:                       # force ties
            cand = np.round(cand * 4) / 4
        tau = float(rng.choice([0.0, 0.3, 0.5, 0.8, 0.9, 0.95, 0.999, 1.0]))
        total = cand.sum()
        kept = oracle.minimal_set(cand, tau)
        if tau >= 1.0:
            assert len(kept) == n
            continue
        best = None
        for size in range(0, n + 1):
            for sub in itertools.combinations(range(n), size):
                if cand[list(sub)].sum() >= tau * total:
                    best = size
                    break
            if best is not None:
                break
        assert len(kept) == best, (cand, tau, kept)
        assert cand[kept].sum() >= tau * total


def test_minimal_set_tie_break_by_ascending_index():
    cand = np.array([0.25, 0.25, 0.25, 0.25])
    np.testing.assert_array_equal(oracle.minimal_set(cand, 0.5), [0, 1])
    cand = np.array([0.1, 0.3, 0.3, 0.3])
    np.testing.assert_array_equal(oracle.minimal_set(cand, 0.6), [1, 2])


def test_select_invariants():
    rng = _rng(4)
    q = rng.standard_normal((1, 2, 512, 16))
    k = rng.standard_normal((1, 1, 512, 16))
    sc = oracle.block_scores(q, k, 32, 4, 0.5, True)
    nb = sc.shape[-1]
    lower = np.tril(np.ones((nb, nb), dtype=bool))
    prev = None
    for tau in [0.0, 0.5, 0.8, 0.9, 0.99, 1.0]:
        mk = oracle.select(sc, [tau, tau], True).astype(bool)
        assert mk[..., np.arange(nb), np.arange(nb)].all()          # diagonal kept
        assert not mk[..., ~lower].any()                              # causal candidates only
        if prev is not None:
            assert (mk >= prev).all()                                 # monotone in tau
        prev = mk
    assert prev[..., lower].all()                                     # tau = 1: everything
    only_diag = oracle.select(sc, [0.0, 0.0], True).astype(bool)
    assert only_diag.sum() == 2 * nb


def _candidates(nb, causal):
    return [(i, j) for i in range(nb) for j in range(i + 1 if causal else nb)]


@pytest.mark.parametrize("causal", [True, False])
def test_global_selection_matches_exhaustive_search(causal):
    # the kept set is the top-m* candidates in (score desc, (I, J) row-major)
    # order, m* the smallest size any candidate subset needs to reach tau * T,
    # found by enumerating subsets; then every diagonal block is added
    rng = _rng(31 if causal else 32)
    for trial in range(120):
        nb = int(rng.integers(1, 5 if causal else 4))
        sc = rng.dirichlet(np.full(nb, 0.6), size=nb)
        if causal:
            sc = np.tril(sc)
            sc /= sc.sum(axis=1, keepdims=True)
        if trial % 4 == 0:
            sc = np.round(sc * 4) / 4                      # ties, zeros
        tau = float(rng.choice([0.0, 0.3, 0.6, 0.8, 0.9, 0.97, 1.0]))
        got = oracle.select_global_head(sc, tau, causal)
        cands = _candidates(nb, causal)
        vals = np.array([sc[i, j] for i, j in cands])
        total = vals.sum()
        if tau >= 1.0:
            m_star = len(cands)
        else:
            m_star = None
            for size in range(len(cands) + 1):
                if any(vals[list(sub)].sum() >= tau * total
                       for sub in itertools.combinations(range(len(cands)), size)):
                    m_star = size
                    break
        order = sorted(range(len(cands)), key=lambda t: (-vals[t], t))
        want = np.zeros((nb, nb), dtype=bool)
        for t in order[:m_star]:
            want[cands[t]] = True
        want[np.arange(nb), np.arange(nb)] = True
        np.testing.assert_array_equal(got, want, err_msg=f"{sc} tau={tau}")


def test_global_selection_invariants():
    rng = _rng(5)
    q = rng.standard_normal((1, 1, 512, 16))
    k = rng.standard_normal((1, 1, 512, 16))
    sc = oracle.block_scores(q, k, 32, 4, 0.5, True)
    nb = sc.shape[-1]
    lower = np.tril(np.ones((nb, nb), dtype=bool))
    prev = None
    for tau in [0.0, 0.4, 0.8, 0.95, 1.0]:
        mk = oracle.select(sc, [tau], True, mode="global").astype(bool)[0, 0]
        assert mk[np.arange(nb), np.arange(nb)].all()
        assert not mk[~lower].any()
        # the kept mass reaches tau * T (T = NB: every row sums to 1)
        assert sc[0, 0][mk].sum() >= tau * nb - 1e-12
        if prev is not None:
            assert (mk >= prev).all()
        prev = mk
    assert prev[lower].all()
    # global differs from per-row selection on the same scores (mass moves
    # between rows), yet keeps a comparable number of blocks
    row = oracle.select(sc, [0.8], True).astype(bool)[0, 0]
    glob = oracle.select(sc, [0.8], True, mode="global").astype(bool)[0, 0]
    assert (row != glob).any()


def test_gqa_union_groups_consecutive_heads():
    # head h marks only block (h + 1, 0); with Hkv = 2 the groups are heads
    # {0, 1, 2} and {3, 4, 5} (h // 3), not h % 2
    b, hq, hkv, nb = 1, 6, 2, 8
    mk = np.zeros((b, hq, nb, nb), dtype=np.uint8)
    for h in range(hq):
        mk[0, h, h + 1, 0] = 1
    u = oracle.gqa_union(mk, hkv).astype(bool)
    for h in range(hq):
        group = range(3 * (h // 3), 3 * (h // 3) + 3)
        want = np.zeros((nb, nb), dtype=bool)
        for hh in group:
            want[hh + 1, 0] = True
        np.testing.assert_array_equal(u[0, h], want)


def test_gqa_union_selection_contains_each_head():
    rng = _rng(6)
    q = rng.standard_normal((1, 4, 256, 16))
    k = rng.standard_normal((1, 2, 256, 16))
    sc = oracle.block_scores(q, k, 32, 4, 0.5, True)
    tau = [0.5, 0.9, 0.7, 0.3]
    row = oracle.select(sc, tau, True).astype(bool)
    uni = oracle.select(sc, tau, True, mode="gqa_union", hkv=2).astype(bool)
    assert (uni >= row).all()
    assert (uni[0, 0] == uni[0, 1]).all() and (uni[0, 2] == uni[0, 3]).all()
    assert (uni[0, 0] == (row[0, 0] | row[0, 1])).all()
    # with one head per KV head the union is the per-row selection
    k4 = rng.standard_normal((1, 4, 256, 16))
    sc4 = oracle.block_scores(q, k4, 32, 4, 0.5, True)
    np.testing.assert_array_equal(oracle.select(sc4, tau, True, mode="gqa_union", hkv=4),
                                  oracle.select(sc4, tau, True))


def test_tau_one_keeps_underflowed_blocks():
    row = np.array([1.0, 0.0, 0.0, 0.0])
    keep = oracle.select_row(row, 3, 1.0, True)
    assert keep.all()


def test_mask_to_index():
    mk = np.array([[[[1, 0, 1, 0], [0, 1, 0, 0], [1, 1, 1, 0], [0, 0, 0, 1]]]], dtype=np.uint8)
    idx, cnt = oracle.mask_to_index(mk)
    np.testing.assert_array_equal(cnt[0, 0], [2, 1, 3, 1])
    np.testing.assert_array_equal(idx[0, 0, 0, :2], [0, 2])
    np.testing.assert_array_equal(idx[0, 0, 2, :3], [0, 1, 2])
    assert idx[0, 0, 1, 1] == -1


# --------------------------------------------------------------- attention

def _sdpa_masked(q, k, v, mask, block, scale, causal):
    """torch SDPA on the CPU in float64 with the block mask expanded to elements
    (cropped to Mq x Mk; causal with the queries the last Mq of Mk tokens)."""
    hq, hkv = q.shape[1], k.shape[1]
    mq, mk = q.shape[2], k.shape[2]
    kr = torch.from_numpy(np.repeat(k, hq // hkv, axis=1))
    vr = torch.from_numpy(np.repeat(v, hq // hkv, axis=1))
    elem = np.repeat(np.repeat(mask.astype(bool), block, axis=-2), block, axis=-1)[..., :mq, :mk]
    if causal:
        elem = elem & np.tril(np.ones((mq, mk), dtype=bool), k=mk - mq)
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), kr, vr, attn_mask=torch.from_numpy(elem), scale=scale)
    logits = scale * torch.from_numpy(q) @ kr.transpose(-1, -2)
    logits = logits.masked_fill(~torch.from_numpy(elem), float("-inf"))
    return out.numpy(), torch.logsumexp(logits, dim=-1).numpy()


@pytest.mark.parametrize("causal", [True, False])
def test_attend_matches_sdpa_with_element_mask(causal):
    rng = _rng(13)
    q = rng.standard_normal((1, 4, 128, 16))
    k = rng.standard_normal((1, 2, 128, 16))
    v = rng.standard_normal((1, 2, 128, 16))
    nb = 8
    mask = (rng.random((1, 4, nb, nb)) < 0.4).astype(np.uint8)
    mask[..., np.arange(nb), np.arange(nb)] = 1
    if causal:
        mask = mask * np.tril(np.ones((nb, nb), dtype=np.uint8))
    out, lse = oracle.attend(q, k, v, mask, 16, 0.25, causal)
    ref, ref_lse = _sdpa_masked(q, k, v, mask, 16, 0.25, causal)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_tau_one_equals_dense_causal_sdpa():
    rng = _rng(17)
    q = rng.standard_normal((1, 2, 128, 16))
    k = rng.standard_normal((1, 1, 128, 16))
    v = rng.standard_normal((1, 1, 128, 16))
    sc, mk, out, lse = oracle.prefill(q, k, v, 16, 4, [1.0, 1.0], 0.0625, 0.25, True)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(np.repeat(k, 2, axis=1)),
        torch.from_numpy(np.repeat(v, 2, axis=1)), is_causal=True, scale=0.25).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    d_out, _ = oracle.dense(q, k, v, 16, 0.25, True)
    np.testing.assert_allclose(d_out, ref, rtol=1e-10, atol=1e-12)


def test_density_counts_candidates():
    nb = 4
    mk = np.tril(np.ones((1, 1, nb, nb), dtype=np.uint8))
    assert oracle.density(mk, True) == 1.0
    eye = np.eye(nb, dtype=np.uint8)[None, None]
    assert oracle.density(eye, True) == pytest.approx(4 / 10)
    assert oracle.density(eye, False) == pytest.approx(4 / 16)


@pytest.mark.parametrize("stride,m,c", [(2, 16, 3), (4, 32, 5), (8, 64, 2)])
def test_diagonal_pattern_equals_bruteforce_diagonal(stride, m, c):
    # the older diagonal variant: main diagonal of each stride x stride tile
    rng = _rng(40 + stride)
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    full = q @ k.T
    r = m // stride
    brute = np.array([[sum(full[i * stride + a, j * stride + a] for a in range(stride))
                       for j in range(r)] for i in range(r)])
    got = oracle.strided_logits(q, k, stride, 1.0, causal=False, pattern="diagonal")
    np.testing.assert_allclose(got, brute, rtol=1e-12, atol=1e-12)
    anti = oracle.strided_logits(q, k, stride, 1.0, causal=False)
    assert np.abs(anti - got).max() > 1e-3


def test_diagonal_pattern_block_scores_are_normalised():
    rng = _rng(44)
    q = rng.standard_normal((1, 2, 256, 16))
    k = rng.standard_normal((1, 1, 256, 16))
    sc = oracle.block_scores(q, k, 32, 4, 0.3, True, pattern="diagonal")
    np.testing.assert_allclose(sc.sum(-1), 1.0, rtol=1e-12)
    assert (sc >= 0).all()


# ------------------------------------------------ ragged and chunked lengths

@pytest.mark.parametrize("stride,mq,mk,c", [(4, 30, 30, 3), (8, 61, 61, 2), (2, 7, 15, 4), (4, 13, 29, 3)])
@pytest.mark.parametrize("causal", [True, False])
def test_ragged_strided_logits_equal_bruteforce(stride, mq, mk, c, causal):
    # tokens past the end of a partial stride group count as zero vectors; the
    # queries are the last mq of mk tokens (strided offset (mk - mq) / stride)
    rng = _rng(stride + mq)
    q = rng.standard_normal((mq, c))
    k = rng.standard_normal((mk, c))
    rq, rk = -(-mq // stride), -(-mk // stride)
    off_s = (mk - mq) // stride
    brute = np.zeros((rq, rk))
    for i in range(rq):
        for j in range(rk):
            for a in range(stride):
                qi, kj = i * stride + stride - 1 - a, j * stride + a
                if qi < mq and kj < mk:
                    brute[i, j] += q[qi] @ k[kj]
            if causal and j > i + off_s:
                brute[i, j] = -np.inf
    got = oracle.strided_logits(q, k, stride, 1.0, causal)
    np.testing.assert_allclose(got, brute, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_stride_one_ragged_equals_textbook_block_attention_mass(causal):
    # S = 1, M = 61 with 16-row blocks: the last block holds 13 queries and 13
    # keys; its score row averages over its 13 real rows
    rng = _rng(12)
    m, c, block = 61, 8, 16
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    scale = 0.6
    logits = scale * (q @ k.T)
    if causal:
        logits = np.where(np.tril(np.ones((m, m), dtype=bool)), logits, -np.inf)
    p = scipy.special.softmax(logits, axis=1)
    nb = -(-m // block)
    expect = np.zeros((nb, nb))
    for big_i in range(nb):
        rows = p[big_i * block:(big_i + 1) * block]
        for big_j in range(nb):
            expect[big_i, big_j] = rows[:, big_j * block:(big_j + 1) * block].sum() / rows.shape[0]
    got = oracle.block_scores(q[None, None], k[None, None], block, 1, scale, causal)[0, 0]
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(got.sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_chunk_equals_last_rows_of_full_sequence(causal):
    # queries = the last mq tokens of the sequence: the chunk's block scores,
    # per-row selection and attention equal the last rows of the full run
    rng = _rng(14)
    mk, off, block, stride, c = 200, 64, 32, 4, 8      # NBk = 7 (last block 8 keys)
    q = rng.standard_normal((1, 2, mk, c))
    k = rng.standard_normal((1, 1, mk, c))
    v = rng.standard_normal((1, 1, mk, c))
    qc = q[:, :, off:]
    full = oracle.block_scores(q, k, block, stride, 0.4, causal)
    chunk = oracle.block_scores(qc, k, block, stride, 0.4, causal)
    assert chunk.shape == (1, 2, 5, 7)
    np.testing.assert_allclose(chunk, full[:, :, off // block:], rtol=1e-12, atol=1e-15)
    tau = [0.8, 0.95]
    mf = oracle.select(full, tau, causal)
    mc = oracle.select(chunk, tau, causal)
    np.testing.assert_array_equal(mc, mf[:, :, off // block:])
    of, lf = oracle.attend(q, k, v, mf, block, 0.3, causal)
    oc, lc = oracle.attend(qc, k, v, mc, block, 0.3, causal)
    np.testing.assert_allclose(oc, of[:, :, off:], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lc, lf[:, :, off:], rtol=1e-12, atol=1e-13)
    assert oracle.density(mc, causal) > 0


@pytest.mark.parametrize("causal", [True, False])
def test_attend_ragged_chunk_matches_sdpa(causal):
    rng = _rng(15)
    mq, mk, block = 100, 164, 32                         # NBq = 4, NBk = 6, offset 2 blocks
    q = rng.standard_normal((1, 2, mq, 16))
    k = rng.standard_normal((1, 1, mk, 16))
    v = rng.standard_normal((1, 1, mk, 16))
    nbq, nbk = 4, 6
    mask = (rng.random((1, 2, nbq, nbk)) < 0.4).astype(np.uint8)
    mask[..., np.arange(nbq), np.arange(nbq) + 2] = 1
    if causal:
        mask = mask * np.tril(np.ones((nbq, nbk), dtype=np.uint8), k=2)
    out, lse = oracle.attend(q, k, v, mask, block, 0.25, causal)
    ref, ref_lse = _sdpa_masked(q, k, v, mask, block, 0.25, causal)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)
    # tau = 1 keeps every candidate: dense attention over the chunk
    sc = oracle.block_scores(q, k, block, 4, 0.3, causal)
    np.testing.assert_allclose(sc.sum(axis=-1), 1.0, rtol=1e-12)
    mk1 = oracle.select(sc, [1.0, 1.0], causal)
    full = np.ones((1, 2, nbq, nbk), dtype=np.uint8)
    if causal:
        full = full * np.tril(np.ones((nbq, nbk), dtype=np.uint8), k=2)
    np.testing.assert_array_equal(mk1, full)
    o1, _ = oracle.attend(q, k, v, mk1, block, 0.25, causal)
    d1, _ = _sdpa_masked(q, k, v, full, block, 0.25, causal)
    np.testing.assert_allclose(o1, d1, rtol=1e-10, atol=1e-12)


def test_global_selection_chunk_exhaustive():
    # rectangular (chunked) block matrices: candidates J <= I + NBk - NBq
    rng = _rng(33)
    for trial in range(80):
        nbq = int(rng.integers(1, 3))
        qoff = int(rng.integers(1, 3))
        nbk = nbq + qoff
        sc = np.tril(rng.dirichlet(np.full(nbk, 0.6), size=nbq), k=qoff)
        if trial % 4 == 0:
            sc = np.round(sc * 4) / 4
        tau = float(rng.choice([0.0, 0.5, 0.8, 0.95, 1.0]))
        got = oracle.select_global_head(sc, tau, True)
        cands = [(i, j) for i in range(nbq) for j in range(i + qoff + 1)]
        vals = np.array([sc[i, j] for i, j in cands])
        if tau >= 1.0:
            m_star = len(cands)
        else:
            m_star = next(size for size in range(len(cands) + 1)
                          if any(vals[list(sub)].sum() >= tau * vals.sum()
                                 for sub in itertools.combinations(range(len(cands)), size)))
        order = sorted(range(len(cands)), key=lambda t: (-vals[t], t))
        want = np.zeros((nbq, nbk), dtype=bool)
        for t in order[:m_star]:
            want[cands[t]] = True
        want[np.arange(nbq), np.arange(nbq) + qoff] = True
        np.testing.assert_array_equal(got, want)


# ------------------------------------------------------- DuSA1 multi-stride scoring

@pytest.mark.parametrize("stride,r", [(2, 2), (2, 4), (4, 2), (4, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_dusa1_block_scores_bruteforce(stride, r, causal):
    # From the token-level logits with loops: phase s keeps tokens s, s+S, ...;
    # each phase row is softmaxed over the phase's keys (j <= i when causal),
    # and the probabilities of the S * r phase rows of a query block are summed
    # per key block and divided by S * r.
    rng = _rng(300 + 10 * stride + r)
    block = stride * r
    nb, c = 3, 4
    m = nb * block
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    scale = 0.45
    big_r = m // stride
    expect = np.zeros((nb, nb))
    for s in range(stride):
        for i in range(big_r):
            keys = range(i + 1) if causal else range(big_r)
            vals = [scale * float(q[i * stride + s] @ k[j * stride + s]) for j in keys]
            top = max(vals)
            z = sum(math.exp(v - top) for v in vals)
            for j, v in zip(keys, vals):
                expect[i // r, j // r] += math.exp(v - top) / z / (stride * r)
    got = oracle.block_scores(q[None, None], k[None, None], block, stride, scale, causal, pattern="dusa1")[0, 0]
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-15)
    # not the diagonal XAttention pattern, which sums the phases' logits before
    # one softmax per strided row
    diag = oracle.block_scores(q[None, None], k[None, None], block, stride, scale, causal, pattern="diagonal")[0, 0]
    assert np.abs(got - diag).max() > 1e-3


@pytest.mark.parametrize("causal", [True, False])
def test_dusa1_stride_one_is_the_block_attention_mass(causal):
    # one phase: the textbook per-block attention mass averaged over the block's rows
    rng = _rng(17)
    m, c, block = 48, 5, 8
    q = rng.standard_normal((m, c))
    k = rng.standard_normal((m, c))
    logits = 0.6 * (q @ k.T)
    if causal:
        logits = np.where(np.tril(np.ones((m, m), dtype=bool)), logits, -np.inf)
    p = scipy.special.softmax(logits, axis=1)
    nb = m // block
    expect = p.reshape(nb, block, nb, block).sum(axis=(1, 3)) / block
    got = oracle.block_scores(q[None, None], k[None, None], block, 1, 0.6, causal, pattern="dusa1")[0, 0]
    np.testing.assert_allclose(got, expect, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_dusa1_invariants_and_chunk(causal):
    rng = _rng(23)
    q = rng.standard_normal((1, 2, 256, 8))
    k = rng.standard_normal((1, 1, 256, 8))
    sc = oracle.block_scores(q, k, 32, 4, 0.5, causal, pattern="dusa1")
    assert (sc >= 0).all()
    np.testing.assert_allclose(sc.sum(-1), 1.0, rtol=1e-12)
    if causal:
        assert (sc[..., np.triu(np.ones((8, 8), dtype=bool), 1)] == 0).all()
    # the last 96 queries against all 256 keys score like the last 3 rows of the full run
    part = oracle.block_scores(q[:, :, 160:], k, 32, 4, 0.5, causal, pattern="dusa1")
    np.testing.assert_allclose(part, sc[:, :, 5:], rtol=1e-12, atol=1e-15)
    with pytest.raises(ValueError):
        oracle.block_scores(q[:, :, :250], k[:, :, :250], 32, 4, 0.5, causal, pattern="dusa1")
