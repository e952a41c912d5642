"""GPU parity: every stage of the HIP path against the CPU oracle, element by
element, through the C ABI (via the thin ctypes binding).

Tolerances (from the method's acceptance bar):
  block scores |g - o| <= 1e-4 |o| + 1e-7;  bf16 outputs max-abs <= 2e-2;
  fp32 outputs max-abs <= 1e-3;  masks identical up to near-tau blocks.
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


def _rand(shape, seed, dtype, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    t = torch.randn(shape, generator=g) * scale
    return t.to(dtype)


def _inputs(B, Hq, Hkv, M, C, dtype, seed, structured=False):
    if structured:
        fam = "llama" if dtype == torch.bfloat16 else "tiny"
        w = wl.WORKLOADS["llama8k" if fam == "llama" else "tiny"].scaled(B=B, Hq=Hq, Hkv=Hkv, M=M, C=C)
        x = wl.make_inputs(w)
        return x["q"], x["k"], x["v"]
    q = _rand((B, Hq, M, C), seed, dtype)
    k = _rand((B, Hkv, M, C), seed + 1, dtype)
    v = _rand((B, Hkv, M, C), seed + 2, dtype)
    return q, k, v


def _bf16_tol(dtype):
    return 2e-2 if dtype == torch.bfloat16 else 1e-3


# ------------------------------------------------------------------ attention

ATTN_CASES = [
    # B, Hq, Hkv, M, C, block, causal, dtype
    (1, 4, 2, 512, 128, 128, True, torch.bfloat16),
    (1, 4, 4, 384, 128, 128, False, torch.bfloat16),
    (2, 2, 1, 256, 64, 64, True, torch.bfloat16),
    (1, 2, 2, 256, 64, 128, False, torch.bfloat16),
    (1, 8, 2, 128, 128, 128, True, torch.bfloat16),   # a single block
    (1, 2, 1, 256, 128, 64, True, torch.bfloat16),
    (1, 3, 1, 640, 128, 128, True, torch.bfloat16),   # odd group, odd block count
    (1, 2, 2, 896, 64, 128, True, torch.bfloat16),    # one query head per KV head
    (1, 1, 1, 512, 64, 64, True, torch.float32),
    (1, 2, 1, 256, 128, 128, False, torch.float32),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c[:7])) + str(c[7])[-4:])
def test_dense_fwd_matches_oracle(xa, case):
    B, Hq, Hkv, M, C, block, causal, dtype = case
    q, k, v = _inputs(B, Hq, Hkv, M, C, dtype, 100 + M)
    scale = 1.0 / math.sqrt(C)
    out, lse = xa.dense_fwd(q.to(DEV), k.to(DEV), v.to(DEV), block, scale, causal, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.dense(f64(q), f64(k), f64(v), block, scale, causal)
    err = np.abs(f64(out) - ref).max()
    assert err <= _bf16_tol(dtype), err
    assert np.abs(f64(lse) - ref_lse).max() <= 2e-3


@pytest.mark.parametrize("case", ATTN_CASES, ids=lambda c: "-".join(map(str, c[:7])) + str(c[7])[-4:])
def test_bsa_fwd_matches_oracle_with_given_mask(xa, case):
    B, Hq, Hkv, M, C, block, causal, dtype = case
    q, k, v = _inputs(B, Hq, Hkv, M, C, dtype, 200 + M)
    nb = M // block
    rng = np.random.default_rng(M + Hq)
    mask = (rng.random((B, Hq, nb, nb)) < 0.35).astype(np.uint8)
    mask[..., np.arange(nb), np.arange(nb)] = 1
    if causal:
        mask *= np.tril(np.ones((nb, nb), dtype=np.uint8))
    idx, cnt = oracle.mask_to_index(mask)
    scale = 1.0 / math.sqrt(C)
    out, lse = xa.bsa_fwd(q.to(DEV), k.to(DEV), v.to(DEV), torch.from_numpy(idx).to(DEV),
                          torch.from_numpy(cnt).to(DEV), block, scale, causal, want_lse=True)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attend(f64(q), f64(k), f64(v), mask, block, scale, causal)
    err = np.abs(f64(out) - ref).max()
    assert err <= _bf16_tol(dtype), err
    assert np.abs(f64(lse) - ref_lse).max() <= 2e-3


# ------------------------------------------------------------------ scoring

SCORE_CASES = [
    # B, Hq, Hkv, M, C, block, stride, causal, dtype, structured
    (1, 4, 1, 2048, 128, 128, 8, True, torch.bfloat16, True),
    (1, 4, 2, 2048, 128, 128, 16, True, torch.bfloat16, True),
    (1, 2, 2, 1280, 128, 128, 8, False, torch.bfloat16, False),
    (1, 2, 1, 1024, 64, 64, 8, True, torch.bfloat16, False),
    (1, 2, 1, 512, 128, 128, 4, True, torch.bfloat16, False),    # r = 32
    (1, 2, 1, 512, 64, 64, 32, True, torch.bfloat16, False),     # r = 2
    (1, 1, 1, 256, 128, 128, 32, False, torch.bfloat16, False),  # r = 4, R < one tile
    (1, 2, 1, 512, 64, 64, 2, True, torch.bfloat16, False),      # S*C = 128: four 32-element chunks
    (1, 2, 2, 768, 128, 64, 2, False, torch.bfloat16, False),    # S*C = 256, 1.5 tiles of strided rows
    (1, 1, 1, 1024, 64, 64, 8, True, torch.float32, True),       # the tiny fp32 workload
    (1, 2, 1, 512, 128, 128, 16, False, torch.float32, False),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=lambda c: "-".join(map(str, c[:8])) + str(c[8])[-4:])
def test_score_matches_oracle(xa, case):
    B, Hq, Hkv, M, C, block, stride, causal, dtype, structured = case
    q, k, _ = _inputs(B, Hq, Hkv, M, C, dtype, 300 + M, structured)
    sscale = 1.0 / (stride * math.sqrt(C))
    got = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, sscale, causal)
    torch.cuda.synchronize()
    ref = oracle.block_scores(f64(q), f64(k), block, stride, sscale, causal)
    g = got.cpu().numpy().astype(np.float64)
    assert (g >= 0).all()
    viol = np.abs(g - ref) > score_tol(ref)
    assert not viol.any(), (np.argwhere(viol)[:5], np.abs(g - ref).max())
    np.testing.assert_allclose(g.sum(-1), 1.0, rtol=1e-4)


ROW_FORM_CASES = [
    # block, stride, C, causal, M: rows of up to 256 candidate blocks and longer
    # rows are normalised by two different finalisation forms; these layers
    # hold both, for r = block / stride of 2, 4, 16 and 32 strided rows
    (64, 32, 64, True, 300 * 64),          # r = 2
    (128, 32, 128, False, 300 * 128 - 37),  # r = 4, non-causal, ragged tail
    (128, 8, 128, True, 300 * 128),        # r = 16
    (128, 4, 64, True, 300 * 128),         # r = 32
    (64, 4, 128, False, 257 * 64),         # r = 16, one candidate over the boundary
]


@pytest.mark.parametrize("case", ROW_FORM_CASES, ids=lambda c: "-".join(map(str, c)))
def test_short_and_long_score_rows(xa, case):
    block, stride, C, causal, M = case
    w = wl.WORKLOADS["llama8k"].scaled(Hq=2, Hkv=1, M=M, C=C, block=block, stride=stride, causal=causal)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    print(f"[row-forms] block={block} S={stride} C={C} causal={causal} M={M}", flush=True)
    sep = xa.xattn_score(x["q"], x["k"], block, stride, sscale, causal)
    bufs = xa.xattn_prefill(x["q"], x["k"], x["v"], x["tau"], block, stride, sscale, smscale, causal)
    torch.cuda.synchronize()
    nb = -(-M // block)
    rows = [0, 200, 255, 256, nb - 1] if causal else [0, 255, nb - 1]
    kh = f64(x["k"][0, 0])
    tau = x["tau"].numpy().astype(np.float64)
    for h in range(2):
        qh = f64(x["q"][0, h])
        for big_i in rows:
            ref = oracle.block_score_row(qh, kh, big_i, block, stride, sscale, causal)
            for label, got in (("score", f64(sep[0, h, big_i])), ("prefill", f64(bufs.block_scores[0, h, big_i]))):
                bad = np.abs(got - ref) > score_tol(ref)
                assert not bad.any(), (label, h, big_i, np.nonzero(bad)[0][:5], np.abs(got - ref).max())
            got = f64(bufs.block_scores[0, h, big_i])
            gmask = bufs.mask[0, h, big_i].cpu().numpy().astype(bool)
            same = oracle.select_row(got, big_i, float(tau[h]), causal)
            diff = np.nonzero(same != gmask)[0]
            ok = near_tau_blocks(got, big_i, float(tau[h]), causal, 1e-5)
            assert all(int(j) in ok for j in diff), (h, big_i, diff[:5])


# Layers of at most 256 key blocks are selected by one wave per row (sorting
# 64, 128 or 256 slots); larger ones by the radix passes: block counts on
# every side of those sizes.
@pytest.mark.parametrize("nb", [40, 130, 300])
@pytest.mark.parametrize("tau", [0.0, 0.5, 0.9, 0.95, 1.0])
@pytest.mark.parametrize("causal", [True, False])
def test_select_matches_oracle_on_same_scores(xa, tau, causal, nb):
    B, Hq = 1, 3
    rng = np.random.default_rng(int(tau * 100) + causal + nb)
    raw = rng.gamma(0.3, size=(B, Hq, nb, nb))
    raw[..., :, 3] *= 0.0       # exact zeros
    raw[..., :, 5] = raw[..., :, 6]  # exact ties
    if causal:
        raw *= np.tril(np.ones((nb, nb)))
    raw /= raw.sum(-1, keepdims=True)
    scores = torch.from_numpy(raw.astype(np.float32))
    taus = [tau, min(1.0, tau + 0.03), max(0.0, tau - 0.2)]
    mask, idx, cnt = xa.xattn_select(scores.to(DEV), taus, 128, 8, causal, Hkv=Hq)
    torch.cuda.synchronize()
    s64 = scores.numpy().astype(np.float64)
    ref = oracle.select(s64, taus, causal)
    m = mask.cpu().numpy()
    check_mask(f"select tau={tau} causal={causal}", m, ref, s64, np.array(taus), causal, 1e-5)
    check_index(m, idx.cpu().numpy(), cnt.cpu().numpy())


def _cut_case_rows(nb):
    """Rows whose cut is decided exactly in float64 and in any exact fixed-point
    sum (scores that are short binary fractions): ties, a cut landing exactly
    on tau * T, one dominant block, scores far below 2^-50, an all-zero row."""
    rows = []
    rows.append(np.full(nb, 1.0 / nb))                   # all tied
    r = np.full(nb, 0.125 / (nb - 1)); r[7] = 0.875       # one dominant block
    rows.append(r)
    r = np.zeros(nb); r[10:18] = 1.0 / 16; r[20:52] = 1.0 / 64   # big block run, then a tie run
    rows.append(r)
    r = np.where(np.arange(nb) % 2 == 0, 2.0 ** -60, 1.0 / 32)   # tiny scores beside large ones
    rows.append(r)
    rows.append(np.zeros(nb))                              # no mass: only the diagonal
    return rows


@pytest.mark.parametrize("nb", [64, 100, 200, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_select_exact_cuts(xa, causal, nb):
    # per-head tau: 0.5 and 0.625 land exactly on cumulative masses of these rows
    # (c_k = tau * T), 0.51 and 0.85 between them, 0.99 near the total
    taus = [0.5, 0.51, 0.625, 0.85, 0.99, 0.0, 1.0]
    cases = _cut_case_rows(nb)
    raw = np.zeros((1, len(taus), nb, nb))
    for h in range(len(taus)):
        for i in range(nb):
            row = cases[(i + h) % len(cases)].copy()
            if causal:
                # the causal row I sees blocks 0..I: place the pattern's last
                # I+1 entries there (tail mass dropped)
                row = np.concatenate([row[nb - (i + 1):], np.zeros(nb - (i + 1))])
            raw[0, h, i] = row
    raw = raw.astype(np.float32).astype(np.float64)  # the oracle sees the GPU's float32 scores
    scores = torch.from_numpy(raw.astype(np.float32))
    mask, idx, cnt = xa.xattn_select(scores.to(DEV), taus, 128, 8, causal, Hkv=1)
    torch.cuda.synchronize()
    # the C ABI takes tau as float32, so the oracle is given that same value:
    # with 1/nb scores a cut can land exactly on a cumulative mass (0.85 * 100
    # blocks), where float32 and float64 tau fall on either side of it
    ref = oracle.select(raw, np.float32(taus).astype(np.float64), causal)
    m = mask.cpu().numpy()
    bad = np.argwhere(m.astype(bool) != ref.astype(bool))
    assert bad.size == 0, bad[:8]
    check_index(m, idx.cpu().numpy(), cnt.cpu().numpy())


@pytest.mark.parametrize("nb", [200, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_select_keeps_diagonal_that_is_an_unkept_tie(xa, nb, causal):
    # Every candidate of a row tied: tau cuts through the ties, which are kept
    # by ascending J, so the diagonal block (high J on the later rows) is an
    # unkept tie and kept only by the diagonal rule. Its flag belongs to a
    # thread of a later wave than the one that sets the diagonal. 200 blocks
    # take the short-row selection, 300 the radix passes.
    taus = [0.5, 0.25, 0.75]
    rows = np.arange(nb)
    raw = np.zeros((1, len(taus), nb, nb))
    for i in rows:
        n = i + 1 if causal else nb
        raw[0, :, i, :n] = 1.0 / 256  # a binary fraction: sums are exact in float32 and float64
    scores = torch.from_numpy(raw.astype(np.float32))
    mask, idx, cnt = xa.xattn_select(scores.to(DEV), taus, 128, 8, causal, Hkv=1)
    torch.cuda.synchronize()
    ref = oracle.select(raw, taus, causal)
    m = mask.cpu().numpy()
    assert (m[0, :, rows, rows] == 1).all()
    bad = np.argwhere(m.astype(bool) != ref.astype(bool))
    assert bad.size == 0, bad[:8]
    check_index(m, idx.cpu().numpy(), cnt.cpu().numpy())


# ------------------------------------------------------------------ end to end

E2E_CASES = [
    # workload name, overrides
    ("tiny", {}),
    ("llama8k", dict(M=2048, Hq=8, Hkv=2)),
    ("llama32k", dict(M=2048, Hq=8, Hkv=2)),
    ("llama128k", dict(M=4096, Hq=4, Hkv=1)),
    ("video", dict(M=2560, Hq=2, Hkv=2)),
    # other seeds of the same generators (other sink, band and column draws)
    ("llama8k", dict(M=2048, Hq=8, Hkv=2, seed=101)),
    ("llama8k", dict(M=2048, Hq=8, Hkv=2, seed=102)),
    ("llama32k", dict(M=3072, Hq=4, Hkv=1, seed=103)),
    ("llama128k", dict(M=4096, Hq=4, Hkv=2, seed=104)),
    ("video", dict(M=2560, Hq=2, Hkv=2, seed=105)),
]


@pytest.mark.parametrize("name,over", E2E_CASES,
                         ids=[c[0] + (f"-seed{c[1]['seed']}" if "seed" in c[1] else "") for c in E2E_CASES])
def test_prefill_end_to_end(xa, name, over):
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    bufs = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    torch.cuda.synchronize()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    tau = x["tau"].numpy().astype(np.float64)
    ref_sc = oracle.block_scores(q, k, w.block, w.stride, sscale, w.causal)
    g_sc = bufs.block_scores.cpu().numpy().astype(np.float64)
    assert not (np.abs(g_sc - ref_sc) > score_tol(ref_sc)).any()
    g_mask = bufs.mask.cpu().numpy()
    # selection parity on the GPU's own scores
    same = oracle.select(g_sc, tau, w.causal)
    check_mask(f"{name} select on GPU scores", g_mask, same, g_sc, tau, w.causal, 1e-5)
    # end to end: differences only where the score tolerance can move the cut
    ref_mask = oracle.select(ref_sc, tau, w.causal)
    band = 1e-5 + 1e-4 + w.nb * 1e-7
    check_mask(f"{name} end to end", g_mask, ref_mask, ref_sc, tau, w.causal, band)
    check_index(g_mask, bufs.kv_idx.cpu().numpy(), bufs.kv_cnt.cpu().numpy())
    # attention parity with the GPU's mask (isolates the attention stage)
    ref_out, _ = oracle.attend(q, k, v, g_mask, w.block, smscale, w.causal)
    err = np.abs(f64(bufs.out) - ref_out).max()
    assert err <= (2e-2 if w.dtype == "bf16" else 1e-3), err
    # invariants
    nb = w.nb
    assert g_mask[..., np.arange(nb), np.arange(nb)].all()
    if w.causal:
        assert not g_mask[..., np.triu(np.ones((nb, nb), dtype=bool), 1)].any()


def test_tau_one_selects_all_and_equals_dense(xa):
    w = wl.WORKLOADS["llama8k"].scaled(M=1024, Hq=4, Hkv=1)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    bufs = xa.xattn_prefill(qd, kd, vd, [1.0] * 4, w.block, w.stride, sscale, smscale, True)
    dense, _ = xa.dense_fwd(qd, kd, vd, w.block, smscale, True)
    torch.cuda.synchronize()
    nb = w.nb
    assert (bufs.mask.cpu().numpy() == np.tril(np.ones((nb, nb), dtype=np.uint8))).all()
    assert torch.equal(bufs.out, dense)


def test_repeat_runs_are_bitwise_identical(xa):
    w = wl.WORKLOADS["llama32k"].scaled(M=2048, Hq=8, Hkv=2)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    a = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, True)
    b = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, True)
    torch.cuda.synchronize()
    assert torch.equal(a.block_scores, b.block_scores)
    assert torch.equal(a.mask, b.mask)
    assert torch.equal(a.out, b.out)


def test_concurrent_streams_with_separate_buffers(xa):
    # The library keeps no state: two different layers in flight at once on
    # two streams, each with its own buffers and workspace, give bitwise what
    # they give one after the other.
    ws = [wl.WORKLOADS["llama32k"].scaled(M=4096, Hq=8, Hkv=2),
          wl.WORKLOADS["llama128k"].scaled(M=6144, Hq=4, Hkv=1)]
    xs = [wl.make_inputs(w, device=DEV) for w in ws]
    args = []
    for w, x in zip(ws, xs):
        sscale, smscale = wl.default_scales(w)
        args.append((x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal))
    refs = []
    for a in args:
        refs.append(xa.xattn_prefill(*a))
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    bufs = [None, None]
    for _ in range(3):
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                bufs[i] = xa.xattn_prefill(*args[i], buffers=bufs[i])
        torch.cuda.synchronize()
        for ref, got in zip(refs, bufs):
            assert torch.equal(ref.block_scores, got.block_scores)
            assert torch.equal(ref.mask, got.mask)
            assert torch.equal(ref.kv_cnt, got.kv_cnt)
            nb = ref.kv_idx.shape[-1]
            valid = torch.arange(nb, device=DEV) < ref.kv_cnt[..., None]
            assert torch.equal(ref.kv_idx[valid], got.kv_idx[valid])
            assert torch.equal(ref.out, got.out)


@pytest.mark.parametrize("name,over", [("llama32k", dict(M=4096, Hq=8, Hkv=2)),
                                       ("llama128k", dict(M=131072, Hq=2, Hkv=1))],
                         ids=["llama32k-4096", "llama128k-2heads"])
def test_prefill_replays_from_a_hip_graph(xa, name, over):
    # xattn_prefill enqueues kernels only (the work queues are cleared by a
    # kernel, not a memset), so it can be captured in a graph. Every replay,
    # with eager work and synchronisations in between, equals the eager call.
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    ref = xa.xattn_prefill(*args)
    bufs = xa.PrefillBuffers(x["q"], x["k"], w.block, w.stride, w.causal)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        xa.xattn_prefill(*args, buffers=bufs)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        xa.xattn_prefill(*args, buffers=bufs)
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


def test_outputs_stay_inside_buffers(xa):
    # guard regions around every output must be untouched
    B, Hq, Hkv, M, C, block = 1, 4, 1, 1024, 128, 128
    q, k, v = _inputs(B, Hq, Hkv, M, C, torch.bfloat16, 7)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    nb = M // block
    guard = 4096
    def guarded(n, dtype, fill):
        t = torch.full((n + 2 * guard,), fill, dtype=dtype, device=DEV)
        return t, t[guard:guard + n]
    sc_all, sc = guarded(B * Hq * nb * nb, torch.float32, -7.0)
    mk_all, mk = guarded(B * Hq * nb * nb, torch.uint8, 0xAB)
    ix_all, ix = guarded(B * Hq * nb * nb, torch.int32, -5)
    ct_all, ct = guarded(B * Hq * nb, torch.int32, -5)
    out_all, out = guarded(B * Hq * M * C, torch.bfloat16, 3.0)
    lse_all, lse = guarded(B * Hq * M, torch.float32, -7.0)
    p = xa.problem(B, Hq, Hkv, M, C, block, 8, 1, torch.bfloat16)
    ws_all, ws = guarded(xa.prefill_workspace_bytes(p), torch.uint8, 0x5A)
    tau = torch.full((Hq,), 0.9)
    import ctypes
    st = torch.cuda.current_stream().cuda_stream
    rc = xa._lib.xattn_prefill(ctypes.byref(p), qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), tau.data_ptr(),
                               1 / (8 * math.sqrt(C)), 1 / math.sqrt(C), sc.data_ptr(), mk.data_ptr(),
                               ix.data_ptr(), ct.data_ptr(), ws.data_ptr(), ws.numel(), out.data_ptr(),
                               lse.data_ptr(), st)
    assert rc == 0
    torch.cuda.synchronize()
    for full, fill in ((sc_all, -7.0), (mk_all, 0xAB), (ix_all, -5), (ct_all, -5), (out_all, 3.0),
                       (lse_all, -7.0), (ws_all, 0x5A)):
        assert (full[:guard] == fill).all() and (full[-guard:] == fill).all()


def test_nonfinite_inputs_terminate(xa):
    B, Hq, Hkv, M, C, block = 1, 2, 1, 512, 128, 128
    q, k, v = _inputs(B, Hq, Hkv, M, C, torch.bfloat16, 9)
    q[0, 0, 5, 3] = float("nan")
    k[0, 0, 17, 0] = float("inf")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    bufs = xa.xattn_prefill(qd, kd, vd, [0.9, 0.9], block, 8, 0.01, 0.08, True)
    torch.cuda.synchronize()
    assert bufs.kv_cnt.min().item() >= 1
    assert bufs.kv_cnt.max().item() <= M // block


@pytest.mark.parametrize("name,over", [("llama32k", dict(M=4096, Hq=8, Hkv=2)),
                                       ("llama128k", dict(M=4096, Hq=4, Hkv=1)),
                                       ("video", dict(M=2560, Hq=2, Hkv=2)),
                                       ("tiny", {})])
def test_fused_prefill_equals_stagewise_calls(xa, name, over):
    # xattn_prefill normalises and selects in one launch; it must reproduce the
    # separate xattn_score + xattn_select + bsa_fwd calls bit for bit
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    qd, kd, vd = x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV)
    fused = xa.xattn_prefill(qd, kd, vd, x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    sc = xa.xattn_score(qd, kd, w.block, w.stride, sscale, w.causal)
    mk, idx, cnt = xa.xattn_select(sc, x["tau"], w.block, w.stride, w.causal, Hkv=w.Hkv, C=w.C,
                                   dtype=qd.dtype)
    out, _ = xa.bsa_fwd(qd, kd, vd, idx, cnt, w.block, smscale, w.causal)
    torch.cuda.synchronize()
    assert torch.equal(fused.block_scores, sc)
    assert torch.equal(fused.mask, mk)
    assert torch.equal(fused.kv_cnt, cnt)
    c = cnt.cpu().numpy().reshape(-1)
    fi = fused.kv_idx.cpu().numpy().reshape(len(c), -1)
    si = idx.cpu().numpy().reshape(len(c), -1)
    for row, n in enumerate(c):
        assert (fi[row, :n] == si[row, :n]).all()
    assert torch.equal(fused.out, out)


@pytest.mark.parametrize("case", [
    (1, 4, 1, 2048, 128, 128, 8, True, torch.bfloat16, True),
    (1, 2, 2, 1280, 128, 128, 16, False, torch.bfloat16, False),
    (1, 2, 1, 512, 64, 64, 4, True, torch.bfloat16, False),
    (1, 1, 1, 1024, 64, 64, 8, True, torch.float32, True),
], ids=["bf16-s8-causal", "bf16-s16-noncausal", "bf16-c64-s4", "f32-tiny"])
def test_diagonal_pattern_score_matches_oracle(xa, case):
    B, Hq, Hkv, M, C, block, stride, causal, dtype, structured = case
    q, k, _ = _inputs(B, Hq, Hkv, M, C, dtype, 500 + M, structured)
    sscale = 1.0 / (stride * math.sqrt(C))
    got = xa.xattn_score(q.to(DEV), k.to(DEV), block, stride, sscale, causal, pattern=xa.DIAGONAL)
    torch.cuda.synchronize()
    ref = oracle.block_scores(f64(q), f64(k), block, stride, sscale, causal, pattern="diagonal")
    g = got.cpu().numpy().astype(np.float64)
    viol = np.abs(g - ref) > score_tol(ref)
    assert not viol.any(), (np.argwhere(viol)[:5], np.abs(g - ref).max())
    if not structured:   # (sink-dominated structured rows score alike under both patterns)
        anti = oracle.block_scores(f64(q), f64(k), block, stride, sscale, causal)
        assert np.abs(anti - ref).max() > 1e-4   # the two patterns really differ here


def test_diagonal_pattern_prefill_end_to_end(xa):
    w = wl.WORKLOADS["llama32k"].scaled(M=2048, Hq=4, Hkv=1)
    x = wl.make_inputs(w)
    sscale, smscale = wl.default_scales(w)
    bufs = xa.xattn_prefill(x["q"].to(DEV), x["k"].to(DEV), x["v"].to(DEV), x["tau"], w.block, w.stride,
                            sscale, smscale, w.causal, pattern=xa.DIAGONAL)
    torch.cuda.synchronize()
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    tau = x["tau"].numpy().astype(np.float64)
    g_sc = bufs.block_scores.cpu().numpy().astype(np.float64)
    ref_sc = oracle.block_scores(q, k, w.block, w.stride, sscale, w.causal, pattern="diagonal")
    assert not (np.abs(g_sc - ref_sc) > score_tol(ref_sc)).any()
    g_mask = bufs.mask.cpu().numpy()
    check_mask("diagonal pattern select on GPU scores", g_mask, oracle.select(g_sc, tau, w.causal), g_sc,
               tau, w.causal, 1e-5)
    ref_out, _ = oracle.attend(q, k, v, g_mask, w.block, smscale, w.causal)
    assert np.abs(f64(bufs.out) - ref_out).max() <= 2e-2


@pytest.mark.parametrize("name,over", [("llama32k", dict(M=4096, Hq=8, Hkv=2)),
                                       ("video", dict(M=2560, Hq=2, Hkv=2)),
                                       ("llama128k", dict(M=8192, Hq=4, Hkv=1, selection="gqa_union"))],
                         ids=["llama32k-4096", "video-2560", "llama128k-8192-gqa-union"])
def test_prefill_without_block_scores(xa, name, over):
    # block scores are an optional output of xattn_prefill: with a NULL pointer
    # the fused normalise+select pass skips their write, and the selection and
    # output are bitwise those of the call that writes them
    over = dict(over)
    sel = over.pop("selection", "row")
    w = wl.WORKLOADS[name].scaled(**over)
    x = wl.make_inputs(w, device=DEV)
    sscale, smscale = wl.default_scales(w)
    args = (x["q"], x["k"], x["v"], x["tau"], w.block, w.stride, sscale, smscale, w.causal)
    ref = xa.xattn_prefill(*args, selection=sel)
    got = xa.xattn_prefill(*args, selection=sel, want_scores=False)
    torch.cuda.synchronize()
    assert got.block_scores is None
    assert torch.equal(ref.mask, got.mask)
    assert torch.equal(ref.kv_cnt, got.kv_cnt)
    valid = torch.arange(ref.kv_idx.shape[-1], device=DEV) < ref.kv_cnt[..., None]
    assert torch.equal(ref.kv_idx[valid], got.kv_idx[valid])
    assert torch.equal(ref.out, got.out)
    # and the selection is the oracle's on these scores
    g_sc = f64(ref.block_scores)
    tau = x["tau"].numpy().astype(np.float64)
    rows = oracle.select(g_sc, tau, w.causal, mode=sel, hkv=w.Hkv)
    if sel == "row":
        check_mask(f"{name} no-scores prefill", got.mask.cpu().numpy(), rows, g_sc, tau, w.causal, 1e-5)
    check_index(got.mask.cpu().numpy(), got.kv_idx.cpu().numpy(), got.kv_cnt.cpu().numpy())
    q, k, v = f64(x["q"]), f64(x["k"]), f64(x["v"])
    heads = [0, w.Hq - 1]
    ref_out, _ = oracle.attend(q, k, v, got.mask.cpu().numpy(), w.block, smscale, w.causal, heads=heads)
    err = max(np.abs(f64(got.out[:, h]) - ref_out[:, h]).max() for h in heads)
    assert err <= 2e-2, err
