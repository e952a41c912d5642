"""CPU oracle for XAttention-style block-sparse prefill attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this module:
only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it. It shares no code, constant or helper with the HIP library.

Plain NumPy in float64. Inputs (bf16 values carried in float32, or float32) are
upcast exactly. Every step is written the way the pages describe it, with no
blocking or fusion beyond processing one query-block row at a time so memory
stays O(block * M).

Sources (page title, section):
  [XA-abs]  "XAttention: Block Sparse Attention with Antidiagonal Scoring",
            arXiv abstract as shown on fugumt.com (2503.16428v1).
  [XA-sum]  "XAttention: Block Sparse Attention with Antidiagonal Scoring",
            AI-written summary on atlas.scime.ai: sections "Approach",
            "Key results", "Limitations".
  [DuSA]    "DuSA: Fast and Accurate Dual-Stage Sparse Attention Mechanism
            Accelerating Both Training and Inference", rebuttal on paperhub.cn,
            section "Response to Q2" (the reshape formulation of XAttention).
  [Flex]    "FlexPrefill: A Context-Aware Sparse Attention Mechanism for
            Efficient Long-Sequence Inference", rebuttal on paperhub.cn,
            sections "R Q3" (minimal |S| under a cumulative-mass constraint;
            global, flattened index selection versus query-wise selection).

Notation: Q is (B, Hq, Mq, C); K, V are (B, Hkv, Mk, C) with Mk >= Mq; query
head h reads KV head h // (Hq // Hkv). Query i sits at absolute position
off + i, off = Mk - Mq (chunked prefill: the queries are the last Mq tokens;
off = 0 is the plain prefill), and off must be a multiple of the block size.
Block size Bk, stride S, r = Bk // S strided rows per block,
NBq = ceil(Mq / Bk) query blocks, NBk = ceil(Mk / Bk) key blocks; query block I
is key block I + off // Bk. Lengths need not be multiples of S or Bk.

Readings taken where the pages are silent:
  * score temperature: the caller passes ``score_scale`` explicitly;
  * the antidiagonal pairs query row i*S+s with key row j*S+S-1-s;
  * causal masking of the strided scores is at the strided level (j <= i);
  * softmax runs over keys for each strided query row, before the block sum;
  * block scores are divided by r so each query-block row sums to 1;
  * ties in the sort are broken by ascending block index;
  * tau >= 1 keeps every candidate; the diagonal block is always added after
    the threshold cut;
  * sparse attention is exact softmax attention renormalised over the
    selected keys only;
  * DuSA1 multi-stride scoring (pattern "dusa1"): each of the S phases of the
    (S, M // S, C) reshape is softmaxed on its own and a block's score is the
    phases' summed mass over its S * r rows, divided by S * r; it needs
    lengths that are multiples of S;
  * ragged lengths ([DuSA] rebuttal, "Response to Q1": padding makes the
    sequence length divisible by the block size): the missing tokens of a
    partial stride group are zero vectors; strided key rows and keys past the
    end take no part in any softmax; a partial last query block's scores are
    divided by its count of real strided rows, so its row still sums to 1.

Pins: every function here is checked in tests/test_oracle_pins.py against
something other than itself (brute force, closed forms, library routines).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "strided_query_rows",
    "reversed_key_rows",
    "strided_logits",
    "block_score_row",
    "dusa1_phase_rows",
    "dusa1_block_score_row",
    "block_scores",
    "minimal_set",
    "select_row",
    "select",
    "select_global_head",
    "gqa_union",
    "mask_to_index",
    "attend_row",
    "attend",
    "dense",
    "prefill",
    "density",
]


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def _kv_head(h: int, hq: int, hkv: int) -> int:
    # GQA: consecutive query heads share one KV head.
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (hq // hkv)


# ---------------------------------------------------------------------------
# Stage 1: strided antidiagonal scoring.
# [DuSA] Response to Q2: Q and K of shape (B, H, M, C) are reshaped to
# (B, H, M // stride, stride * C) and an attention is computed on them.
# [XA-abs]: the antidiagonal runs from the lower-left to the upper-right
# corner of each stride x stride tile, so query row i*S + s meets key row
# j*S + (S - 1 - s). Reversing the S key rows inside each stride group before
# the reshape turns the reshape-matmul into exactly that antidiagonal sum.
# ---------------------------------------------------------------------------

def _pad_rows(x: np.ndarray, mult: int) -> np.ndarray:
    """x (m, c) in float64 with zero rows appended up to a multiple of ``mult``."""
    x = _f64(x)
    m, c = x.shape
    extra = (-m) % mult
    if extra:
        x = np.concatenate([x, np.zeros((extra, c))], axis=0)
    return x


def _cdiv(a: int, b: int) -> int:
    return -(-a // b)


def strided_query_rows(qh: np.ndarray, stride: int) -> np.ndarray:
    """Q' (R, S*C): row i concatenates q[i*S], ..., q[i*S+S-1] (zero past the end)."""
    x = _pad_rows(qh, stride)
    return x.reshape(x.shape[0] // stride, stride * x.shape[1])


def reversed_key_rows(kh: np.ndarray, stride: int) -> np.ndarray:
    """K~' (R, S*C): row j concatenates k[j*S+S-1], ..., k[j*S] (zero past the end)."""
    x = _pad_rows(kh, stride)
    r = x.shape[0] // stride
    return x.reshape(r, stride, x.shape[1])[:, ::-1, :].reshape(r, stride * x.shape[1])


def strided_logits(qh, kh, stride: int, score_scale: float, causal: bool,
                   rows: slice | None = None, pattern: str = "antidiagonal") -> np.ndarray:
    """Scaled strided logits for strided query ``rows`` vs all strided keys.

    ``pattern="antidiagonal"`` (the method) reverses K inside each stride group;
    ``pattern="diagonal"`` (the older variant the DuSA rebuttal, Response to Q2,
    describes: plain (M/stride, stride*C) reshapes of Q and K) does not, which
    sums the main diagonal of each stride x stride tile instead.
    With queries the last Mq of Mk tokens, strided query row i is absolute
    strided row i + (Mk - Mq) / S. Entries with key j > that row are -inf when
    ``causal`` (strided level).
    """
    off = kh.shape[0] - qh.shape[0]
    if off < 0 or off % stride:
        raise ValueError("Mk - Mq must be a non-negative multiple of the stride")
    qs = strided_query_rows(qh, stride)
    if pattern == "antidiagonal":
        ks = reversed_key_rows(kh, stride)
    elif pattern == "diagonal":
        ks = strided_query_rows(kh, stride)
    else:
        raise ValueError(pattern)
    if rows is None:
        rows = slice(0, qs.shape[0])
    lo = rows.start
    a = qs[rows] @ ks.T
    a *= score_scale
    if causal:
        i = np.arange(lo, lo + a.shape[0])[:, None] + off // stride
        j = np.arange(ks.shape[0])[None, :]
        a[j > i] = -np.inf
    return a


# ---------------------------------------------------------------------------
# Stage 2: softmax-normalised block importance.
# [XA-sum] Approach: the strided antidiagonal values inside each attention
# block are summed after softmax normalisation. [DuSA] Response to Q2: the
# softmax runs on the final two dimensions of the reshaped tensors, i.e. over
# keys for each strided query row.
# ---------------------------------------------------------------------------

def dusa1_phase_rows(x: np.ndarray, stride: int) -> np.ndarray:
    """(S, M // S, C): x (M, C) reshaped to (M // S, S, C), then its first two
    axes swapped, so phase s holds rows s, s + S, s + 2S, ... ([DuSA] Response
    to Q2, DuSA1)."""
    x = _f64(x)
    m, c = x.shape
    if m % stride:
        raise ValueError("DuSA1 scoring needs a length that is a multiple of the stride")
    return x.reshape(m // stride, stride, c).transpose(1, 0, 2)


def dusa1_block_score_row(qh, kh, big_i: int, block: int, stride: int,
                          score_scale: float, causal: bool) -> np.ndarray:
    """DuSA1 multi-stride block scores for query block ``big_i`` (length NBk).

    [DuSA] Response to Q2: Q and K are reshaped to (M // S, S, C) and
    transposed to (S, M // S, C); an attention with its softmax on the final
    two dimensions is computed for each of the S phases (they may be folded
    into the head axis without changing the result). Reading taken: every
    phase row is softmaxed over its own phase's strided keys (j <= i at the
    strided level when causal), and block (I, J) scores the probability mass of
    its S * r_I phase rows falling in key block J, summed over the phases and
    divided by S * r_I, so each row of block scores sums to 1.
    """
    if block % stride:
        raise ValueError("block must be a multiple of the stride")
    mq, mk = qh.shape[0], kh.shape[0]
    if (mk - mq) % block:
        raise ValueError("Mk - Mq must be a multiple of the block size")
    qp = dusa1_phase_rows(qh, stride)        # (S, Rq, C)
    kp = dusa1_phase_rows(kh, stride)        # (S, Rk, C)
    r = block // stride
    rq, rk = qp.shape[1], kp.shape[1]
    nbk = _cdiv(mk, block)
    off = (mk - mq) // stride                # strided position of query row 0
    rows = range(big_i * r, min((big_i + 1) * r, rq))
    total = np.zeros(nbk)
    for s in range(stride):
        logits = score_scale * (qp[s, rows.start:rows.stop] @ kp[s].T)   # (r_I, Rk)
        if causal:
            i = np.arange(rows.start, rows.stop)[:, None] + off
            j = np.arange(rk)[None, :]
            logits[j > i] = -np.inf
        mx = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - mx)
        p /= p.sum(axis=1, keepdims=True)                                 # softmax over the phase's keys
        p = np.concatenate([p, np.zeros((p.shape[0], nbk * r - rk))], axis=1)
        total += p.reshape(p.shape[0], nbk, r).sum(axis=2).sum(axis=0)
    return total / (stride * len(rows))


def block_score_row(qh, kh, big_i: int, block: int, stride: int,
                    score_scale: float, causal: bool, pattern: str = "antidiagonal") -> np.ndarray:
    """Block scores S^[I, :] (length NBk) for query block ``big_i`` of one head.
    ``pattern`` is "antidiagonal" (the method), "diagonal" or "dusa1"."""
    if pattern == "dusa1":
        return dusa1_block_score_row(qh, kh, big_i, block, stride, score_scale, causal)
    if block % stride:
        raise ValueError("block must be a multiple of the stride")
    mq, mk = qh.shape[0], kh.shape[0]
    if (mk - mq) % block:
        raise ValueError("Mk - Mq must be a multiple of the block size")
    r = block // stride
    nbk = _cdiv(mk, block)
    rq = _cdiv(mq, stride)
    rows = slice(big_i * r, min((big_i + 1) * r, rq))   # the block's real strided rows
    logits = strided_logits(qh, kh, stride, score_scale, causal, rows=rows, pattern=pattern)
    n_rows = logits.shape[0]
    # row softmax over keys
    mx = logits.max(axis=1, keepdims=True)
    p = np.exp(logits - mx)
    p /= p.sum(axis=1, keepdims=True)
    # sum each tile: strided key j belongs to key block j // r
    p = np.concatenate([p, np.zeros((n_rows, nbk * r - p.shape[1]))], axis=1)
    per_block = p.reshape(n_rows, nbk, r).sum(axis=2).sum(axis=0)
    return per_block / n_rows


def block_scores(q, k, block: int, stride: int, score_scale: float, causal: bool,
                 heads=None, qblocks=None, pattern: str = "antidiagonal") -> np.ndarray:
    """Block scores (B, Hq, NBq, NBk), float64. Rows not in ``qblocks`` stay 0."""
    b_, hq, mq, _ = q.shape
    hkv, mk = k.shape[1], k.shape[2]
    nbq, nbk = _cdiv(mq, block), _cdiv(mk, block)
    heads = range(hq) if heads is None else heads
    qblocks = range(nbq) if qblocks is None else qblocks
    out = np.zeros((b_, hq, nbq, nbk))
    for b in range(b_):
        for h in heads:
            g = _kv_head(h, hq, hkv)
            for big_i in qblocks:
                out[b, h, big_i] = block_score_row(q[b, h], k[b, g], big_i, block,
                                                   stride, score_scale, causal, pattern)
    return out


# ---------------------------------------------------------------------------
# Stage 3: minimal-set threshold selection.
# [XA-sum] Approach: keep the minimal set of blocks whose softmax-normalised
# antidiagonal mass exceeds a (per-head) threshold. [Flex] R Q3: minimising
# |S| subject to the cumulative-mass constraint is solved by taking entries in
# descending order until the constraint holds.
# ---------------------------------------------------------------------------

def minimal_set(cand: np.ndarray, tau: float) -> np.ndarray:
    """Indices of the smallest candidate set whose mass reaches tau * total.

    Candidates are taken in descending score order (ties: ascending index) and
    the prefix stops at the first k with cumulative mass >= tau * total
    (k = 0 when tau <= 0). tau >= 1 keeps every candidate.
    """
    cand = _f64(cand)
    n = cand.shape[0]
    if tau >= 1.0:
        return np.arange(n)
    idx = np.arange(n)
    order = np.lexsort((idx, -cand))          # score descending, index ascending
    csum = np.concatenate([[0.0], np.cumsum(cand[order])])
    total = csum[-1]
    kstar = int(np.argmax(csum >= tau * total))  # first k with mass >= tau * total
    return order[:kstar]


def select_row(scores_row: np.ndarray, big_i: int, tau: float, causal: bool) -> np.ndarray:
    """Boolean keep-mask (length NBk) for one query-block row; ``big_i`` is the
    row's key-block index (its position in the whole sequence)."""
    nb = scores_row.shape[0]
    n_cand = big_i + 1 if causal else nb
    keep = np.zeros(nb, dtype=bool)
    keep[minimal_set(scores_row[:n_cand], tau)] = True
    keep[big_i] = True                               # diagonal block, added after the cut
    return keep


def select_global_head(scores_h: np.ndarray, tau: float, causal: bool) -> np.ndarray:
    """Global (flattened) selection for one head ([Flex] R Q3): keep-mask (NBq, NBk).

    Every candidate block (I, J) of the head (J <= I + NBk - NBq when causal)
    enters one list in row-major order; the minimal set is taken over that list
    exactly as for a single row (score descending, ties by list position, i.e.
    by (I, J) row-major), against tau times the head's total candidate mass. The
    diagonal blocks (I, I + NBk - NBq) are then added.
    """
    nbq, nbk = scores_h.shape
    qoff = nbk - nbq
    rows, cols = [], []
    for big_i in range(nbq):
        n_cand = big_i + qoff + 1 if causal else nbk
        rows.extend([big_i] * n_cand)
        cols.extend(range(n_cand))
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    flat = _f64(scores_h)[rows, cols]
    keep = np.zeros((nbq, nbk), dtype=bool)
    chosen = minimal_set(flat, tau)
    keep[rows[chosen], cols[chosen]] = True
    keep[np.arange(nbq), np.arange(nbq) + qoff] = True
    return keep


def gqa_union(mask: np.ndarray, hkv: int) -> np.ndarray:
    """GQA union of a mask (B, Hq, NB, NB): every head of a KV group gets the
    union of the group's kept blocks, row by row.

    Not from the pages: a reuse variant in which the sibling heads that read
    one KV head share a single block list, so one K/V tile serves all of them.
    """
    b_, hq, nbq, nbk = mask.shape
    g = hq // hkv
    out = mask.astype(bool).reshape(b_, hkv, g, nbq, nbk).any(axis=2, keepdims=True)
    return np.ascontiguousarray(np.broadcast_to(out, (b_, hkv, g, nbq, nbk)).reshape(mask.shape),
                                dtype=np.uint8)


def select(scores: np.ndarray, tau, causal: bool, heads=None, qblocks=None,
           mode: str = "row", hkv: int | None = None) -> np.ndarray:
    """Mask (B, Hq, NB, NB) uint8 from block scores and per-head ``tau`` (len Hq).

    mode "row": the minimal set per query-block row ([XA-sum] Approach);
    "global": per head over all rows at once ([Flex] R Q3), all rows required;
    "gqa_union": "row", then the union over each KV group (``hkv`` heads).
    """
    b_, hq, nbq, nbk = scores.shape
    qoff = nbk - nbq          # key block of query block 0
    tau = np.broadcast_to(np.asarray(tau, dtype=np.float64), (hq,))
    some_heads = heads is not None
    heads = range(hq) if heads is None else heads
    mask = np.zeros(scores.shape, dtype=np.uint8)
    if mode == "global":
        if qblocks is not None:
            raise ValueError("global selection needs every query-block row")
        for b in range(b_):
            for h in heads:
                mask[b, h] = select_global_head(scores[b, h], float(tau[h]), causal)
        return mask
    if mode not in ("row", "gqa_union"):
        raise ValueError(f"unknown selection mode {mode!r}")
    if mode == "gqa_union":
        if hkv is None:
            raise ValueError("gqa_union needs hkv")
        if some_heads:
            # the union needs every sibling of a selected head
            g = hq // hkv
            heads = sorted({hh for h in heads for hh in range((h // g) * g, (h // g + 1) * g)})
    qblocks = range(nbq) if qblocks is None else qblocks
    for b in range(b_):
        for h in heads:
            for big_i in qblocks:
                mask[b, h, big_i] = select_row(scores[b, h, big_i], big_i + qoff, float(tau[h]), causal)
    if mode == "gqa_union":
        mask = gqa_union(mask, hkv)
    return mask


def mask_to_index(mask: np.ndarray):
    """Ascending per-row block lists: kv_idx (.., NB) int32 padded with -1, kv_cnt int32."""
    nb = mask.shape[-1]
    cnt = np.ascontiguousarray(mask.astype(bool).sum(axis=-1), dtype=np.int32)
    idx = np.full(mask.shape, -1, dtype=np.int32)
    flat_m = mask.reshape(-1, nb).astype(bool)
    flat_i = idx.reshape(-1, nb)
    for row in range(flat_m.shape[0]):
        sel = np.nonzero(flat_m[row])[0]
        flat_i[row, :sel.size] = sel
    return idx, cnt


# ---------------------------------------------------------------------------
# Stage 4: block-sparse attention.
# [XA-abs]: block-sparse attention computes only on the critical blocks.
# Plain definition: exact softmax attention over the selected keys only
# (causal: key index <= query index), scale sm_scale.
# ---------------------------------------------------------------------------

def attend_row(qh, kh, vh, keep_row: np.ndarray, big_i: int, block: int,
               sm_scale: float, causal: bool):
    """Output (rows, C) and natural-log LSE (rows,) for query block ``big_i``
    (rows = the block's queries, fewer in a partial last block)."""
    mq, mk = qh.shape[0], kh.shape[0]
    off = mk - mq
    qb = _f64(qh[big_i * block:(big_i + 1) * block])
    blocks = np.nonzero(keep_row)[0]
    keys = (blocks[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    keys = keys[keys < mk]
    kk = _f64(kh[keys])
    vv = _f64(vh[keys])
    s = (qb @ kk.T) * sm_scale
    if causal:
        qi = off + big_i * block + np.arange(qb.shape[0])[:, None]
        s[keys[None, :] > qi] = -np.inf
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    den = p.sum(axis=1, keepdims=True)
    out = (p @ vv) / den
    lse = (mx + np.log(den))[:, 0]
    return out, lse


def attend(q, k, v, mask, block: int, sm_scale: float, causal: bool,
           heads=None, qblocks=None):
    """Block-sparse attention with a block mask (B, Hq, NBq, NBk): (out, lse) float64."""
    b_, hq, mq, c = q.shape
    hkv = k.shape[1]
    nbq = _cdiv(mq, block)
    heads = range(hq) if heads is None else heads
    qblocks = range(nbq) if qblocks is None else qblocks
    out = np.zeros((b_, hq, mq, c))
    lse = np.zeros((b_, hq, mq))
    for b in range(b_):
        for h in heads:
            g = _kv_head(h, hq, hkv)
            for big_i in qblocks:
                o, l = attend_row(q[b, h], k[b, g], v[b, g], mask[b, h, big_i], big_i,
                                  block, sm_scale, causal)
                out[b, h, big_i * block:big_i * block + o.shape[0]] = o
                lse[b, h, big_i * block:big_i * block + o.shape[0]] = l
    return out, lse


def dense(q, k, v, block: int, sm_scale: float, causal: bool, heads=None, qblocks=None):
    """Dense attention: every candidate block kept."""
    b_, hq, mq, _ = q.shape
    nbq, nbk = _cdiv(mq, block), _cdiv(k.shape[2], block)
    full = np.ones((b_, hq, nbq, nbk), dtype=np.uint8)
    if causal:
        tri = np.tril(np.ones((nbq, nbk), dtype=np.uint8), k=nbk - nbq)
        full = np.broadcast_to(tri, full.shape).copy()
    return attend(q, k, v, full, block, sm_scale, causal, heads, qblocks)


def prefill(q, k, v, block: int, stride: int, tau, score_scale: float, sm_scale: float,
            causal: bool, heads=None, qblocks=None, pattern: str = "antidiagonal",
            mode: str = "row"):
    """All three stages: (block_scores, mask, out, lse)."""
    if mode == "gqa_union" and heads is not None:
        raise ValueError("gqa_union prefill runs every head")
    sc = block_scores(q, k, block, stride, score_scale, causal, heads, qblocks, pattern)
    mk = select(sc, tau, causal, heads, qblocks, mode=mode, hkv=k.shape[1])
    out, lse = attend(q, k, v, mk, block, sm_scale, causal, heads, qblocks)
    return sc, mk, out, lse


def density(mask: np.ndarray, causal: bool, qblocks=None) -> float:
    """Selected blocks / candidate blocks (diagonal counted as 1)."""
    nbq, nbk = mask.shape[-2:]
    rows = range(nbq) if qblocks is None else list(qblocks)
    sel = 0
    cand = 0
    for big_i in rows:
        sel += int(mask[..., big_i, :].astype(bool).sum())
        cand += (big_i + nbk - nbq + 1 if causal else nbk) * int(np.prod(mask.shape[:-2]))
    return sel / cand
