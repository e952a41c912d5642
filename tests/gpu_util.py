"""Helpers shared by the GPU parity tests: CPU views of device results and the
mask-acceptance rules.

Acceptance (floating point decides an integer here, so the rules say which
differences are allowed):
  * select parity: the oracle's selection run on the GPU's own float32 block
    scores must give the GPU's mask, except blocks whose cumulative mass (in the
    oracle's sorted order, before or after the block) is within 1e-5 of tau
    (relative to the row total);
  * end to end: the same near-tau rule with the band widened by the shift in
    cumulative mass that the 1e-4 relative score tolerance allows.
"""
import numpy as np
import torch

import oracle


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def near_tau_blocks(scores_row: np.ndarray, big_i: int, tau: float, causal: bool, band: float):
    """Blocks whose cumulative mass before or after them is within ``band`` of tau."""
    n = big_i + 1 if causal else scores_row.shape[0]
    cand = scores_row[:n].astype(np.float64)
    order = np.lexsort((np.arange(n), -cand))
    csum = np.concatenate([[0.0], np.cumsum(cand[order])])
    total = csum[-1]
    if total <= 0 or tau >= 1.0:
        return set()
    frac = csum / total
    near = set()
    for p in range(n):
        if abs(frac[p] - tau) <= band or abs(frac[p + 1] - tau) <= band:
            near.add(int(order[p]))
    return near


def mask_mismatches(mask_gpu: np.ndarray, mask_ref: np.ndarray, scores_for_band: np.ndarray,
                    tau: np.ndarray, causal: bool, band: float, rows=None, qoff: int = 0):
    """Return (n_diff_blocks, unexplained (b, h, I, J) list) over (b, h, I) rows;
    query block I is key block I + qoff."""
    B, H, NB, _ = mask_gpu.shape
    n_diff = 0
    bad = []
    it = rows if rows is not None else [(b, h, i) for b in range(B) for h in range(H) for i in range(NB)]
    for (b, h, i) in it:
        d = np.nonzero(mask_gpu[b, h, i].astype(bool) != mask_ref[b, h, i].astype(bool))[0]
        if d.size == 0:
            continue
        n_diff += d.size
        ok = near_tau_blocks(scores_for_band[b, h, i], i + qoff, float(tau[h]), causal, band)
        for J in d:
            if int(J) not in ok:
                bad.append((b, h, i, int(J)))
    return n_diff, bad


def check_mask(tag: str, mask_gpu: np.ndarray, mask_ref: np.ndarray, scores_for_band: np.ndarray,
               tau: np.ndarray, causal: bool, band: float, rows=None, cap_frac: float = 0.02,
               qoff: int = 0):
    """Masks identical except near-tau blocks; print the count of such allowed
    differences and cap the share of rows that hold any.

    Returns (n_diff_blocks, n_rows_with_diffs, n_rows_compared).
    """
    B, H, NB, _ = mask_gpu.shape
    it = list(rows) if rows is not None else [(b, h, i) for b in range(B) for h in range(H) for i in range(NB)]
    n_diff, bad = mask_mismatches(mask_gpu, mask_ref, scores_for_band, tau, causal, band, it, qoff)
    diff_rows = sum(1 for (b, h, i) in it
                    if (mask_gpu[b, h, i].astype(bool) != mask_ref[b, h, i].astype(bool)).any())
    print(f"[mask] {tag}: {len(it)} rows, {n_diff} near-tau block differences in {diff_rows} rows "
          f"(band {band:.2e}), {len(bad)} unexplained", flush=True)
    assert not bad, (tag, bad[:5])
    cap = max(2, int(cap_frac * len(it)))
    assert diff_rows <= cap, (tag, diff_rows, cap)
    return n_diff, diff_rows, len(it)


def check_index(mask: np.ndarray, kv_idx: np.ndarray, kv_cnt: np.ndarray):
    """kv_idx/kv_cnt must list the mask's kept blocks in ascending order."""
    ref_idx, ref_cnt = oracle.mask_to_index(mask)
    np.testing.assert_array_equal(kv_cnt, ref_cnt)
    nb = mask.shape[-1]
    flat_i = kv_idx.reshape(-1, nb)
    flat_r = ref_idx.reshape(-1, nb)
    for row, c in enumerate(ref_cnt.reshape(-1)):
        np.testing.assert_array_equal(flat_i[row, :c], flat_r[row, :c])


def score_tol(ref: np.ndarray) -> np.ndarray:
    return 1e-4 * np.abs(ref) + 1e-7
