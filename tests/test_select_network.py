"""The one-wave selection of short rows, modelled on the CPU.

Layers of at most 256 key blocks are selected on the GPU by one wave per row:
candidate p sits in slot e = 64 k + lane (k < 4), keyed by (score bits << 32 |
~p); a bitonic network sorts the first 64, 128 or 256 slots in place (partners
in the same lane's registers for distances 64 and 128, in lane ^ j below);
then each slot is kept while the fixed-point mass before it, in slot order, is
below ceil(tau * T). This model runs the same slot layout, partner rule and
cut on the CPU and checks it against the oracle's minimal sets, so a wrong
network index or a wrong cut shows without a GPU. (The GPU tests check the
kernel itself against the oracle.)
"""
import math

import numpy as np
import pytest

import oracle


def _fx(s: np.float32) -> int:
    # score * 2^50 truncated (scores are in [0, 1])
    return int(math.floor(float(s) * 2.0 ** 50))


def _network(keys: np.ndarray, nk: int) -> np.ndarray:
    """keys: (4, 64) uint64 in slot layout [k, lane]; sorts slots 0 .. 64 nk - 1."""
    kv = keys.copy()
    lane = np.arange(64)
    size = 2
    while size <= 64 * nk:
        j = size >> 1
        while j > 0:
            new = kv.copy()
            if j >= 64:
                kj = j >> 6
                for k in range(nk):
                    if k & kj:
                        continue
                    k2 = k | kj
                    big_first = ((64 * k + lane) & size) == 0
                    a, b = kv[k], kv[k2]
                    sw = np.where(big_first, a < b, a > b)
                    new[k] = np.where(sw, b, a)
                    new[k2] = np.where(sw, a, b)
            else:
                lower = (lane & j) == 0
                for k in range(nk):
                    other = kv[k][lane ^ j]
                    big_first = ((64 * k + lane) & size) == 0
                    keep_max = lower == big_first
                    new[k] = np.where(keep_max, np.maximum(kv[k], other), np.minimum(kv[k], other))
            kv = new
            j >>= 1
        size <<= 1
    return kv


def _select_one_wave(sc: np.ndarray, n: int, nb: int, diag: int, tau: np.float32) -> np.ndarray:
    flags = np.zeros(nb, dtype=bool)
    if tau >= 1.0:
        flags[:n] = True
    else:
        keys = np.zeros((4, 64), dtype=np.uint64)
        total = 0
        for p in range(n):
            bits = int(np.float32(sc[p]).view(np.uint32))
            keys[p // 64, p % 64] = (bits << 32) | (0xFFFFFFFF - p)
            total += _fx(sc[p])
        thr = int(math.ceil(float(tau) * float(total)))
        if not (tau <= 0.0 or total == 0 or thr == 0):
            nk = 1 if n <= 64 else (2 if n <= 128 else 4)
            kv = _network(keys, nk)
            flat = [int(kv[k, lane]) for k in range(4) for lane in range(64)]
            assert flat[:64 * nk] == sorted(flat[:64 * nk], reverse=True)
            assert all(v == 0 for v in flat[64 * nk:])
            before = 0
            for key in flat:
                if key == 0:
                    continue
                if before < thr:
                    flags[0xFFFFFFFF - (key & 0xFFFFFFFF)] = True
                before += _fx(np.uint32(key >> 32).view(np.float32))
    flags[diag] = True
    return flags


def _rows(seed: int, count: int):
    rng = np.random.default_rng(seed)
    for t in range(count):
        nb = int(rng.integers(1, 257))
        causal = bool(rng.integers(0, 2))
        big_i = int(rng.integers(0, nb))
        n = big_i + 1 if causal else nb
        kind = t % 4
        if kind == 0:
            sc = rng.random(nb)
        elif kind == 1:
            sc = rng.integers(0, 4, nb) / 8.0          # many exact ties
        elif kind == 2:
            sc = np.exp(rng.normal(0, 3, nb))          # a wide range
        else:
            sc = np.zeros(nb)
            sc[rng.integers(0, nb, 3)] = 1.0           # few non-zeros, many zero candidates
        sc[n:] = 0.0
        sc = (sc / max(sc[:n].sum(), 1e-30)).astype(np.float32)
        tau = np.float32(rng.choice([0.0, 0.5, 0.8, 0.9, 0.95, 1.0, rng.random()]))
        yield nb, causal, big_i, n, sc, tau


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_one_wave_selection_model_matches_oracle(seed):
    for nb, causal, big_i, n, sc, tau in _rows(seed, 60):
        got = _select_one_wave(sc, n, nb, big_i, tau)
        # the oracle gets the same float32 scores and tau the kernel receives
        ref = oracle.select_row(sc.astype(np.float64), big_i, float(tau), causal).astype(bool)
        assert np.array_equal(got, ref), (nb, causal, big_i, float(tau), np.nonzero(got != ref)[0][:5])


@pytest.mark.parametrize("nb", [40, 64, 100, 128, 200, 256])
def test_one_wave_selection_model_exact_cuts(nb):
    # binary-fraction scores whose cumulative masses land exactly on tau * T
    # (tau 0.5 and 0.625 over runs of 1/64 and 1/16), and all-equal rows cut
    # through their ties: a cut taken one slot early or late shows here
    rows = []
    r = np.zeros(nb, np.float32); r[:min(nb, 64)] = 1.0 / 64; rows.append(r)
    r = np.zeros(nb, np.float32); r[nb - 16:] = 1.0 / 16; r[:8] = 1.0 / 64; rows.append(r)
    rows.append(np.full(nb, np.float32(1.0 / 256)))
    for sc in rows:
        for tau in (np.float32(0.5), np.float32(0.625), np.float32(0.25)):
            got = _select_one_wave(sc, nb, nb, 0, tau)
            ref = oracle.select_row(sc.astype(np.float64), 0, float(tau), False).astype(bool)
            assert np.array_equal(got, ref), (nb, float(tau), np.nonzero(got != ref)[0][:5])
