"""Calibrate the structure strength gamma of a workload family on the oracle.

Runs the oracle's scoring and selection on evenly spaced query-block rows of
every head and reports the head-mean block density for each gamma tried. The
targets are the densities the XAttention summary page reports ("Key results":
7.32% at 256K tokens, tau=0.9; 45.5% for the video model at tau=0.95). The
chosen gamma is then frozen in workloads.GAMMA; it is never tuned against GPU
time.

Usage: python tests/calibrate_gamma.py llama256k 0.5 1 2 [--rows 16] [--heads 32]
"""
from __future__ import annotations

import argparse
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads as wl  # noqa: E402


def density_for(name: str, gamma: float, rows: int, heads: int) -> tuple[float, list[float]]:
    w = wl.WORKLOADS[name]
    x = wl.make_inputs(w, gamma=gamma)
    sscale, _ = wl.default_scales(w)
    q = x["q"]
    k = x["k"]
    tau = x["tau"].numpy().astype(np.float64)
    nb = w.nb
    qb = sorted(set(np.linspace(0, nb - 1, rows).round().astype(int).tolist()))
    G = w.Hq // w.Hkv
    per_head = []
    for h in range(min(heads, w.Hq)):
        qh = q[0, h].float().numpy()
        kh = k[0, h // G].float().numpy()
        sel = cand = 0
        for big_i in qb:
            row = oracle.block_score_row(qh, kh, big_i, w.block, w.stride, sscale, w.causal)
            keep = oracle.select_row(row, big_i, float(tau[h]), w.causal)
            sel += int(keep.sum())
            cand += big_i + 1 if w.causal else nb
        per_head.append(sel / cand)
    return float(np.mean(per_head)), per_head


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("name")
    ap.add_argument("gammas", type=float, nargs="+")
    ap.add_argument("--rows", type=int, default=16)
    ap.add_argument("--heads", type=int, default=32)
    a = ap.parse_args()
    for g in a.gammas:
        t0 = time.time()
        d, ph = density_for(a.name, g, a.rows, a.heads)
        print(f"{a.name} gamma={g:g} density={d * 100:.2f}% per-head min/max="
              f"{min(ph) * 100:.2f}/{max(ph) * 100:.2f}% ({time.time() - t0:.0f}s)", flush=True)


if __name__ == "__main__":
    main()
