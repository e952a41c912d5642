"""bench.py's host-side logic, without a GPU: the one-GPU guard, the FLOP
counts behind the reported rates, and the rule that traffic is read from the
committed profile only while it was taken on the current kernel sources."""
import os
import subprocess
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_score_and_dense_flops_match_the_size_table():
    # strided GEMM FLOPs Hq * 2SC * R(R+1)/2 and dense causal 2 Hq M^2 C at
    # 256K, 128K and 32K (exact values of the configuration sizes)
    w = wl.WORKLOADS["llama256k"]
    assert bench.score_flops(w) == pytest.approx(1.76e13, rel=3e-3)
    assert w.dense_flops == pytest.approx(5.63e14, rel=2e-3)
    assert bench.score_flops(wl.WORKLOADS["llama128k"]) == pytest.approx(4.40e12, rel=3e-3)
    assert bench.score_flops(wl.WORKLOADS["llama32k"]) == pytest.approx(5.50e11, rel=3e-3)
    # non-causal: the whole square
    v = wl.WORKLOADS["video"]
    R = v.M // v.stride
    assert bench.score_flops(v) == v.B * v.Hq * 2.0 * v.stride * v.C * R * R


def test_useful_attention_flops_count_diagonal_tiles_half():
    w = wl.WORKLOADS["llama8k"].scaled(Hq=2, M=512)   # 4 blocks of 128
    kv_cnt = torch.tensor([[[1, 2, 1, 4], [1, 1, 3, 2]]], dtype=torch.int32)
    per = 4.0 * 128 * 128 * 128
    # 15 kept tiles, 8 of them diagonal (one per row)
    assert bench.useful_attn_flops(kv_cnt, w) == (15 - 0.5 * 8) * per
    v = wl.WORKLOADS["video"].scaled(Hq=2, Hkv=2, M=512)
    assert bench.useful_attn_flops(kv_cnt, v) == 15 * per


def test_traffic_is_read_only_for_the_current_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "traffic_bsa_fwd_llama256k.md")
    text = open(path).read()
    sha = [l.split(":")[1].strip() for l in text.splitlines() if l.startswith("kernel_source_sha:")][0]
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: sha)
    got = bench.traffic_from_profile("bsa_fwd", "llama256k")
    assert got is not None and got > 5 * 2 ** 30   # above the 5 GiB floor
    monkeypatch.setattr(bench, "kernel_source_sha", lambda: "0" * 16)
    assert bench.traffic_from_profile("bsa_fwd", "llama256k") is None
    assert bench.traffic_from_profile("bsa_fwd", "no_such_workload") is None
