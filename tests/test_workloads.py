"""Seeded synthetic inputs: shapes, dtypes, determinism, and the structure they carry."""
import numpy as np
import pytest
import torch

import workloads as wl


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_shapes_dtypes_and_determinism(name):
    w = wl.WORKLOADS[name]
    small = w.scaled(M=min(w.M, 2 * 2560 if w.family == "video" else 2048),
                     Hq=min(w.Hq, 4), Hkv=min(w.Hkv, 4 if w.Hq == w.Hkv else 1))
    a = wl.make_inputs(small)
    b = wl.make_inputs(small)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    assert a["q"].shape == (1, small.Hq, small.M, w.C) and a["q"].dtype == dt
    assert a["k"].shape == (1, small.Hkv, small.M, w.C) and a["v"].dtype == dt
    assert a["tau"].shape == (small.Hq,)
    for key in ("q", "k", "v", "tau"):
        assert wl.sha256(a[key]) == wl.sha256(b[key])
    assert torch.isfinite(a["q"].float()).all() and torch.isfinite(a["k"].float()).all()


def test_per_head_tau_drawn_from_choices():
    w = wl.WORKLOADS["llama32k"].scaled(M=1024)
    t = wl.make_inputs(w)["tau"].numpy().astype(np.float64)
    assert set(np.round(t, 4)).issubset({0.8, 0.85, 0.9, 0.95})
    assert len(set(np.round(t, 4))) > 1


def test_sink_keys_dominate_plain_keys():
    w = wl.WORKLOADS["llama8k"].scaled(M=1024, Hq=4, Hkv=1)
    x = wl.make_inputs(w)
    q = x["q"].float()[0, 0]
    k = x["k"].float()[0, 0]
    logits = (q[-1] @ k.T) / w.C ** 0.5
    assert logits[:4].min() > logits[100:500].max()


def test_dense_flops():
    w = wl.WORKLOADS["llama256k"]
    assert w.dense_flops == pytest.approx(5.63e14, rel=2e-3)
    assert wl.WORKLOADS["video"].dense_flops == pytest.approx(7.25e13, rel=2e-3)
