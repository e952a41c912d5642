#!/usr/bin/env python3
"""Prefill-attention benchmark on one MI355X: XAttention-style block-sparse
prefill (strided antidiagonal scoring -> minimal-set selection -> block-sparse
flash attention), all three stages per step, on seeded synthetic Llama-3.1-8B-
shaped layers (32 query / 8 KV heads, C=128, bf16, causal).

One step = one xattn_prefill call over the whole layer (strided scoring
partials, fused normalisation + selection, block-sparse attention), inputs
already resident in HBM. A second timed loop through the stage entry points
(xattn_score, xattn_select, bsa_fwd) gives the per-stage breakdown. Reported value: dense-equivalent TFLOP/s
(2*Hq*M^2*C / step time). Also reported: per-stage times, measured density, our
own dense_fwd time and the speedup over it, the roofline of the dominant kernel,
the CPU oracle timed on a bounded sample of the same workload, the 32K and 128K
lengths, method variants on the headline layer, and the non-causal video-model
layer (24/24 heads, 76,800 tokens, stride 8, tau 0.95) under other_configs.

Prints ONE JSON line on stdout (progress goes to stderr).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill attn ms & dense-equiv TFLOP/s at 32K/128K/256K tokens, 1 MI355X"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_sparse_attention_xattn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def measure_peaks(torch) -> dict:
    """Measured peak rates on this GPU (libxattn_peaks.so): the bf16 matrix-core
    rate of a pure v_mfma_f32_32x32x16_bf16 loop, the core clock sustained under
    it, and an HBM stream copy, next to the published peaks."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "block_sparse_attention_xattn_amd", "libxattn_peaks.so"))
    lib.xattn_peak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.xattn_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    dev = torch.device("cuda:0")
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wpb = lib.xattn_peak_mfma_waves_per_block()
    blocks, iters = 2 * cus, 40000
    sink = torch.empty(blocks * 64 * wpb, dtype=torch.float32, device=dev)
    clk = torch.zeros(2 * blocks, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def mfma():
        rc = lib.xattn_peak_mfma(blocks, iters, ctypes.c_void_p(sink.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                                 ctypes.c_void_p(stream))
        if rc:
            raise RuntimeError(f"xattn_peak_mfma: hip error {rc}")

    ms = timed(mfma, 3)
    flops = blocks * wpb * iters * 16 * 32768.0
    c = clk.view(blocks, 2).double().cpu()
    ghz = float((c[:, 0] / c[:, 1]).median()) * 0.1
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def copy():
        rc = lib.xattn_peak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), nbytes,
                                 ctypes.c_void_p(stream))
        if rc:
            raise RuntimeError(f"xattn_peak_copy: hip error {rc}")

    cms = timed(copy, 5)
    assert torch.equal(dst[:4096], src[:4096])
    del src, dst, sink, clk
    torch.cuda.empty_cache()
    out = {"mfma_bf16_tflops": round(flops / ms / 1e9, 1), "mfma_clock_ghz": round(ghz, 3),
           "hbm_copy_gbs": round(2 * nbytes / cms / 1e6, 1),
           "published": {"bf16_dense_tflops": PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS, "clock_ghz": 2.4},
           "method": (f"MFMA: {blocks} workgroups x {wpb} waves x {iters} x 16 v_mfma_f32_32x32x16_bf16 on four "
                      f"independent accumulators; clock: s_memtime over s_memrealtime (100 MHz) per workgroup, "
                      f"median; copy: {nbytes >> 30} GiB with 16-byte vector loads/stores")}
    log(f"[peaks] {out}")
    return out


def provenance(torch, head) -> dict:
    """Where the numbers come from: the GPU, the software stack, the sources and
    the inputs of the headline layer (SHA-256 of the cast tensors, 16 hex)."""
    import platform
    import subprocess
    import workloads as wl
    props = torch.cuda.get_device_properties(0)
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    try:
        head_sha = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True,
                                  timeout=10).stdout.strip() or None
    except Exception:  # pragma: no cover
        head_sha = None
    w = head["workload"]
    q, k, v = head["_tensors"][:3]
    with open(os.path.join(ROOT, "bench.py"), "rb") as f:
        bench_sha = hashlib.sha256(f.read()).hexdigest()[:16]
    return {"gpu": torch.cuda.get_device_name(0), "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count, "rocm": rocm, "torch": torch.__version__,
            "hip": torch.version.hip, "host": platform.node(), "git_head": head_sha,
            "kernel_source_sha": kernel_source_sha(), "bench_py_sha": bench_sha,
            "inputs": {"workload": w.name, "seed": w.seed, "generator": "workloads.make_inputs (on the GPU)",
                       "sha256_q": wl.sha256(q), "sha256_k": wl.sha256(k), "sha256_v": wl.sha256(v)}}


def traffic_from_profile(kernel: str, workload: str):
    """HBM bytes per launch from a committed rocprofv3 --pmc summary, if it was
    taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != kernel_source_sha():
        return None
    return float(m_b.group(1))


def useful_attn_flops(kv_cnt, w) -> float:
    """4*Bk^2*C per kept (query block, key block) tile; causal diagonal tiles count half."""
    tiles = float(kv_cnt.sum().item())
    per = 4.0 * w.block * w.block * w.C
    if w.causal:
        n_rows = kv_cnt.numel()
        return (tiles - 0.5 * n_rows) * per
    return tiles * per


def score_flops(w) -> float:
    R = w.M // w.stride
    pairs = R * (R + 1) / 2 if w.causal else R * R
    return w.B * w.Hq * 2.0 * w.stride * w.C * pairs


def run_workload(xa, wl, torch, name, steps, warmup, dense_steps):
    w = wl.WORKLOADS[name]
    dev = "cuda:0"
    t0 = time.time()
    x = wl.make_inputs(w, device=dev)
    torch.cuda.synchronize()
    log(f"[{name}] inputs generated on the GPU in {time.time() - t0:.1f}s")
    q, k, v, tau = x["q"], x["k"], x["v"], x["tau"]
    sscale, smscale = wl.default_scales(w)
    B, Hq, M, C = q.shape
    nb = w.nb
    p = xa.problem(B, Hq, w.Hkv, M, C, w.block, w.stride, w.causal, q.dtype)
    ws = torch.empty(xa.workspace_bytes(p), dtype=torch.uint8, device=dev)
    aws = torch.empty(xa.attn_workspace_bytes(p), dtype=torch.uint8, device=dev)
    scores = torch.empty((B, Hq, nb, nb), dtype=torch.float32, device=dev)
    mask = torch.empty((B, Hq, nb, nb), dtype=torch.uint8, device=dev)
    kv_idx = torch.empty((B, Hq, nb, nb), dtype=torch.int32, device=dev)
    kv_cnt = torch.empty((B, Hq, nb), dtype=torch.int32, device=dev)
    out = torch.empty_like(q)

    bufs = xa.PrefillBuffers(q, k, w.block, w.stride, w.causal, want_mask=True)

    def step():
        # the whole hot path in one C-ABI call: partials, fused normalise+select,
        # block-sparse attention
        xa.xattn_prefill(q, k, v, tau, w.block, w.stride, sscale, smscale, w.causal, buffers=bufs)

    def stages(ev):
        # the same path through the three stage entry points, for a per-stage
        # breakdown (xattn_score + xattn_select run normalisation and selection
        # as two kernels where xattn_prefill fuses them)
        ev[0].record()
        xa.xattn_score(q, k, w.block, w.stride, sscale, w.causal, block_scores=scores, ws=ws)
        ev[1].record()
        xa.xattn_select(scores, tau, w.block, w.stride, w.causal, Hkv=w.Hkv, C=C, dtype=q.dtype,
                        mask=mask, kv_idx=kv_idx, kv_cnt=kv_cnt)
        ev[2].record()
        xa.bsa_fwd(q, k, v, kv_idx, kv_cnt, w.block, smscale, w.causal, out=out, ws=aws)
        ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    ms = total_ms / steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    stages(evs[0])
    torch.cuda.synchronize()
    for i in range(steps):
        stages(evs[i])
    torch.cuda.synchronize()
    # per-stage medians over the steps (the whole-step value above is the mean
    # over exactly `steps` timed steps)
    st = {
        "xattn_score": statistics.median(e[0].elapsed_time(e[1]) for e in evs),
        "xattn_select": statistics.median(e[1].elapsed_time(e[2]) for e in evs),
        "bsa_fwd": statistics.median(e[2].elapsed_time(e[3]) for e in evs),
    }
    assert torch.equal(bufs.kv_cnt, kv_cnt), "fused and stage-wise selections differ"
    cand = B * Hq * (nb * (nb + 1) // 2 if w.causal else nb * nb)
    density = float(kv_cnt.sum().item()) / cand
    attn_flops = useful_attn_flops(kv_cnt, w)
    dense_flops = w.dense_flops
    # selection bytes (HBM-bound stage): the candidates' block scores read, the
    # mask row, the kept indices and the count written
    select_bytes = 4.0 * cand + B * Hq * nb * nb + 4.0 * float(kv_cnt.sum().item()) + 4.0 * B * Hq * nb
    log(f"[{name}] step {ms:.3f} ms (xattn_prefill)  stage calls " + " ".join(f"{k}={v:.3f}" for k, v in st.items())
        + f"  density={density * 100:.2f}%")

    dense_ms = None
    if dense_steps > 0:
        dense_out = torch.empty_like(q)
        xa.dense_fwd(q, k, v, w.block, smscale, w.causal, out=dense_out)
        torch.cuda.synchronize()
        d0 = torch.cuda.Event(enable_timing=True)
        d1 = torch.cuda.Event(enable_timing=True)
        d0.record()
        for _ in range(dense_steps):
            xa.dense_fwd(q, k, v, w.block, smscale, w.causal, out=dense_out)
        d1.record()
        torch.cuda.synchronize()
        dense_ms = d0.elapsed_time(d1) / dense_steps
        del dense_out
        log(f"[{name}] dense_fwd {dense_ms:.3f} ms ({dense_flops / dense_ms / 1e9:.1f} TFLOP/s)")

    res = {
        "workload": w,
        "ms": ms,
        "stages_ms": st,
        "density": density,
        "attn_flops": attn_flops,
        "score_flops": score_flops(w),
        "select_bytes": select_bytes,
        "dense_flops": dense_flops,
        "tflops": dense_flops / ms / 1e9,
        "dense_ms": dense_ms,
        "kv_cnt_sum": int(kv_cnt.sum().item()),
    }
    res["_tensors"] = (q, k, v, tau, kv_idx, kv_cnt)
    return res


def cpu_baseline(wl, torch, res, budget_s):
    """The oracle, as it stands, on a bounded sample of the layer: query-block
    rows in a stratified order (bit-reversed positions, so every prefix spreads
    over the sequence) of the query heads of KV group 0 in turn, until budget_s
    seconds of oracle time; the per-row cost is fitted as a + b*I (causal
    scoring and attention grow with the row index) and extrapolated to every
    row of every head."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = os.cpu_count()
    w = res["workload"]
    q, k, v, tau, _, _ = res["_tensors"]
    sscale, smscale = wl.default_scales(w)
    G = w.Hq // w.Hkv
    kh = k[0, 0].float().cpu().numpy().astype(np.float64)
    vh = v[0, 0].float().cpu().numpy().astype(np.float64)
    nb = w.nb
    bits = max(1, (nb - 1).bit_length())
    order = [r for r in (int(format(x, f"0{bits}b")[::-1], 2) for x in range(1 << bits)) if r < nb]
    qh = np.zeros((w.M, w.C))
    times = []
    spent = 0.0
    for j, big_i in enumerate(order):
        h = j % G
        rows = slice(big_i * w.block, (big_i + 1) * w.block)
        qh[rows] = q[0, h, rows].float().cpu().numpy()
        t0 = time.perf_counter()
        sc = oracle.block_score_row(qh, kh, big_i, w.block, w.stride, sscale, w.causal)
        keep = oracle.select_row(sc, big_i, float(tau[h]), w.causal)
        oracle.attend_row(qh, kh, vh, keep, big_i, w.block, smscale, w.causal)
        dt = time.perf_counter() - t0
        qh[rows] = 0.0
        times.append((big_i, h, dt))
        spent += dt
        if spent > budget_s and len(times) >= 2:
            break
    Is = np.array([t[0] for t in times], dtype=np.float64)
    ts = np.array([t[2] for t in times])
    if w.causal and len(times) >= 2 and np.ptp(Is) > 0:
        b, a = np.polyfit(Is, ts, 1)
        per_head = max(a * nb + b * nb * (nb - 1) / 2, ts.mean() * nb)
    else:
        per_head = ts.mean() * nb
    total_s = per_head * w.B * w.Hq
    cpu_model = None
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [f"{i.get('internal_api')} {i.get('version')} ({i.get('threading_layer')})" for i in threadpool_info()
                if i.get("user_api") == "blas"]
    except Exception:  # pragma: no cover
        blas = []
    return {
        "value": w.dense_flops / total_s / 1e12,
        "unit": "TFLOP/s (dense-equivalent)",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{len(times)} query-block rows (stratified over I = 0..{nb - 1}, query heads 0..{G - 1} in "
                   f"turn) of {w.name}, score+select+attend in float64 NumPy, {ts.sum():.1f}s of oracle time; "
                   f"per-row cost fitted as a + b*I and extrapolated to {nb} rows x {w.Hq} heads = "
                   f"{total_s:.0f}s per layer"),
        "ms_per_step_extrapolated": total_s * 1e3,
        "nproc": os.cpu_count(),
        "cpu_model": cpu_model,
        "blas": blas,
        "note": ("the oracle is unoptimised by design: each row re-derives the head's whole reversed-K view "
                 "(Mk x C float64) before its strided logits, so much of its time is that copy"),
    }


def run_variants(xa, torch, head, steps):
    """The headline layer through xattn_prefill with each method variant:
    per-row selection on the same buffers (no mask output, the reference for
    the others), selection inside the scoring launch, global and GQA-union
    selection, the diagonal and DuSA1 scoring patterns, a chunked prefill step
    and a ragged length."""
    w = head["workload"]
    q, k, v, tau = head["_tensors"][:4]
    sscale, smscale = 1.0 / (w.stride * math.sqrt(w.C)), 1.0 / math.sqrt(w.C)
    cand = w.B * w.Hq * (w.nb * (w.nb + 1) // 2 if w.causal else w.nb * w.nb)
    res = {}
    for label, kw in (("select_row", {}),
                      ("select_in_score", dict(select_in_score=True)),
                      ("select_global", dict(selection="global")),
                      ("select_gqa_union", dict(selection="gqa_union")),
                      ("pattern_diagonal", dict(pattern=xa.DIAGONAL)),
                      ("pattern_dusa1", dict(pattern=xa.DUSA1))):
        bufs = xa.PrefillBuffers(q, k, w.block, w.stride, w.causal, want_mask=False, **kw)
        # a DuSA1 phase logit is one dot product: the attention scale
        ss = smscale if kw.get("pattern") == xa.DUSA1 else sscale

        def step():
            xa.xattn_prefill(q, k, v, tau, w.block, w.stride, ss, smscale, w.causal, buffers=bufs, **kw)

        step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        dens = float(bufs.kv_cnt.sum().item()) / cand
        res[label] = {"ms": round(ms, 4), "density": round(dens, 5),
                      "dense_equiv_tflops": round(w.dense_flops / ms / 1e9, 2)}
        log(f"[{w.name}] variant {label}: {ms:.3f} ms, density {dens * 100:.2f}%")
        del bufs
        torch.cuda.empty_cache()
    # chunked prefill (the last 32K queries against the whole context) and a
    # ragged length (not a multiple of the block or the stride)
    chunk = min(32768, w.M // 2)
    for label, mq, mk in ((f"chunk_last{chunk // 1024}k", chunk, w.M), ("ragged_" + str(w.M - 12101), w.M - 12101,
                                                                        w.M - 12101)):
        qv = q[:, :, mk - mq:mk].contiguous()
        kv = k[:, :, :mk].contiguous()
        vv = v[:, :, :mk].contiguous()
        bufs = xa.PrefillBuffers(qv, kv, w.block, w.stride, w.causal, want_mask=False)

        def step():
            xa.xattn_prefill(qv, kv, vv, tau, w.block, w.stride, sscale, smscale, w.causal, buffers=bufs)

        step()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        nbq, nbk = -(-mq // w.block), -(-mk // w.block)
        qoff = nbk - nbq
        cand_v = w.B * w.Hq * (sum(i + qoff + 1 for i in range(nbq)) if w.causal else nbq * nbk)
        dens = float(bufs.kv_cnt.sum().item()) / cand_v
        off = mk - mq
        pairs = mq * off + mq * (mq + 1) / 2 if w.causal else mq * mk
        flops = 4.0 * w.B * w.Hq * w.C * pairs
        res[label] = {"ms": round(ms, 4), "density": round(dens, 5), "Mq": mq, "Mk": mk,
                      "dense_equiv_tflops": round(flops / ms / 1e9, 2)}
        log(f"[{w.name}] variant {label} (Mq={mq}, Mk={mk}): {ms:.3f} ms, density {dens * 100:.2f}%")
        del bufs, qv, kv, vv
        torch.cuda.empty_cache()
    return res


def library_context(xa, wl, torch):
    """Library routines on the path's shapes, for context only (never part of a
    step): a plain hipBLASLt GEMM (torch.mm, bf16) of one head's strided
    operands at 256K, the whole square where the scoring kernel computes the
    causal triangle with its epilogue, and torch's flash SDPA backend on the
    dense causal 32K and 128K layers next to dense_fwd."""
    dev = "cuda:0"
    out = {}

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    w = wl.WORKLOADS["llama256k"]
    R, D = w.M // w.stride, w.stride * w.C
    g = torch.Generator(device=dev).manual_seed(0)
    kp = torch.randn((R, D), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    qt = torch.randn((D, R), generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty((R, R), device=dev, dtype=torch.bfloat16)
    ms = timed(lambda: torch.mm(kp, qt, out=c), 10)
    flops = 2.0 * R * R * D
    out["gemm_strided_256k_one_head"] = {"routine": "torch.mm (hipBLASLt), bf16 in/out", "shape": [R, D, R],
                                         "ms": round(ms, 4), "tflops": round(flops / ms / 1e9, 1)}
    log(f"[library] torch.mm {R}x{D}x{R}: {ms:.3f} ms, {flops / ms / 1e9:.0f} TFLOP/s")
    del kp, qt, c
    torch.cuda.empty_cache()

    from torch.nn.attention import SDPBackend, sdpa_kernel
    import torch.nn.functional as F
    for name in ("llama32k", "llama128k"):
        w = wl.WORKLOADS[name]
        x = wl.make_inputs(w, device=dev)
        q, k, v = x["q"], x["k"], x["v"]
        _, smscale = wl.default_scales(w)
        g = w.Hq // w.Hkv
        ke = k.repeat_interleave(g, dim=1).contiguous()
        ve = v.repeat_interleave(g, dim=1).contiguous()
        ours = torch.empty_like(q)
        n = 3 if w.M <= 32768 else 1
        ms_ours = timed(lambda: xa.dense_fwd(q, k, v, w.block, smscale, True, out=ours), n)
        rec = {"dense_fwd_ms": round(ms_ours, 3), "dense_fwd_tflops": round(w.dense_flops / ms_ours / 1e9, 1)}
        try:
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                ref = [None]

                def sdpa():
                    ref[0] = F.scaled_dot_product_attention(q, ke, ve, is_causal=True, scale=smscale)
                ms = timed(sdpa, n)
            diff = (ref[0].float() - ours.float()).abs().max().item()
            rec.update({"routine": "torch SDPA, flash backend, K/V repeated to 32 heads",
                        "sdpa_ms": round(ms, 3), "sdpa_tflops": round(w.dense_flops / ms / 1e9, 1),
                        "max_abs_diff_vs_dense_fwd": diff})
            log(f"[library] {name} SDPA flash {ms:.3f} ms, dense_fwd {ms_ours:.3f} ms, max|diff| {diff:.3g}")
        except RuntimeError as e:
            rec["sdpa_error"] = str(e).splitlines()[0][:200]
            log(f"[library] {name} SDPA flash unavailable: {rec['sdpa_error']}")
        out[name] = rec
        del x, q, k, v, ke, ve, ours
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama256k")
    ap.add_argument("--also", default="llama8k,llama32k,llama128k",
                    help="other lengths reported under by_length (comma list, '' for none)")
    ap.add_argument("--extra", default="video,tiny",
                    help="other configurations reported under other_configs (comma list, '' for none)")
    ap.add_argument("--dense-steps", type=int, default=2)
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the peak-rate microbenchmarks")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip timing the selection and scoring variants on the headline layer")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain elementwise kernel of known size (1 GiB read, 1 GiB "
                         "written), the reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--library-context", action="store_true",
                    help="only time library routines on the path's shapes (hipBLASLt GEMM, torch's flash "
                         "SDPA) next to dense_fwd, as context; prints one JSON line")
    a = ap.parse_args()

    if a.copy_calibration:
        import torch
        x = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            torch.mul(x, 2.0, out=y)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "torch.mul(x, 2.0, out=y)", "launches": 3,
                          "bytes_read_per_launch": 1 << 30, "bytes_written_per_launch": 1 << 30}))
        return

    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only (--gpus 1): the library runs a layer on a single "
              "MI355X; across GPUs a layer shards by KV-head group with no communication, which "
              "this benchmark does not run.", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_sparse_attention_xattn_amd as xa
    import workloads as wl

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)

    if a.library_context:
        print(json.dumps({"library_context": library_context(xa, wl, torch)}))
        return

    others = {}
    for n in [n for n in a.extra.split(",") if n and n != a.workload]:
        others[n] = run_workload(xa, wl, torch, n, max(3, a.steps // 2), a.warmup, a.dense_steps)
        others[n].pop("_tensors", None)
        torch.cuda.empty_cache()

    names = [a.workload] + [n for n in a.also.split(",") if n and n != a.workload]
    results = {}
    for n in names[1:] + names[:1]:  # headline workload last so its tensors stay for the CPU leg
        if results:
            for r in results.values():
                r.pop("_tensors", None)
            torch.cuda.empty_cache()
        results[n] = run_workload(xa, wl, torch, n, a.steps if n == a.workload else max(3, a.steps // 2),
                                  a.warmup, a.dense_steps)
    head = results[a.workload]
    w = head["workload"]

    # roofline of the dominant kernel
    st = head["stages_ms"]
    dom = max(st, key=st.get)
    if dom == "bsa_fwd":
        ach = head["attn_flops"] / (st[dom] * 1e-3) / 1e12
        roof = {"kernel": "bsa_fwd (attn_fwd_bf16_kernel<128,128,causal,sparse>)", "bound": "mfma", "achieved": ach,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS}
    else:
        ach = head["score_flops"] / (st[dom] * 1e-3) / 1e12
        roof = {"kernel": "xattn_score (score_partials_dma_kernel + score_finalize_kernel)", "bound": "mfma",
                "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS}
    roof["traffic"] = traffic_from_profile("bsa_fwd" if dom == "bsa_fwd" else "xattn_score", w.name)

    variants = None if a.no_variants else run_variants(xa, torch, head, max(2, a.steps // 3))

    prov = provenance(torch, head)
    peaks = None if a.no_peaks else measure_peaks(torch)

    cpu = None
    if not a.no_cpu_baseline:
        log("[cpu] timing the oracle on a bounded sample ...")
        cpu = cpu_baseline(wl, torch, head, a.cpu_budget)

    def summary(r):
        sel_tf = r["attn_flops"] / (r["stages_ms"]["bsa_fwd"] * 1e-3) / 1e12
        d = {"ms": round(r["ms"], 4), "dense_equiv_tflops": round(r["tflops"], 2),
             # dense-equivalent rate over the bf16 peak: above 1 whenever sparsity
             # saves more than the kernels lose; not a roofline fraction
             "dense_equiv_over_bf16_peak": round(r["tflops"] / PEAK_BF16_TFLOPS, 4),
             "selected_tile_frac_of_bf16_peak": round(sel_tf / PEAK_BF16_TFLOPS, 4),
             "stages_ms": {k: round(v, 4) for k, v in r["stages_ms"].items()},
             "density": round(r["density"], 5),
             "selected_tile_tflops": round(sel_tf, 2),
             "score_tflops": round(r["score_flops"] / (r["stages_ms"]["xattn_score"] * 1e-3) / 1e12, 2),
             "select_gbs": round(r["select_bytes"] / (r["stages_ms"]["xattn_select"] * 1e-3) / 1e9, 1)}
        if r["dense_ms"]:
            d["dense_fwd_ms"] = round(r["dense_ms"], 3)
            d["dense_fwd_tflops"] = round(r["dense_flops"] / r["dense_ms"] / 1e9, 2)
            d["speedup_vs_dense_fwd"] = round(r["dense_ms"] / r["ms"], 3)
        return d

    line = {
        "metric": METRIC,
        "value": round(head["tflops"], 3),
        "unit": "TFLOP/s (dense-equivalent)",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded generators: sinks, slash bands, random vertical columns; no dataset)",
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "M": w.M, "C": w.C,
                   "block": w.block, "stride": w.stride, "tau": w.tau, "causal": w.causal,
                   "density": round(head["density"], 5)},
        **{k: v for k, v in summary(head).items() if k not in ("ms", "dense_equiv_tflops")},
        "roofline": roof,
        "cpu_baseline": cpu,
        "by_length": {n: summary(r) for n, r in results.items()},
        "variants": variants,
        "other_configs": {n: {"config": {"Hq": r["workload"].Hq, "Hkv": r["workload"].Hkv, "M": r["workload"].M,
                                          "C": r["workload"].C, "block": r["workload"].block,
                                          "stride": r["workload"].stride, "tau": r["workload"].tau,
                                          "causal": r["workload"].causal, "dtype": r["workload"].dtype},
                              **summary(r)}
                          for n, r in others.items()},
        "peaks_measured": peaks,
        "provenance": prov,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
