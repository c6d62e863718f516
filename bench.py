#!/usr/bin/env python3
"""Benchmark of the FP16 fused-attention forward hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--only NAME] [--no-cpu] [--no-extra]

Headline (one step = one attn_fwd_dense call over the whole workload): the
dense non-causal D128 attention of a video diffusion transformer, B1 H8
L36864, FP16 inputs N(0,1), FP32 accumulation, FP16 output. `value` is its
algorithmic throughput, 4*D FLOP per (query, key) pair, in TFLOP/s.

The same JSON line carries, under "extra", the other workloads of the hot
path, each timed with HIP events on the launch stream:
  * causal prefill D256 Hq6/Hkv1 Q8000 KV128000 (split-KV + merge), TFLOP/s
    over the visible pairs only;
  * the dense D128 shape of the GB10 page, H56 Lq15360 Lkv29678 with LSE,
    on FP16 and on BF16 operands;
  * the same prefill reading a paged E4M3 cache, KV256000, non-unit scales;
  * the exact paged E4M3 -> FP16 bridge, GB/s over the bytes it must move;
  * decode: 16 new positions of all 6 heads against the same 256000-token
    E4M3 cache, GB/s over the cache read once (HBM-bound);
  * the FP8 round trip of prefix keys with the valid-row gather (B1 N36864
    H8, 32768 rows), GB/s over K and V rows read and written;
  * the FP8-MFMA prefix attention (per-row E4M3 queries and keys, BF16 V) at
    the video shape, TFLOP/s and its fraction of the mixed FP8/BF16 peak;
  * VSA block selection (pool, score, top-k), GB/s over Q and K read once
    plus the indices written, and VSA block-sparse attention, TFLOP/s over
    the selected pairs.
HBM-bound kernels run after a 512 MiB buffer read that evicts the 256 MB
last-level cache, outside the timed events.

"cpu_baseline" times the FP64 CPU oracle on a sample of query rows of the
headline workload on this host's cores (a reported baseline, not a target),
and "parity_sample" compares those rows with the GPU output.

"roofline.measured_ceiling" is the rate of fa_mfma_ceiling, a kernel of
nothing but FP16 MFMAs on operands varied per lane: the matrix throughput the
chip sustains on data like these inputs, timed right after the headline and
reported beside the published peak.

Only one GPU is supported: --gpus N with N > 1 exits with an error.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense FP16 MFMA, published
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
METRIC = "attention TFLOP/s and % FP16 MFMA peak (D128 dense, D256 causal prefix)"
# The pages publish no kernel-level attention timings; their nearest figures are
# whole-model runs on four V100 SXM2 32GB (tensor parallel 4). Context only:
# other hardware, other work, not a target.
PAGES_CONTEXT = {
    "hardware": "4x V100 SXM2 32GB, TP4 (whole-model runs)",
    "dense_fa_denoise_median_s": 58.293218,
    "vsa_fp16_denoise_median_s": 30.990756,
    "prefill_256000_tokens_model_s": 106.985,
    "prefill_v37_port_speed_ratio_kv128000": 0.998963,
}


def log(*msg):
    print("[bench]", *msg, file=sys.stderr, flush=True)


# ------------------------------------------------------------------ FLOP / byte accounting

def dense_flops(w):
    return 4 * w["D"] * w["B"] * w["H"] * w["Lq"] * w["Lkv"]


def causal_flops(w):
    """4*D per visible pair; query row i sees keys 0 .. (kv_len - q_real) + i."""
    off = w["kv_len"] - w["q_real"]
    vis = np.minimum(off + np.arange(w["q_rows"], dtype=np.int64) + 1, w["kv_len"])
    return 4 * w["D"] * w["B"] * w["Hq"] * int(vis.sum())


def vsa_flops(w):
    nb, blk, dp = w["L"] // w["block"], w["block"], w["dense_prefix"]
    pairs = dp * blk * w["L"] + (nb - dp) * blk * w["topk"] * blk
    return 4 * w["D"] * w["B"] * w["H"] * pairs


def bridge_bytes(w):
    n = w["B"] * w["Hkv"] * w["kv_len"] * w["D"]
    return 2 * n + 2 * 2 * n + 4 * (w["kv_len"] // w["page_size"]) * w["B"]


def decode_bytes(w):
    """The cache codes of every key read once, the page table, q read and o written."""
    return (2 * w["B"] * w["Hkv"] * w["kv_len"] * w["D"] + 4 * w["B"] * (w["kv_len"] // w["page_size"])
            + 2 * 2 * w["B"] * w["Hq"] * w["q_rows"] * w["D"])


def select_bytes(w):
    nb = w["L"] // w["block"]
    return 2 * 2 * w["B"] * w["H"] * w["L"] * w["D"] + 4 * w["B"] * w["H"] * nb * w["topk"]


def dense_traffic(path):
    """HBM bytes per launch of the dense kernel from the recorded rocprofv3
    FETCH_SIZE / WRITE_SIZE runs (scaled by a 1 GiB copy's readings), or None
    when there is no record or the kernel source has changed since."""
    if not os.path.exists(path):
        return None
    import hashlib
    with open(path) as f:
        t = json.load(f)
    with open(os.path.join(ROOT, "fp16_attention_amd", "csrc", "attn_fwd.hip"), "rb") as f:
        src = hashlib.sha256(f.read()).hexdigest()
    if t.get("kernel_source_sha256") != src:
        log("traffic record is for another version of attn_fwd.hip: reporting null")
        return None
    return t.get("attn_fwd_dense_video")


# ------------------------------------------------------------------------------ timing

class Timer:
    """HIP events around each launch on torch's current stream (the stream the
    library enqueues on)."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, fn, iters, warmup, flush=None):
        torch = self.torch
        for _ in range(warmup):
            if flush is not None:
                flush()
            fn()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(iters)]
        t0 = time.perf_counter()
        for s, e in ev:
            if flush is not None:
                flush()
            s.record()
            fn()
            e.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = np.array([s.elapsed_time(e) for s, e in ev])
        return ms, wall


def stats(ms):
    return {"median_ms": float(np.median(ms)), "mean_ms": float(ms.mean()),
            "cv": float(ms.std() / ms.mean()) if ms.mean() > 0 else 0.0}


# --------------------------------------------------------------------------- workloads

def bench_copy(torch, timer, iters, flush=None):
    """The runtime's device copy of 1 GiB: the measured HBM copy rate that
    the HBM-bound kernels are also reported against."""
    src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms, _ = timer.run(lambda: dst.copy_(src), iters, 2, flush=flush)
    gbs = 2 * src.numel() / (np.median(ms) * 1e-3) / 1e9
    log(f"copy 1 GiB: {np.median(ms):.3f} ms  {gbs:.0f} GB/s")
    rec = {"workload": "device copy of 1 GiB (read 1 GiB, write 1 GiB)", "bytes_read": src.numel(),
           "bytes_written": dst.numel(), **stats(ms), "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
           "llc_flushed": flush is not None}
    del src, dst
    torch.cuda.empty_cache()
    return rec


def bench_dense(fa, torch, W, steps, warmup, timer):
    import synth.workloads as wl
    w = wl.VIDEO_DENSE
    log("generating", w["name"])
    q, k, v = wl.dense_inputs(w)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    out = torch.empty_like(dq)
    fn = lambda: fa.attn_fwd_dense(dq, dk, dv, out=out)
    log(f"dense: warmup {warmup}, {steps} timed steps")
    ms, wall = timer.run(fn, steps, warmup)
    return w, (q, k, v), out, ms, wall


def bench_ragged(fa, torch, iters, timer):
    import synth.workloads as wl
    w = wl.RAGGED_DENSE
    log("generating", w["name"])
    q, k, v = wl.dense_inputs(w)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(dq)
    lse = torch.empty((w["B"], w["H"], w["Lq"]), dtype=torch.float32, device="cuda")
    ms, _ = timer.run(lambda: fa.attn_fwd_dense(dq, dk, dv, out=out, lse=lse), iters, 2)
    f = dense_flops(w)
    tf = f / (np.median(ms) * 1e-3) / 1e12
    log(f"ragged dense: {np.median(ms):.3f} ms  {tf:.1f} TFLOP/s")
    res = {"workload": w["name"] + ", FP32 LSE", "flop": f, **stats(ms), "tflops": tf,
           "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS}
    # the same shape on BF16 operands (BF16 MFMA; same dense peak)
    for t in (dq, dk, dv):
        t.copy_(t.to(torch.bfloat16).view(torch.float16))
    dq, dk, dv = (t.view(torch.bfloat16) for t in (dq, dk, dv))
    outb = out.view(torch.bfloat16)
    ms, _ = timer.run(lambda: fa.attn_fwd_dense(dq, dk, dv, out=outb, lse=lse), iters, 2)
    tf = f / (np.median(ms) * 1e-3) / 1e12
    log(f"ragged dense bf16: {np.median(ms):.3f} ms  {tf:.1f} TFLOP/s")
    bf = {"workload": w["name"] + ", BF16 operands, FP32 LSE", "flop": f, **stats(ms), "tflops": tf,
          "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS}
    return res, bf


FP8_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published


def bench_prefix_fp8_attn(fa, torch, iters, timer):
    """The FP8-MFMA prefix attention (per-row E4M3 queries and keys, BF16 values) at the
    video shape: B1 H8 D128 Lq = Lkv = 36864, the dense workload's draws rounded to BF16.
    Half of the algorithmic FLOPs (QK^T) run at the FP8 rate, half (PV) at the BF16 rate,
    so the mixed peak is 1 / (0.5 / 5.0 + 0.5 / 2.5) PFLOP/s = 3.33 PFLOP/s. The timed call
    includes the per-row quantization of Q and K."""
    import synth.workloads as wl
    w = wl.VIDEO_DENSE
    log("generating", w["name"], "(BF16 operands for the FP8 prefix path)")
    q, k, v = wl.dense_inputs(w)
    dq, dk, dv = (torch.from_numpy(x).cuda().to(torch.bfloat16) for x in (q, k, v))
    del q, k, v
    out = torch.empty_like(dq)
    ws = torch.empty(fa.prefix_fp8_workspace(w["B"], w["H"], w["Lq"], w["Lkv"]), dtype=torch.uint8, device="cuda")
    ms, _ = timer.run(lambda: fa.attn_fwd_prefix_fp8(dq, dk, dv, out=out, workspace=ws), iters, 2)
    f = dense_flops(w)
    tf = f / (np.median(ms) * 1e-3) / 1e12
    mixed_peak = 1.0 / (0.5 / FP8_PEAK_TFLOPS + 0.5 / MFMA_F16_PEAK_TFLOPS)
    log(f"prefix fp8 attention: {np.median(ms):.3f} ms  {tf:.1f} TFLOP/s = {100 * tf / mixed_peak:.1f}% of "
        f"the mixed FP8/BF16 peak")
    return {"workload": "FP8-QK prefix attention B1 H8 D128 Lq36864 Lkv36864, BF16 operands, per-row E4M3 Q and K "
                        "(quantization included)", "flop": f, **stats(ms), "tflops": tf,
            "peak_tflops": mixed_peak, "frac_mixed_peak": tf / mixed_peak,
            "frac_fp16_peak": tf / MFMA_F16_PEAK_TFLOPS}


def bench_causal(fa, torch, iters, timer):
    import synth.workloads as wl
    w = wl.PREFIX_CAUSAL
    log("generating", w["name"])
    q, k, v = wl.causal_inputs(w)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    del q, k, v
    ws_bytes = fa.prefix_causal_workspace(w["B"], w["Hq"], w["Hkv"], w["D"], w["q_rows"], w["kv_len"])
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dq)
    fn = lambda: fa.attn_fwd_prefix_causal(dq, dk, dv, w["q_real"], out=out, workspace=ws)
    ms, _ = timer.run(fn, iters, 2)
    f = causal_flops(w)
    tf = f / (np.median(ms) * 1e-3) / 1e12
    log(f"causal: {np.median(ms):.3f} ms  {tf:.1f} TFLOP/s")
    return {"workload": w["name"], "flop": f, **stats(ms), "tflops": tf,
            "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS, "workspace_bytes": ws_bytes,
            "kernels": "attn split-KV + merge"}


def bench_paged(fa, torch, iters, timer, flush):
    import synth.workloads as wl
    w = wl.PAGED_E4M3
    log("generating", w["name"])
    q, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    dq, dkc, dvc, dt = (torch.from_numpy(x).cuda() for x in (q, kc, vc, table))
    del q, kc, vc
    shape = (w["B"], w["Hq"], w["Hkv"], w["D"], w["q_rows"], w["kv_len"])
    out = torch.empty_like(dq)
    f = causal_flops(w)
    plans = {}
    # the library's plans for this non-power-of-two k_scale: with the workspace the bridged plan needs
    # (the exact bridge into FP16 K/V, then the FP16 causal kernel), and with the split-KV states only
    # (the cache attended in place, K converted per workgroup in LDS)
    for name, k_arg in (("bridged", ks), ("in_place", None)):
        ws_bytes = fa.paged_e4m3_workspace(*shape, k_scale=k_arg)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        fn = lambda: fa.attn_fwd_paged_e4m3(dq, dkc, dvc, dt, w["kv_len"], w["q_real"], ks, vs, out=out,
                                            workspace=ws)
        ms, _ = timer.run(fn, iters, 2)
        tf = f / (np.median(ms) * 1e-3) / 1e12
        log(f"paged e4m3 ({name}): {np.median(ms):.3f} ms  {tf:.1f} TFLOP/s")
        plans[name] = {"workload": w["name"] + f" k_scale={ks:.6g} v_scale={vs:.6g}, {name} plan", "flop": f,
                       **stats(ms), "tflops": tf, "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS,
                       "workspace_bytes": ws_bytes}
        del ws
    fused = plans["bridged"]
    fused["in_place_plan"] = plans["in_place"]

    ko = torch.empty((w["B"], w["Hkv"], w["kv_len"], w["D"]), dtype=torch.float16, device="cuda")
    vo = torch.empty_like(ko)
    fn = lambda: fa.kv_e4m3_paged_to_fp16(dkc, dvc, dt, w["B"], w["kv_len"], ks, vs, k_out=ko, v_out=vo)
    ms, _ = timer.run(fn, iters, 2, flush=flush)
    nb = bridge_bytes(w)
    gbs = nb / (np.median(ms) * 1e-3) / 1e9
    log(f"bridge: {np.median(ms) * 1e3:.1f} us  {gbs:.0f} GB/s")
    bridge = {"workload": "exact paged E4M3 -> FP16 bridge, K and V, KV256000 D256 page32", "bytes": nb,
              **stats(ms), "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS, "llc_flushed": True}
    # decode: 16 new positions per head against the same cache, HBM-bound
    wd = wl.PAGED_DECODE
    qd = torch.from_numpy(wl.paged_inputs(wd, unit_scales=False)[0]).cuda()
    ws_d = torch.empty(fa.load().attn_fwd_paged_e4m3_decode_workspace(wd["B"], wd["Hq"], wd["Hkv"], wd["D"],
                                                                       wd["q_rows"], wd["kv_len"]),
                       dtype=torch.uint8, device="cuda")
    od = torch.empty_like(qd)
    fn = lambda: fa.attn_fwd_paged_e4m3_decode(qd, dkc, dvc, dt, wd["kv_len"], wd["q_real"], ks, vs, out=od,
                                               workspace=ws_d)
    ms, _ = timer.run(fn, iters, 2, flush=flush)
    nb = decode_bytes(wd)
    gbs = nb / (np.median(ms) * 1e-3) / 1e9
    log(f"paged decode: {np.median(ms) * 1e3:.1f} us  {gbs:.0f} GB/s")
    decode = {"workload": wd["name"] + f" k_scale={ks:.6g} v_scale={vs:.6g}", "bytes": nb, **stats(ms),
              "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS, "llc_flushed": True,
              "workspace_bytes": int(ws_d.numel())}
    # the same cache decoded for fewer new positions per head, timing only: one
    # (6 packed rows: one-wave workgroups) and eight (48 rows: 16-row waves)
    for n, key in ((1, "one_position"), (8, "eight_positions")):
        qn = qd[:, :, :n].contiguous()
        ws_n = torch.empty(fa.load().attn_fwd_paged_e4m3_decode_workspace(wd["B"], wd["Hq"], wd["Hkv"], wd["D"], n,
                                                                           wd["kv_len"]),
                           dtype=torch.uint8, device="cuda")
        on = torch.empty_like(qn)
        fn = lambda: fa.attn_fwd_paged_e4m3_decode(qn, dkc, dvc, dt, wd["kv_len"], n, ks, vs, out=on, workspace=ws_n)
        msn, _ = timer.run(fn, iters, 2, flush=flush)
        gbsn = nb / (np.median(msn) * 1e-3) / 1e9
        log(f"paged decode, {n} position{'s' if n > 1 else ''}: {np.median(msn) * 1e3:.1f} us  {gbsn:.0f} GB/s")
        decode[key] = {"q_rows": n, **stats(msn), "gbs": gbsn, "frac_hbm_peak": gbsn / HBM_PEAK_GBS,
                       "workspace_bytes": int(ws_n.numel())}
    return fused, bridge, decode


def bench_prefix_fp8(fa, torch, iters, timer, flush):
    import synth.workloads as wl
    w = wl.PREFIX_FP8
    log("generating", w["name"])
    k, v, index = wl.prefix_fp8_inputs(w)
    dk, dv = (torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16) for x in (k, v))
    di = torch.from_numpy(index).cuda()
    del k, v
    ko = torch.empty((w["B"], w["rows"], w["H"], w["D"]), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)
    ms, _ = timer.run(lambda: fa.kv_prefix_fp8_gather(dk, dv, di, k_out=ko, v_out=vo), iters, 2, flush=flush)
    nb = 4 * w["B"] * w["rows"] * w["H"] * w["D"] * 2 + 4 * w["rows"]
    gbs = nb / (np.median(ms) * 1e-3) / 1e9
    log(f"prefix fp8 gather: {np.median(ms) * 1e3:.1f} us  {gbs:.0f} GB/s")
    return {"workload": w["name"], "bytes": nb, **stats(ms), "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS,
            "llc_flushed": True}


def bench_vsa(fa, torch, iters, timer, flush):
    import synth.workloads as wl
    w = wl.VSA
    log("generating", w["name"])
    q, k, v = wl.vsa_inputs(w)
    dq, dk, dv = (torch.from_numpy(x).cuda() for x in (q, k, v))
    del q, k, v
    nb = w["L"] // w["block"]
    idx = torch.empty((w["B"], w["H"], nb, w["topk"]), dtype=torch.int32, device="cuda")
    ws = torch.empty(fa.load().vsa_block_select_workspace(w["B"], w["H"], w["L"], w["D"], w["block"]),
                     dtype=torch.uint8, device="cuda")
    sel = lambda: fa.vsa_block_select(dq, dk, w["topk"], block=w["block"], workspace=ws, out=idx)
    ms_s, _ = timer.run(sel, iters, 2, flush=flush)
    sb = select_bytes(w)
    gbs = sb / (np.median(ms_s) * 1e-3) / 1e9
    log(f"vsa select: {np.median(ms_s) * 1e3:.1f} us  {gbs:.0f} GB/s")
    out = torch.empty_like(dq)
    att = lambda: fa.vsa_block_sparse_attn(dq, dk, dv, idx, dense_prefix_qblocks=w["dense_prefix"],
                                           block=w["block"], out=out)
    ms_a, _ = timer.run(att, iters, 2)
    f = vsa_flops(w)
    tf = f / (np.median(ms_a) * 1e-3) / 1e12
    log(f"vsa sparse: {np.median(ms_a):.3f} ms  {tf:.1f} TFLOP/s")
    return ({"workload": w["name"] + " (pool + FP64 block scores + top-k)", "bytes": sb, **stats(ms_s),
             "gbs": gbs, "frac_hbm_peak": gbs / HBM_PEAK_GBS, "llc_flushed": True},
            {"workload": w["name"] + " (sparse attention)", "flop": f, **stats(ms_a), "tflops": tf,
             "frac_mfma_peak": tf / MFMA_F16_PEAK_TFLOPS,
             "selected_fraction_of_dense": f / (4 * w["D"] * w["B"] * w["H"] * w["L"] * w["L"])})


# -------------------------------------------------------------------------- CPU oracle

def bench_mfma_ceiling(fa, torch, timer, iters=16384, launches=5):
    """FP16 MFMA rate the chip sustains on varied operands (fa_mfma_ceiling, a
    measurement aid in its own library): the attainable matrix throughput
    beside the published peak."""
    from fp16_attention_amd import measure
    out = torch.empty(measure.MFMA_CEILING_OUT, dtype=torch.float32, device="cuda")
    ms, _ = timer.run(lambda: measure.mfma_ceiling(out, iters), launches, 2)
    tf = measure.mfma_ceiling_flop(iters) / (np.median(ms) * 1e-3) / 1e12
    log(f"MFMA ceiling (varied FP16 operands): {np.median(ms):.3f} ms, {tf:.0f} TFLOP/s")
    return {"value": tf, "unit": "TFLOP/s", "kind": "fa_mfma_ceiling: FP16 MFMAs only, operands varied per lane",
            "flop_per_launch": measure.mfma_ceiling_flop(iters), **stats(ms)}


def cpu_baseline(w, qkv, out_gpu, rows_per_head):
    """Time the FP64 oracle on a seeded sample of query rows of the headline
    workload and compare the GPU output on those rows."""
    import oracle
    q, k, v = qkv
    rng = np.random.default_rng(1234)
    rows = []
    for h in range(w["H"]):
        # first and last rows, both sides of 16 seeded 128-row tile boundaries,
        # then seeded random rows up to rows_per_head distinct rows
        edges = 128 * rng.integers(1, w["Lq"] // 128, 16)
        sel = {0, w["Lq"] - 1, *(edges - 1).tolist(), *edges.tolist()}
        while len(sel) < rows_per_head:
            sel.add(int(rng.integers(0, w["Lq"])))
        rows += [(0, h, i) for i in sorted(sel)]
    rows = np.array(rows, dtype=np.int32)
    threads = max(1, min(16, os.cpu_count() or 1))
    oracle.build()
    log(f"cpu oracle: {len(rows)} rows on {threads} threads")
    t0 = time.perf_counter()
    ref, _ = oracle.attention(q, k, v, float(np.float32(1.0 / np.sqrt(w["D"]))), rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    flop = 4 * w["D"] * w["Lkv"] * len(rows)
    got = out_gpu[rows[:, 0], rows[:, 1], rows[:, 2]].astype(np.float64)
    err = got - ref
    parity = {"rows": int(len(rows)), "max_abs": float(np.abs(err).max()),
              "rel_l2": float(np.linalg.norm(err) / np.linalg.norm(ref))}
    cpu = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} query rows ({rows_per_head} per head, seeded: first, last, both sides of 16 "
                     f"tile boundaries, random) of the headline workload, "
                     f"each against all {w['Lkv']} keys, FP64; {dt:.2f} s wall",
           "seconds": dt, "host_cpus_online": os.cpu_count(), "cpu_model": _cpu_model(),
           "extrapolated_full_problem_s": dense_flops(w) / (flop / dt),
           "extrapolation": "the whole workload's FLOP at the sampled rate (an extrapolation, not a measurement)"}
    return cpu, parity


def cpu_extra_baselines(rows_per_head: int = 8):
    """The FP64 oracle timed on three more workloads: a seeded sample of query
    rows of the causal prefill, and the whole paged E4M3 -> FP16 bridge and
    the whole VSA block selection (each a few seconds of CPU work)."""
    import oracle
    import synth.workloads as wl
    oracle.build()
    threads = max(1, min(16, os.cpu_count() or 1))
    res = {}

    w = wl.PREFIX_CAUSAL
    q, k, v = wl.causal_inputs(w)
    rng = np.random.default_rng(4321)
    off = w["kv_len"] - w["q_real"]
    rows = []
    for h in range(w["Hq"]):
        sel = {0, w["q_real"] - 1, *rng.integers(0, w["q_real"], rows_per_head - 2).tolist()}
        rows += [(0, h, i) for i in sorted(sel)]
    rows = np.array(rows, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.attention(q, k, v, float(np.float32(1.0 / np.sqrt(w["D"]))), mode=oracle.MODE_CAUSAL, offset=off,
                     rows=rows, threads=threads)
    dt = time.perf_counter() - t0
    flop = 4 * w["D"] * int(np.minimum(off + rows[:, 2].astype(np.int64) + 1, w["kv_len"]).sum())
    res["prefix_causal"] = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                            "sample": f"{len(rows)} query rows ({rows_per_head} per head, seeded) of {w['name']}, "
                                      f"each against its visible keys, FP64; {dt:.2f} s wall",
                            "seconds": dt, "extrapolated_full_problem_s": causal_flops(w) / (flop / dt)}
    del q, k, v

    w = wl.PAGED_E4M3
    _, kc, vc, table, ks, vs = wl.paged_inputs(w, unit_scales=False)
    t0 = time.perf_counter()
    for cache, sc in ((kc, ks), (vc, vs)):
        oracle.e4m3_to_f16(oracle.paged_gather(cache, table, w["kv_len"]), sc)
    dt = time.perf_counter() - t0
    nb = bridge_bytes(w)
    res["e4m3_bridge"] = {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                          "sample": f"the whole bridge of {w['name']} (K and V), {dt:.2f} s wall",
                          "seconds": dt}
    del kc, vc

    w = wl.VSA
    q, k, _ = wl.vsa_inputs(w)
    t0 = time.perf_counter()
    oracle.vsa_select(q, k, w["block"], w["topk"])
    dt = time.perf_counter() - t0
    nb = select_bytes(w)
    res["vsa_select"] = {"value": nb / dt / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "sample": f"the whole block selection (pool, FP64 scores, top-k) of {w['name']}, "
                                   f"{dt:.2f} s wall", "seconds": dt}
    return res


def _cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unavailable)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


# --------------------------------------------------------------------------------- main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--iters", type=int, default=20, help="timed launches of each extra workload")
    ap.add_argument("--only", choices=["dense", "causal", "ragged", "paged", "prefix", "fp8", "vsa", "copy", "ceiling"],
                    default=None,
                    help="run one workload only (for profiling); 'copy' runs the plain 1 GiB "
                         "device copy that calibrates the HBM byte counters")
    ap.add_argument("--no-extra", action="store_true", help="skip the non-headline workloads")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-rows", type=int, default=512, help="oracle rows per head for cpu_baseline")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic.json"),
                    help="measured HBM bytes per launch of the dense kernel (from rocprofv3 PMC runs)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the attention path has no multi-GPU mode", file=sys.stderr)
        sys.exit(2)

    import torch

    import fp16_attention_amd as fa
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    fa.load()  # raises if the HIP library is not built
    props = torch.cuda.get_device_properties(0)
    log(f"device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")
    timer = Timer(torch)
    flush_buf = None
    flush_sink = []

    def flush():
        # evict the 256 MB last-level cache by reading 512 MiB (a write-based
        # flush would leave dirty lines whose write-back lands in the timed run)
        flush_sink.append(flush_buf.view(torch.int64).sum())
        if len(flush_sink) > 64:
            flush_sink.clear()

    extra = {}
    result = None
    if args.only == "ceiling":
        print(json.dumps({"metric": "fp16 mfma ceiling", "partial": True, "only": "ceiling",
                          **bench_mfma_ceiling(fa, torch, timer)}), flush=True)
        return
    if args.only == "copy":
        # A plain copy of a known size: the kernel whose FETCH_SIZE / WRITE_SIZE
        # readings scale the attention kernel's counters to bytes.
        rec = bench_copy(torch, timer, args.iters)
        print(json.dumps({"metric": "device copy", "partial": True, "only": "copy", **rec}), flush=True)
        return
    if args.only in (None, "dense"):
        w, qkv, out, ms, wall = bench_dense(fa, torch, None, args.steps, args.warmup, timer)
        flop = dense_flops(w)
        avg_ms = float(ms.mean())
        value = flop * args.steps / wall / 1e12
        achieved = flop / (avg_ms * 1e-3) / 1e12
        log(f"dense: {avg_ms:.3f} ms/launch (events), {wall / args.steps * 1e3:.3f} ms/step (wall), "
            f"{achieved:.1f} TFLOP/s = {100 * achieved / MFMA_F16_PEAK_TFLOPS:.1f}% of peak")
        traffic = dense_traffic(args.traffic)
        result = {
            "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "f16", "data": "synthetic",
            "config": {"workload": w["name"], "B": w["B"], "H": w["H"], "D": w["D"], "Lq": w["Lq"],
                       "Lkv": w["Lkv"], "causal": False, "scale": "1/sqrt(128) in FP32",
                       "inputs": "N(0,1) FP16, counter-based generator seed 2"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": MFMA_F16_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": achieved / MFMA_F16_PEAK_TFLOPS, "traffic": traffic,
                         "traffic_unit": "HBM bytes per call, both kernels (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                         "kernel": "attn_fwd_kernel (dense, D128): the whole rounds, then the last half round "
                                   "with each item's keys split between the halves of 8-wave workgroups",
                         "launch_ms_mean": avg_ms,
                         "algorithmic_flop_per_launch": flop},
        }
        result["headline_stats"] = stats(ms)
        ceiling = bench_mfma_ceiling(fa, torch, timer)
        result["roofline"]["measured_ceiling"] = ceiling["value"]
        result["roofline"]["frac_of_measured_ceiling"] = achieved / ceiling["value"]
        result["mfma_ceiling"] = ceiling
        if not args.no_cpu:
            out_np = out.cpu().numpy()
            cpu, parity = cpu_baseline(w, qkv, out_np, args.cpu_rows)
            result["cpu_baseline"] = cpu
            result["parity_sample"] = parity
            log(f"cpu oracle {cpu['value'] * 1e3:.3f} GFLOP/s; GPU vs oracle on the sample: {parity}")
        del qkv, out
        torch.cuda.empty_cache()

    if not args.no_extra or args.only not in (None, "dense"):
        flush_buf = torch.ones(512 << 20, dtype=torch.uint8, device="cuda")
        if args.only in (None, "causal"):
            extra["prefix_causal"] = bench_causal(fa, torch, args.iters, timer)
            torch.cuda.empty_cache()
        if args.only in (None, "ragged"):
            extra["ragged_dense"], extra["ragged_dense_bf16"] = bench_ragged(fa, torch, args.iters, timer)
            torch.cuda.empty_cache()
        if args.only in (None, "paged"):
            extra["paged_e4m3"], extra["e4m3_bridge"], extra["paged_e4m3_decode"] = bench_paged(
                fa, torch, args.iters, timer, flush)
            torch.cuda.empty_cache()
        if args.only in (None, "fp8"):
            extra["prefix_fp8_attention"] = bench_prefix_fp8_attn(fa, torch, args.iters, timer)
            torch.cuda.empty_cache()
        if args.only in (None, "prefix"):
            extra["prefix_fp8_gather"] = bench_prefix_fp8(fa, torch, args.iters, timer, flush)
            torch.cuda.empty_cache()
        if args.only in (None, "vsa"):
            extra["vsa_select"], extra["vsa_sparse_attn"] = bench_vsa(fa, torch, args.iters, timer, flush)
            torch.cuda.empty_cache()
        if args.only is None:
            extra["hbm_copy"] = copy = bench_copy(torch, timer, args.iters, flush)
            for rec in extra.values():
                if "gbs" in rec and rec is not copy:
                    rec["frac_of_measured_copy"] = rec["gbs"] / copy["gbs"]

    if result is None:
        print(json.dumps({"metric": METRIC, "partial": True, "only": args.only, "extra": extra}), flush=True)
        return
    if not args.no_cpu and not args.no_extra and args.only is None:
        log("cpu oracle: causal prefill sample, bridge, VSA selection")
        result["cpu_baseline_extra"] = cpu_extra_baselines()
    # FP16 MFMA-bound workloads against the same measured (FP16) ceiling as the headline
    for rec in extra.values():
        if "tflops" in rec and "BF16" not in rec["workload"] and "peak_tflops" not in rec:
            rec["frac_of_measured_ceiling"] = rec["tflops"] / result["mfma_ceiling"]["value"]
    result["extra"] = extra
    result["device"] = {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                        "compute_units": props.multi_processor_count}
    result["context"] = PAGES_CONTEXT
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
