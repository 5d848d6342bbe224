#!/usr/bin/env python3
"""Benchmark of the fused GEMM-epilogue hot path on one MI355X.

A step is one forward GEMM-RMSNorm-GEMM (GEMM1 with the residual / gamma / row-partial
epilogue, the auxiliary row reduction, GEMM2 with the deferred row scale) on the
Llama-3-8B-shaped workload: M = 8192 tokens, x[8192, 14336] W0[14336, 4096] (FFN
down-projection), residual z[8192, 4096], W1[4096, 6144] (GQA QKV), eps = 1e-5, bf16
inputs with fp32 accumulation, synthetic seeded data already resident in HBM.

Prints ONE JSON line. `value` is the algorithmic TFLOP/s of the step (2MKD + 2MDN1 per
step) over the synchronize-bracketed wall time of `--steps` steps. Per-kernel durations
come from HIP events recorded on the stream the kernels run on: GEMM1's (the roofline
kernel's) in every timed step, the other two kernels' in as many steps after the timed
ones, so the timed steps carry no events between the row reduction and GEMM2. The other fused paths
(GEMM+RoPE at 4096 and 8192 under both schedules, GEMM+SwiGLU, the backward statistic,
the rest of the RMSNorm backward, the SwiGLU and RoPE backward maps, GEMM+cross-entropy)
and the unfused baselines are timed after the headline and reported under "paths"
(context, not the headline); so is the register-only MFMA rate the chip sustains on
Gaussian operands under its power limit ("mfma_power_ceiling").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused GEMM-epilogue TFLOP/s (% bf16 MFMA peak), 8192-class GEMM-RMSNorm-GEMM"
PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm1_residual_rmsnorm_llama8k.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


# The sources that define GEMM1's kernel (main loop, residual epilogue) and its launch.
GEMM1_SOURCES = ("coda_common.hpp", "coda_abi.hpp", "coda_gemm.hpp", "coda_gemm.hip")


def source_hash() -> str:
    """Hash of GEMM1's HIP sources; stored HBM-traffic counters are used only while it matches."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_gemm_epilogue_amd", "csrc")
    for name in GEMM1_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def event_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def time_reps(fn, reps, warmup=3):
    """Median / mean / min milliseconds of fn() over reps, from HIP events on the current stream."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = np.array(event_ms(evs))
    return dict(median_ms=float(np.median(t)), mean_ms=float(t.mean()), min_ms=float(t.min()))


def time_interleaved(fns, reps, rounds=4, warmup=2):
    """Median milliseconds per callable, all timed in alternating rounds (forward order on
    even rounds, reverse on odd) so that every variant sees the same clock and thermal
    state; back-to-back blocks of one variant would compare different clocks."""
    import torch
    names = list(fns)
    for n in names:
        for _ in range(warmup):
            fns[n]()
    torch.cuda.synchronize()
    times = {n: [] for n in names}
    per = max(1, reps // rounds)
    for k in range(rounds):
        for n in (names if k % 2 == 0 else names[::-1]):
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(per)]
            for a, b in evs:
                a.record()
                fns[n]()
                b.record()
            torch.cuda.synchronize()
            times[n] += event_ms(evs)
    return {n: float(np.median(t)) for n, t in times.items()}


# --------------------------------------------------------------------------- headline
def headline(args, coda, torch):
    import workloads as W
    wl = W.llama_fwd()
    M, K, D, N1, eps = wl["M"], wl["K"], wl["D"], wl["N1"], wl["eps"]
    x, w0, z, g, w1 = (to_dev(wl[k]) for k in ("x", "w0", "z", "gamma", "w1"))
    h1 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    h2 = torch.empty_like(h1)
    part = torch.empty((M, coda.num_partials(D)), dtype=torch.float32, device="cuda")
    r = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N1), dtype=torch.bfloat16, device="cuda")

    def step(ev=None, each=False):
        # ev[0], ev[1] bracket GEMM1 (the roofline kernel); with `each`, ev[2] and ev[3]
        # also close the row reduction and GEMM2
        if ev is not None:
            ev[0].record()
        coda.coda_gemm_residual_rmsnorm_partials(x, w0, z, g, h1=h1, h2=h2, partials=part)
        if ev is not None:
            ev[1].record()
        coda.coda_rowstat_reduce(part, D, eps, coda.ROWSTAT_RSQRT_MEAN_EPS, out=r)
        if each:
            ev[2].record()
        coda.coda_gemm_rowscale(h2, w1, r, y=y)
        if each:
            ev[3].record()

    # Clock settle: the MI355X ramps its clocks over the first tens of milliseconds of
    # MFMA load, so untimed steps run for `--settle-s` seconds before the warm-up steps.
    t_end = time.perf_counter() + args.settle_s
    while time.perf_counter() < t_end:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps carry only GEMM1's two events (the roofline's launch duration)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    g1 = np.array([e[0].elapsed_time(e[1]) for e in evs])
    # the row reduction and GEMM2, timed in as many further steps with events between
    # all three kernels
    evs_each = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for e in evs_each:
        step(e, each=True)
    torch.cuda.synchronize()
    rs = np.array([e[1].elapsed_time(e[2]) for e in evs_each])
    g2 = np.array([e[2].elapsed_time(e[3]) for e in evs_each])

    # the single fused entry point (same three launches), for cross-checking
    fused = time_reps(lambda: coda.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, eps, h1=h1, h2=h2, partials=part,
                                                         r=r, y=y), reps=max(5, args.steps // 2))

    flop1 = 2.0 * M * K * D
    flop2 = 2.0 * M * D * N1
    flops = flop1 + flop2
    ms_step = wall * 1e3 / args.steps
    value = flops / (ms_step * 1e-3) / 1e12
    g1_us = float(g1.mean() * 1e3)
    achieved = flop1 / (g1.mean() * 1e-3) / 1e12

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        rec = json.load(open(TRAFFIC_FILE))
        if rec.get("source_hash") == source_hash():
            traffic = rec.get("hbm_bytes_per_launch")
    nb = coda.num_partials(D)
    aux_bytes = M * nb * 4 + M * 4
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama3_8b_gemm_rmsnorm_gemm_fwd", "M": M, "K": K, "D": D, "N1": N1, "eps": eps,
                   "seed": 3, "tokens_per_step": M, "inputs": "bf16, N(0,1) activations, N(0,1/fan_in) weights",
                   "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": "gemm_epilogue_kernel<KN, EpiResidualRmsPartials> (GEMM1)",
                     "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "algorithmic_flop_per_launch": flop1, "avg_launch_us": round(g1_us, 2)},
        "kernels_us": {"gemm1_residual_rmsnorm_partials": round(g1_us, 2),
                       "rowstat_reduce": round(float(rs.mean() * 1e3), 2),
                       "gemm2_rowscale": round(float(g2.mean() * 1e3), 2),
                       "fused_entry_point_median": round(fused["median_ms"] * 1e3, 2)},
        "gemm1_us_median_min": [round(float(np.median(g1)) * 1e3, 2), round(float(g1.min()) * 1e3, 2)],
        "kernels_tflops": {"gemm1": round(flop1 / (g1.mean() * 1e-3) / 1e12, 1),
                           "gemm2": round(flop2 / (g2.mean() * 1e-3) / 1e12, 1)},
        "rowstat_reduce_gbps_at_config": round(aux_bytes / (rs.mean() * 1e-3) / 1e9, 1),
    }
    bufs = dict(x=x, w0=w0, z=z, g=g, w1=w1, h1=h1, h2=h2, part=part, r=r, y=y, eps=eps)
    return res, bufs


def mall_flushed(coda, torch, b, reps):
    """The forward step with the caches cold: before each timed step a 512 MiB buffer is
    written (twice the 256 MiB Infinity Cache), so the step's inputs come from HBM. HIP
    events bracket the step alone (GEMM1's start to GEMM2's end); median and min."""
    x, w0, z, g, w1, eps = b["x"], b["w0"], b["z"], b["g"], b["w1"], b["eps"]
    M, D = b["h1"].shape
    K, N1 = x.shape[1], w1.shape[1]
    flush = torch.empty((512 << 20,), dtype=torch.uint8, device="cuda")
    ms = []
    for i in range(reps + 2):
        flush.fill_(i & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        coda.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, eps, h1=b["h1"], h2=b["h2"], partials=b["part"], r=b["r"],
                                   y=b["y"])
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            ms.append(e0.elapsed_time(e1))
    del flush
    fl = 2.0 * M * K * D + 2.0 * M * D * N1
    med, mn = float(np.median(ms)), float(np.min(ms))
    return dict(flush_bytes=512 << 20, steps=reps, ms_median=round(med, 4), ms_min=round(mn, 4),
                tflops_median=round(fl / (med * 1e-3) / 1e12, 1))


# ------------------------------------------------------------------- unfused baseline
def unfused_fwd(coda, torch, b, reps):
    """The fused forward entry point against (a) the same MFMA main loop with a plain
    store, then a separate residual+RMSNorm kernel, then the plain GEMM again (bf16
    intermediates), and (b) torch (hipBLASLt) + eager ops; the three are timed
    interleaved."""
    x, w0, z, g, w1, eps = b["x"], b["w0"], b["z"], b["g"], b["w1"], b["eps"]
    M, D = b["h1"].shape
    h0 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    h1 = torch.empty_like(h0)
    o = torch.empty_like(h0)
    r = torch.empty((M,), dtype=torch.float32, device="cuda")
    y = torch.empty_like(b["y"])

    def ours():
        coda.coda_baseline_gemm(x, w0, c=h0)
        coda.coda_baseline_residual_rmsnorm(h0, z, g, eps, h1=h1, r=r, o=o)
        coda.coda_baseline_gemm(o, w1, c=y)

    def torch_path():
        hh = torch.matmul(x, w0) + z
        oo = torch.nn.functional.rms_norm(hh, (D,), weight=g, eps=eps)
        return torch.matmul(oo, w1)

    def fused():
        coda.coda_gemm_rmsnorm_fwd(x, w0, z, g, w1, eps, h1=b["h1"], h2=b["h2"], partials=b["part"], r=b["r"],
                                   y=b["y"])

    t = time_interleaved({"fused": fused, "ours": ours, "torch": torch_path}, 2 * reps)
    t_norm = time_reps(lambda: coda.coda_baseline_residual_rmsnorm(h0, z, g, eps, h1=h1, r=r, o=o), reps)
    t_mm1 = time_reps(lambda: torch.matmul(x, w0), reps)
    t_mm2 = time_reps(lambda: torch.matmul(o, w1), reps)
    # GEMM1 alone, three ways in one interleaved run: the fused kernel (residual, gamma, row
    # partials), the same main loop with a plain store, and hipBLASLt's plain GEMM
    g1 = time_interleaved({
        "fused": lambda: coda.coda_gemm_residual_rmsnorm_partials(x, w0, z, g, h1=b["h1"], h2=b["h2"],
                                                                  partials=b["part"]),
        "plain": lambda: coda.coda_baseline_gemm(x, w0, c=h0),
        "hipblaslt": lambda: torch.matmul(x, w0, out=h0)}, 2 * reps)
    fl1 = 2.0 * M * x.shape[1] * D
    return dict(gemm1_interleaved={k: dict(us=round(v * 1e3, 1), tflops=round(fl1 / (v * 1e-3) / 1e12, 1))
                                   for k, v in g1.items()},
                gemm1_fused_vs_hipblaslt_plain=round(g1["hipblaslt"] / g1["fused"], 3),
                fused_entry_point_ms=t["fused"],
                same_mainloop_plus_separate_kernels_ms=t["ours"],
                torch_hipblaslt_eager_ms=t["torch"],
                separate_residual_rmsnorm_kernel_us=round(t_norm["median_ms"] * 1e3, 2),
                separate_residual_rmsnorm_gbps=round(4 * M * D * 2 / (t_norm["median_ms"] * 1e-3) / 1e9, 1),
                hipblaslt_gemm1_tflops=round(2 * M * x.shape[1] * D / (t_mm1["median_ms"] * 1e-3) / 1e12, 1),
                hipblaslt_gemm2_tflops=round(2 * M * D * w1.shape[1] / (t_mm2["median_ms"] * 1e-3) / 1e12, 1))


def shard_share(coda, torch, b, reps):
    """The forward on one GPU's share of the headline workload under token sharding over
    G GPUs (M/G rows; every step is row-independent, so a shard runs the same kernels with
    no exchange), through coda_gemm_rmsnorm_fwd (one kernel per GEMM) and through
    coda_gemm_rmsnorm_fwd_ws (split depth for GEMMs with fewer tiles than CUs), timed
    interleaved. One GPU only: no multi-GPU figure is implied."""
    x, w0, z, g, w1, eps = b["x"], b["w0"], b["z"], b["g"], b["w1"], b["eps"]
    M, D = b["h1"].shape
    K, N1 = x.shape[1], w1.shape[1]
    fns, ws = {}, {}
    for G in (1, 2, 4, 8):
        m = M // G
        outs = dict(h1=b["h1"][:m], h2=b["h2"][:m], partials=b["part"][:m], r=b["r"][:m], y=b["y"][:m])
        fns[(G, "one_kernel")] = (lambda m=m, outs=outs: coda.coda_gemm_rmsnorm_fwd(x[:m], w0, z[:m], g, w1, eps,
                                                                                 **outs))
        need = coda.coda_gemm_rmsnorm_fwd_workspace_bytes(m, K, D, N1)
        ws[G] = torch.empty((max(need, 16),), dtype=torch.uint8, device="cuda")
        fns[(G, "split_depth")] = (lambda m=m, outs=outs, G=G: coda.coda_gemm_rmsnorm_fwd_ws(
            x[:m], w0, z[:m], g, w1, eps, workspace=ws[G], **outs))
    t = time_interleaved(fns, reps)
    out = {}
    for (G, how), ms in t.items():
        m = M // G
        fl = 2.0 * m * K * D + 2.0 * m * D * N1
        out.setdefault(f"G{G}", dict(rows=m, workspace_bytes=coda.coda_gemm_rmsnorm_fwd_workspace_bytes(m, K, D, N1)))
        out[f"G{G}"][how] = dict(ms=round(ms, 4), tflops=round(fl / (ms * 1e-3) / 1e12, 1))
    del ws
    return out


def token_shares(torch, reps, M, flops_per_row, one, split, need, G_list=(4, 8)):
    """One GPU's share (M/G rows) of a row-independent GEMM under token sharding, through
    the one-kernel entry point `one(m, ws)` and the split-depth one `split(m, ws)`, timed
    interleaved; `need(m)` is the split workspace in bytes (allocated before timing)."""
    ws = torch.empty((max([need(M // G) for G in G_list] + [16]),), dtype=torch.uint8, device="cuda")
    fns = {}
    for G in G_list:
        m = M // G
        fns[(G, "one_kernel")] = lambda m=m: one(m, ws)
        fns[(G, "split_depth")] = lambda m=m: split(m, ws)
    res = {}
    for (G, how), ms in time_interleaved(fns, reps).items():
        m = M // G
        rec = res.setdefault(f"G{G}", dict(rows=m, workspace_bytes=need(m)))
        rec[how] = dict(ms=round(ms, 4), tflops=round(flops_per_row * m / (ms * 1e-3) / 1e12, 1))
    del ws
    return res


# ------------------------------------------------------------------ other fused paths
def path_record(t, fl):
    rec = dict(fused_us=round(t["fused"] * 1e3, 1), tflops=round(fl / (t["fused"] * 1e-3) / 1e12, 1),
               unfused_us=round(t["unfused"] * 1e3, 1), speedup_vs_unfused=round(t["unfused"] / t["fused"], 3),
               hipblaslt_gemm_only_us=round(t["hipblaslt"] * 1e3, 1),
               hipblaslt_gemm_only_tflops=round(fl / (t["hipblaslt"] * 1e-3) / 1e12, 1))
    if "persistent" in t:  # the same fused computation under the persistent schedule
        rec.update(persistent_us=round(t["persistent"] * 1e3, 1),
                   persistent_tflops=round(fl / (t["persistent"] * 1e-3) / 1e12, 1),
                   persistent_vs_per_tile=round(t["fused"] / t["persistent"], 3))
    return rec


def other_paths(coda, torch, reps):
    import workloads as W
    out = {}
    # GEMM + RoPE (QKV projection)
    wl = W.rope_qkv()
    x, w = to_dev(wl["x"]), to_dev(wl["w"])
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    M, K, N = wl["M"], wl["K"], wl["n_q"] + wl["n_k"] + wl["n_v"]
    qkv = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    h = torch.empty_like(qkv)
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], 0)
    t = time_interleaved({
        "fused": lambda: coda.coda_gemm_rope(x, w, c, s, *args, out=qkv),
        "persistent": lambda: coda.coda_gemm_rope_persistent(x, w, c, s, *args, out=qkv),
        "unfused": lambda: (coda.coda_baseline_gemm(x, w, c=h), coda.coda_baseline_rope(h, c, s, *args, out=qkv)),
        "hipblaslt": lambda: torch.matmul(x, w)}, reps)
    fl = 2.0 * M * K * N
    out["gemm_rope_qkv_4096x12288x4096"] = path_record(t, fl)
    # one GPU's share of it under token sharding (M/G rows, pos_offset = the share's first
    # row), one kernel against the split-depth schedule
    fns, wss, shares = {}, {}, {}
    for G in (4, 8):
        m = M // G
        wss[G] = torch.empty((max(coda.coda_split_workspace_bytes(m, N, K), 16),), dtype=torch.uint8, device="cuda")
        sargs = args[:-1] + (M - m,)
        fns[(G, "one_kernel")] = (lambda m=m, sargs=sargs: coda.coda_gemm_rope(x[M - m:], w, c, s, *sargs,
                                                                               out=qkv[:m]))
        fns[(G, "split_depth")] = (lambda m=m, sargs=sargs, G=G: coda.coda_gemm_rope_ws(
            x[M - m:], w, c, s, *sargs, out=qkv[:m], workspace=wss[G]))
    for (G, how), ms in time_interleaved(fns, reps).items():
        m = M // G
        shares.setdefault(f"G{G}", dict(rows=m))[how] = dict(ms=round(ms, 4),
                                                             tflops=round(2.0 * m * K * N / (ms * 1e-3) / 1e12, 1))
    out["gemm_rope_qkv_4096x12288x4096"]["one_gpu_share_of_token_shards"] = shares
    del x, w, qkv, h, wss
    torch.cuda.empty_cache()
    # GEMM + RoPE at the 8192 class (M = K = 8192, QKV width 3 x 8192), both schedules
    log("paths: rope 8192 (generating inputs) ...")
    wl = W.rope_qkv_8k()
    x, w = to_dev(wl["x"]), to_dev(wl["w"])
    c, s = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    M, K, N = wl["M"], wl["K"], wl["n_q"] + wl["n_k"] + wl["n_v"]
    qkv = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    h = torch.empty_like(qkv)
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], 0)
    t = time_interleaved({
        "fused": lambda: coda.coda_gemm_rope(x, w, c, s, *args, out=qkv),
        "persistent": lambda: coda.coda_gemm_rope_persistent(x, w, c, s, *args, out=qkv),
        "unfused": lambda: (coda.coda_baseline_gemm(x, w, c=h), coda.coda_baseline_rope(h, c, s, *args, out=qkv)),
        "hipblaslt": lambda: torch.matmul(x, w)}, reps)
    out["gemm_rope_qkv_8192x24576x8192"] = path_record(t, 2.0 * M * K * N)
    del x, w, qkv, h, wl
    torch.cuda.empty_cache()
    # GEMM + SwiGLU at the pages' two shapes
    for wl in (W.swiglu_4k(), W.swiglu()):
        x, w = to_dev(wl["x"]), to_dev(wl["w"])
        M, K, F = wl["M"], wl["K"], wl["F"]
        o = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
        h = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
        t = time_interleaved({
            "fused": lambda: coda.coda_gemm_swiglu(x, w, out=o),
            "unfused": lambda: (coda.coda_baseline_gemm(x, w, c=h), coda.coda_baseline_swiglu(h, out=o)),
            "hipblaslt": lambda: torch.matmul(x, w)}, reps)
        fl = 2.0 * M * K * 2 * F
        out[f"gemm_swiglu_{M}x{2 * F}x{K}"] = path_record(t, fl)
        del x, w, o, h
    # backward statistic
    wl = W.bwd_stats()
    dy, w1, h2 = to_dev(wl["dy"]), to_dev(wl["w1"]), to_dev(wl["h2"])
    M, D, N = wl["M"], wl["D"], wl["N"]
    dh2 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    part = torch.empty((M, coda.num_partials(D)), dtype=torch.float32, device="cuda")
    sv = torch.empty((M,), dtype=torch.float32, device="cuda")
    w1t = w1.t().contiguous()
    t = time_interleaved({
        "fused": lambda: coda.coda_gemm_rmsnorm_bwd_stats(dy, w1, h2, dh2=dh2, partials=part, s=sv),
        "unfused": lambda: (coda.coda_baseline_gemm(dy, w1, b_kn=False, c=dh2),
                            coda.coda_baseline_rowdot(dh2, h2, s=sv)),
        "hipblaslt": lambda: torch.matmul(dy, w1t)}, reps)
    fl = 2.0 * M * N * D
    out["gemm_rmsnorm_bwd_stats_8192x4096x6144"] = path_record(t, fl)
    out["gemm_rmsnorm_bwd_stats_8192x4096x6144"]["one_gpu_share_of_token_shards"] = token_shares(
        torch, reps, M, 2.0 * N * D,
        lambda m, ws: coda.coda_gemm_rmsnorm_bwd_stats(dy[:m], w1, h2[:m], dh2=dh2[:m], partials=part[:m], s=sv[:m]),
        lambda m, ws: coda.coda_gemm_rmsnorm_bwd_stats_ws(dy[:m], w1, h2[:m], dh2=dh2[:m], partials=part[:m],
                                                          s=sv[:m], workspace=ws),
        lambda m: coda.coda_split_workspace_bytes(m, D, N))
    del dy, w1, h2, dh2, part, sv, w1t
    torch.cuda.empty_cache()
    # rest of the RMSNorm backward (dh1 with the residual-stream gradient, dgamma)
    wl = W.rmsnorm_bwd_full()
    dy, w1, h1, g, gres = (to_dev(wl[k]) for k in ("dy", "w1", "h1", "gamma", "g_res"))
    M, D, N, eps = wl["M"], wl["D"], wl["N"], wl["eps"]
    hf = h1.float()
    r = torch.rsqrt((hf * hf).mean(dim=1) + eps).contiguous()
    y = coda.coda_gemm_rowscale((hf * g.float()).to(torch.bfloat16).contiguous(), w1, r)
    sv = torch.empty((M,), dtype=torch.float32, device="cuda")
    dh1 = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    pg = torch.empty((coda.num_row_tiles(M), D), dtype=torch.float32, device="cuda")
    dg = torch.empty((D,), dtype=torch.float32, device="cuda")
    dO = torch.empty((M, D), dtype=torch.bfloat16, device="cuda")
    w1t = w1.t().contiguous()

    def unfused():
        # grad GEMM storing dO, then the RMSNorm backward as separate (torch eager) operators
        coda.coda_baseline_gemm(dy, w1, b_kn=False, c=dO)
        d = dO.float()
        rr = r[:, None]
        o = hf * rr * g.float()
        ss = (d * o).mean(dim=1, keepdim=True)
        out_dh1 = (rr * g.float() * d - rr * rr * ss * hf + gres.float()).to(torch.bfloat16)
        out_dg = (d * rr * hf).sum(dim=0)
        return out_dh1, out_dg

    t = time_interleaved({
        "fused": lambda: coda.coda_rmsnorm_bwd(dy, w1, h1, g, r, y, g_res=gres, s=sv, dh1=dh1, dgamma_partials=pg,
                                               dgamma=dg),
        "unfused": unfused,
        "hipblaslt": lambda: torch.matmul(dy, w1t)}, reps)
    out["rmsnorm_bwd_dx_dgamma_8192x4096x6144"] = path_record(t, fl)
    # the grad GEMM with the dh1 / dgamma-partial epilogue alone, on one GPU's share
    out["rmsnorm_bwd_dx_dgamma_8192x4096x6144"]["one_gpu_share_of_token_shards"] = token_shares(
        torch, reps, M, 2.0 * N * D,
        lambda m, ws: coda.coda_gemm_rmsnorm_bwd_dx(dy[:m], w1, h1[:m], g, r[:m], sv[:m], g_res=gres[:m],
                                                    dh1=dh1[:m], dgamma_partials=pg[:(m + 255) // 256]),
        lambda m, ws: coda.coda_gemm_rmsnorm_bwd_dx_ws(dy[:m], w1, h1[:m], g, r[:m], sv[:m], g_res=gres[:m],
                                                       dh1=dh1[:m], dgamma_partials=pg[:(m + 255) // 256],
                                                       workspace=ws),
        lambda m: coda.coda_split_workspace_bytes(m, D, N))
    del dy, w1, h1, g, gres, hf, r, y, sv, dh1, pg, dg, dO, w1t
    torch.cuda.empty_cache()
    # SwiGLU backward on the down projection's grad GEMM
    wl = W.swiglu_bwd()
    dy, wd, h = (to_dev(wl[k]) for k in ("dy", "w_down", "h"))
    M, Dm, F = wl["M"], wl["Dm"], wl["F"]
    dh = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
    dout = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
    wdt = wd.t().contiguous()

    def swiglu_bwd_unfused():
        coda.coda_baseline_gemm(dy, wd, b_kn=False, c=dout)
        d = dout.float()
        gg, uu = h[:, 0::2].float(), h[:, 1::2].float()
        sg = torch.sigmoid(gg)
        return torch.stack((d * uu * sg * (1 + gg * (1 - sg)), d * gg * sg), dim=2).reshape(M, 2 * F).to(torch.bfloat16)

    t = time_interleaved({
        "fused": lambda: coda.coda_gemm_swiglu_bwd(dy, wd, h, dh=dh),
        "unfused": swiglu_bwd_unfused,
        "hipblaslt": lambda: torch.matmul(dy, wdt)}, reps)
    out["gemm_swiglu_bwd_8192x8192x4096"] = path_record(t, 2.0 * M * Dm * F)
    out["gemm_swiglu_bwd_8192x8192x4096"]["one_gpu_share_of_token_shards"] = token_shares(
        torch, reps, M, 2.0 * Dm * F,
        lambda m, ws: coda.coda_gemm_swiglu_bwd(dy[:m], wd, h[:m], dh=dh[:m]),
        lambda m, ws: coda.coda_gemm_swiglu_bwd_ws(dy[:m], wd, h[:m], dh=dh[:m], workspace=ws),
        lambda m: coda.coda_split_workspace_bytes(m, F, Dm))
    del dy, wd, h, dh, dout, wdt
    torch.cuda.empty_cache()
    # RoPE backward (inverse rotation) in the epilogue of the GEMM producing dQKV
    wl = W.rope_bwd()
    x, w = to_dev(wl["x"]), to_dev(wl["w"])
    c, sn = coda.coda_rope_tables(wl["seq_len"], wl["head_dim"], wl["theta"])
    sneg = (-sn).contiguous()
    M, K, N = wl["M"], wl["K"], wl["n_q"] + wl["n_k"] + wl["n_v"]
    q = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    hh = torch.empty_like(q)
    args = (wl["n_q"], wl["n_k"], wl["n_v"], wl["head_dim"], wl["seq_len"], 0)
    t = time_interleaved({
        "fused": lambda: coda.coda_gemm_rope_bwd(x, w, c, sn, *args, out=q),
        # the separate rotation kernel with a negated sine table is the same inverse rotation
        "unfused": lambda: (coda.coda_baseline_gemm(x, w, c=hh), coda.coda_baseline_rope(hh, c, sneg, *args, out=q)),
        "hipblaslt": lambda: torch.matmul(x, w)}, reps)
    out["gemm_rope_bwd_4096x12288x4096"] = path_record(t, 2.0 * M * K * N)
    out["gemm_rope_bwd_4096x12288x4096"]["one_gpu_share_of_token_shards"] = token_shares(
        torch, reps, M, 2.0 * K * N,
        lambda m, ws: coda.coda_gemm_rope_bwd(x[M - m:], w, c, sn, *args[:-1], M - m, out=q[:m]),
        lambda m, ws: coda.coda_gemm_rope_bwd_ws(x[M - m:], w, c, sn, *args[:-1], M - m, out=q[:m], workspace=ws),
        lambda m: coda.coda_split_workspace_bytes(m, N, K))
    del x, w, c, sn, sneg, q, hh
    torch.cuda.empty_cache()
    # GEMM + cross-entropy at the pages' two shapes (M x vocab x K); logits never stored
    for M_, K_ in ((4096, 4096), (8192, 8192)):
        wl = W.cross_entropy(M=M_, K=K_, ignore_every=97)
        x, w = to_dev(wl["x"]), to_dev(wl["w"])
        lab = torch.from_numpy(wl["labels"]).cuda()
        lab64 = lab.long()
        M, K, V = wl["M"], wl["K"], wl["V"]
        tl = torch.empty((M, coda.num_partials(V)), dtype=torch.float32, device="cuda")
        tg, ls, lo = (torch.empty((M,), dtype=torch.float32, device="cuda") for _ in range(3))
        logits = torch.empty((M, V), dtype=torch.bfloat16, device="cuda")

        def ce_unfused():
            coda.coda_baseline_gemm(x, w, c=logits)
            return torch.nn.functional.cross_entropy(logits.float(), lab64, reduction="none", ignore_index=-1)

        t = time_interleaved({
            "fused": lambda: coda.coda_gemm_cross_entropy(x, w, lab, tile_lse=tl, target=tg, lse=ls, loss=lo),
            "unfused": ce_unfused,
            "hipblaslt": lambda: torch.matmul(x, w)}, reps)
        out[f"gemm_cross_entropy_{M}x{V}x{K}"] = path_record(t, 2.0 * M * K * V)
        del x, w, lab, lab64, tl, tg, ls, lo, logits
        torch.cuda.empty_cache()
    return out


def mfma_ceiling(coda, torch):
    """Register-only MFMA rate (no memory traffic; the GEMM's per-wave shape and
    occupancy) with operands drawn like the workloads' data (bf16 N(0,1)) and with
    constant operands: under its power limit the chip's clock, and so the MFMA rate,
    depends on how much the operands toggle. The Gaussian figure is the practical
    ceiling for the headline workload beside the nominal peak."""
    import workloads as W
    rng = np.random.default_rng(17)
    ops = {"gaussian": to_dev(W.normal_bf16(rng, (1 << 20, 8), 1.0)),
           "constant_1.0": torch.ones((1 << 20) * 8, dtype=torch.bfloat16, device="cuda")}
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    grid, iters = 4 * cus, 5000
    out = torch.empty((grid * 512,), dtype=torch.float32, device="cuda")
    fl = grid * 8.0 * iters * 32 * 16384
    res = {}
    for name, o in ops.items():
        t_end = time.perf_counter() + 0.5  # clock settle under this load
        while time.perf_counter() < t_end:
            coda.coda_baseline_mfma_loop(o, iters, grid, out=out)
            torch.cuda.synchronize()
        t = time_reps(lambda: coda.coda_baseline_mfma_loop(o, iters, grid, out=out), reps=5, warmup=1)
        res[f"{name}_tflops"] = round(fl / (t["median_ms"] * 1e-3) / 1e12, 1)
    return res


def aux_reduce_sweep(coda, torch, reps):
    """Bandwidth of the auxiliary row reduction on partial buffers far above the 256 MiB
    Infinity Cache (at the forward workload the buffer is 0.5 MiB and latency-bound)."""
    res = {}
    for mib in (256, 1024):
        nb = 16
        M = mib * 1024 * 1024 // (nb * 4)
        P = torch.rand((M, nb), dtype=torch.float32, device="cuda")
        o = torch.empty((M,), dtype=torch.float32, device="cuda")
        t = time_reps(lambda: coda.coda_rowstat_reduce(P, 4096, 1e-5, coda.ROWSTAT_RSQRT_MEAN_EPS, out=o), reps)
        byts = M * nb * 4 + M * 4
        res[f"{mib}MiB"] = dict(us=round(t["median_ms"] * 1e3, 1),
                                gbps=round(byts / (t["median_ms"] * 1e-3) / 1e9, 1),
                                frac_of_hbm_peak=round(byts / (t["median_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBPS, 3))
        del P, o
    return res


# ------------------------------------------------------- GEMM1 against hipBLASLt (counters)
def gemm1_compare(coda, torch, reps):
    """GEMM1 of the Llama-shaped forward three ways, for counter runs: the fused kernel
    (residual, gamma, row partials), the same main loop with a plain store, and
    hipBLASLt's plain GEMM (torch.matmul); then the plain kernel on 1/32 .. all of the
    token rows, i.e. 16 .. 512 concurrent tiles, to see how one tile's time depends on
    how many CUs run at once (at most one tile per CU up to 256 tiles)."""
    wl_shape = dict(M=8192, K=14336, D=4096)
    M, K, D = wl_shape["M"], wl_shape["K"], wl_shape["D"]
    g = torch.Generator(device="cuda").manual_seed(3)
    x = (torch.randn((M, K), generator=g, device="cuda")).to(torch.bfloat16)
    w0 = (torch.randn((K, D), generator=g, device="cuda") * K ** -0.5).to(torch.bfloat16)
    z = torch.randn((M, D), generator=g, device="cuda").to(torch.bfloat16)
    gam = (1 + 0.1 * torch.randn((D,), generator=g, device="cuda")).to(torch.bfloat16)
    h1, h2 = torch.empty_like(z), torch.empty_like(z)
    part = torch.empty((M, coda.num_partials(D)), dtype=torch.float32, device="cuda")
    out = torch.empty_like(z)
    fns = {"fused_gemm1": lambda: coda.coda_gemm_residual_rmsnorm_partials(x, w0, z, gam, h1=h1, h2=h2,
                                                                          partials=part),
           "plain_gemm1": lambda: coda.coda_baseline_gemm(x, w0, c=out),
           "hipblaslt_gemm1": lambda: torch.matmul(x, w0, out=out)}
    fl = 2.0 * M * K * D
    settle = time.time() + 1.0  # clock settle before any timing
    while time.time() < settle:
        fns["plain_gemm1"]()
        torch.cuda.synchronize()
    t = time_interleaved(fns, max(reps, 8))
    res = {name: dict(us=round(ms * 1e3, 1), tflops=round(fl / (ms * 1e-3) / 1e12, 1)) for name, ms in t.items()}
    sweep = {}
    for m in (256, 512, 1024, 2048, 4096, 8192):
        xs, os_ = x[:m], out[:m]
        t = time_reps(lambda: coda.coda_baseline_gemm(xs, w0, c=os_), reps)
        tiles = (m // 256) * (D // 256)
        sweep[f"{tiles}_tiles"] = dict(M=m, us=round(t["median_ms"] * 1e3, 1),
                                       tflops=round(2.0 * m * K * D / (t["median_ms"] * 1e-3) / 1e12, 1))
    res["plain_gemm1_by_concurrent_tiles"] = sweep
    return res


def schedule_probe(coda, torch, steps=20000):
    """The main loop's LDS reads and MFMAs alone (coda_baseline_schedule_probe: a fixed LDS
    image of hashed values, no DMA): cycles per 32-deep step of a workgroup (its slowest
    wave; median over workgroups), on one workgroup and on 256 (one per CU), for each
    kind; 1024 cycles per step is the nominal MFMA time (64 MFMAs of 16 cycles per SIMD
    at the published peak)."""
    kinds = {0: "reads_kn_mfma_barrier", 1: "reads_kn_mfma_no_barrier", 2: "reads_nk_mfma_barrier",
             3: "reads_kn_only", 4: "mfma_only", 5: "w_reads_only_kn_mfma_barrier", 6: "x_reads_only_mfma_barrier",
             7: "reads_kn_mfma_barrier_zero_fill_dma"}
    res = {}
    for grid in (1, 256):
        for kind, name in list(kinds.items()) + [(4, "mfma_only_constant_image"), (0, "reads_kn_mfma_barrier_constant_image")]:
            seed = 0 if name.endswith("constant_image") or kind == 7 else 11
            fill = 0.0 if kind == 7 else 0.125   # the zero-filling DMA runs on the zero image only
            out = torch.empty((grid * 512,), dtype=torch.float32, device="cuda")
            cyc = torch.empty((grid * 8,), dtype=torch.int64, device="cuda")
            coda.coda_baseline_schedule_probe(kind, 50, grid, fill=fill, seed=seed, out=out, cycles=cyc)  # warm-up
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            coda.coda_baseline_schedule_probe(kind, steps, grid, fill=fill, seed=seed, out=out, cycles=cyc)
            e1.record()
            torch.cuda.synchronize()
            # a workgroup's time is its slowest wave's (without the per-step barrier the
            # two waves of a SIMD drift apart, and one may finish long before the other)
            c = cyc.cpu().numpy().astype(np.float64).reshape(grid, 8).max(axis=1)
            per = float(np.median(c)) / steps
            res[f"{name}_grid{grid}"] = dict(cycles_per_step=round(per, 1),
                                             mfma_occupancy=round(1024.0 / per, 3) if kind != 3 else None,
                                             clock_ghz=round(float(c.max()) / (e0.elapsed_time(e1) * 1e6), 2))
    return res


# --------------------------------------------------------------------- CPU oracle leg
def cpu_baseline(target_s: float):
    """The fp64 oracle, as it stands, on a row sample of the same workload (every op is
    row-independent), timed on this host's cores; scaled to the metric's unit."""
    import oracle as O
    import workloads as W
    blas = "unknown BLAS"
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        cores = max([int(i.get("num_threads", 1)) for i in info] or [1])
        if info:
            blas = f"{info[0].get('internal_api', '?')} {info[0].get('version', '?')}"
    except Exception:
        cores = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next(ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name"))
    except Exception:
        pass
    wl = W.llama_fwd()
    M, K, D, N1 = wl["M"], wl["K"], wl["D"], wl["N1"]

    def run(n):
        rows = np.arange(n) * (M // n)
        t0 = time.perf_counter()
        O.gemm_rmsnorm_fwd(wl["x"], wl["w0"], wl["z"], wl["gamma"], wl["w1"], wl["eps"], rows=rows)
        return time.perf_counter() - t0

    t = run(512)
    n = int(min(M, max(512, 512 * target_s / max(t, 1e-3))))
    if n != 512:
        t = run(n)
    passes = 1
    if n == M and t < target_s:  # the whole workload is shorter than the target: repeat it
        passes = int(np.ceil(target_s / max(t, 1e-3)))
        t = sum(run(n) for _ in range(passes))
    flops = passes * (2.0 * n * K * D + 2.0 * n * D * N1)
    what = f"{n} of {M} rows" if n < M else f"all {M} rows, {passes} passes"
    # wall time of one oracle pass over each stated workload in full (inputs generated
    # beforehand, not timed)
    per = {}
    if n == M:
        per["llama3_8b_gemm_rmsnorm_gemm_fwd"] = round(t / passes, 3)
    else:
        per[f"llama3_8b_gemm_rmsnorm_gemm_fwd ({n} of {M} rows)"] = round(t, 3)
    del wl
    for name, make, call in (
            ("tiny_gemm_rmsnorm_gemm_256", W.tiny_fwd,
             lambda w: O.gemm_rmsnorm_fwd(w["x"], w["w0"], w["z"], w["gamma"], w["w1"], w["eps"])),
            ("gemm_rope_qkv_4096x12288x4096", W.rope_qkv,
             lambda w: O.gemm_rope(w["x"], w["w"], w["n_q"], w["n_k"], w["n_v"], w["head_dim"], w["seq_len"],
                                   w["pos_offset"], w["theta"])),
            ("gemm_swiglu_8192x8192x8192", W.swiglu, lambda w: O.gemm_swiglu(w["x"], w["w"])),
            ("gemm_rmsnorm_bwd_stats_8192x4096x6144", W.bwd_stats,
             lambda w: O.gemm_rmsnorm_bwd_stats(w["dy"], w["w1"], w["h2"]))):
        w = make()
        t0 = time.perf_counter()
        call(w)
        per[name] = round(time.perf_counter() - t0, 3)
        del w
    return {"value": round(flops / t / 1e12, 5), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "wall_s_per_workload": per,
            "sample": f"{what} of the same workload (all five fp64 outputs per row, incl. "
                      f"weight decode), {t:.1f} s wall",
            "implementation": f"numpy fp64, matrix products through {blas} with {cores} threads",
            "host": {"nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=20, help="repetitions for the context measurements")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--settle-s", type=float, default=1.0, help="untimed clock-settle time before warm-up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the plain 1 GiB copy kernel (reference for HBM traffic counters)")
    ap.add_argument("--aux-sweep-only", action="store_true",
                    help="only run the auxiliary row reduction's bandwidth sweep (for profiling it)")
    ap.add_argument("--gemm1-compare", action="store_true",
                    help="only run GEMM1 fused / plain / hipBLASLt and the concurrent-tile sweep (counter runs)")
    ap.add_argument("--schedule-probe", action="store_true",
                    help="only run the main loop's reads and MFMAs on a fixed LDS image (no DMA)")
    ap.add_argument("--shard-share", action="store_true",
                    help="only run the headline and one GPU's share of it under token sharding (M/G rows)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the fused GEMM-epilogue path is row-independent and "
              "shards over tokens with no exchange; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    import transformer_gemm_epilogue_amd as coda
    if not torch.cuda.is_available():
        print("bench.py needs a GPU (there is no CPU path)", file=sys.stderr)
        sys.exit(1)
    coda.lib()
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_calibration:
        src = torch.ones((1 << 29,), dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            coda.coda_baseline_copy(src, dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": src.numel() * 2, "launches": args.steps}), flush=True)
        return
    if args.aux_sweep_only:
        print(json.dumps({"aux_reduce_sweep": aux_reduce_sweep(coda, torch, args.reps)}), flush=True)
        return
    if args.gemm1_compare:
        print(json.dumps({"gemm1_compare": gemm1_compare(coda, torch, args.reps)}), flush=True)
        return
    if args.schedule_probe:
        print(json.dumps({"schedule_probe": schedule_probe(coda, torch)}), flush=True)
        return
    aux_cool = None if args.headline_only else aux_reduce_sweep(coda, torch, args.reps)
    torch.cuda.empty_cache()
    res, bufs = headline(args, coda, torch)
    log(f"headline: {res['value']} TFLOP/s, {res['ms_per_step']} ms/step")
    if args.shard_share:
        print(json.dumps({"one_gpu_share_of_token_shards": shard_share(coda, torch, bufs, args.reps)}), flush=True)
        return
    if not args.headline_only:
        res["mall_flushed_step"] = mall_flushed(coda, torch, bufs, args.reps)
        res["unfused_fwd"] = unfused_fwd(coda, torch, bufs, args.reps)
        res["one_gpu_share_of_token_shards"] = shard_share(coda, torch, bufs, args.reps)
        u = res["unfused_fwd"]
        res["speedup_vs_unfused_same_mainloop"] = round(u["same_mainloop_plus_separate_kernels_ms"] / u["fused_entry_point_ms"], 3)
        res["speedup_vs_torch_hipblaslt"] = round(u["torch_hipblaslt_eager_ms"] / u["fused_entry_point_ms"], 3)
        del bufs
        torch.cuda.empty_cache()
        res["paths"] = other_paths(coda, torch, args.reps)
        torch.cuda.empty_cache()
        res["mfma_power_ceiling"] = mfma_ceiling(coda, torch)
        g = res["mfma_power_ceiling"]["gaussian_tflops"]
        res["roofline"]["practical_peak_gaussian_operands"] = g
        res["roofline"]["frac_of_practical_peak"] = round(res["roofline"]["achieved"] / g, 4)
        # the same sweep before any GEMM ran and after the GEMM paths (sustained MFMA load
        # leaves the GPU in a lower power state that also slows pure streaming kernels)
        res["aux_reduce_sweep"] = dict(before_gemms=aux_cool, after_gemms=aux_reduce_sweep(coda, torch, args.reps))
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
