"""Benchmark of the KDA hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--no-decode] [--no-extras]

A step is one kda_chunk_fwd call (intra-chunk stage + chain stage) over the
1M-token prefill workload: B=1, H=16, T=1,048,576, d_k=d_v=128, C=64, bf16 q/k/v,
fp32 g/beta and state, recurring address keys, fast/slow channel gates (seeded
synthetic inputs, resident in HBM before timing).  Prints one JSON line.  The
same step with the log-gate in bf16 too is timed beside it ("bf16_log_gates"),
the mid (B=4, H=16, T=8192, C=64) and long (B=1, H=32, T=65536, C=128) prefill
workloads as well ("workloads"), and the decode step (256 sequences x 32 heads,
in-place 128x128 fp32 states) is reported under "decode".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E, GB/s
CSRC = os.path.join(ROOT, "linear_attention_sequence_chunk_amd", "csrc")
# HBM bytes per launch measured with rocprofv3 FETCH_SIZE / WRITE_SIZE (scaled by a
# plain copy of known size); valid only while the kernel's sources are unchanged
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic_1m_prefill.txt")
# MFMA counters per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16, SQ_VALU_MFMA_BUSY_CYCLES,
# GRBM_GUI_ACTIVE), under the same rule
MFMA_FILE = os.path.join(ROOT, "profiles", "mfma_valu_1m_prefill.txt")
PROFILED_WORKLOAD = "1m"    # the workload both counter summaries were taken on
MFMA_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
SIMDS = 1024                # 256 CUs x 4
XCDS = 8                    # GRBM_GUI_ACTIVE is summed over them
KERNEL_SOURCES = {
    "chunk_intra64_kernel": ["kda_common.h", "kda_launch.h", "kda_chunk.h", "kda_chunk_intra.hip"],
    "chunk_chain64_kernel": ["kda_common.h", "kda_launch.h", "kda_chunk.h", "kda_chunk_chain64.hip"],
    "chain_maps64_kernel": ["kda_common.h", "kda_launch.h", "kda_chunk.h", "kda_chunk_chain64.hip"],
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="1m")
    p.add_argument("--no-workloads", action="store_true",
                   help="only the headline workload: no mid and long prefill lines")
    p.add_argument("--decode-steps", type=int, default=200)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-extras", action="store_true",
                   help="only the step (and decode): no bf16-gate, gate-layout, fused, varlen or backward lines")
    p.add_argument("--copy-calibration", action="store_true",
                   help="only run a plain 4 GiB device copy (to scale FETCH_SIZE/WRITE_SIZE counters)")
    p.add_argument("--survey", action="store_true",
                   help="only time the prefill step of other head sizes, chunk sizes and dtypes "
                        "(one JSON line each)")
    return p.parse_args()


def source_digest(names):
    """sha256 over the kernel's source files, in order."""
    import hashlib
    hsh = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            hsh.update(f.read())
    return hsh.hexdigest()


def measured_traffic(kernel):
    """HBM bytes per launch (fetch + write) from the committed counter summary,
    or None when there is none or the kernel's sources changed since."""
    if kernel not in KERNEL_SOURCES or not os.path.exists(TRAFFIC_FILE):
        return None
    digest = source_digest(KERNEL_SOURCES[kernel])
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) < 2 or parts[0] != "traffic" or parts[1] != kernel:
                continue
            kv = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
            if kv.get("sha256") == digest:
                return int(kv["fetch_bytes"]) + int(kv["write_bytes"])
    return None


def counted_mfma(kernel):
    """bf16 MFMA flops of one launch (512 per MOPS unit) and its MFMA-busy share of
    all SIMD cycles, from the committed counter summary; None when absent or stale."""
    if kernel not in KERNEL_SOURCES or not os.path.exists(MFMA_FILE):
        return None
    digest = source_digest(KERNEL_SOURCES[kernel])
    with open(MFMA_FILE) as f:
        for line in f:
            parts = line.split()
            if len(parts) < 2 or parts[0] != "mfma" or parts[1] != kernel:
                continue
            kv = dict(p.split("=", 1) for p in parts[2:] if "=" in p)
            if kv.get("sha256") != digest:
                continue
            flops = 512.0 * float(kv["mops_bf16"])
            busy = float(kv["busy_cycles"]) / (float(kv["gui_active"]) / XCDS * SIMDS)
            return flops, busy
    return None


def measured_mfma(kernel, seconds):
    """bf16 MFMA work and utilisation of one launch from the committed counter
    summary, the rate at the live duration; None when absent or stale."""
    c = counted_mfma(kernel)
    if c is None:
        return None
    flops, busy = c
    tflops = flops / seconds / 1e12
    return {"kernel": kernel, "flops_per_launch": round(flops), "tflops": round(tflops, 1),
            "frac_bf16_peak": round(tflops / MFMA_PEAK_TFLOPS, 4), "busy_pct": round(100 * busy, 2),
            "source": os.path.relpath(MFMA_FILE, ROOT)}


def mfma_summary(names, t_intra, t_chain, t_step):
    """Counted bf16 MFMA work of both prefill kernels at the live durations, and
    over the whole step; None when the counters are absent or stale."""
    intra, chain = measured_mfma(names[0], t_intra), measured_mfma(names[1], t_chain)
    if intra is None or chain is None:
        return None
    step = (intra["flops_per_launch"] + chain["flops_per_launch"]) / t_step / 1e12
    return {"intra": intra, "chain": chain, "step_tflops": round(step, 1),
            "step_frac_bf16_peak": round(step / MFMA_PEAK_TFLOPS, 4)}


def mfma_summary_segmented(t_intra, t_step):
    """bf16 MFMA work when the chain runs in segments: the intra kernel at its live
    duration, the chain's first launch (segment 0 and the maps) and outputs launch
    from their counters, and all three over the live step time; None when absent or stale."""
    intra = measured_mfma("chunk_intra64_kernel", t_intra)
    maps, outs = counted_mfma("chain_maps64_kernel"), counted_mfma("chunk_chain64_kernel")
    if intra is None:
        return None
    out = {"intra": intra}
    if maps is not None and outs is not None:
        flops = intra["flops_per_launch"] + maps[0] + outs[0]
        out["chain"] = {"maps_flops_per_launch": round(maps[0]), "maps_busy_pct": round(100 * maps[1], 2),
                        "outputs_flops_per_launch": round(outs[0]), "outputs_busy_pct": round(100 * outs[1], 2)}
        out["step_tflops"] = round(flops / t_step / 1e12, 1)
        out["step_frac_bf16_peak"] = round(flops / t_step / 1e12 / MFMA_PEAK_TFLOPS, 4)
    return out


def prefill_bytes_per_token_head(dk, dv, in_bytes, out_bytes):
    """Bytes the method has to move per (token, head): q, k, v in, g, beta in, o out."""
    return (2 * dk + dv) * in_bytes + dk * 4 + 4 + dv * out_bytes


def device_inputs(torch, inputs, w, dev, t0=0, t1=None):
    """A workload's inputs for tokens [t0, t1), generated block by block on the
    host and copied into device tensors (a few GB at a time for the 1M workload)."""
    t1 = w.T if t1 is None else t1
    Tn = t1 - t0
    sd = w.torch_dtype
    g = {"q": torch.empty((w.B, Tn, w.H, w.dk), dtype=sd, device=dev),
         "k": torch.empty((w.B, Tn, w.H, w.dk), dtype=sd, device=dev),
         "v": torch.empty((w.B, Tn, w.H, w.dv), dtype=sd, device=dev),
         "g": torch.empty((w.B, Tn, w.H, w.dk), dtype=torch.float32, device=dev),
         "beta": torch.empty((w.B, Tn, w.H), dtype=torch.float32, device=dev)}
    piece = 1 << 16
    for a in range(t0, t1, piece):
        b = min(t1, a + piece)
        d = inputs.make_prefill(w, t0=a, t1=b)
        for n in ("q", "k", "v", "g", "beta"):
            g[n][:, a - t0:b - t0].copy_(d[n])
    S0 = inputs.make_state(w)
    g["S0"] = None if S0 is None else S0.to(dev)
    return g


def time_step(torch, plan, steps, warmup):
    """Warm-up steps, then ``steps`` timed steps with HIP events on the launch
    stream around each stage: (mean step ms, mean intra ms, mean chain ms, host ms)."""
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t_host0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        plan.intra()
        ev[i][1].record(stream)
        plan.chain()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    t_host = (time.perf_counter() - t_host0) / steps * 1e3
    intra = sum(ev[i][0].elapsed_time(ev[i][1]) for i in range(steps)) / steps
    chain = sum(ev[i][1].elapsed_time(ev[i][2]) for i in range(steps)) / steps
    step = sum(ev[i][0].elapsed_time(ev[i][2]) for i in range(steps)) / steps
    return step, intra, chain, t_host


def alg_bytes(w, has_s0):
    """Algorithmic bytes of one call (intra stage, chain stage): q, k, v, g, beta
    read once; o written once, the initial state read (when given) and the
    final state written."""
    units = w.B * w.T * w.H                          # token-heads
    ib = 2 if w.dtype == "bf16" else 4
    state = w.B * w.H * w.dk * w.dv * 4
    intra = units * ((2 * w.dk + w.dv) * ib + w.dk * 4 + 4)
    chain = units * (w.dv * ib) + (2 if has_s0 else 1) * state
    return intra, chain


def workload_label(w, chunk_used=None):
    keys = ", recurring address keys" if w.keys == "address" else ""
    ran = f" (run as {chunk_used}-token chunks)" if chunk_used and chunk_used != w.C else ""
    gates = {"tiny": "channel gates", "long": "fast/slow channel gates", "none": "no gate",
             "scalar": "per-head gates"}[w.gates]
    return (f"{w.name} prefill B={w.B} H={w.H} T={w.T} dk={w.dk} dv={w.dv} C={w.C}{ran} "
            f"{'bf16' if w.dtype == 'bf16' else 'fp32'} q/k/v, fp32 g/beta/state, {gates}{keys}")


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    from linear_attention_sequence_chunk_amd import ChunkPlan, decode_step, inputs

    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 4 << 30          # 16x the 256 MB memory-side cache: every byte comes from HBM
        x = torch.ones(n // 4, dtype=torch.float32, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return
    if args.survey:
        bench_survey(torch, ChunkPlan, dev, args.steps)
        return
    w = inputs.WORKLOADS[args.workload]
    g = device_inputs(torch, inputs, w, dev)
    plan = ChunkPlan(g["q"], g["k"], g["v"], g["g"], g["beta"], g["S0"], chunk_size=w.C)

    K = args.steps
    ms_per_step, intra_ms, chain_ms, host_ms = time_step(torch, plan, K, args.warmup)
    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3)

    intra_alg, chain_alg = alg_bytes(w, g["S0"] is not None)
    step_alg = intra_alg + chain_alg
    t_intra, t_chain = intra_ms / 1e3, chain_ms / 1e3
    hot = w.dtype == "bf16" and w.dk == 128 and plan.chunk_used == 64
    names = ("chunk_intra64_kernel", "chunk_chain64_kernel") if hot else ("chunk_intra_kernel", "chunk_chain_kernel")
    # The dominant kernel: the intra stage is one kernel; the chain stage is one
    # kernel, or three (segment 0 with the maps, scan, outputs) when the sequence runs in segments,
    # none of them longer than the intra kernel there (profiles/kernel_stats_1m_prefill.txt).
    segmented = plan.segmented
    dom = (names[0], intra_alg, t_intra) if (t_intra >= t_chain or segmented) else (names[1], chain_alg, t_chain)
    achieved = dom[1] / dom[2] / 1e9
    profiled = args.workload == PROFILED_WORKLOAD
    traffic = measured_traffic(dom[0]) if profiled else None
    roofline = {"bound": "hbm", "kernel": dom[0], "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic, "alg_bytes": dom[1], "ms": round(dom[2] * 1e3, 4)}
    if traffic:
        # the counter bytes (inputs and the workspace the kernel writes) at the same
        # measured duration: how close the kernel runs to the HBM limit for what it moves
        roofline["traffic_GBps"] = round(traffic / dom[2] / 1e9, 1)
        roofline["traffic_frac"] = round(traffic / dom[2] / 1e9 / HBM_PEAK_GBS, 4)

    out = {
        "metric": "KDA chunked-prefill tokens/s (MFMA util %); decode step state GB/s (% HBM)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": f"synthetic (seeded; shapes and distributions of the {w.name} prefill workload)",
        "config": {"workload": workload_label(w, plan.chunk_used), "global_batch": w.B, "seq_len": w.T, "heads": w.H,
                   "chunk": w.C, "parallelism": "single GPU"},
        "roofline": roofline,
        "mfma": mfma_summary(names, t_intra, t_chain, ms_per_step / 1e3) if hot and profiled and not segmented else None,
        "path": {"step_alg_bytes": step_alg, "step_alg_GBps": round(step_alg / (ms_per_step / 1e3) / 1e9, 1),
                 "step_frac_hbm": round(step_alg / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                 "intra_ms": round(intra_ms, 4), "chain_ms": round(chain_ms, 4),
                 "chain_segments": plan.segments, "host_wall_ms_per_step": round(host_ms, 4)},
    }
    if segmented and profiled:
        out["mfma"] = mfma_summary_segmented(t_intra, ms_per_step / 1e3)

    out["gpu_clocks"] = gpu_clocks(torch, plan, steps=min(5000, max(60, int(1200 / ms_per_step))))
    if not args.no_extras:
        out["bf16_log_gates"] = bench_bf16_gates(torch, ChunkPlan, g, w, K, args.warmup)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(torch, inputs, w, g, dev)
    del plan, g
    torch.cuda.empty_cache()

    if not args.no_workloads:
        out["workloads"] = {}
        for name in ("mid", "long"):
            if name != args.workload:
                out["workloads"][name] = bench_workload(torch, inputs, ChunkPlan, inputs.WORKLOADS[name], dev, K,
                                                        args.warmup)

    if not args.no_extras:
        wm = inputs.WORKLOADS["mid"]
        gm = device_inputs(torch, inputs, wm, dev)
        out["gate_layouts"] = bench_gate_layouts(torch, ChunkPlan, gm, wm, K, args.warmup)
        out["fused_pre"] = bench_fused_pre(torch, ChunkPlan, gm, wm, K, args.warmup)
        out["varlen"] = bench_varlen(torch, gm, wm, K, args.warmup)
        out["backward"] = bench_backward(torch, gm, wm)
        del gm
        torch.cuda.empty_cache()

    if not args.no_decode:
        out["decode"] = bench_decode(torch, inputs, decode_step, dev, args.decode_steps)

    if cpu is not None:
        out["cpu_baseline"] = cpu

    print(json.dumps(out), flush=True)


def gpu_clocks(torch, plan, steps=60, samples=12):
    """GPU clocks while the step runs (amd-smi's library, in this process, after
    the timed region): about 1.2 s of untimed steps are queued, and the graphics
    and memory clocks are sampled only while the stream still has work pending,
    from 0.3 s after the queueing on.  None where the library is missing."""
    try:
        import amdsmi
    except Exception:
        return None
    try:
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
        gmax = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)["max_clk"]
        stream = torch.cuda.current_stream()
        for _ in range(steps):
            plan.run()
        time.sleep(0.3)          # both readings refresh about every 0.1 s: skip those taken while idle
        gfx, mem, sleep, xcd = [], [], [], []
        while len(gfx) < samples and not stream.query():
            g = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
            gfx.append(g["clk"])
            sleep.append(g.get("clk_deep_sleep"))
            mem.append(amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.MEM)["clk"])
            xcd.append(_current_gfx_mhz(amdsmi, h))
            time.sleep(0.02)
        torch.cuda.synchronize()
        return {"gfx_mhz_samples": gfx, "gfx_deep_sleep": sleep, "gfx_max_mhz": gmax,
                "mem_mhz": max(mem) if mem else None,
                "gfx_mhz_current_xcd_mean": xcd,
                "note": "sampled while untimed steps ran, after the timed region: the clock the "
                        "management library reports (with its deep-sleep flag), and the mean over "
                        "the XCDs of the instantaneous clocks in its metrics table"}
    except Exception as e:                 # a clock reading must never fail the bench
        torch.cuda.synchronize()
        return {"error": type(e).__name__}
    finally:
        try:
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def _current_gfx_mhz(amdsmi, h):
    """Mean over the XCDs of the instantaneous graphics clocks in the metrics
    table (entries the table marks as not available skipped), or None."""
    try:
        m = amdsmi.amdsmi_get_gpu_metrics_info(h)
    except Exception:
        return None
    vals = m.get("current_gfxclks")
    if not isinstance(vals, (list, tuple)):
        vals = [m.get("current_gfxclk")]
    vals = [v for v in vals if isinstance(v, (int, float)) and 0 < v < 0xFFFF]
    return round(sum(vals) / len(vals)) if vals else None


def bench_workload(torch, inputs, ChunkPlan, w, dev, steps, warmup):
    """One more prefill workload: step time, tokens/s and the fraction of the HBM
    roofline the whole step reaches for its algorithmic bytes."""
    g = device_inputs(torch, inputs, w, dev)
    plan = ChunkPlan(g["q"], g["k"], g["v"], g["g"], g["beta"], g["S0"], chunk_size=w.C)
    ms, intra, chain, _ = time_step(torch, plan, steps, warmup)
    ia, ca = alg_bytes(w, g["S0"] is not None)
    res = {"config": workload_label(w, plan.chunk_used), "ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1),
           "intra_ms": round(intra, 4), "chain_ms": round(chain, 4), "chain_segments": plan.segments,
           "step_alg_bytes": ia + ca, "step_frac_hbm": round((ia + ca) / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "hbm_floor_ms": round((ia + ca) / HBM_PEAK_GBS / 1e6, 4)}
    del plan, g
    torch.cuda.empty_cache()
    return res


def bench_bf16_gates(torch, ChunkPlan, g, w, steps, warmup):
    """The same step with the log-gate stored in bf16 as well, so that every input
    is bf16 (the kernels widen the gate to fp32 on load): 1028 instead of 1284
    bytes read per token-head.  The gate values are the workload's, rounded."""
    gb = g["g"].to(torch.bfloat16)
    plan = ChunkPlan(g["q"], g["k"], g["v"], gb, g["beta"], g["S0"], chunk_size=w.C)
    ms, intra, chain, _ = time_step(torch, plan, steps, warmup)
    del plan, gb
    torch.cuda.empty_cache()
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1),
            "intra_ms": round(intra, 4), "chain_ms": round(chain, 4),
            "note": "q, k, v and the log-gate g in bf16; beta and the state fp32"}


def bench_gate_layouts(torch, ChunkPlan, g, w, steps, warmup):
    """The same step with one gate per head (g [B,T,H]: the first channel's
    gates) and with no gate (alpha = 1, g not read)."""
    res = {}
    for layout in ("head", "none"):
        gl = g["g"][..., 0].contiguous() if layout == "head" else None
        plan = ChunkPlan(g["q"], g["k"], g["v"], gl, g["beta"], g["S0"], chunk_size=w.C, gate_layout=layout)
        for _ in range(warmup):
            plan.run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            plan.run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[layout] = {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1)}
        del plan
    return res


def bench_fused_pre(torch, ChunkPlan, g, w, steps, warmup):
    """The same step with the fused pre-processing: q and k normalised in the
    kernels and the gate given as a bf16 pre-activation a = log(e^{-g} - 1),
    whose -softplus is the workload's log-gate (up to bf16 rounding)."""
    a = torch.log(torch.expm1(-g["g"])).to(torch.bfloat16)
    plan = ChunkPlan(g["q"], g["k"], g["v"], a, g["beta"], g["S0"], chunk_size=w.C, qk_l2norm=True,
                     gate_act="softplus")
    for _ in range(warmup):
        plan.run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        plan.run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del plan, a
    return {"ms_per_step": round(ms, 4), "tokens_per_s": round(w.B * w.T / (ms / 1e3), 1),
            "note": "raw q/k L2-normalised and g = -softplus(a), bf16 a, inside the intra kernel"}


def bench_varlen(torch, g, w, steps, warmup):
    """A packed batch of mixed lengths: the mid workload's tokens of batch row 0
    and 1 (16384 tokens per head) cut into sequences of 64..2047 tokens (seeded),
    one kda_chunk_fwd_varlen call."""
    import numpy as np

    from linear_attention_sequence_chunk_amd import chunk_fwd_varlen
    T = 2 * w.T
    rs = np.random.default_rng(11)
    cuts = [0]
    while cuts[-1] < T:
        cuts.append(min(T, cuts[-1] + int(rs.integers(64, 2048))))
    cu = torch.tensor(cuts, dtype=torch.int32, device=g["q"].device)
    N = len(cuts) - 1
    pk = {key: g[key][:2].reshape((T,) + tuple(g[key].shape[2:])).contiguous() for key in ("q", "k", "v", "g", "beta")}
    from linear_attention_sequence_chunk_amd import _lib
    code = _lib.BF16 if pk["q"].dtype == torch.bfloat16 else _lib.F32
    nbytes = int(_lib.lib().kda_chunk_varlen_workspace_bytes(N, T, w.H, w.dk, w.dv, code, w.C))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=g["q"].device)   # allocated once, outside timing
    o, S = chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu, chunk_size=w.C, workspace=ws)
    for _ in range(warmup):
        chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu, chunk_size=w.C, final_state=S,
                         workspace=ws)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu, chunk_size=w.C, final_state=S,
                         workspace=ws)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"sequences": N, "tokens": T, "heads": w.H, "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms / 1e3), 1),
            "note": "workspace allocated once, outside the timed calls"}


def bench_backward(torch, g, w, steps=5, warmup=2):
    """kda_chunk_bwd on the same workload: gradients of sum(dO * o) for every
    input (the forward stages are re-run inside the call); and kda_chunk_bwd_pre,
    the same through the fused pre-processing (raw q, k; bf16 gate
    pre-activation a = log(e^{-g} - 1))."""
    from linear_attention_sequence_chunk_amd import chunk_bwd
    gen = torch.Generator(device=g["q"].device).manual_seed(0)
    dO = torch.randn(g["v"].shape, generator=gen, device=g["q"].device, dtype=torch.float32)
    a = torch.log(torch.expm1(-g["g"])).to(torch.bfloat16)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    ms = timed(lambda: chunk_bwd(g["q"], g["k"], g["v"], g["g"], g["beta"], dO, g["S0"], chunk_size=w.C))
    ms_pre = timed(lambda: chunk_bwd(g["q"], g["k"], g["v"], a, g["beta"], dO, g["S0"], chunk_size=w.C,
                                     qk_l2norm=True, gate_act="softplus"))
    del a, dO
    tps = lambda t: round(w.B * w.T / (t / 1e3), 1)
    return {"ms_per_call": round(ms, 3), "tokens_per_s": tps(ms), "calls": steps,
            "note": "gradients accumulated in fp32 (fp32 operands of bf16 MFMA split into hi + lo parts); "
                    "includes re-running the forward stages",
            "fused_pre": {"ms_per_call": round(ms_pre, 3), "tokens_per_s": tps(ms_pre),
                          "note": "gradients of raw q, k and the bf16 gate pre-activation"}}


SURVEY_CONFIGS = [(128, 128, 64, "bf16"), (128, 64, 64, "bf16"), (64, 64, 64, "bf16"), (64, 128, 64, "bf16"),
                  (128, 128, 32, "bf16"), (128, 128, 16, "bf16"), (128, 128, 128, "bf16"),
                  (128, 128, 64, "fp32"), (64, 64, 64, "fp32")]


def bench_survey(torch, ChunkPlan, dev, steps):
    """The prefill step (both stages) for other head sizes, chunk sizes and input
    dtypes, at the mid workload's B=4, T=8192, H=16: random inputs drawn on the
    device (timing only), unit-norm q/k rows, log-gates in (-0.05, 0)."""
    B, T, H = 4, 8192, 16
    for dk, dv, C, dt in SURVEY_CONFIGS:
        dtype = torch.bfloat16 if dt == "bf16" else torch.float32
        gen = torch.Generator(device=dev).manual_seed(0)
        rn = lambda *shape: torch.randn(shape, generator=gen, device=dev)
        q = torch.nn.functional.normalize(rn(B, T, H, dk), dim=-1).to(dtype)
        k = torch.nn.functional.normalize(rn(B, T, H, dk), dim=-1).to(dtype)
        v = rn(B, T, H, dv).to(dtype)
        g = -0.05 * torch.rand((B, T, H, dk), generator=gen, device=dev)
        beta = torch.rand((B, T, H), generator=gen, device=dev)
        plan = ChunkPlan(q, k, v, g, beta, None, chunk_size=C)
        for _ in range(2):
            plan.run()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ti = tc = 0.0
        for _ in range(steps):
            ev[0].record(stream)
            plan.intra()
            ev[1].record(stream)
            plan.chain()
            ev[2].record(stream)
            torch.cuda.synchronize()
            ti += ev[0].elapsed_time(ev[1])
            tc += ev[1].elapsed_time(ev[2])
        ti, tc = ti / steps, tc / steps
        print(json.dumps({"survey": {"dk": dk, "dv": dv, "chunk": C, "dtype": dt, "B": B, "T": T, "H": H,
                                     "intra_ms": round(ti, 4), "chain_ms": round(tc, 4),
                                     "tokens_per_s": round(B * T / ((ti + tc) / 1e3), 1)}}), flush=True)
        del plan, q, k, v, g, beta
        torch.cuda.empty_cache()


def bench_decode(torch, inputs, decode_step, dev, steps):
    """Decode: 256 sequences x 32 heads, in-place fp32 states; a pool of 16
    input sets is cycled (the kernel has no data-dependent control flow)."""
    wd = inputs.WORKLOADS["decode"]
    S = inputs.decode_state(wd).to(dev)
    pool = inputs.make_decode_steps(wd, 16)
    pool = {k: v.to(dev) for k, v in pool.items()}
    o = torch.empty((wd.B, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)
    for i in range(5):
        decode_step(pool["q"][i], pool["k"][i], pool["v"][i], pool["g"][i], pool["beta"][i], S, o=o)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        j = i % 16
        decode_step(pool["q"][j], pool["k"][j], pool["v"][j], pool["g"][j], pool["beta"][j], S, o=o)
    e1.record(stream)
    torch.cuda.synchronize()
    t = e0.elapsed_time(e1) / 1e3 / steps
    nh = wd.B * wd.H
    per_tok = (2 * wd.dk + wd.dv) * 2 + wd.dk * 4 + 4 + wd.dv * 2
    byts = nh * (2 * wd.dk * wd.dv * 4 + per_tok)
    gbs = byts / t / 1e9
    out = {"metric": "decode step state GB/s", "GBps": round(gbs, 1),
           "frac_hbm": round(gbs / HBM_PEAK_GBS, 4), "us_per_step": round(t * 1e6, 2),
           "tokens_per_s": round(wd.B / t, 1), "bytes_per_step": byts, "steps": steps,
           "config": "256 sequences x 32 heads, dk=dv=128, bf16 q/k/v, fp32 state in place"}

    # four tokens per call (kda_decode_tokens): the state moves once per call
    from linear_attention_sequence_chunk_amd import decode_tokens
    TT = 4
    seq = lambda x: x.transpose(0, 1).contiguous()
    tk = {key: seq(pool[key][:TT]) for key in pool}
    o4 = torch.empty((wd.B, TT, wd.H, wd.dv), dtype=torch.bfloat16, device=dev)
    calls = max(1, steps // TT)
    for _ in range(3):
        decode_tokens(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S, o=o4)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(calls):
        decode_tokens(tk["q"], tk["k"], tk["v"], tk["g"], tk["beta"], S, o=o4)
    e1.record(stream)
    torch.cuda.synchronize()
    t4 = e0.elapsed_time(e1) / 1e3 / calls
    b4 = nh * (2 * wd.dk * wd.dv * 4 + TT * per_tok)
    out["tokens4"] = {"tokens_per_call": TT, "us_per_call": round(t4 * 1e6, 2),
                      "tokens_per_s": round(wd.B * TT / t4, 1), "GBps": round(b4 / t4 / 1e9, 1),
                      "bytes_per_call": b4}
    return out


CPU_TAIL = 65536       # tokens of the 1M workload the oracle baseline runs


def cpu_baseline(torch, inputs, w, g, dev):
    """The fp64 oracle (as it stands) timed on the host cores.  For the 1M-token
    workload: the last CPU_TAIL tokens of all 16 heads, from the GPU state at
    T - CPU_TAIL (a split call, untimed), about 25 CPU-seconds; for the smaller
    workloads the whole workload.  Threads: os.cpu_count(); the oracle runs one
    (batch, head) sequence per thread, so ``cores`` is the threads it used.  Also
    one thread on one sequence, and the host's CPU model."""
    import numpy as np

    import oracle
    from linear_attention_sequence_chunk_amd import chunk_fwd

    host_cpus = os.cpu_count() or 1
    # a tail from the GPU state needs the prefix call on a contiguous slice: B = 1
    t0 = max(0, w.T - CPU_TAIL) if (w.T > 4 * CPU_TAIL and w.B == 1) else 0
    if t0:
        _, S_mid = chunk_fwd(g["q"][:, :t0], g["k"][:, :t0], g["v"][:, :t0], g["g"][:, :t0], g["beta"][:, :t0],
                             g["S0"], chunk_size=w.C)
        torch.cuda.synchronize()
        S0 = oracle.to_f64(S_mid.cpu())
        sample = (f"the last {w.T - t0} tokens of all {w.B * w.H} (batch, head) sequences, from the GPU "
                  f"state at token {t0}")
    else:
        S0 = None if g["S0"] is None else oracle.to_f64(g["S0"].cpu())
        sample = f"the whole workload: {w.B}x{w.H} (batch x head) sequences of {w.T} tokens"
    d = inputs.make_prefill(w, t0=t0, t1=w.T)
    args = [oracle.to_f64(d[k]) for k in ("q", "k", "v", "g", "beta")]
    oracle._lib()
    ta = time.perf_counter()
    oracle.recurrent(*args, S0=S0, nthreads=host_cpus)
    dt = time.perf_counter() - ta
    used = min(oracle.last_threads(), w.B * w.H)
    one = [np.ascontiguousarray(a[:1, :, :1]) for a in args]
    s0 = None if S0 is None else np.ascontiguousarray(S0[:1, :1])
    tb = time.perf_counter()
    oracle.recurrent(*one, S0=s0, nthreads=1)
    dt1 = time.perf_counter() - tb
    tokens = w.B * (w.T - t0)
    return {"value": round(tokens / dt, 1), "unit": "tokens/s", "cores": used, "threads": used,
            "host_cpus": host_cpus, "kind": "oracle", "seconds": round(dt, 3),
            "cpu_seconds": round(dt * used, 1), "sample": sample,
            "single_thread_value": round((w.T - t0) / w.H / dt1, 1),
            "single_thread_sample": f"1 of the {w.H} heads of one batch row, one thread (a token is all heads)",
            "cpu_model": _cpu_model()}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


if __name__ == "__main__":
    main()
