#!/usr/bin/env python3
"""Benchmark of the channel-wise gated delta rule on one MI355X.

A step is one chunkwise forward (gdr_chunk_fwd: intra-chunk, chain and
output kernels, in segments of chunks) over the long-context stress
workload: B1 H16 T32768 dk=dv=128, bf16 inputs, fp32 output and state, chunk
128 (default) -- inputs resident in HBM before the timed region.  Timed in
the same run and reported beside it: the decode step (256 sequences x 16
heads, fp32 128 x 128 states, 1024 consecutive steps), the same long-context
shape with scalar gates (one decay and one beta per token, Gated DeltaNet),
the layer path around the recurrence (the five-gate low-rank projection,
then the forward with the fused RMSNorm + output gate), and the backward
pass (gdr_chunk_bwd) over the long-context shape.

Prints one JSON line.  Per-kernel durations come from HIP events recorded on
the stream the kernels run on; the roofline object describes the kernel with
the largest share of the step (the intra-chunk kernel), over the launches the
whole call makes (one per segment of chunks).  The same long-context shape at
the other chunk size (64 when the headline uses 128) is measured beside it.
The fp64 CPU oracle is timed on a bounded sample of the same workload (rank
0, N = 1 only) as `cpu_baseline`.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk 64|128]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
METRIC = "tokens/s + % bf16 MFMA peak, chunk fwd T=32K H=16 d=128; decode HBM GB/s"
# HBM bytes per dispatch of the intra-chunk kernel as the whole call launches
# it (one segment of chunks; the launches the roofline times), from two
# rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE) over this benchmark,
# each scaled by what the same counter reads for a plain 1 GiB device copy
# (fetch x2.0, write x1.0).  Valid only for the sources they were taken on
# (digest below: the kernel's sources, the ABI and the build flags);
# otherwise reported as null.
MEASURED_TRAFFIC = {
    "sources": "498a932e0b5eff7c",
    "chunk_intra_kernel_C128_seg": 269411824,   # 512 chunks of 128 tokens per launch
    "chunk_intra_kernel_C64_seg": 168479491,    # 512 chunks of 64 tokens per launch
}


def flops_per_token_head(C, dk, dv):
    """Algorithmic flops of the chunk path per (token, head): the three
    state products (Y S, Qt S, K'^T U: 2 C dk dv each per chunk) plus the
    intra-chunk work (Gram and scores C^2 dk each, triangular solve with
    dk + dv right-hand sides C^2 (dk + dv), A U C^2 dv), triangles counted
    once, divided by C."""
    return 6 * dk * dv + C * (3 * dk + 2 * dv)


def chunk_bytes_per_token_head(dk, dv, in_bytes=2, out_bytes=4, gain=True):
    """HBM bytes that must move per (token, head): q, k, v, b, w (+ z) in the
    input dtype, fp32 log-decay, o in the output dtype."""
    n_in = 5 + (1 if gain else 0)
    return n_in * dk * in_bytes - (dk - dv) * 2 * in_bytes + 4 * dk + out_bytes * dv


def sources_digest():
    """Digest of every source the measured intra-chunk kernel and its launch
    are built from: the kernel's translation unit and the headers it
    includes, the C ABI that sets its arguments, and the build flags."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "channel_wise_gated_amd", "csrc")
    files = [os.path.join(csrc, n) for n in ("gdr_chunk.hip", "gdr_abi.hip", "gdr_device.h", "gdr_launch.h")]
    files += [os.path.join(ROOT, "include", "gdr.h"), os.path.join(ROOT, "channel_wise_gated_amd", "build.py")]
    for path in files:
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def timed_chunk(call, steps, warmup):
    """Wall time of `steps` whole calls (gdr_chunk_fwd, which runs a long
    batch in segments of chunks), then HIP-event times of the same number of
    phase-call pairs over every chunk in one launch each (gdr_chunk_fwd_intra,
    gdr_chunk_fwd_scan), recorded on the stream the kernels run on."""
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call.intra()
        e[1].record()
        call.scan()
        e[2].record()
    torch.cuda.synchronize()
    intra = sorted(e[0].elapsed_time(e[1]) for e in ev)
    scan = sorted(e[1].elapsed_time(e[2]) for e in ev)
    return wall, intra, scan


def timed_segments(x, C, steps, warmup):
    """The kernels of a whole call, launched as gdr_chunk_fwd launches them.
    The library reports its segment length (chunks per stream); the inputs of
    every segment are copied to contiguous tensors of seg * C tokens, and
    each segment's intra-chunk phase call (one launch over B * H * seg
    chunks: the grid of the whole call's intra launches) and scan call (chain
    and output kernels) are issued in order, the fp32 state handed from one
    segment to the next.  HIP events on the stream the kernels run on, around
    every launch.  Returns (seg, [intra ms per segment launch], [scan ms])."""
    import torch

    from channel_wise_gated_amd import gdr
    B, H, T, dk = x["q"].shape
    desc = gdr.make_desc(B, H, T, dk, x["v"].shape[-1], C)
    seg = gdr.gdr_chunk_fwd_segment_chunks(desc)
    L = seg * C
    nseg = -(-T // L)
    if nseg < 2:
        return seg, [], []
    calls, S = [], x["S0"]
    ws = None
    for s in range(nseg):
        part = {k: (v[:, :, s * L:(s + 1) * L].contiguous() if (v is not None and v.dim() == 4 and k != "S0")
                    else v) for k, v in x.items()}
        c = gdr.ChunkCall(part["q"], part["k"], part["v"], part["log_alpha"], part["b"], part["w"],
                          part["gamma"], part["z"], S, chunk=C, workspace=ws)
        ws = c.workspace
        calls.append(c)
        S = c.S_T
    for _ in range(max(1, warmup // 2)):
        for c in calls:
            c.intra()
            c.scan()
    torch.cuda.synchronize()
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in calls] for _ in range(steps)]
    for rep in ev:
        for c, e in zip(calls, rep):
            e[0].record()
            c.intra()
            e[1].record()
            c.scan()
            e[2].record()
    torch.cuda.synchronize()
    intra = [e[0].elapsed_time(e[1]) for rep in ev for e in rep]
    scan = [e[1].elapsed_time(e[2]) for rep in ev for e in rep]
    del calls
    return seg, intra, scan


def measure_chunk(x, wl, C, steps, warmup):
    """One forward configuration: whole-call throughput (wall clock over
    `steps` gdr_chunk_fwd calls), algorithmic rates, and the roofline of the
    dominant kernel over the launches the whole call runs."""
    from channel_wise_gated_amd import gdr
    call = gdr.ChunkCall(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], x["gamma"],
                         x["z"], x["S0"], chunk=C)
    wall, intra1, scan1 = timed_chunk(call, steps, warmup)
    del call
    seg, intra_s, scan_s = timed_segments(x, C, steps, warmup)
    ms_step = 1e3 * wall / steps
    BH = wl.B * wl.H
    per_th = chunk_bytes_per_token_head(wl.dk, wl.dv)
    fl = flops_per_token_head(C, wl.dk, wl.dv) * BH * wl.T
    byt = per_th * BH * wl.T + 2 * BH * wl.dk * wl.dv * 4
    med = lambda a: sorted(a)[len(a) // 2]
    mean = lambda a: sum(a) / len(a)
    in_per_th = per_th - 4 * wl.dv          # the intra-chunk kernel reads every input once
    out = {"workload": f"stress B{wl.B} H{wl.H} T{wl.T} dk{wl.dk} dv{wl.dv} chunk{C}",
           "steps": steps, "ms_per_step": round(ms_step, 4), "tokens_s": round(wl.B * wl.T / (ms_step / 1e3), 1),
           "tflops_algorithmic": round(fl / (ms_step / 1e3) / 1e12, 2),
           "mfma_frac": round(fl / (ms_step / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
           "hbm_gbs_algorithmic": round(byt / (ms_step / 1e3) / 1e9, 1),
           "hbm_frac": round(byt / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
           "segment_chunks": seg}
    kb1 = in_per_th * BH * wl.T
    single = {"launch": f"one launch over all {BH * -(-wl.T // C)} chunks (gdr_chunk_fwd_intra)",
              "avg_ms": round(mean(intra1), 4), "achieved": round(kb1 / (mean(intra1) / 1e3) / 1e9, 1),
              "algorithmic_bytes_per_launch": kb1}
    single["frac"] = round(single["achieved"] / HBM_PEAK_GBS, 4)
    if intra_s:
        ntok = seg * C
        kb = in_per_th * BH * ntok
        avg = mean(intra_s)
        ach = kb / (avg / 1e3) / 1e9
        traffic = None
        if MEASURED_TRAFFIC["sources"] == sources_digest():
            traffic = MEASURED_TRAFFIC.get(f"chunk_intra_kernel_C{C}_seg")
        out["roofline"] = {
            "bound": "hbm", "kernel": "chunk_intra_kernel", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
            "launch": f"one segment: {BH * seg} chunks of {C} tokens ({seg} per stream), as gdr_chunk_fwd "
                      f"launches it; HIP events around each of the {len(intra_s) // steps} segment launches "
                      f"of {steps} calls",
            "algorithmic_bytes_per_launch": kb, "avg_ms": round(avg, 4)}
        out["kernels_ms"] = {"chunk_intra_kernel": round(med(intra_s), 4), "chain_and_output": round(med(scan_s), 4),
                             "per": f"segment launch ({BH * seg} chunks), median"}
    else:  # the whole call runs in one pass
        out["roofline"] = dict(bound="hbm", kernel="chunk_intra_kernel", achieved=single["achieved"],
                               peak=HBM_PEAK_GBS, unit="GB/s", frac=single["frac"], traffic=None,
                               launch=single["launch"], algorithmic_bytes_per_launch=kb1, avg_ms=single["avg_ms"])
        out["kernels_ms"] = {"chunk_intra_kernel": round(med(intra1), 4), "chain_and_output": round(med(scan1), 4),
                             "per": "whole launch, median"}
    out["roofline_single_launch"] = single
    return out


def timed_decode(wl, steps, warmup):
    import ctypes

    import torch

    from channel_wise_gated_amd import gdr
    from channel_wise_gated_amd.inputs import make_inputs_device
    lib = gdr.load()
    x = make_inputs_device(wl, "cuda", steps=steps)
    S = x["S0"].clone()
    o = torch.empty((wl.B, wl.H, wl.dv), dtype=torch.float32, device="cuda")
    desc = gdr.make_desc(wl.B, wl.H, 1, wl.dk, wl.dv, 64, gdr.GDR_BF16, gdr.GDR_F32)
    stream = ctypes.c_void_p(int(torch.cuda.current_stream().cuda_stream))
    # marshal every step's arguments before timing
    args = []
    for s in range(steps):
        p = [ctypes.c_void_p(x[n][s].data_ptr()) for n in ("q", "k", "v", "log_alpha", "b", "w")]
        args.append((ctypes.byref(desc), ctypes.c_void_p(S.data_ptr()), *p,
                     ctypes.c_void_p(x["gamma"].data_ptr()), ctypes.c_void_p(x["z"][s].data_ptr()),
                     ctypes.c_void_p(o.data_ptr()), stream))
    for s in range(warmup):
        if lib.gdr_decode_step(*args[s % steps]) != 0:
            raise RuntimeError("gdr_decode_step failed")
    S.copy_(x["S0"])
    torch.cuda.synchronize()
    # one pair of events around the consecutive steps (an event between every
    # two steps would add its own packet to the stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for s in range(steps):
        lib.gdr_decode_step(*args[s])
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = e0.elapsed_time(e1)
    del x
    return wall, total_ms


def timed_layer(x, C, steps, warmup):
    """The layer path around the recurrence at the long-context shape: the
    five-gate projection (d_model 2048, ranks 64/64/128/128/128, 16 heads of
    128, bf16 gates, fp32 log-decay) of a [1, 32768, 2048] bf16 input, then
    the chunkwise forward with the fused RMSNorm + output gate on the
    stress workload's q, k, v and those gates.  Random-init weights; the
    decay gate's bias is +4 (alpha ~ 0.98 per token).  HIP events on the
    stream the kernels run on, median over `steps`."""
    import torch

    from channel_wise_gated_amd import gdr
    B, H, T, d = 1, 16, x["q"].shape[2], 128
    dm, ranks = 2048, (64, 64, 128, 128, 128)
    R = sum(ranks)
    gen = torch.Generator(device="cuda").manual_seed(20251)
    rn = lambda *s: torch.randn(*s, generator=gen, device="cuda")
    xin = rn(B, T, dm).to(torch.bfloat16)
    wd = (rn(R, dm) / dm ** 0.5).to(torch.bfloat16)
    wu = gdr.pack_gate_up({n: (rn(H * d, r) / r ** 0.5).to(torch.bfloat16) for n, r in zip(gdr.GATE_ORDER, ranks)})
    bias = 0.5 * rn(5, H * d)
    bias[0] += 4.0
    gates = gdr.gdr_gate_proj(xin, wd, wu, bias, ranks, H, d)
    gws = torch.empty(B * T * R * 4, dtype=torch.uint8, device="cuda")
    nw = 1.0 + 0.1 * rn(H, d)
    y = torch.empty(B, T, H, d, device="cuda")
    sT = torch.empty(B, H, d, d, device="cuda")
    probe = gdr.ChunkCall(x["q"], x["k"], x["v"], gates["f"], gates["b"], gates["w"], x["gamma"], gates["q"],
                          x["S0"], chunk=C)
    cws = probe.workspace
    proj = lambda: gdr.gdr_gate_proj(xin, wd, wu, bias, ranks, H, d, outs=gates, workspace=gws)
    gated = lambda: gdr.gdr_chunk_fwd_gated(x["q"], x["k"], x["v"], gates["f"], gates["b"], gates["w"], gates["g"],
                                            gamma=x["gamma"], z=gates["q"], S0=x["S0"], norm_weight=nw,
                                            chunk=C, y=y, S_T=sT, workspace=cws)
    for _ in range(warmup):
        proj()
        gated()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        proj()
        e[1].record()
        gated()
        e[2].record()
    torch.cuda.synchronize()
    med = lambda a: sorted(a)[len(a) // 2]
    p_ms = med([e[0].elapsed_time(e[1]) for e in ev])
    g_ms = med([e[1].elapsed_time(e[2]) for e in ev])
    # algorithmic HBM bytes of the projection: x in, five gate tensors out
    p_bytes = B * T * dm * 2 + B * T * H * d * (4 + 4 * 2)
    return {"workload": f"layer B{B} T{T} d_model {dm} ranks {'/'.join(map(str, ranks))} H{H} d{d} chunk{C}",
            "steps": steps, "gate_proj_ms": round(p_ms, 4), "gated_chunk_fwd_ms": round(g_ms, 4),
            "layer_tokens_s": round(B * T / ((p_ms + g_ms) / 1e3), 1),
            "gate_proj_hbm_gbs": round(p_bytes / (p_ms / 1e3) / 1e9, 1),
            "gate_proj_bytes": p_bytes}


def timed_bwd(x, steps, warmup):
    """The backward pass over the long-context inputs (chunk 64, every
    gradient incl. dS0 from an upstream dS_T): random fp32 dO; and the output
    gate's backward at the same shape.  HIP events on
    the current stream, median over `steps`; gradients and workspace come
    from torch's caching allocator (no device allocation after warm-up)."""
    import torch

    from channel_wise_gated_amd import gdr
    B, H, T, dk = x["q"].shape
    dv = x["v"].shape[-1]
    gen = torch.Generator(device="cuda").manual_seed(4099)
    dO = torch.randn(B, H, T, dv, generator=gen, device="cuda")
    dST = 0.1 * torch.randn(B, H, dk, dv, generator=gen, device="cuda")
    call = lambda: gdr.gdr_chunk_bwd(x["q"], x["k"], x["v"], x["log_alpha"], x["b"], x["w"], dO,
                                     gamma=x["gamma"], z=x["z"], S0=x["S0"], dS_T=dST)
    for _ in range(max(warmup, 1)):
        call()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    ms = sorted(e[0].elapsed_time(e[1]) for e in ev)[steps // 2]
    # the output gate's backward at the same shape (o fp32, bf16 gate logits and
    # dy, norm weight): the step before the recurrence's backward in a layer
    o = torch.randn(B, H, T, dv, generator=gen, device="cuda")
    gl = torch.randn(B, H, T, dv, generator=gen, device="cuda").to(torch.bfloat16)
    dy = torch.randn(B, T, H, dv, generator=gen, device="cuda").to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn(H, dv, generator=gen, device="cuda")
    ogb = lambda: gdr.gdr_output_gate_bwd(o, gl, dy, nw, eps=1e-6)
    ogb()
    torch.cuda.synchronize()
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in ev2:
        e[0].record()
        ogb()
        e[1].record()
    torch.cuda.synchronize()
    og_ms = sorted(e[0].elapsed_time(e[1]) for e in ev2)[steps // 2]
    og_bytes = B * H * T * dv * (4 + 2 + 2 + 4 + 4)  # o, g, dy in; do, dg out
    # algorithmic HBM bytes: bf16 q, k, v, b, w, z and fp32 log-decay, dO in;
    # seven fp32 gradients out (dS0 and dgamma are negligible)
    byt = B * H * T * (6 * 2 * dk + 4 * dk + 4 * dv + 7 * 4 * dk)
    return {"workload": f"bwd B{B} H{H} T{T} dk{dk} dv{dv} chunk64, grads of q,k,v,log-decay,b,w,z,gain,S0",
            "steps": steps, "ms_per_step": round(ms, 4), "tokens_s": round(B * T / (ms / 1e3), 1),
            "bytes_algorithmic": byt, "hbm_gbs_algorithmic": round(byt / (ms / 1e3) / 1e9, 1),
            "out_gate_bwd_ms": round(og_ms, 4), "out_gate_bwd_hbm_gbs": round(og_bytes / (og_ms / 1e3) / 1e9, 1)}


def copy_calibration(mib):
    """A plain device-to-device copy of `mib` MiB (fp32), three times: the
    reference dispatch against which HBM byte counters are scaled."""
    import torch
    src = torch.ones(mib * (1 << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def cpu_baseline(x, target_s=12.0):
    """The fp64 oracle, as it stands, on the host cores: the first Ts tokens of
    every head, or -- when the whole sequence takes less than `target_s` --
    the whole workload repeated until about `target_s` of CPU work."""
    import oracle

    def sample(Ts):
        return {k: (v[:, :, :Ts].cpu() if (v is not None and v.dim() == 4 and k != "S0")
                    else (v.cpu() if v is not None else None)) for k, v in x.items()}

    def run(s):
        oracle.forward(s["q"], s["k"], s["v"], s["log_alpha"], s["b"], s["w"], gamma=s["gamma"],
                       z=s["z"], S0=s["S0"], threads=threads)

    B, H, T = x["q"].shape[:3]
    threads = oracle.default_threads(H * B)
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        avail = os.cpu_count() or 1
    probe = 512
    s = sample(probe)
    t0 = time.perf_counter()
    run(s)
    rate = probe / (time.perf_counter() - t0)
    Ts = int(min(T, max(probe, (rate * target_s) // 64 * 64)))
    reps = 1 if Ts < T else max(1, int(round(target_s / (T / rate))))
    s = sample(Ts)
    t0 = time.perf_counter()
    for _ in range(reps):
        run(s)
    dt = time.perf_counter() - t0
    what = f"first {Ts} of {T} tokens" if Ts < T else f"all {T} tokens, {reps} runs"
    return {"value": round(reps * Ts * B / dt, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "seconds": round(dt, 2), "cpu_model": cpu_model(),
            "cores_available": avail, "threads_used": threads,
            "sample": f"{what}, all {H} heads (one thread per stream, at most one per core), "
                      f"fp64 token recurrence"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--chunk", type=int, default=128, choices=(64, 128))
    ap.add_argument("--no-both-chunks", dest="both_chunks", action="store_false",
                    help="skip the leg at the other chunk size (64 when --chunk 128)")
    ap.add_argument("--decode-steps", type=int, default=1024, help="0 skips the decode leg")
    ap.add_argument("--gdn-steps", type=int, default=20,
                    help="whole calls of the scalar-gate (Gated DeltaNet) leg; 0 skips it")
    ap.add_argument("--layer-steps", type=int, default=20,
                    help="steps of the gate projection + gated forward leg; 0 skips it")
    ap.add_argument("--bwd-steps", type=int, default=10, help="0 skips the backward leg")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain MIB-MiB copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} requested, but this benchmark runs on exactly one GPU "
              "(the recurrence shards over (batch, head) streams with no communication; the "
              "library has no multi-GPU path). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from channel_wise_gated_amd import gdr
    from channel_wise_gated_amd.inputs import WORKLOADS, make_inputs_device

    torch.cuda.set_device(0)
    gdr.load()
    if args.calibrate_copy > 0:
        copy_calibration(args.calibrate_copy)
    wl = WORKLOADS["stress"]
    C = args.chunk
    x = make_inputs_device(wl, "cuda")
    main_leg = measure_chunk(x, wl, C, args.steps, args.warmup)
    other_c = 64 if C == 128 else 128
    other_leg = measure_chunk(x, wl, other_c, args.steps, args.warmup) if args.both_chunks else None
    ms_step = main_leg["ms_per_step"]
    tok_s = wl.B * wl.T / (ms_step / 1e3)

    # scalar-gate leg: the same shape with one decay and one beta per token
    gsteps = args.gdn_steps
    if gsteps > 0:
        gwl = WORKLOADS["gdn"]
        xg = make_inputs_device(gwl, "cuda")
        callg = gdr.ChunkCall(xg["q"], xg["k"], xg["v"], xg["log_alpha"], xg["b"], xg["w"], xg["gamma"],
                              xg["z"], xg["S0"], chunk=C)
        for _ in range(args.warmup):
            callg()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(gsteps):
            callg()
        torch.cuda.synchronize()
        g_ms = 1e3 * (time.perf_counter() - t0) / gsteps
        del callg, xg

    # layer: gate projection + gated chunk forward on the stress inputs
    if args.layer_steps > 0:
        layer = timed_layer(x, C, args.layer_steps, min(args.warmup, 5))
        torch.cuda.empty_cache()

    # backward over the stress inputs
    if args.bwd_steps > 0:
        bwd = timed_bwd(x, args.bwd_steps, min(args.warmup, 3))
        torch.cuda.empty_cache()

    # decode
    dwl = WORKLOADS["decode"]
    dsteps = args.decode_steps
    if dsteps > 0:
        dwall, dtotal = timed_decode(dwl, dsteps, warmup=min(16, dsteps))
        dbytes = dwl.B * dwl.H * (2 * dwl.dk * dwl.dv * 4 + 6 * dwl.dk * 2 + 4 * dwl.dk + 4 * dwl.dv)
        d_us = 1e3 * dtotal / dsteps
        d_gbs = dbytes / (d_us / 1e6) / 1e9

    line = {
        "metric": METRIC, "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_leg["workload"],
                   "inputs": "bf16 q,k,v,b,w,z; fp32 log-decay, gain, state and o",
                   "arith": "bf16 hi/lo-split MFMA, fp32 accumulate and state"},
        "tflops_algorithmic": main_leg["tflops_algorithmic"], "mfma_frac": main_leg["mfma_frac"],
        "mfma_target_frac": 0.40,
        "hbm_gbs_algorithmic": main_leg["hbm_gbs_algorithmic"], "hbm_frac": main_leg["hbm_frac"],
        "segment_chunks": main_leg["segment_chunks"],
        "kernels_ms": main_leg["kernels_ms"],
        "roofline": main_leg["roofline"],
        "roofline_single_launch": main_leg["roofline_single_launch"],
    }
    if other_leg is not None:
        line[f"chunk{other_c}"] = other_leg
    if gsteps > 0:
        line["gdn"] = {"workload": f"gdn B{gwl.B} H{gwl.H} T{gwl.T} dk{gwl.dk} dv{gwl.dv} chunk{C}, "
                                   "one decay and one beta per token (b = w)",
                       "steps": gsteps, "ms_per_step": round(g_ms, 4),
                       "tokens_s": round(gwl.B * gwl.T / (g_ms / 1e3), 1)}
    if args.layer_steps > 0:
        line["layer"] = layer
    if args.bwd_steps > 0:
        line["bwd"] = bwd
    if dsteps > 0:
        line["decode"] = {"workload": f"decode {dwl.B} seq x H{dwl.H}, fp32 state {dwl.dk}x{dwl.dv}, "
                                      f"{dsteps} steps", "us_per_step": round(d_us, 2),
                          "gbs": round(d_gbs, 1), "hbm_frac": round(d_gbs / HBM_PEAK_GBS, 4),
                          "bytes_per_step": dbytes, "wall_s": round(dwall, 3)}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
