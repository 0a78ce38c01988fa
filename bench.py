#!/usr/bin/env python3
"""Benchmark of the KDA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--chunk 32]

A step is one chunkwise forward call (prep, intra-chunk and inter-chunk
kernels) over the layer-shaped workload B=4, T=4096, H=16, Dk=Dv=128, bf16
inputs and fp32 state, with the inputs already resident in HBM.  Four input
sets (about 1.1 GB) rotate from step to step so the 256 MB Infinity Cache
cannot serve them.  The call is kda_chunk_fwd on one stream.  The state chunk is a
tiling choice of the kernels (results agree to rounding for 16, 32 and 64);
32 is the fastest here.  The step time (value, ms_per_step) comes from the
calls alone; the JSON line also reports, measured in the same run:
  * per-call times (median, p10, p90) from an event pair around each call;
  * per-kernel times from HIP events the library records around each of its
    kernels, over a third timed region of the same calls (the records add
    GPU time between kernels: ms_per_step_with_kernel_events);
  * the roofline of the whole call (its compulsory bytes over the step time)
    and the dominant kernel's own-byte rate per launch;
  * MFMA % of the whole call under both flop counts, HBM % on compulsory bytes;
  * the decode step (B=256, H=32, D=128, fp32 state) and its HBM %;
  * the long-context segmented flow (B=1, T=65536, H=32, 8 segments);
  * grouped value heads with the gate bias (4 q/k heads, 16 value heads);
  * the layer body around the core: the input side (SiLU of the kernel-4
    short convolution of q, k, v), the output side (sigmoid gate times per-head
    RMS norm), each with its HBM %, and input side + core + output side;
  * the fp64 oracle timed on the host cores: the whole layer workload, the
    first 2048 tokens of the long workload and 8 full decode steps.
Only the JSON line goes to stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk_kda fwd tokens/s (H=16,Dk=Dv=128,T=4096) + % MFMA peak; decode % HBM"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_layer.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def percentile(sorted_vals, p):
    """Linear-interpolated percentile of an ascending list."""
    if not sorted_vals:
        return None
    x = (len(sorted_vals) - 1) * p / 100.0
    lo = int(x)
    hi = min(lo + 1, len(sorted_vals) - 1)
    return sorted_vals[lo] + (sorted_vals[hi] - sorted_vals[lo]) * (x - lo)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ work model

def chunk_flops(B, T, H, Dk, Dv, C):
    """Algorithmic flops of the chunkwise forward (per chunk-head, triangle
    exact): C^2 (3 Dk + 2 Dv) + 6 C Dk Dv (+ C^3/3 for the solve); and the
    count with full C x C tiles: 2 C^2 (3 Dk + 2 Dv) + 6 C Dk Dv."""
    nch = B * H * ((T + C - 1) // C)
    tri = C * C * (3 * Dk + 2 * Dv) + 6 * C * Dk * Dv + C ** 3 / 3
    full = 2 * C * C * (3 * Dk + 2 * Dv) + 6 * C * Dk * Dv
    return nch * tri, nch * full


def chunk_bytes(B, T, H, Dk, Dv, esize=2):
    """Compulsory HBM bytes of one call: q, k, z, v, beta_raw read once, o and
    the final fp32 state written once."""
    rows = B * T * H
    return rows * (3 * Dk + Dv + 1) * esize + rows * Dv * esize + B * H * Dk * Dv * 4 + H * 4


def block_bytes(Dk, C, esize=2):
    """Bytes of one per-chunk block the intra kernel hands to the inter kernel:
    Kd, Qp (C x Dk), KpT (Dk x C), Tb, Aqk (C x C) as 512-element operand tiles
    (contraction steps of 32 tokens), of which tiles that are zero by
    construction are not stored (Tb and Aqk: steps above the diagonal; the
    diagonal step of an even row block, and a KpT step with no second 16
    tokens, as half tiles), then the fp32 chunk decay (Dk), rounded to 256."""
    nbk, ksd, nbd, ksc = C // 16, (Dk + 31) // 32, Dk // 16, (C + 31) // 32
    tri = sum((256 if 2 * s == ib else 512) for ib in range(nbk) for s in range(ksc) if 2 * s <= ib)
    kpt = nbd * sum((256 if 2 * s + 1 >= nbk else 512) for s in range(ksc))
    elems = 2 * nbk * ksd * 512 + kpt + 2 * tri
    return (elems * esize + Dk * 4 + 255) // 256 * 256


def kernel_bytes(B, T, H, Dk, Dv, C, esize=2):
    """Algorithmic bytes of each kernel over the whole sequence, every byte
    touched once: intra reads q, k, z, beta_raw and A_log and writes the
    per-chunk blocks; inter reads the blocks and v and writes o and the final
    state.  (The fp32 state carried between slices is not counted.)"""
    rows = B * T * H
    blocks = B * H * ((T + C - 1) // C) * block_bytes(Dk, C, esize)
    intra = rows * (3 * Dk + 1) * esize + H * 4 + blocks
    inter = blocks + rows * Dv * esize + rows * Dv * esize + B * H * Dk * Dv * 4
    return {"kda_intra": intra, "kda_inter": inter}


def decode_bytes(B, H, Dk, Dv, esize=2):
    return 2 * B * H * Dk * Dv * 4 + B * H * (3 * Dk + Dv + 1) * esize + B * H * Dv * esize + H * 4


def source_sha():
    h = hashlib.sha256()
    for f in ("kda_chunk.hip", "kda_chunk_kernels.h", "kda_device.h", "kda_internal.h"):
        with open(os.path.join(ROOT, "gated_delta_rule_82_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, chunk, launches):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel sources, the chunk or the launch count per step
    differ from the run the counters were taken on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != source_sha() or kv.get("chunk") != str(chunk):
        return None
    if kv.get(f"{kernel}_launches") != str(launches):
        return None
    val = kv.get(f"{kernel}_hbm_bytes")
    return float(val) if val else None


# ------------------------------------------------------------------ CPU baseline

def _oracle_slice(args):
    from threadpoolctl import threadpool_limits
    from oracle import kda_oracle as ora
    q, k, v, z, br, A = args
    with threadpool_limits(1):
        ora.forward(q, k, v, z, br, A, None)
    return True


def _oracle_decode_slice(args):
    from threadpoolctl import threadpool_limits
    from oracle import kda_oracle as ora
    S, steps, A = args
    with threadpool_limits(1):
        for q, k, v, z, br in steps:
            _, S = ora.step(S, q, k, v, z, br, A)
    return True


def _pool_run(fn, jobs):
    import multiprocessing as mp
    n_proc = min(max(1, min(16, len(os.sched_getaffinity(0)))), len(jobs))
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(n_proc) as pool:
        pool.map(fn, jobs)
    return time.perf_counter() - t0, n_proc


def cpu_baseline_long(inputs, T_sample=2048):
    """The fp64 oracle on the first T_sample tokens of the long workload (B1
    H32 D128), one process per head group."""
    w = inputs.WORKLOADS["long"]
    inp = inputs.make_workload(w, T=T_sample)
    f = lambda n: inp[n].double().numpy()
    q, k, v, z, br = (f(n) for n in ("q", "k", "v", "z", "beta_raw"))
    A = inp["A_log"].double().numpy()
    H = q.shape[2]
    hg = max(1, H // 16)
    jobs = [(q[:, :, h:h + hg], k[:, :, h:h + hg], v[:, :, h:h + hg], z[:, :, h:h + hg], br[:, :, h:h + hg],
             A[h:h + hg]) for h in range(0, H, hg)]
    wall, n_proc = _pool_run(_oracle_slice, jobs)
    return {"value": w.B * T_sample / wall, "unit": "tokens/s", "cores": n_proc,
            "sample": f"long workload, all {w.B * H} heads, first {T_sample} of {w.T} tokens", "wall_s": round(wall, 3)}


def cpu_baseline_decode(inputs, n_steps=8):
    """n_steps full-size decode steps (B256 H32 D128) of the fp64 oracle, one
    process per group of batch rows; per-step time."""
    w = inputs.WORKLOADS["decode"]
    S0, A_log = inputs.make_decode_state(w)
    S = S0.double().numpy()
    A = A_log.double().numpy()
    steps = [inputs.make_decode_step(w, s) for s in range(n_steps)]
    per = max(1, w.B // 16)
    jobs = [(S[b:b + per], [tuple(st[n][b:b + per].double().numpy() for n in ("q", "k", "v", "z", "beta_raw"))
                            for st in steps], A) for b in range(0, w.B, per)]
    wall, n_proc = _pool_run(_oracle_decode_slice, jobs)
    return {"us_per_step": round(wall / n_steps * 1e6, 1), "tokens_per_s": w.B * n_steps / wall, "cores": n_proc,
            "sample": f"decode workload, {n_steps} full steps of B{w.B} H{w.H} D{w.Dk}", "wall_s": round(wall, 3)}


def device_clocks(dev_index=0):
    """Peak shader and memory clocks (MHz) and the CU count from the HIP runtime."""
    import ctypes
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        return {}
    out = {}
    # hipDeviceAttribute_t values of hip_runtime_api.h
    for key, attr in (("clock_mhz", 5), ("mem_clock_mhz", 60), ("cus", 63)):
        v = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), attr, dev_index) == 0:
            out[key] = v.value // 1000 if key.endswith("mhz") else v.value
    return out


def cpu_baseline(inp, T_sample, T_full):
    """Time the fp64 oracle on all heads of the layer workload, first T_sample
    tokens (all of them by default), split over (b, head group) across worker
    processes."""
    import multiprocessing as mp

    import numpy as np
    f = lambda t: t[:, :T_sample].double().numpy()
    q, k, v, z = (f(inp[n]) for n in ("q", "k", "v", "z"))
    br = inp["beta_raw"][:, :T_sample].double().numpy()
    A = inp["A_log"].double().numpy()
    B, _, H, _ = q.shape
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    per_b = max(1, workers // B)
    hg = max(1, H // per_b)
    jobs = [(q[b:b + 1, :, h:h + hg], k[b:b + 1, :, h:h + hg], v[b:b + 1, :, h:h + hg],
             z[b:b + 1, :, h:h + hg], br[b:b + 1, :, h:h + hg], A[h:h + hg])
            for b in range(B) for h in range(0, H, hg)]
    n_proc = min(workers, len(jobs))
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(n_proc) as pool:
        pool.map(_oracle_slice, jobs)
    wall = time.perf_counter() - t0
    return {"value": B * T_sample / wall, "unit": "tokens/s", "cores": n_proc, "kind": "oracle",
            "cpu_model": cpu_model(), "host_cpus_visible": len(os.sched_getaffinity(0)),
            "sample": f"layer workload, all {B * H} (b,h) heads, first {T_sample} of {T_full} tokens, "
                      f"fp64 token recurrence, {len(jobs)} slices over {n_proc} processes",
            "wall_s": round(wall, 3)}


# ------------------------------------------------------------------ GPU legs

def bench_layer(torch, kda, inputs, steps, warmup, chunk=None):
    """Time `steps` calls over rotating input sets (one stream).  Per-kernel
    launch times come from the events the library records around each of its
    kernels on the launch stream (kda_chunk_fwd_timed)."""
    w = inputs.WORKLOADS["layer"]
    dev = torch.device("cuda:0")
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    C = chunk or w.chunk
    base = inputs.make_workload(w)
    sets = [{n: base[n].to(dev) for n in ("q", "k", "v", "z", "beta_raw")}]
    gen = torch.Generator(device=dev)
    for i in range(1, 4):
        gen.manual_seed(w.seed * 100 + i)
        sets.append({n: torch.randn(*base[n].shape, generator=gen, device=dev).to(torch.bfloat16)
                     for n in ("q", "k", "v", "z", "beta_raw")})
    A = base["A_log"].to(dev)
    o = torch.empty(B, T, H, Dv, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    ws_n = kda.workspace_bytes(B, T, H, Dk, Dv, C, torch.bfloat16)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev)
    nk = kda.kernel_count(B, T, H, Dk, Dv, C, torch.bfloat16)
    n_ev = nk + 1

    def step(i, evs=None):
        s = sets[i % len(sets)]
        kda.chunk_fwd(s["q"], s["k"], s["v"], s["z"], s["beta_raw"], A, None, chunk=C,
                      o=o, S_out=S, workspace=ws, events=evs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region 1: the calls alone, back to back (the step time; no
    # per-kernel events, whose records add GPU time between the kernels)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    # timed region 1b: the same calls, each bracketed by its own pair of
    # events on the launch stream (distribution of the call time)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        pairs[i][0].record()
        step(i)
        pairs[i][1].record()
    torch.cuda.synchronize()
    call_ms = sorted(a.elapsed_time(b) for a, b in pairs)
    # timed region 2: the same calls with the library recording an event
    # around each of its kernels on the kernel's stream (per-launch durations)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    start2, end2 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start2.record()
    for i in range(steps):
        step(i, evs[i])
    end2.record()
    torch.cuda.synchronize()
    timed_ms = start2.elapsed_time(end2)
    # kernel k: intra for even k, inter for odd k (they alternate over the slices)
    dur = lambda e, k: e[k].elapsed_time(e[k + 1])
    launches = {"kda_intra": [dur(e, k) for e in evs for k in range(0, nk, 2)],
                "kda_inter": [dur(e, k) for e in evs for k in range(1, nk, 2)]}
    return {"B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "C": C, "ws_bytes": ws_n,
            "schedule": "one stream",
            "ms_per_step": total_ms / steps,
            "call_ms": {"median": percentile(call_ms, 50), "p10": percentile(call_ms, 10),
                        "p90": percentile(call_ms, 90), "mean": sum(call_ms) / len(call_ms), "n": len(call_ms)},
            "ms_per_step_with_kernel_events": timed_ms / steps,
            "kernel_ms": {k: sum(v) / steps for k, v in launches.items()},
            "launch_ms": {k: sum(v) / len(v) for k, v in launches.items()},
            "launches_per_step": {k: len(v) // steps for k, v in launches.items()}}


def bench_decode(torch, kda, inputs, steps, warmup):
    w = inputs.WORKLOADS["decode"]
    dev = torch.device("cuda:0")
    S0, A_log = inputs.make_decode_state(w)
    S = S0.to(dev)
    A = A_log.to(dev)
    pool = [{n: t.to(dev) for n, t in inputs.make_decode_step(w, s).items()} for s in range(8)]
    o = torch.empty(w.B, w.H, w.Dv, dtype=torch.bfloat16, device=dev)

    def step(i):
        p = pool[i % len(pool)]
        kda.step(p["q"], p["k"], p["v"], p["z"], p["beta_raw"], A, S, o=o)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(steps):
        step(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    # each step timed on its own (event pair per launch)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) * 1e3 for a, b in evs)
    nbytes = decode_bytes(w.B, w.H, w.Dk, w.Dv)
    return {"workload": "decode: B256 H32 Dk=Dv=128, bf16 q/k/v/z, fp32 state in place",
            "steps": steps, "us_per_step": round(ms * 1e3, 2),
            "us_per_step_each": {"median": round(percentile(per, 50), 2), "p10": round(percentile(per, 10), 2),
                                 "p90": round(percentile(per, 90), 2)},
            "tokens_per_s": w.B / (ms / 1e3),
            "hbm_gbs": nbytes / (ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS}


def bench_layer_body(torch, kda, inputs, steps, warmup, chunk):
    """The layer's body around the core on the layer workload: SiLU(ShortConv(.))
    of q, k and v (kernel 4, [B, T, H*D] bf16 each); those then the core; the
    output side (sigmoid gate times per-head RMS norm) alone; and all three in a
    row (the layer without its projections).  Algorithmic bytes: each
    convolution reads its input and writes its output once (the three-row
    halo of each 32-token tile is not counted); the output side reads o and
    the gate and writes y once."""
    w = inputs.WORKLOADS["layer"]
    dev = torch.device("cuda:0")
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    base = inputs.make_workload(w)
    gen = torch.Generator(device=dev)
    sets = [{n: base[n].to(dev) for n in ("q", "k", "v", "z", "beta_raw")}]
    for i in range(1, 4):
        gen.manual_seed(w.seed * 100 + 50 + i)
        sets.append({n: torch.randn(*base[n].shape, generator=gen, device=dev).to(torch.bfloat16)
                     for n in ("q", "k", "v", "z", "beta_raw")})
    A = base["A_log"].to(dev)
    gen.manual_seed(w.seed * 100 + 99)
    cw = {n: (torch.randn(H * (Dv if n == "v" else Dk), 4, generator=gen, device=dev) * 0.5).float()
          for n in ("q", "k", "v")}
    cb = {n: (torch.randn(cw[n].shape[0], generator=gen, device=dev) * 0.1).float() for n in ("q", "k", "v")}
    outs = {n: torch.empty_like(sets[0][n]) for n in ("q", "k", "v")}
    gates = [torch.randn(B, T, H, Dv, generator=gen, device=dev).to(torch.bfloat16) for _ in range(2)]
    gw = (torch.rand(Dv, generator=gen, device=dev) + 0.5).float()
    y = torch.empty(B, T, H, Dv, dtype=torch.bfloat16, device=dev)
    o = torch.empty(B, T, H, Dv, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, Dk, Dv, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(B, T, H, Dk, Dv, chunk, torch.bfloat16), dtype=torch.uint8, device=dev)

    def convs(i):
        s = sets[i % len(sets)]
        for n in ("q", "k", "v"):
            kda.short_conv(s[n], cw[n], cb[n], silu=True, y=outs[n])

    def full(i):
        convs(i)
        s = sets[i % len(sets)]
        kda.chunk_fwd(outs["q"], outs["k"], outs["v"], s["z"], s["beta_raw"], A, None, chunk=chunk,
                      o=o, S_out=S, workspace=ws)

    def gate(i):
        kda.output_gate(o, gates[i % 2], gw, y=y)

    def body(i):
        full(i)
        gate(i)

    cw_all = torch.cat([cw["q"], cw["k"], cw["v"]]).contiguous()
    cb_all = torch.cat([cb["q"], cb["k"], cb["v"]]).contiguous()

    def fused_core(i):
        s = sets[i % len(sets)]
        kda.chunk_fwd_conv(s["q"], s["k"], s["v"], s["z"], s["beta_raw"], A, cw_all, cb_all, None, None,
                           chunk=chunk, o=o, S_out=S, workspace=ws)

    def fused_body(i):
        fused_core(i)
        gate(i)

    lws = torch.empty(kda.layer_workspace_bytes(B, T, H, Dk, Dv, chunk, torch.bfloat16), dtype=torch.uint8,
                      device=dev)

    def layer_call(i):
        s = sets[i % len(sets)]
        kda.layer_fwd(s["q"], s["k"], s["v"], s["z"], s["beta_raw"], A, gates[i % 2], gw, None, conv_w=cw_all,
                      conv_b=cb_all, chunk=chunk, y=y, S_out=S, workspace=lws)

    def layer_call_noconv(i):
        s = sets[i % len(sets)]
        kda.layer_fwd(s["q"], s["k"], s["v"], s["z"], s["beta_raw"], A, gates[i % 2], gw, None, chunk=chunk,
                      y=y, S_out=S, workspace=lws)

    def core_then_gate(i):
        s = sets[i % len(sets)]
        kda.chunk_fwd(s["q"], s["k"], s["v"], s["z"], s["beta_raw"], A, None, chunk=chunk, o=o, S_out=S,
                      workspace=ws)
        gate(i)

    res = {}
    for name, fn in (("convs", convs), ("input_side_and_core", full), ("output_gate", gate), ("body", body),
                     ("fused_input_side_and_core", fused_core), ("fused_body", fused_body),
                     ("layer_fwd", layer_call), ("layer_fwd_noconv", layer_call_noconv),
                     ("core_then_gate", core_then_gate)):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        res[name] = e0.elapsed_time(e1) / steps
    conv_bytes = 3 * 2 * B * T * H * Dk * 2
    gate_bytes = 3 * B * T * H * Dv * 2   # o and the gate read, y written
    return {"workload": "layer workload body: SiLU(ShortConv_4(.)) of q, k, v (B4 T4096, 16 x 128 channels "
                        "each, bf16), kda_chunk_fwd (chunk %d), sigmoid(gate) * HeadRMSNorm(o)" % chunk,
            "convs_us": round(res["convs"] * 1e3, 2),
            "convs_hbm_gbs": round(conv_bytes / (res["convs"] / 1e3) / 1e9, 1),
            "convs_hbm_frac": round(conv_bytes / (res["convs"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "input_side_and_core_ms": round(res["input_side_and_core"], 4),
            "input_side_and_core_tokens_per_s": B * T / (res["input_side_and_core"] / 1e3),
            "output_gate_us": round(res["output_gate"] * 1e3, 2),
            "output_gate_hbm_frac": round(gate_bytes / (res["output_gate"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "layer_body_ms": round(res["body"], 4),
            "layer_body_tokens_per_s": B * T / (res["body"] / 1e3),
            "fused_input_side_and_core_ms": round(res["fused_input_side_and_core"], 4),
            "fused_layer_body_ms": round(res["fused_body"], 4),
            "fused_layer_body_tokens_per_s": B * T / (res["fused_body"] / 1e3),
            "fused": "kda_chunk_fwd_conv: the short convolutions and SiLU inside the chunk kernels, then the output side",
            "layer_fwd_ms": round(res["layer_fwd"], 4),
            "layer_fwd_tokens_per_s": B * T / (res["layer_fwd"] / 1e3),
            "layer_fwd_noconv_ms": round(res["layer_fwd_noconv"], 4),
            "core_then_output_gate_ms": round(res["core_then_gate"], 4),
            "layer_fwd": "kda_layer_fwd: the convolutions in the chunk kernels and the output side in the inter "
                         "kernel's output stores (one call, o never stored); _noconv: the output side only, "
                         "against kda_chunk_fwd then kda_output_gate"}


def bench_grouped(torch, kda, steps, warmup, chunk):
    """Grouped value heads with the gate bias at the layer size: B4 T4096, 4
    q/k heads shared by 16 value heads, D128, bf16 (kda_chunk_fwd_grouped)."""
    dev = torch.device("cuda:0")
    B, T, H, HV, D = 4, 4096, 4, 16, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(20260)
    mk = lambda *shape: torch.randn(*shape, generator=gen, device=dev).to(torch.bfloat16)
    sets = [dict(q=mk(B, T, H, D), k=mk(B, T, H, D), v=mk(B, T, HV, D), z=mk(B, T, HV, D), br=mk(B, T, HV))
            for _ in range(4)]
    A = (torch.randn(HV, generator=gen, device=dev) * 0.5).float()
    db = (torch.randn(HV, D, generator=gen, device=dev) * 0.5).float()
    o = torch.empty(B, T, HV, D, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, HV, D, D, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(B, T, HV, D, D, chunk, torch.bfloat16), dtype=torch.uint8, device=dev)

    def step(i):
        s = sets[i % 4]
        kda.chunk_fwd(s["q"], s["k"], s["v"], s["z"], s["br"], A, None, chunk=chunk, o=o, S_out=S,
                      workspace=ws, dt_bias=db)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": "grouped: kda_chunk_fwd_grouped B4 T4096, 4 q/k heads for 16 value heads, "
                        "D128 bf16, with dt_bias (chunk %d)" % chunk,
            "ms": round(ms, 4), "tokens_per_s": B * T / (ms / 1e3)}


def bench_v1_gate(torch, kda, steps, warmup, chunk):
    """The unbounded KDA v1 gate g = -exp(A_log) softplus(z) at the layer size
    (B4 T4096 H16 D128 bf16): ordinary logits z ~ N(0, 1), and logits shifted
    by +8 and spread by 4, where most 16-token blocks decay past the factored
    range and take the element-by-element diagonal products."""
    dev = torch.device("cuda:0")
    B, T, H, D = 4, 4096, 16, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(20261)
    mk = lambda *shape: torch.randn(*shape, generator=gen, device=dev)
    base = [dict(q=mk(B, T, H, D).bfloat16(), k=mk(B, T, H, D).bfloat16(), v=mk(B, T, H, D).bfloat16(),
                 z=mk(B, T, H, D), br=mk(B, T, H).bfloat16()) for _ in range(4)]
    A = (torch.randn(H, generator=gen, device=dev) * 0.5).float()
    o = torch.empty(B, T, H, D, dtype=torch.bfloat16, device=dev)
    S = torch.empty(B, H, D, D, dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(B, T, H, D, D, chunk, torch.bfloat16), dtype=torch.uint8, device=dev)
    flags = kda.FLAGS_DEFAULT | kda.GATE_SOFTPLUS
    res = {"workload": "v1 gate: kda_chunk_fwd with -exp(A_log) softplus(z), B4 T4096 H16 D128 bf16 (chunk %d)"
                       % chunk}
    for name, shift, scale in (("ordinary", 0.0, 1.0), ("strong_decay", 8.0, 4.0)):
        zs = [(b["z"] * scale + shift).bfloat16() for b in base]

        def step(i):
            s = base[i % 4]
            kda.chunk_fwd(s["q"], s["k"], s["v"], zs[i % 4], s["br"], A, None, chunk=chunk, flags=flags, o=o,
                          S_out=S, workspace=ws)

        for i in range(warmup):
            step(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"ms": round(ms, 4), "tokens_per_s": B * T / (ms / 1e3)}
    return res


def bench_backward(torch, kda, inputs, steps, warmup):
    """The backward (kda_chunk_bwd) at the layer size: B4 T4096 H16 D128 bf16,
    a random output gradient, no final-state gradient."""
    w = inputs.WORKLOADS["layer"]
    dev = torch.device("cuda:0")
    inp = {k: (None if v is None else v.to(dev)) for k, v in inputs.make_workload(w).items()}
    gen = torch.Generator(device=dev)
    gen.manual_seed(20262)
    do = torch.randn(w.B, w.T, w.H, w.Dv, generator=gen, device=dev).to(torch.bfloat16)
    ws = torch.empty(kda.bwd_workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv), dtype=torch.uint8, device=dev)

    def step():
        kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["z"], inp["beta_raw"], inp["A_log"], do, inp["S0"],
                      None, workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    # algorithmic flops per chunk-head of the products the backward runs
    # (state and adjoint passes, gradients, operators); the bf16 path runs them
    # on bf16 matrix-core operands with fp32 accumulation, except the operator
    # triangles (fp32, element by element):
    # 2 C Dk Dv x 10 + 2 C^2 Dv x 8 + 2 C^2 Dk
    C = 32
    nch = w.B * w.H * ((w.T + C - 1) // C)
    flops = nch * (2 * C * w.Dk * w.Dv * 10 + 2 * C * C * w.Dv * 8 + 2 * C * C * w.Dk)
    tflops = flops / (ms * 1e-3) / 1e12
    return {"workload": "backward: kda_chunk_bwd B4 T4096 H16 D128 bf16 (bf16 matrix-core operands, fp32 accumulation "
                        "and states, 32-token chunks)",
            "ms": round(ms, 4), "tokens_per_s": w.B * w.T / (ms / 1e3),
            "algorithmic_gflop": round(flops / 1e9, 2), "tflops": round(tflops, 2),
            "frac_bf16_mfma_peak": round(tflops / BF16_PEAK_TFLOPS, 4),
            "workspace_bytes": int(ws.numel())}


def bench_long(torch, kda, inputs, reps, chunk):
    w = inputs.WORKLOADS["long"]
    dev = torch.device("cuda:0")
    n, Tseg = w.segments, w.T // w.segments
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed)
    x = {nm: torch.randn(w.B, w.T, w.H, d, generator=gen, device=dev).to(torch.bfloat16)
         for nm, d in (("q", w.Dk), ("k", w.Dk), ("v", w.Dv), ("z", w.Dk))}
    x["beta_raw"] = torch.randn(w.B, w.T, w.H, generator=gen, device=dev).to(torch.bfloat16)
    A = (torch.randn(w.H, generator=gen, device=dev) * w.a_std).float()
    seg = {k: v.view(n, Tseg, *v.shape[2:]) for k, v in x.items()}
    o_full = torch.empty_like(x["v"])
    S_full = torch.empty(w.B, w.H, w.Dk, w.Dv, device=dev)
    ws = torch.empty(max(kda.workspace_bytes(w.B, w.T, w.H, w.Dk, w.Dv, chunk),
                         kda.workspace_bytes(n, Tseg, w.H, w.Dk, w.Dv, chunk)), dtype=torch.uint8, device=dev)
    o0 = torch.empty(n, 1, Tseg, w.H, w.Dv, dtype=torch.bfloat16, device=dev)
    P = torch.empty(n, 1, Tseg, w.H, w.Dk, dtype=torch.bfloat16, device=dev)
    M = torch.empty(n, 1, w.H, w.Dk, w.Dk, device=dev)
    St = torch.empty(n, 1, w.H, w.Dk, w.Dv, device=dev)
    Sp = torch.empty_like(St)

    def full():
        kda.chunk_fwd(x["q"], x["k"], x["v"], x["z"], x["beta_raw"], A, None, chunk=chunk, o=o_full, S_out=S_full,
                      workspace=ws)

    def segmented():
        kda.chunk_fwd(seg["q"], seg["k"], seg["v"], seg["z"], seg["beta_raw"], A, None, chunk=chunk,
                      want_M=True, want_P=True, o=o0.view(n, Tseg, w.H, w.Dv), S_out=St.view(n, w.H, w.Dk, w.Dv),
                      M_out=M.view(n, w.H, w.Dk, w.Dk), P_out=P.view(n, Tseg, w.H, w.Dk), workspace=ws)
        kda.segment_compose(M, St, S_prefix=Sp)
        kda.segment_fixup(P, Sp, o0)

    res = {}
    for name, fn in (("full", full), ("segmented", segmented)):
        fn()
        torch.cuda.synchronize()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            fn()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        res[name] = {"ms": round(ms, 3), "tokens_per_s": w.T / (ms / 1e3)}
    diff = float((o0.view(w.B, w.T, w.H, w.Dv).float() - o_full.float()).abs().max())
    res["max_abs_diff_vs_full"] = diff
    res["workload"] = (f"long: B1 T65536 H32 Dk=Dv=128 bf16, chunk {chunk}; segmented = 8 x 8192 fragments "
                       "+ compose + fixup")
    return res


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-tokens", type=int, default=4096, help="oracle sample length (0 = skip)")
    ap.add_argument("--decode-steps", type=int, default=1024)  # the decode workload: 1024 successive steps
    ap.add_argument("--long-reps", type=int, default=3)
    ap.add_argument("--only-layer", action="store_true", help="time the layer workload only")
    ap.add_argument("--chunk", type=int, default=32, help="state chunk length (16, 32 or 64)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run 3 device copies of 1 GiB (a counter reference of known size)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the KDA heads are independent, so a multi-GPU run "
              "is B x H sharding with no exchange (see the design notes); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from gated_delta_rule_82_amd import inputs, kda

    kda.load()  # fails loudly if libkda.so is missing

    cpu = None
    if args.cpu_tokens > 0 and not args.only_layer:
        log(f"[bench] oracle CPU baseline on {args.cpu_tokens} tokens ...")
        wl = inputs.WORKLOADS["layer"]
        cpu = cpu_baseline(inputs.make_workload(wl, T=args.cpu_tokens), args.cpu_tokens, wl.T)
        log(f"[bench] oracle: {cpu['value']:.1f} tokens/s on {cpu['cores']} processes")
        cpu["long_sample"] = cpu_baseline_long(inputs)
        cpu["decode_sample"] = cpu_baseline_decode(inputs)
        log(f"[bench] oracle long {cpu['long_sample']}, decode {cpu['decode_sample']}")

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name}, {props.multi_processor_count} CUs")

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 1 GiB device copies done")

    log("[bench] layer workload ...")
    C = args.chunk or 32
    L = bench_layer(torch, kda, inputs, args.steps, args.warmup, C)
    B, T, H, Dk, Dv = L["B"], L["T"], L["H"], L["Dk"], L["Dv"]
    ms = L["ms_per_step"]
    tok_s = B * T / (ms / 1e3)
    f_tri, f_full = chunk_flops(B, T, H, Dk, Dv, C)
    f_tri64, f_full64 = chunk_flops(B, T, H, Dk, Dv, 64)
    cbytes = chunk_bytes(B, T, H, Dk, Dv)
    kb = kernel_bytes(B, T, H, Dk, Dv, C)
    dom = max(L["kernel_ms"], key=L["kernel_ms"].get)
    n_launch = L["launches_per_step"][dom]
    launch_ms = L["launch_ms"][dom]
    bytes_per_launch = kb[dom] / n_launch
    dom_rate = bytes_per_launch / (launch_ms / 1e3) / 1e9
    # the roofline of the whole call: its compulsory bytes (q, k, v, z,
    # beta_raw read once; o and the final state written once) over the step
    # time; the counted traffic is the sum over the call's kernels
    achieved = cbytes / (ms / 1e3) / 1e9
    traffic = None
    per_kernel_traffic = {kn: read_traffic(kn, C, L["launches_per_step"][kn]) for kn in L["launches_per_step"]}
    if per_kernel_traffic and all(v is not None for v in per_kernel_traffic.values()):
        traffic = sum(v * L["launches_per_step"][kn] for kn, v in per_kernel_traffic.items())
    log(f"[bench] layer {ms:.3f} ms/step ({L['schedule']}), {tok_s:.3e} tokens/s; kernels {L['kernel_ms']}")

    extra = {}
    if not args.only_layer:
        log("[bench] decode workload ...")
        extra["decode"] = bench_decode(torch, kda, inputs, args.decode_steps, 10)
        log(f"[bench] decode {extra['decode']['us_per_step']} us/step")
        log("[bench] long workload ...")
        extra["long"] = bench_long(torch, kda, inputs, args.long_reps, C)
        log(f"[bench] long {extra['long']}")
        log("[bench] input side ...")
        extra["layer_body"] = bench_layer_body(torch, kda, inputs, args.steps, args.warmup, C)
        log(f"[bench] layer body {extra['layer_body']}")
        extra["grouped"] = bench_grouped(torch, kda, args.steps, args.warmup, C)
        extra["v1_gate"] = bench_v1_gate(torch, kda, args.steps, args.warmup, C)
        extra["backward"] = bench_backward(torch, kda, inputs, max(3, args.steps // 4), 2)
        log(f"[bench] grouped {extra['grouped']}")

    out = {
        "metric": METRIC,
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, A_log ~ N(0,0.5); 4 rotating input sets in HBM)",
        "config": {"workload": f"layer: chunk_kda fwd B4 T4096 H16 Dk=Dv=128, bf16 in, fp32 state "
                               f"(state chunk {C}; {L['schedule']})",
                   "B": B, "T": T, "H": H, "Dk": Dk, "Dv": Dv, "chunk": C, "g_min": -5.0},
        "roofline": {"bound": "hbm", "kernel": "kda_chunk_fwd call (all kernels)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes": cbytes, "launch_ms": round(ms, 4), "launches_per_step": 1,
                     "basis": "compulsory bytes of the call / ms_per_step"},
        "call_ms": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in L["call_ms"].items()},
        "dominant_kernel": {"kernel": dom, "launch_ms": round(launch_ms, 4), "launches_per_step": n_launch,
                            "own_bytes_per_launch": round(bytes_per_launch),
                            "own_bytes_rate_gbs": round(dom_rate, 1),
                            "own_bytes_frac": round(dom_rate / HBM_PEAK_GBS, 4),
                            "own_bytes": "the kernel's own algorithmic reads and writes, workspace blocks included"},
        "kernel_ms": {k: round(v, 4) for k, v in L["kernel_ms"].items()},
        "ms_per_step_with_kernel_events": round(L["ms_per_step_with_kernel_events"], 4),
        "mfma_frac": {"algorithmic": round(f_tri64 / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "tile_count": round(f_full64 / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "flop_basis": "C = 64 counts of the chunk form whatever chunk runs: triangles exact with the C^3/3 solve (36.9 GFLOP), full C x C tiles (47.2 GFLOP)",
                      "algorithmic_at_run_chunk": round(f_tri / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4),
                      "tile_count_at_run_chunk": round(f_full / (ms / 1e3) / 1e12 / BF16_PEAK_TFLOPS, 4)},
        "hbm_frac_compulsory": round(cbytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "cpu_baseline": cpu,
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count, **{f"hip_{k}": v for k, v in device_clocks().items()}},
    }
    out.update(extra)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
