"""Benchmark: selective-scan layer core, forward + backward, on one MI355X.

A step is one training pass of the layer core over one batch of synthetic
input: zero the accumulated gradients, forward (conv+SiLU when the workload
has it, softplus, exp(delta*A) recurrence, C.h + D*u, gate), backward (the
full reverse-time adjoint).  Inputs are resident in HBM before timing
starts.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--workload NAME]

``--layer NAME`` instead times one whole Mamba-1 layer (RMSNorm,
projections, conv, scan core, residual; include/mamba_layer.h), forward +
backward per step, at a shape of ``workloads.LAYER_CONFIGS``.

``--m3 NAME`` instead times the Mamba-3 SISO core (include/mamba3.h),
forward + backward per step, at a shape of ``workloads.M3_CONFIGS``.

``--recurrent`` instead times the recurrent-step path: one-step forward
calls of the fused entry (conv state and SSM state in, new states out, the
state ping-ponging between two buffers as in decoding), one JSON line per
(batch, d_inner) shape.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBPS = 8000.0            # MI355X HBM3E
# VALU issue rate without packed-FP32 instructions: 256 CUs x 4 SIMDs x 16
# lanes x 2.4 GHz = 39.3 T lane-slots/s (one fp32 FMA, mul or add per slot;
# v_exp_f32 measured at half rate, i.e. 2 slots)
VALU_LANE_SLOTS_PER_S = 256 * 4 * 16 * 2.4e9
# Checkpoint interval of the algorithmic byte model: the backward reads one
# f32 state per 64 steps and channel, whatever interval a run uses.
MODEL_CHUNK = 64
# Algorithmic VALU slots per (t, channel, state) element, exp = 2:
#   forward : delta*A, exp, delta*u*B, h = dA*h + .., y += C*h               ->  6
#   backward: recompute (delta*A, exp, delta*u*B, h update)                  ->  5
#             adjoint (dh, dA*h_prev, q, d_A sum, carry, sum dh*B, sum q*A,
#             d_B and d_C products)                                          ->  9
#             the two sums over channels (d_B, d_C)                          ->  2
# Per-(t, channel) work (softplus, gate, D*u, ...) is spread over the states
# and not counted: the figures are lower bounds of the work the method needs.
SLOTS_FWD_ELEM = 6
SLOTS_BWD_ELEM = 16


def kernel_source_hash():
    """sha256 over the sources the core's backward kernels are built from
    (file names and contents, sorted): every csrc file but the forward's
    (scan_fwd.h, scan_step.h, inst_fwd_*), the whole-layer kernels' (layer_*)
    and the Mamba-3 core's (m3*), since the counters it guards are those of
    the backward."""
    import hashlib
    csrc = os.path.join(ROOT, "state_space_sequence_selective_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")) and not f.startswith(("layer_", "scan_fwd", "scan_step", "inst_fwd_", "m3")):
            h.update(f.encode())
            h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, chunk: int):
    """HBM bytes per backward launch from the committed rocprofv3 counter runs
    (profiles/traffic.json), or None when the kernels or the launch
    configuration changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(workload)
    if not rec or rec.get("kernel_src_sha256") != kernel_source_hash() or rec.get("chunk", 16) != chunk:
        return None
    return rec["bwd_entry_bytes"]


def act_bytes(act):
    return 4 if act == "f32" else 2


def io_bytes(w: workloads.Workload):
    """Activation I/O the method must move, (forward, backward), inputs read
    once and outputs written once.

    Per token-channel: the forward reads x|u, delta_raw, [z] and writes out;
    the backward reads x|u, delta_raw, [z], dout and writes d_x|d_u,
    d_delta_raw, [d_z].  Per token: the B and C rows (activation dtype) in
    both passes, and d_B / d_C (f32) out of the backward."""
    s = act_bytes(w.act)
    N, Di, Ds = w.batch * w.seqlen, w.d_inner, w.d_state
    g = 1 if w.gate else 0
    fwd = N * Di * s * (3 + g) + N * 2 * Ds * s
    bwd = N * Di * s * (5 + 2 * g) + N * 2 * Ds * s + N * 2 * Ds * 4
    return fwd, bwd


def ckpt_bytes(w: workloads.Workload, L: int):
    """f32 states saved every L steps: [B, ceil(T/L), d_inner, d_state]."""
    return w.batch * -(-w.seqlen // L) * w.d_inner * w.d_state * 4


def algorithmic_bytes(w: workloads.Workload):
    """(forward, backward) bytes of the byte model: the activation I/O plus
    checkpoints at MODEL_CHUNK, written by the forward and read by the
    backward."""
    fio, bio = io_bytes(w)
    c = ckpt_bytes(w, MODEL_CHUNK)
    return fio + c, bio + c


def overhead_bytes(w: workloads.Workload, L: int):
    """Bytes a run moves beyond the model, per pass: checkpoints at the run's
    interval beyond those at MODEL_CHUNK, and the y the forward saves for the
    gate's adjoint (written, then read)."""
    extra_ckpt = ckpt_bytes(w, L) - ckpt_bytes(w, MODEL_CHUNK)
    y = w.batch * w.seqlen * w.d_inner * act_bytes(w.act) if w.gate else 0
    return {"fwd": extra_ckpt + y, "bwd": extra_ckpt + y, "extra_ckpt_each_way": extra_ckpt, "y_saved_each_way": y}


def device_inputs(torch, w, inp):
    at = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act]
    dev = {}
    for k in ("x", "delta_raw", "z", "dout", "xdbl"):
        if inp.get(k) is not None:
            dev[k] = torch.from_numpy(inp[k]).to("cuda", at)
    for k in ("a_log", "D", "conv_w", "conv_b"):
        if inp.get(k) is not None:
            dev[k] = torch.from_numpy(inp[k]).to("cuda", torch.float32)
    return dev


# (batch, d_inner) of the recurrent-step timings; d_state 16, dt_rank
# d_inner / 32, conv width 4, bf16 activations, gate on
RECURRENT_SHAPES = [(1, 2048), (64, 2048), (1, 5120), (16, 5120), (64, 5120)]
GRAPH_STEPS = 64   # one-step calls captured per HIP graph


def recurrent_bytes(w: workloads.Workload):
    """Bytes one step call must move: per channel the SSM state and conv
    state in and out (f32), x, delta_raw, z read and out written; per batch
    row the B/C row; per channel the parameters (a_log, D, conv_w, conv_b)."""
    s = act_bytes(w.act)
    per_chan = 2 * w.d_state * 4 + 2 * w.d_conv * 4 + 4 * s
    params = w.d_inner * (w.d_state + 1 + w.d_conv + 1) * 4
    return w.batch * w.d_inner * per_chan + w.batch * 2 * w.d_state * s + params


def recurrent(torch, pkg, calls: int, warmup: int):
    from state_space_sequence_selective_amd import _lib
    stream = torch.cuda.current_stream()
    for B, Di in RECURRENT_SHAPES:
        w = workloads.Workload("recurrent_step_b%d_di%d_bf16" % (B, Di), B, 1, Di, 16, Di // 32, 4, "bf16", True)
        inp = workloads.make_inputs(w, 0, h0=True, conv_state0=True)
        dev = device_inputs(torch, w, inp)
        dims = pkg.Dims.make(B, 1, Di, w.d_state, w.dt_rank, w.d_conv, 16, w.act)
        f32 = dict(device="cuda", dtype=torch.float32)
        h = [torch.from_numpy(inp["h0"]).to(**f32), torch.empty((B, Di, w.d_state), **f32)]
        cs = [torch.from_numpy(inp["conv_state0"]).to(**f32), torch.empty((B, Di, w.d_conv), **f32)]
        out = torch.empty((B, 1, Di), device="cuda", dtype=torch.bfloat16)
        ws = torch.empty(_lib.workspace_bytes(dims), device="cuda", dtype=torch.uint8)

        def call(k):
            _lib.conv_scan_gate_fwd(dims, dev["x"], dev["conv_w"], dev["conv_b"], cs[k % 2], dev["delta_raw"],
                                    dev["a_log"], dev["xdbl"], dev["D"], dev["z"], h[k % 2], out=out,
                                    h_last=h[(k + 1) % 2], conv_state_last=cs[(k + 1) % 2], workspace=ws)

        for k in range(warmup):
            call(k)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(calls):
            call(k)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / calls
        # the same ping-pong captured as one HIP graph of GRAPH_STEPS calls and
        # replayed: the per-step cost without the host-side launch path
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for k in range(2):
                call(k)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for k in range(GRAPH_STEPS):
                call(k)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        reps = max(1, calls // GRAPH_STEPS)
        e0.record(stream)
        for _ in range(reps):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us_graph = e0.elapsed_time(e1) * 1e3 / (reps * GRAPH_STEPS)
        nb = recurrent_bytes(w)
        print(json.dumps({"metric": "recurrent step latency (one-step fused forward, state in/out)",
                          "value": round(us, 2), "unit": "us/call", "higher_is_better": False, "calls": calls,
                          "dtype": w.act, "data": "synthetic",
                          "config": {"workload": w.name, "batch": B, "d_inner": Di, "d_state": w.d_state,
                                     "dt_rank": w.dt_rank, "d_conv": w.d_conv},
                          "algorithmic_bytes_per_call": nb,
                          "GBps_at_algorithmic_bytes": round(nb / (us / 1e6) / 1e9, 1),
                          "us_per_step_graph": round(us_graph, 2), "graph_steps": GRAPH_STEPS}), flush=True)


def layer_flops(w: workloads.LayerWorkload):
    """Dense-projection flops of one layer step (forward + both backward
    products of every projection), 2 per multiply-add."""
    N, dm, Di, R = w.batch * w.seqlen, w.d_model, w.d_inner, w.dt_rank
    X = R + 2 * w.d_state
    per_pass = 2 * N * (dm * 2 * Di + Di * X + R * Di + Di * dm)
    return 3 * per_pass


def layer_bench(torch, pkg, name: str, steps: int, warmup: int, no_cpu: bool, budget_s: float):
    w = workloads.LAYER_CONFIGS[name]
    inp = workloads.make_layer_inputs(w, 0)
    at = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act]
    weights = {n: torch.from_numpy(inp[n]).to("cuda", at if n in pkg.LAYER_TYPED else torch.float32)
               for n in pkg.LAYER_PARAMS}
    dims = pkg.LayerDims.make(w.batch, w.seqlen, w.d_model, w.d_inner, w.d_state, w.dt_rank, w.d_conv, 16, w.act)
    layer = pkg.MambaLayer(dims, weights)
    resid = torch.from_numpy(inp["resid"]).cuda()
    d_out = torch.from_numpy(inp["d_resid_out"]).cuda()
    stream = torch.cuda.current_stream()

    def step(ev=None):
        # the current stream: the caller's here, the capture stream below
        cur = torch.cuda.current_stream()
        layer.zero_grads()
        if ev:
            ev[0].record(cur)
        layer.forward(resid, stream=cur)
        if ev:
            ev[1].record(cur)
        layer.backward(resid, d_out, stream=cur)
        if ev:
            ev[2].record(cur)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # eager calls: each step enqueues about 50 kernels, library calls and the
    # second stream's forks and joins from the host
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(steps):
        step(evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / steps
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # the same step captured once as a HIP graph and replayed: the identical
    # kernels without the host's per-call launch work (the replay test checks
    # replays bit for bit against the eager step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        step()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        graph.replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    tokens = w.batch * w.seqlen
    res = {"metric": "Mamba-1 layer fwd+bwd tokens/sec", "value": round(tokens / (ms / 1e3), 1), "unit": "tokens/s",
           "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": w.act, "data": "synthetic (seeded)",
           "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_model": w.d_model,
                      "d_inner": w.d_inner, "d_state": w.d_state, "dt_rank": w.dt_rank, "d_conv": w.d_conv,
                      "chunk": 16, "parallelism": "single GPU", "step": "HIP graph replay"},
           "ms_per_step_eager": round(ms_eager, 4), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
           "projection_flops_per_step": layer_flops(w)}
    # the dense products (rocBLAS, bf16 / f16 on the matrix cores) against the
    # dense 16-bit peak; their flops over the whole step's time, so a lower
    # bound on their own rate (they share the step with the core and the
    # elementwise kernels; the kernel-trace profile gives their own time)
    pt = layer_flops(w) / (ms / 1e3) / 1e12
    res["roofline"] = {"bound": "mfma", "achieved": round(pt, 1), "peak": 2500.0, "unit": "TFLOP/s",
                       "frac": round(pt / 2500.0, 4), "traffic": None,
                       "kernel": "the layer's dense products, averaged over the whole step",
                       "algorithmic_flops_per_step": layer_flops(w)}
    if not no_cpu:
        res["cpu_baseline"] = layer_cpu_baseline(w, budget_s)
    print(json.dumps(res), flush=True)


def layer_cpu_baseline(w: workloads.LayerWorkload, budget_s: float):
    """The layer oracle as it stands (float64), forward + backward, on a
    bounded sample of the same widths (fewer steps), scaled to the tokens of
    the workload."""
    from oracle import layer as OL
    T = 64
    while True:
        sw = w.with_(batch=1, seqlen=T)
        inp = workloads.make_layer_inputs(sw, 0)
        p = {n: inp[n].astype(np.float64) for n in ("norm_w", "w_in", "conv_w", "conv_b", "w_x", "w_dt", "b_dt",
                                                   "a_log", "D", "w_out")}
        t0 = time.perf_counter()
        out, saved = OL.layer_forward(inp["resid"].astype(np.float64), p, act=w.act)
        OL.layer_backward(inp["resid"].astype(np.float64), p, saved, inp["d_resid_out"].astype(np.float64), act=w.act)
        dt = time.perf_counter() - t0
        if dt > 0.25 * budget_s or T >= w.seqlen * w.batch:
            break
        T = min(w.seqlen * w.batch, T * max(2, int(0.5 * budget_s / max(dt, 1e-3))))
    return {"value": T / dt, "unit": "tokens/s", "cores": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": "1 batch row x %d steps of the same widths, fwd+bwd in %.1f s" % (T, dt)}


def m3_flops(w: workloads.M3Workload):
    """(forward, backward) flops of the per-chunk contractions, 2 per
    multiply-add, per 64-step chunk and head (L = 64 steps, P = headdim,
    N = d_state):
      forward : chunk state L*P*N, Q K^T L*L*N, (G o M) V L*L*P, Q S_in L*P*N
      backward: chunk state of (dY, Q) L*P*N, Q K^T L*L*N, dY V^T L*L*P,
                dV = (G o M)^T dY L*L*P, dQ and dK from (DV o M) 2*L*L*N, the
                entering-state and outgoing-gradient terms of dQ, dK, dV 3*L*P*N."""
    L, P, N = 64, w.headdim, w.d_state
    chunks = w.batch * w.heads * -(-w.seqlen // L)
    fwd = 2 * L * (2 * P * N + L * N + L * P) * chunks
    bwd = 2 * L * (4 * P * N + 3 * L * N + 2 * L * P) * chunks
    return fwd, bwd


def m3_bytes(w: workloads.M3Workload):
    """(forward, backward) algorithmic bytes: inputs read once, outputs
    written once, the f32 chunk states written by the forward and read by the
    backward."""
    s = act_bytes(w.act)
    N_tok = w.batch * w.seqlen
    x = N_tok * w.heads * w.headdim * s
    bc = 2 * N_tok * w.groups * w.d_state * s
    scal = 3 * N_tok * w.heads * 4 + N_tok * w.n_angles * 4
    params = (2 * w.heads * w.d_state + 2 * w.heads) * 4
    states = w.batch * w.heads * -(-w.seqlen // 64) * w.headdim * w.d_state * 4
    fwd = x + bc + scal + params + x + states
    bwd = (x + bc + scal + params + states + x) + (x + bc + scal + params)
    return fwd, bwd


def m3_bench(torch, pkg, name: str, steps: int, warmup: int, no_cpu: bool, budget_s: float):
    w = workloads.M3_CONFIGS[name]
    dims = pkg.M3Dims.make(w.batch, w.seqlen, w.heads, w.headdim, w.d_state, w.groups, w.n_angles, w.act, w.a_floor)
    core = pkg.Mamba3Core(dims)
    at = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act]
    sets = []
    for k in range(INPUT_SETS):
        inp = workloads.make_m3_inputs(w, k)
        sets.append({n: torch.from_numpy(v).to("cuda", at if n in ("x", "b_in", "c_in", "dy") else torch.float32)
                     for n, v in inp.items()})
    stream = torch.cuda.current_stream()

    def step(k, ev=None):
        cur = torch.cuda.current_stream()   # the capture stream while a graph is captured
        dev = sets[k % len(sets)]
        core.zero_grads()
        if ev:
            ev[0].record(cur)
        core.forward(dev, stream=cur)
        if ev:
            ev[1].record(cur)
        core.backward(dev, dev["dy"], stream=cur)
        if ev:
            ev[2].record(cur)

    for k in range(warmup):
        step(k)
    torch.cuda.synchronize()
    # eager calls: each step enqueues about 25 kernels from the host
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for k in range(steps):
        step(warmup + k, evs[k])
    end.record(stream)
    torch.cuda.synchronize()
    ms_eager = start.elapsed_time(end) / steps
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    # the same step captured as a HIP graph, one per input set, and the K
    # steps replayed in the eager order: the identical kernels without the
    # host's per-call launch work (the replay test checks replays bit for bit
    # against the eager step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for k in range(len(sets)):
            step(k)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for k in range(len(sets)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(k)
        graphs.append(g)
    torch.cuda.synchronize()
    for k in range(warmup):
        graphs[k % len(graphs)].replay()
    torch.cuda.synchronize()
    start.record(stream)
    for k in range(steps):
        graphs[(warmup + k) % len(graphs)].replay()
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / steps
    tokens = w.batch * w.seqlen
    ff, fb = m3_flops(w)
    bf, bb = m3_bytes(w)
    # the dominant launch is the backward entry point; at the byte model's
    # bytes and the flop count above, its ideal time at the HBM and matrix (or,
    # for f32 / f16 activations, VALU) peaks puts it on the HBM side
    gbps = bb / (bwd / 1e3) / 1e9
    tflops = fb / (bwd / 1e3) / 1e12
    mfma = w.act == "bf16"
    cpeak = 2500.0 if mfma else 78.6
    res = {"metric": "Mamba-3 SISO core fwd+bwd tokens/sec", "value": round(tokens / (ms / 1e3), 1),
           "unit": "tokens/s", "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": round(ms, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.act,
           "data": "synthetic (seeded; %d input sets rotated)" % len(sets),
           "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "heads": w.heads,
                      "headdim": w.headdim, "d_state": w.d_state, "groups": w.groups, "n_angles": w.n_angles,
                      "chunk": 64, "parallelism": "single GPU", "step": "HIP graph replay"},
           "ms_per_step_eager": round(ms_eager, 4), "fwd_ms": round(fwd, 4), "bwd_ms": round(bwd, 4),
           "hbm_GBps": round((bf + bb) / (ms / 1e3) / 1e9, 1),
           "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                        "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": None,
                        "kernel": "mamba3_siso_bwd entry point", "launch_ms": round(bwd, 4),
                        "algorithmic_bytes_per_launch": bb},
           "compute_roofline": {"bound": "mfma" if mfma else "alu", "achieved": round(tflops, 2), "peak": cpeak,
                                "unit": "TFLOP/s", "frac": round(tflops / cpeak, 4),
                                "algorithmic_flops_per_launch": fb,
                                "note": "bf16 products on the matrix cores (f32 operands as two bf16 parts)"
                                        if mfma else "products on f32 VALU FMA"},
           "fwd_flops": ff, "fwd_bytes": bf}
    if not no_cpu:
        res["cpu_baseline"] = m3_cpu_baseline(w, budget_s)
    print(json.dumps(res), flush=True)


def m3_cpu_baseline(w: workloads.M3Workload, budget_s: float):
    """The Mamba-3 oracle as it stands (numpy, float64), forward + backward,
    on one batch row of the same widths and a bounded number of steps, scaled
    to the workload's tokens (its cost per step does not depend on T)."""
    from oracle import mamba3 as m3o
    T = 16
    while True:
        sw = w.with_(batch=1, seqlen=T)
        inp = workloads.make_m3_inputs(sw, 0)
        args = {k: inp[k] for k in ("x", "b_in", "c_in", "dd_dt_raw", "dd_a_raw", "trap_raw", "angles_raw", "b_bias",
                                    "c_bias", "dt_bias", "D")}
        t0 = time.perf_counter()
        m3o.forward(a_floor=w.a_floor, heads=w.heads, headdim=w.headdim, **args)
        m3o.backward(inp["dy"], a_floor=w.a_floor, heads=w.heads, headdim=w.headdim, **args)
        dt = time.perf_counter() - t0
        if dt > 0.25 * budget_s or T >= w.seqlen:
            break
        T = min(w.seqlen, T * max(2, int(0.5 * budget_s / max(dt, 1e-3))))
    ncpu, model = host_info()
    return {"value": T / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle", "precision": "f64",
            "host_logical_cpus": ncpu, "cpu_model": model,
            "sample": "1 batch row x %d steps of the same widths (all %d heads), fwd+bwd in %.1f s on one thread"
                      % (T, w.heads, dt)}


def host_info():
    """Logical CPUs and CPU model of the host the baseline runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return os.cpu_count(), model


def cpu_baseline(w: workloads.Workload, L: int, budget_s: float):
    """The CPU oracle as it stands, in its single-precision build (the same
    source with float in place of double), threaded over channel ranges on
    the host's cores; timed on a bounded channel sample of the same workload
    (all batch rows and steps) and scaled to the full channel count."""
    import oracle
    oracle.build(force=False)
    threads = oracle.default_threads()
    chans = min(w.d_inner, 64 * threads)
    while True:
        sw = w.with_(d_inner=chans)
        inp = workloads.make_inputs(sw, 0)
        kw = dict(x=inp["x"], delta_raw=inp["delta_raw"], a_log=inp["a_log"], xdbl=inp["xdbl"], D=inp["D"],
                  z=inp.get("z"), threads=threads, precision="f32")
        if w.d_conv:
            kw.update(conv_w=inp["conv_w"], conv_b=inp["conv_b"])
        t0 = time.perf_counter()
        oracle.forward(chunk=L, **kw)
        oracle.backward(dout=inp["dout"], **kw)
        dt = time.perf_counter() - t0
        if dt > 0.25 * budget_s or chans >= w.d_inner:
            break
        chans = min(w.d_inner, chans * max(2, int(0.5 * budget_s / max(dt, 1e-3))))
    full_s = dt * (w.d_inner / chans) * w.layers
    tokens = w.batch * w.seqlen
    ncpu, model = host_info()
    return {"value": tokens / full_s, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "precision": "f32", "host_logical_cpus": ncpu, "cpu_model": model,
            "sample": "%d of %d channels, all %d batch rows x %d steps%s, fwd+bwd in %.1f s on %d threads; "
                      "scaled by %d/%d%s"
                      % (chans, w.d_inner, w.batch, w.seqlen, "" if w.layers == 1 else " (one layer)", dt, threads,
                         w.d_inner, chans, "" if w.layers == 1 else " x %d layers" % w.layers)}


def copy_bandwidth(torch, stream, mib: int = 1024, reps: int = 10):
    """HBM bandwidth of a plain device copy of `mib` MiB (read + write bytes
    over the event-timed copies)."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        b.copy_(a)
    e1.record(stream)
    torch.cuda.synchronize()
    gbps = 2 * n * 4 * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, b
    return gbps


# input sets rotated step by step, so that a step's inputs are not still in
# the 256 MB last-level cache (MALL) from the step before
INPUT_SETS = 3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="scan_2p8b_t8192_bf16", choices=sorted(workloads.CONFIGS))
    ap.add_argument("--chunk", type=int, default=16, help="checkpoint interval of the run")
    ap.add_argument("--segments", type=int, default=0,
                    help="sequence segments scanned in parallel (0: chosen by the library)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--layer", default=None, choices=sorted(workloads.LAYER_CONFIGS),
                    help="time one whole Mamba-1 layer at this shape and exit")
    ap.add_argument("--m3", default=None, choices=sorted(workloads.M3_CONFIGS),
                    help="time the Mamba-3 SISO core (include/mamba3.h), forward + backward per step")
    ap.add_argument("--recurrent", action="store_true",
                    help="time one-step forward calls with state in/out (see RECURRENT_SHAPES) and exit")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (HBM counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the kernel on one GPU's share); "
              "--gpus %d is not supported" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import state_space_sequence_selective_amd as pkg

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 5}))
        return

    torch.cuda.set_device(0)
    pkg.load()
    if args.recurrent:
        recurrent(torch, pkg, calls=max(args.steps, 200), warmup=max(args.warmup, 20))
        return
    if args.m3:
        m3_bench(torch, pkg, args.m3, args.steps, args.warmup, args.no_cpu_baseline, args.cpu_budget)
        return
    if args.layer:
        layer_bench(torch, pkg, args.layer, args.steps, args.warmup, args.no_cpu_baseline, args.cpu_budget)
        return

    stream = torch.cuda.current_stream()
    copy_gbps = copy_bandwidth(torch, stream)

    w = workloads.CONFIGS[args.workload]
    L = args.chunk
    nsets = INPUT_SETS if w.layers == 1 else 1   # many layers: each layer's inputs are its own already
    layers = []
    for l in range(w.layers):
        dims = pkg.Dims.make(w.batch, w.seqlen, w.d_inner, w.d_state, w.dt_rank, w.d_conv, L, w.act,
                             args.segments)
        sets = [device_inputs(torch, w, workloads.make_inputs(w, args.seed + l + 7919 * k)) for k in range(nsets)]
        layers.append((pkg.LayerCore(dims, gate=w.gate), sets))

    def step(k, evs=None):
        for core, _ in layers:
            core.zero_grads()
        for j, (core, sets) in enumerate(layers):
            if evs is not None and j == 0:
                evs[0].record(stream)
            core.forward(sets[k % nsets], stream=stream)
            if evs is not None and j == 0:
                evs[1].record(stream)
        for j, (core, sets) in reversed(list(enumerate(layers))):
            dev = sets[k % nsets]
            if evs is not None and j == 0:
                evs[2].record(stream)
            core.backward(dev, dev["dout"], stream=stream)
            if evs is not None and j == 0:
                evs[3].record(stream)

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record(stream)
    for k in range(args.steps):
        step(args.warmup + k, ev[k])
    end.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    ms_step = total_ms / args.steps
    fwd_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[2].elapsed_time(e[3]) for e in ev]))

    tokens = w.batch * w.seqlen
    value = tokens / (ms_step / 1e3)
    fb, bb = algorithmic_bytes(w)
    over = overhead_bytes(w, L)
    elems = w.batch * w.seqlen * w.d_inner * w.d_state
    step_bytes = (fb + bb) * w.layers
    hbm_gbps = step_bytes / (ms_step / 1e3) / 1e9
    # dominant launch: the backward entry point of one layer (its segment
    # carry pass and fold when segmented, scan_bwd_kernel, the fused entry's
    # conv adjoint and the fixed-order reduce),
    # event-timed on the stream its kernels run on
    bwd_gbps = bb / (bwd_ms / 1e3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(bwd_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(bwd_gbps / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(w.name, L),
                "kernel": ("mamba_conv_scan_gate_bwd" if w.d_conv else "mamba_scan_bwd")
                          + " entry point (scan_bwd_carry_kernel + mscan_carry_fold_kernel + scan_bwd_kernel + "
                          + ("conv_bwd_kernel + " if w.d_conv else "") + "mscan_reduce_kernel), layer 0",
                "launch_ms": round(bwd_ms, 4), "algorithmic_bytes_per_launch": bb,
                "overhead_bytes_per_launch": over["bwd"]}
    bwd_slots = elems * SLOTS_BWD_ELEM / (bwd_ms / 1e3)
    alu = {"bound": "alu", "achieved": round(bwd_slots / 1e12, 2), "peak": round(VALU_LANE_SLOTS_PER_S / 1e12, 2),
           "unit": "T lane-slots/s", "frac": round(bwd_slots / VALU_LANE_SLOTS_PER_S, 4),
           "slots_per_element": SLOTS_BWD_ELEM, "elements_per_launch": elems,
           "kernel": roofline["kernel"]}
    res = {
        "metric": "selective-scan fwd+bwd tokens/sec and achieved HBM GB/s (% of MI355X peak)",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.act,
        "data": "synthetic (seeded, distributions of the workload; %d input sets rotated)" % nsets,
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen, "d_inner": w.d_inner,
                   "d_state": w.d_state, "dt_rank": w.dt_rank, "d_conv": w.d_conv, "gate": w.gate,
                   "layers": w.layers, "chunk": L, "segments": args.segments or "auto",
                   "parallelism": "single GPU"},
        "hbm_GBps": round(hbm_gbps, 1),
        "hbm_frac_of_peak": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "copy_GBps": round(copy_gbps, 1),
        "hbm_frac_of_copy": round(hbm_gbps / copy_gbps, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "overhead_bytes_per_step": (over["fwd"] + over["bwd"]) * w.layers,
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        # the forward alone (one layer's, timed on layer 0): tokens/s and HBM
        # GB/s at its algorithmic bytes
        "fwd_tokens_per_s": round(tokens / (fwd_ms / 1e3), 1),
        "fwd_hbm_GBps": round(fb / (fwd_ms / 1e3) / 1e9, 1),
        "wall_s": round(t_wall, 3),
        "roofline": roofline,
        "alu_roofline": alu,
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, L, args.cpu_budget)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
