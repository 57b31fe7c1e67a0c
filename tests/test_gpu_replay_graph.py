"""HIP-graph capture of the hot path.  The core entry points only enqueue
kernels (no allocation, no memset, no synchronisation), so a whole training
step of the layer core (clear the accumulated gradients, forward, backward)
and a chain of recurrent decode steps can be captured once and replayed.
Every replay is compared bit for bit with the eager result, with eager
work (the outputs overwritten with NaN) and synchronisations between the
replays.  Inputs come from the seeded workload generator; the oracle is not
needed here (the eager path is pinned to it by test_gpu_parity.py)."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def mscan():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import state_space_sequence_selective_amd as m
    m.load()
    return m


def _device_inputs(w, inp):
    at = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act]
    dev = {}
    for k, v in inp.items():
        if v is None:
            continue
        dt = at if k in ("x", "delta_raw", "z", "dout", "xdbl", "d_u_extra") else torch.float32
        dev[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to("cuda", dt)
    return dev


def _replay_and_compare(graph, outputs: dict, ref: dict):
    for r in range(REPLAYS):
        for t in outputs.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for k, t in outputs.items():
            assert torch.equal(t, ref[k]), "replay %d: %s differs from the eager step" % (r, k)


def _capture(fn):
    """Warm up on a side stream (default priority), then capture fn."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("name,seg", [("scan_gate_bf16", 0), ("scan_gate_bf16", 3), ("fused_f16", 0)])
def test_training_step_replays(mscan, name, seg):
    """zero_grads + forward + backward of LayerCore, captured and replayed:
    the scan entry (unsplit and with 3 backward / forward segments, which
    adds the aggregate passes) and the fused conv entry."""
    if name == "fused_f16":
        w = workloads.Workload("graph_fused", 2, 150, 96, 16, 6, 4, "f16", True)
    else:
        w = workloads.Workload("graph_scan", 2, 300, 160, 16, 6, 0, "bf16", True)
    inp = workloads.make_inputs(w, 11)
    dev = _device_inputs(w, inp)
    dims = mscan.Dims.make(w.batch, w.seqlen, w.d_inner, w.d_state, w.dt_rank, w.d_conv, 16, w.act, seg)
    core = mscan.LayerCore(dims, gate=True)

    def step():
        core.zero_grads()
        core.forward(dev)
        core.backward(dev, dev["dout"])

    names = ["out", "y", "h_last", "ckpt", "d_x", "d_delta_raw", "d_z", "d_xdbl", "d_a_log", "d_D"]
    if w.d_conv:
        names += ["conv_state_last", "d_conv_w", "d_conv_b"]
    step()
    torch.cuda.synchronize()
    ref = {n: getattr(core, n).clone() for n in names}
    for n, t in ref.items():
        assert torch.isfinite(t.float()).all(), n
    g = _capture(step)
    _replay_and_compare(g, {n: getattr(core, n) for n in names}, ref)


def test_decode_chain_replays(mscan):
    """Eight one-step fused forward calls, each reading the previous call's
    SSM and conv state (decoding), captured as one graph."""
    from state_space_sequence_selective_amd import _lib
    B, Di, Ds, K, steps = 4, 256, 16, 4, 8
    w = workloads.Workload("graph_decode", B, steps, Di, Ds, 8, K, "bf16", True)
    inp = workloads.make_inputs(w, 12, h0=True, conv_state0=True)
    dev = _device_inputs(w, inp)
    per = [{k: dev[k][:, t:t + 1].contiguous() for k in ("x", "delta_raw", "z", "xdbl")} for t in range(steps)]
    dims = mscan.Dims.make(B, 1, Di, Ds, w.dt_rank, K, 16, "bf16")
    f32 = dict(device="cuda", dtype=torch.float32)
    h = [dev["h0"]] + [torch.empty((B, Di, Ds), **f32) for _ in range(steps)]
    cs = [dev["conv_state0"]] + [torch.empty((B, Di, K), **f32) for _ in range(steps)]
    outs = [torch.empty((B, 1, Di), device="cuda", dtype=torch.bfloat16) for _ in range(steps)]
    ws = torch.empty(_lib.workspace_bytes(dims), device="cuda", dtype=torch.uint8)

    def chain():
        for t in range(steps):
            _lib.conv_scan_gate_fwd(dims, per[t]["x"], dev["conv_w"], dev["conv_b"], cs[t], per[t]["delta_raw"],
                                    dev["a_log"], per[t]["xdbl"], dev["D"], per[t]["z"], h[t], out=outs[t],
                                    h_last=h[t + 1], conv_state_last=cs[t + 1], workspace=ws)

    chain()
    torch.cuda.synchronize()
    tensors = {"out%d" % t: outs[t] for t in range(steps)}
    tensors.update({"h%d" % (t + 1): h[t + 1] for t in range(steps)})
    tensors.update({"cs%d" % (t + 1): cs[t + 1] for t in range(steps)})
    ref = {k: v.clone() for k, v in tensors.items()}
    # the chain equals one 8-step call (the same step kernel, state kept in registers)
    core = mscan.LayerCore(mscan.Dims.make(B, steps, Di, Ds, w.dt_rank, K, 16, "bf16"), gate=True)
    core.forward(dev)
    torch.cuda.synchronize()
    assert torch.equal(torch.cat(outs, 1), core.out)
    assert torch.equal(h[steps], core.h_last)
    g = _capture(chain)
    _replay_and_compare(g, tensors, ref)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_layer_step_replays(mscan, act):
    """zero_grads + mamba_layer_fwd + mamba_layer_bwd captured as one graph:
    the library products, the weight-gradient products forked onto the
    second stream and joined back, the column sums and (bf16) the
    matrix-core projection and weight-gradient kernels.  1041 token rows, so
    the wide weight products take their K split with a 1-row tail."""
    w = workloads.LayerWorkload("graph_layer_" + act, 3, 347, 96, 192, 16, 8, 4, act)
    inp = workloads.make_layer_inputs(w, 13)
    at = {"f32": torch.float32, "bf16": torch.bfloat16}[act]
    weights = {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to("cuda", at if n in mscan.LAYER_TYPED else
                                                                      torch.float32) for n in mscan.LAYER_PARAMS}
    dims = mscan.LayerDims.make(w.batch, w.seqlen, w.d_model, w.d_inner, w.d_state, w.dt_rank, w.d_conv, 16, w.act)
    layer = mscan.MambaLayer(dims, weights)
    resid = torch.from_numpy(inp["resid"]).cuda()
    d_out = torch.from_numpy(inp["d_resid_out"]).cuda()

    def step():
        layer.zero_grads()
        layer.forward(resid)
        layer.backward(resid, d_out)

    step()
    torch.cuda.synchronize()
    outs = {"resid_out": layer.resid_out, "d_resid_in": layer.d_resid_in}
    outs.update({"d_" + k: v for k, v in layer.grads.items()})
    ref = {k: v.clone() for k, v in outs.items()}
    for k, t in ref.items():
        assert torch.isfinite(t).all(), k
    g = _capture(step)
    _replay_and_compare(g, outs, ref)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_m3_step_replays(mscan, act):
    """zero_grads + the Mamba-3 SISO forward and backward (the chunked
    passes, the angle scans, the fixed-order sums: about 25 kernels)
    captured as one graph.  137 steps, so the last 64-step chunk is ragged;
    two B/C groups of two heads."""
    w = workloads.M3Workload("graph_m3_" + act, 2, 137, 4, 64, 64, 2, 16, act)
    inp = workloads.make_m3_inputs(w, 21)
    at = {"f32": torch.float32, "bf16": torch.bfloat16}[act]
    dev = {k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda", at if k in ("x", "b_in", "c_in", "dy") else
                                                             torch.float32)
           for k, v in inp.items() if v is not None}
    dims = mscan.M3Dims.make(w.batch, w.seqlen, w.heads, w.headdim, w.d_state, w.groups, w.n_angles, w.act,
                             w.a_floor)
    core = mscan.Mamba3Core(dims)

    def step():
        core.zero_grads()
        core.forward(dev)
        core.backward(dev, dev["dy"])

    step()
    torch.cuda.synchronize()
    outs = {"y": core.y, "states": core.states}
    outs.update({"d_" + k: v for k, v in core.grads.items()})
    ref = {k: v.clone() for k, v in outs.items()}
    for k, t in ref.items():
        assert torch.isfinite(t).all(), k
    g = _capture(step)
    _replay_and_compare(g, outs, ref)
