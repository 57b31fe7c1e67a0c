"""mamba_scan_bwd_static (scratch in a static device array, no workspace
argument, nothing allocated) against mamba_scan_bwd (caller's workspace) on
the same inputs and forward state.  Both run the same kernels on the same
partial-sum layout, so every output must agree bit for bit.  Two calls in a
row on one GPU, the second with a smaller input (other d_state, width and
length), so the second reads scratch the first left behind."""
import numpy as np
import pytest

import workloads

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mscan():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import state_space_sequence_selective_amd as m
    m.load()
    return m


def _dev(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda", dtype)


def _compare_static_with_workspace(m, w, seed, segments):
    at = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.act]
    inp = workloads.make_inputs(w, seed, h0=True)
    dev = {k: _dev(inp[k], at) for k in ("x", "delta_raw", "z", "dout", "xdbl")}
    for k in ("a_log", "D", "h0"):
        dev[k] = _dev(inp[k], torch.float32)
    dims = m.Dims.make(w.batch, w.seqlen, w.d_inner, w.d_state, w.dt_rank, 0, 16, w.act, segments)
    assert m.workspace_bytes(dims) <= 64 << 20
    core = m.LayerCore(dims, gate=True)
    core.forward(dev)
    core.zero_grads()
    core.backward(dev, dev["dout"])
    ref = {k: getattr(core, k).clone() for k in ("d_x", "d_delta_raw", "d_z", "d_xdbl", "d_a_log", "d_D")}
    out = {k: torch.full_like(v, float("nan")) for k, v in ref.items()}
    for k in ("d_xdbl", "d_a_log", "d_D"):   # accumulated outputs start from zero
        out[k].zero_()
    print("static backward", w, "segments", segments, flush=True)
    m.scan_bwd_static(dims, dev["x"], dev["delta_raw"], dev["a_log"], dev["xdbl"], dev["D"], dev["z"], core.y,
                      core.ckpt, dev["dout"], d_u=out["d_x"], d_delta_raw=out["d_delta_raw"], d_z=out["d_z"],
                      d_xdbl=out["d_xdbl"], d_a_log=out["d_a_log"], d_D=out["d_D"])
    torch.cuda.synchronize()
    for k in ref:
        assert torch.equal(out[k], ref[k]), k


def test_static_backward_equals_workspace_backward_twice(mscan):
    big = workloads.Workload("static_big", 2, 1000, 512, 16, 3, 0, "bf16", True)
    small = workloads.Workload("static_small", 1, 300, 100, 8, 0, 0, "f16", True)
    _compare_static_with_workspace(mscan, big, 41, 0)
    _compare_static_with_workspace(mscan, small, 42, 3)


def test_static_backward_rejects_oversized_dims(mscan):
    """Dims whose scratch exceeds the static array fail with
    MAMBA_ERR_CAPACITY before anything is enqueued."""
    import ctypes
    d = mscan.Dims.make(2, 8192, 5120, 16, 0, 0, 16, "bf16")
    assert mscan.workspace_bytes(d) > 64 << 20
    p = torch.empty(64, device="cuda").data_ptr()
    rc = mscan.load().mamba_scan_bwd_static(ctypes.byref(d), p, p, p, p, p, None, None, p, p, p, p, None, p, p, p,
                                            None)
    assert rc == 3 and "static array" in mscan.last_error()
