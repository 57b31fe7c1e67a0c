"""Host logic of bench.py (no GPU): the one-GPU refusal, the algorithmic
byte and flop counts the roofline divides by, and the guard that keeps
stored HBM counters from being reported for kernels that changed since."""
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_t8192():
    """B=2, T=8192, d_inner 5120, d_state 16, bf16, gate, no conv, listed
    tensor by tensor, checkpoints at the model's 64-step interval whatever
    interval a run uses."""
    w = workloads.CONFIGS["scan_2p8b_t8192_bf16"]
    tok = 2 * 8192                      # token rows
    act = tok * 5120 * 2                # one [B, T, d_inner] bf16 tensor
    bc_rows = tok * 32 * 2              # B and C columns, bf16
    ckpt = 2 * (8192 // 64) * 16 * 5120 * 4
    # The model counts what the method must move.  The y the forward saves
    # for d_z is not in it (the backward could form it again from the states
    # it recomputes), so neither its write nor its read is counted.
    fwd = 3 * act + act + bc_rows + ckpt                   # u, delta_raw, z in; out; B/C in; ckpt written
    bwd = (4 * act                                          # u, delta_raw, z, dout in
           + 3 * act                                        # d_u, d_delta_raw, d_z out
           + bc_rows + tok * 32 * 4 + ckpt)                 # B/C in, d_B/d_C f32 out, ckpt read
    assert bench.algorithmic_bytes(w) == (fwd, bwd)
    assert bwd == 1261436928 and fwd + bwd == 2017460224
    # a run at L = 16 moves four times the checkpoint bytes, and the saved y
    over = bench.overhead_bytes(w, 16)
    assert over["extra_ckpt_each_way"] == 3 * ckpt and over["y_saved_each_way"] == act
    assert over["bwd"] == 3 * ckpt + act


def test_algorithmic_bytes_other_workloads():
    """The 130M shape (B=4, T=2048, d_inner 1536) and one fused f16 layer of
    the 24-layer workload (B=8, T=4096, d_inner 2048; the conv adds no
    activation tensor)."""
    f, b = bench.algorithmic_bytes(workloads.CONFIGS["scan_130m_bf16"])
    assert f + b == 304087040
    f, b = bench.algorithmic_bytes(workloads.CONFIGS["fused_24l_f16"])
    assert f == 538968064 + 67108864 and b == 945815552 + 67108864


def test_alu_slots_and_layer_flops():
    elems = 2 * 8192 * 5120 * 16
    assert bench.SLOTS_BWD_ELEM * elems == 21474836480
    assert bench.VALU_LANE_SLOTS_PER_S == pytest.approx(39.32e12, rel=1e-3)
    # 130M layer widths: B=4, T=2048, d_model 768, d_inner 1536, dt_rank 48,
    # d_state 16 (xdbl row 80): in_proj, x_proj, dt_proj, out_proj, each
    # run forward, for the input gradient and for the weight gradient
    lw = workloads.LAYER_CONFIGS["layer_130m_bf16"]
    N = 4 * 2048
    macs = N * 768 * 3072 + N * 1536 * 80 + N * 48 * 1536 + N * 1536 * 768
    assert bench.layer_flops(lw) == 3 * 2 * macs == 183609851904


@pytest.fixture
def tree(tmp_path, monkeypatch):
    """A copy of the kernel sources and profiles that bench.py is pointed at."""
    src = os.path.join(ROOT, "state_space_sequence_selective_amd", "csrc")
    dst = tmp_path / "state_space_sequence_selective_amd" / "csrc"
    shutil.copytree(src, dst)
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    return tmp_path


def test_traffic_guard_follows_the_backward_sources(tree):
    csrc = tree / "state_space_sequence_selective_amd" / "csrc"
    h0 = bench.kernel_source_hash()
    # the forward's, the layer's and the Mamba-3 core's sources are not part of it
    for name in ("scan_fwd.h", "scan_step.h", "inst_fwd_bf16.hip", "layer_kernels.hip", "m3.hip"):
        with open(csrc / name, "a") as f:
            f.write("\n// edited\n")
        assert bench.kernel_source_hash() == h0, name
    # the backward's are
    with open(csrc / "scan_bwd.h", "a") as f:
        f.write("\n// edited\n")
    assert bench.kernel_source_hash() != h0


def test_measured_traffic_is_none_for_other_sources(tree):
    wl = "scan_2p8b_t8192_bf16"
    rec = {wl: {"kernel_src_sha256": bench.kernel_source_hash(), "bwd_entry_bytes": 123, "chunk": 16}}
    path = tree / "profiles" / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(wl, 16) == 123
    assert bench.measured_traffic(wl, 64) is None          # counters of another launch configuration
    assert bench.measured_traffic("scan_130m_bf16", 16) is None
    rec[wl]["kernel_src_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(wl, 16) is None
    path.unlink()
    assert bench.measured_traffic(wl, 16) is None


def test_m3_flops_and_bytes():
    """The Mamba-3 core's counts, by hand for the measured shape (B=4,
    T=2048, 24 heads of 64, d_state 128, one group, 32 angles, bf16):
    3072 chunk-heads; per chunk 2*64*(2*64*128 + 64*128 + 64*64) forward and
    2*64*(4*64*128 + 3*64*128 + 2*64*64) backward flops."""
    w = workloads.M3_CONFIGS["m3_siso_bf16"]
    f, b = bench.m3_flops(w)
    assert f == 3072 * 2 * 64 * (2 * 64 * 128 + 64 * 128 + 64 * 64)
    assert b == 3072 * 2 * 64 * (4 * 64 * 128 + 3 * 64 * 128 + 2 * 64 * 64)
    x = 4 * 2048 * 1536 * 2
    bc = 2 * 4 * 2048 * 128 * 2
    scal = 3 * 4 * 2048 * 24 * 4 + 4 * 2048 * 32 * 4
    par = (2 * 24 * 128 + 2 * 24) * 4
    states = 4 * 24 * 32 * 64 * 128 * 4
    fb, bb = bench.m3_bytes(w)
    assert fb == 2 * x + bc + scal + par + states
    assert bb == 3 * x + 2 * (bc + scal + par) + states
