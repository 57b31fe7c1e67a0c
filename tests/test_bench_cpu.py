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
    """B=2, T=8192, d_inner 5120, d_state 16, bf16, gate, no conv, L = 16,
    listed tensor by tensor."""
    w = workloads.CONFIGS["scan_2p8b_t8192_bf16"]
    tok = 2 * 8192                      # token rows
    act = tok * 5120 * 2                # one [B, T, d_inner] bf16 tensor
    bc_rows = tok * 32 * 2              # B and C columns, bf16
    ckpt = 2 * (8192 // 16) * 16 * 5120 * 4
    # The model counts what the method must move.  The y the forward saves
    # for d_z is not in it (the backward could form it again from the states
    # it recomputes), so neither its write nor its read is counted.
    fwd = 3 * act + act + bc_rows + ckpt                   # u, delta_raw, z in; out; B/C in; ckpt written
    bwd = (4 * act                                          # u, delta_raw, z, dout in
           + 3 * act                                        # d_u, d_delta_raw, d_z out
           + bc_rows + tok * 32 * 4 + ckpt)                 # B/C in, d_B/d_C f32 out, ckpt read
    assert bench.algorithmic_bytes(w, 16) == (fwd, bwd)
    assert bwd == 1513095168


def test_algorithmic_flops_and_layer_flops():
    w = workloads.CONFIGS["scan_2p8b_t8192_bf16"]
    elems = 2 * 8192 * 5120 * 16
    assert bench.FLOPS_BWD_ELEM * elems == 28185722880
    # 130M layer widths: B=4, T=2048, d_model 768, d_inner 1536, dt_rank 48,
    # d_state 16 (xdbl row 80): in_proj, x_proj, dt_proj, out_proj, each
    # run forward, for the input gradient and for the weight gradient
    lw = workloads.LAYER_CONFIGS["layer_130m_bf16"]
    N = 4 * 2048
    macs = N * 768 * 3072 + N * 1536 * 80 + N * 48 * 1536 + N * 1536 * 768
    assert bench.layer_flops(lw) == 3 * 2 * macs == 183609851904
    assert w.d_state == 16


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
    assert h0 == json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))["scan_2p8b_t8192_bf16"][
        "kernel_src_sha256"], "the committed HBM counters were taken on other backward sources"
    # the forward's and the layer's sources are not part of it
    for name in ("scan_fwd.h", "scan_step.h", "inst_fwd_bf16.hip", "layer_kernels.hip"):
        with open(csrc / name, "a") as f:
            f.write("\n// edited\n")
        assert bench.kernel_source_hash() == h0, name
    # the backward's are
    with open(csrc / "scan_bwd.h", "a") as f:
        f.write("\n// edited\n")
    assert bench.kernel_source_hash() != h0


def test_measured_traffic_is_none_for_other_sources(tree):
    wl = "scan_2p8b_t8192_bf16"
    rec = {wl: {"kernel_src_sha256": bench.kernel_source_hash(), "bwd_entry_bytes": 123}}
    path = tree / "profiles" / "traffic.json"
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(wl) == 123
    assert bench.measured_traffic("scan_130m_bf16") is None
    rec[wl]["kernel_src_sha256"] = "0" * 64
    path.write_text(json.dumps(rec))
    assert bench.measured_traffic(wl) is None
    path.unlink()
    assert bench.measured_traffic(wl) is None
