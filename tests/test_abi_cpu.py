"""CPU-side checks of the C ABI: the library loads, exports every entry
point the header declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]


@pytest.fixture(scope="module")
def pkg():
    import state_space_sequence_selective_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libmamba_scan.so not built")
    m.load()
    return m


def declared_functions():
    src = "\n".join(open(h).read() for h in HEADERS)
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mamba3?_\w+)\s*\(", src)))


def test_header_declares_the_binding_entry_points(pkg):
    assert declared_functions() == sorted(pkg.EXPORTED)


def test_library_exports_every_declared_symbol(pkg):
    lib = ctypes.CDLL(pkg.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen("nm -D --defined-only %s" % pkg.LIB_PATH).read()
    for name in declared_functions():
        assert re.search(r"\bT %s\b" % name, out), name


def test_abi_version(pkg):
    assert pkg.abi_version() == 3


def _dims(pkg, **kw):
    base = dict(batch=2, seqlen=100, d_inner=64, d_state=16, dt_rank=0, d_conv=0, chunk=32, act="bf16")
    base.update(kw)
    return pkg.Dims.make(**base)


def test_sizes(pkg):
    d = _dims(pkg)
    assert pkg.ckpt_bytes(d) == 2 * 4 * 16 * 64 * 4            # ceil(100/32) = 4 checkpoints
    # per-group d_B|d_C partials (groups of 32 channels: 2) padded to 256 B,
    # then per-row param partials
    bc = 2 * 2 * 100 * 32 * 4
    assert pkg.workspace_bytes(d) == ((bc + 255) // 256) * 256 + 2 * 64 * 17 * 4
    # fused: the same, plus d_u (f32) for the conv adjoint pass and its weight
    # / bias partials per (batch row, 64-step tile)
    dc = _dims(pkg, d_conv=4, d_inner=128)
    al = lambda x: (x + 255) // 256 * 256
    bc = 4 * 2 * 100 * 32 * 4
    assert pkg.workspace_bytes(dc) == (al(bc) + al(2 * 128 * 17 * 4) + al(2 * 100 * 128 * 4)
                                       + al(2 * 2 * 128 * 5 * 4))


@pytest.mark.parametrize("kw,status,msg", [
    (dict(batch=0), 1, "batch"),
    (dict(batch=70000), 3, "batch"),
    (dict(seqlen=0), 1, "seqlen"),
    (dict(d_inner=66), 1, "d_inner"),
    (dict(d_inner=0), 1, "d_inner"),
    (dict(d_state=12), 2, "d_state"),
    (dict(d_state=128), 2, "d_state"),
    (dict(chunk=20), 2, "chunk"),
    (dict(chunk=8), 2, "chunk"),
    (dict(chunk=-16), 1, "chunk"),
    (dict(chunk=4096 + 16), 2, "chunk"),
    (dict(dt_rank=-1), 1, "dt_rank"),
    (dict(dt_rank=(1 << 24) + 1), 3, "dt_rank"),
    (dict(d_inner=(1 << 24) + 4), 3, "d_inner"),
    (dict(act=5), 1, "act"),
    (dict(seqlen=1 << 40), 3, "2^46"),
    # within the element cap, but the tiled launches would exceed 2^32 - 1 threads
    (dict(batch=65535, seqlen=1, d_inner=1 << 24), 3, "threads"),
    (dict(batch=4096, seqlen=1 << 16, d_inner=64), 3, "threads"),
])
def test_bad_dims_rejected(pkg, kw, status, msg):
    d = _dims(pkg, **kw)
    with pytest.raises(pkg.MambaScanError) as ei:
        pkg.ckpt_bytes(d)
    assert ei.value.status == status
    assert msg in str(ei.value) and "mamba_ckpt_bytes" in str(ei.value)


@pytest.mark.parametrize("segments", [-1, 4097])
def test_segments_range(pkg, segments):
    d = _dims(pkg, segments=segments)
    with pytest.raises(pkg.MambaScanError, match="segments") as ei:
        pkg.ckpt_bytes(d)
    assert ei.value.status == 1


def test_segmented_workspace_layout(pkg):
    # B=1, T=1024, Di=64, Ds=16, L=16: 64 checkpoint tiles, 64 forward tiles;
    # four segments each way.  The carry pass has 2 channel groups x 3 later
    # segments = 6 workgroups, so it halves each 256-step segment down to
    # 4 sub-segments of 64 steps (4 tiles, the least it cuts to): seg_q and
    # seg_sd hold 16 sub-segments, seg_c (the folded carry) 4 segments.
    d = _dims(pkg, batch=1, seqlen=1024, chunk=16, segments=4)
    al = lambda x: (x + 255) // 256 * 256
    fwd = al(1 * 4 * 64 * 16 * 4) + al(1 * 4 * 64 * 4)                  # seg_h | seg_sd
    bwd = (al(2 * 1 * 1024 * 32 * 4) + al(4 * 1 * 64 * 17 * 4)          # part_bc | part_par (4 segments)
           + al(1 * 16 * 64 * 16 * 4) + al(1 * 16 * 64 * 4)             # seg_q | seg_sd (16 sub-segments)
           + al(1 * 4 * 64 * 16 * 4))                                    # seg_c
    assert pkg.workspace_bytes(d) == max(fwd, bwd)
    # a cap above the tile count gives one segment per tile (too short to split)
    d = _dims(pkg, batch=1, seqlen=64, chunk=16, segments=4096)
    fwd = al(1 * 4 * 64 * 16 * 4) + al(1 * 4 * 64 * 4)
    bwd = (al(2 * 1 * 64 * 32 * 4) + al(4 * 1 * 64 * 17 * 4) + al(1 * 4 * 64 * 16 * 4) + al(1 * 4 * 64 * 4)
           + al(1 * 4 * 64 * 16 * 4))
    assert pkg.workspace_bytes(d) == max(fwd, bwd)
    # the fused backward segments like the scan one and adds d_u (f32) and
    # the conv partials per (batch row, 64-step tile)
    d = _dims(pkg, batch=1, seqlen=1024, chunk=16, segments=4, d_conv=4)
    bwd_fused = (al(2 * 1 * 1024 * 32 * 4) + al(4 * 1 * 64 * 17 * 4) + al(1 * 16 * 64 * 16 * 4)
                 + al(1 * 16 * 64 * 4) + al(1 * 4 * 64 * 16 * 4) + al(1 * 1024 * 64 * 4) + al(1 * 16 * 64 * 5 * 4))
    assert pkg.workspace_bytes(d) == bwd_fused


def _raw(pkg):
    return pkg.load()


def test_null_and_misaligned_pointers_rejected_before_launch(pkg):
    lib = _raw(pkg)
    d = _dims(pkg)
    P = ctypes.c_void_p
    good = P(0x10000)           # never dereferenced: the call fails before any launch
    # u NULL
    nows = (None, ctypes.c_size_t(0), None)   # workspace, its size, stream
    rc = lib.mamba_scan_fwd(ctypes.byref(d), None, good, good, good, None, None, None, good, None, None, None, *nows)
    assert rc == 1 and "mamba_scan_fwd: u is NULL" == pkg.last_error()
    # out misaligned (bf16 needs 2-byte alignment)
    rc = lib.mamba_scan_fwd(ctypes.byref(d), good, good, good, good, None, None, None, P(0x10001), None, None,
                            None, *nows)
    assert rc == 1 and "out is not 2-byte aligned" in pkg.last_error()
    # a_log misaligned (f32)
    rc = lib.mamba_scan_fwd(ctypes.byref(d), good, good, P(0x10002), good, None, None, None, good, None, None,
                            None, *nows)
    assert rc == 1 and "a_log" in pkg.last_error()
    # backward: z given but y_saved missing
    args = [ctypes.byref(d), good, good, good, good, None, good, None, good, good, good, good, good, good, good,
            good, good, ctypes.c_size_t(1 << 30), None]
    rc = lib.mamba_scan_bwd(*args)
    assert rc == 1 and "y_saved is NULL" in pkg.last_error()
    # backward: workspace too small
    args = [ctypes.byref(d), good, good, good, good, None, None, None, good, good, good, good, None, good, good,
            good, P(0x100000), ctypes.c_size_t(16), None]
    rc = lib.mamba_scan_bwd(*args)
    assert rc == 3 and "workspace_bytes" in pkg.last_error()
    # a segmented forward needs its workspace
    ds = _dims(pkg, batch=1, seqlen=1024, chunk=16, segments=4)
    rc = lib.mamba_scan_fwd(ctypes.byref(ds), good, good, good, good, None, None, None, good, None, None, None,
                            *nows)
    assert rc == 1 and "mamba_scan_fwd: workspace is NULL" == pkg.last_error()
    rc = lib.mamba_scan_fwd(ctypes.byref(ds), good, good, good, good, None, None, None, good, None, None, None,
                            P(0x100000), ctypes.c_size_t(256), None)
    assert rc == 3 and "workspace_bytes 256 < required" in pkg.last_error()
    # fused: d_conv out of range
    dc = _dims(pkg, d_conv=5)
    rc = lib.mamba_conv_scan_gate_fwd(ctypes.byref(dc), *([good] * 16), *nows)
    assert rc == 2 and "d_conv" in pkg.last_error()
    dc = _dims(pkg, d_conv=0)
    rc = lib.mamba_conv_scan_gate_bwd(ctypes.byref(dc), *([good] * 22), ctypes.c_size_t(1 << 30), None)
    assert rc == 1 and "mamba_conv_scan_gate_bwd: d_conv" in pkg.last_error()


def test_static_backward_rejects_dims_beyond_its_scratch(pkg):
    """mamba_scan_bwd_static refuses dims whose scratch exceeds its static
    array before it touches the device (no GPU here)."""
    lib = _raw(pkg)
    good = ctypes.c_void_p(0x10000)      # never dereferenced
    d = _dims(pkg, batch=2, seqlen=8192, d_inner=5120)
    assert pkg.workspace_bytes(d) > 64 << 20
    rc = lib.mamba_scan_bwd_static(ctypes.byref(d), *([good] * 5), None, None, good, good, good, good, None, good,
                                   good, good, None)
    assert rc == 3
    msg = pkg.last_error()
    assert msg.startswith("mamba_scan_bwd_static: these dims need") and str(64 << 20) in msg
    # argument checks as in mamba_scan_bwd
    small = _dims(pkg)
    rc = lib.mamba_scan_bwd_static(ctypes.byref(small), None, *([good] * 4), None, None, good, good, good, good,
                                   None, good, good, good, None)
    assert rc == 1 and pkg.last_error() == "mamba_scan_bwd_static: u is NULL"


def test_last_error_is_per_thread(pkg):
    """mamba_last_error() is thread-local: two threads whose calls fail for
    different reasons, interleaved, each read back their own message (the
    library drops the interpreter lock during a call, so they do overlap)."""
    import threading
    lib = _raw(pkg)
    good = ctypes.c_void_p(0x10000)      # never dereferenced: the calls fail before any launch
    d = _dims(pkg)
    bad = _dims(pkg, segments=-1)
    wrong = []

    def worker(kind):
        size = ctypes.c_size_t(0)
        for _ in range(3000):
            if kind == 0:
                rc = lib.mamba_scan_fwd(ctypes.byref(d), None, good, good, good, None, None, None, good, None, None,
                                        None, None, ctypes.c_size_t(0), None)
                msg = pkg.last_error()
                ok = rc == 1 and msg == "mamba_scan_fwd: u is NULL"
            else:
                rc = lib.mamba_workspace_bytes(ctypes.byref(bad), ctypes.byref(size))
                msg = pkg.last_error()
                ok = rc == 1 and msg.startswith("mamba_workspace_bytes: dims.segments")
            if not ok:
                wrong.append((kind, rc, msg))

    threads = [threading.Thread(target=worker, args=(k,)) for k in (0, 1, 0, 1)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not wrong, wrong[:3]


def test_binding_rejects_host_tensors(pkg):
    torch = pytest.importorskip("torch")
    d = _dims(pkg, batch=1, seqlen=4)
    t = torch.zeros(1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor"):
        pkg.scan_fwd(d, t, t, torch.zeros(64, 16), torch.zeros(1, 4, 32, dtype=torch.bfloat16), out=t)


def test_product_does_not_touch_the_oracle():
    """The product package never imports the oracle or the input generator."""
    pkgdir = os.path.join(ROOT, "state_space_sequence_selective_amd")
    for dirpath, _, files in os.walk(pkgdir):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower() or f == "__init__.py" and "oracle" not in src, f
                assert "import workloads" not in src and "from workloads" not in src, f


def _ldims(pkg, **kw):
    base = dict(batch=2, seqlen=100, d_model=48, d_inner=64, d_state=16, dt_rank=4, d_conv=4, chunk=16, act="bf16")
    base.update(kw)
    return pkg.LayerDims.make(**base)


@pytest.mark.parametrize("kw,status,msg", [
    (dict(d_model=0), 1, "d_model"),
    (dict(d_model=(1 << 24) + 1), 3, "d_model"),
    (dict(d_conv=0), 1, "d_conv"),
    (dict(dt_rank=0), 1, "dt_rank"),
    (dict(d_state=12), 2, "core dims: mamba_ckpt_bytes: d_state"),
    (dict(batch=0), 1, "core dims"),
])
def test_layer_bad_dims_rejected(pkg, kw, status, msg):
    with pytest.raises(pkg.MambaScanError) as ei:
        pkg.layer_saved_bytes(_ldims(pkg, **kw))
    assert ei.value.status == status
    assert msg in str(ei.value) and "mamba_layer_saved_bytes" in str(ei.value)


def test_layer_buffer_sizes(pkg):
    """The saved buffer holds the typed activations the backward reads (plus
    RMSNorm statistics and the core checkpoints); the workspace is at least
    the backward's temporaries."""
    ld = _ldims(pkg)
    N, dm, Di, X = 200, 48, 64, 4 + 32
    saved = pkg.layer_saved_bytes(ld)
    typed = 2 * (N * dm + N * X + 6 * N * Di)
    assert typed + N * 4 + pkg.ckpt_bytes(ld.core) <= saved <= typed + N * 4 + pkg.ckpt_bytes(ld.core) + 11 * 256
    ws = pkg.layer_workspace_bytes(ld)
    assert ws >= 2 * N * dm + 4 * N * dm + 4 * 2 * N * Di + 4 * N * X
    # f32 activations double the typed parts
    assert pkg.layer_saved_bytes(_ldims(pkg, act="f32")) > 1.9 * typed
