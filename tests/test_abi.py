"""C-ABI checks that run without a GPU: the library loads, exports exactly what the
header declares, sizes its workspace, and rejects bad arguments before touching the
device."""
import ctypes
import os
import re
import subprocess

import pytest

from draft_block_verification_spec_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b((?:sv|spec)_\w+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(b.LIB_PATH):
        from draft_block_verification_spec_amd import build
        build.build()
    return b.load()


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("spec_verify_greedy", "spec_verify_sample", "spec_verify_scheduled", "sv_workspace_bytes"):
        assert n in names
    assert set(names) == set(b.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for n in _declared():
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", b.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert set(_declared()) <= exported
    # nothing else of ours leaks out of the shared object
    ours = {s for s in exported if s.startswith(("sv_", "spec_", "_ZN2sv"))}
    assert ours == set(_declared())


def test_version_and_strerror(lib):
    assert b"gfx950" in lib.sv_version()
    assert lib.sv_strerror(b.SV_EINVAL) == b"invalid argument"
    assert lib.sv_strerror(b.SV_EWORKSPACE) == b"workspace too small"


def _w(d=4096, d_ff=12288, V=151936, mlp=True):
    z = 1 << 20
    return b.SvWeights(z if mlp else None, 2 * z if mlp else None, 3 * z if mlp else None, 4 * z, d, d_ff if mlp else 0, V)


def test_workspace_sizes(lib):
    w = _w()
    g = lib.sv_workspace_bytes(b.SV_MODE_GREEDY, 1, 15, ctypes.byref(w))
    s = lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(w))
    sch = lib.sv_workspace_bytes(b.SV_MODE_SCHEDULED, 64, 15, ctypes.byref(w))
    p = lib.sv_workspace_bytes(b.SV_MODE_PROPOSE, 15, 0, ctypes.byref(w))
    assert 0 < g < s                       # sampled mode keeps fp32 logits of 31 rows
    assert s >= 31 * 151936 * 4
    assert sch >= 64 * 15 * 151936 * 4     # scheduled mode keeps every draft row's logits
    assert p >= 15 * 151936 * 4
    assert all(x % 256 == 0 for x in (g, s, sch, p))
    # larger batches never need less
    assert lib.sv_workspace_bytes(b.SV_MODE_GREEDY, 128, 7, ctypes.byref(w)) > g


@pytest.mark.parametrize("bad", [
    dict(d=100), dict(d=0), dict(d_ff=100), dict(V=0), dict(V=(1 << 19) + 1), dict(mlp=False, d_ff=12288),
])
def test_workspace_rejects_bad_shapes(lib, bad):
    kw = dict(d=4096, d_ff=12288, V=151936, mlp=True)
    kw.update(bad)
    if "mlp" in bad and not bad["mlp"]:
        w = b.SvWeights(None, None, None, 1 << 20, kw["d"], kw["d_ff"], kw["V"])
    else:
        w = _w(kw["d"], kw["d_ff"], kw["V"], kw["mlp"])
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 4, ctypes.byref(w)) == 0
    assert lib.sv_workspace_bytes(7, 1, 4, ctypes.byref(_w())) == 0
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 0, 4, ctypes.byref(_w())) == 0


def _outs():
    z = 1 << 24
    return b.SvOutputs(z, z + 4096, None, z + 8192, None, None, None, None, None)


def test_entry_points_reject_invalid_arguments(lib):
    w, o = _w(), _outs()
    P = 1 << 28
    ws, wsn = 1 << 30, 1 << 40
    # NULL hidden states / outputs / weights
    assert lib.spec_verify_greedy(ctypes.byref(w), None, P, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(None, P, P, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 1, 4, ws, wsn, None, None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(ctypes.byref(w), P, None, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    # misaligned hidden pointer, bad batch
    assert lib.spec_verify_greedy(ctypes.byref(w), P + 2, P, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 0, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 1, -1, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    # temperature must be positive and finite in sampled mode
    for T in (0.0, -1.0, float("inf"), float("nan")):
        assert lib.spec_verify_sample(ctypes.byref(w), P, P, P, P, T, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_sample(ctypes.byref(w), P, P, P, None, 1.0, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_sample(ctypes.byref(w), P, None, P, P, 1.0, 1, 4, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    # scheduled: budget below B, threshold outside (0, 1]
    assert lib.spec_verify_scheduled(ctypes.byref(w), P, P, P, P, 1.0, 0.3, 3, 4, 15, ws, wsn, ctypes.byref(o),
                                     None) == b.SV_EINVAL
    for thr in (0.0, 1.5, float("nan")):
        assert lib.spec_verify_scheduled(ctypes.byref(w), P, P, P, P, 1.0, thr, 64, 4, 15, ws, wsn, ctypes.byref(o),
                                         None) == b.SV_EINVAL
    # K beyond SV_MAX_K = 8190 (the acceptance kernels' LDS), sampled, greedy and scheduled
    assert lib.spec_verify_sample(ctypes.byref(w), P, P, P, P, 1.0, 1, 8191, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 1, 8191, ws, wsn, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_scheduled(ctypes.byref(w), P, P, P, P, 1.0, 0.3, 16, 1, 8192, ws, wsn, ctypes.byref(o),
                                     None) == b.SV_EINVAL
    # scheduled: more than 8192 requests, or more than 8192 draft positions
    for B, K in ((8193, 0), (8193, 1), (4097, 2)):
        assert lib.spec_verify_scheduled(ctypes.byref(w), P, P, P, P, 1.0, 0.3, 16384, B, K, ws, wsn,
                                         ctypes.byref(o), None) == b.SV_EINVAL
    # required outputs
    o2 = b.SvOutputs(None, 1 << 24, None, 1 << 24, None, None, None, None, None)
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 1, 4, ws, wsn, ctypes.byref(o2), None) == b.SV_EINVAL
    # propose
    assert lib.spec_draft_propose(ctypes.byref(w), P, None, 1.0, 4, ws, wsn, P, None, None) == b.SV_EINVAL
    assert lib.spec_draft_propose(ctypes.byref(w), P, P, -1.0, 4, ws, wsn, P, None, None) == b.SV_EINVAL
    assert lib.spec_draft_propose(ctypes.byref(w), P, P, 1.0, 0, ws, wsn, P, None, None) == b.SV_EINVAL


def test_entry_points_reject_small_workspace(lib):
    w, o = _w(), _outs()
    P = 1 << 28
    need = lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(w))
    assert lib.spec_verify_sample(ctypes.byref(w), P, P, P, P, 1.0, 1, 15, 1 << 30, need - 256, ctypes.byref(o),
                                  None) == b.SV_EWORKSPACE
    need = lib.sv_workspace_bytes(b.SV_MODE_GREEDY, 2, 7, ctypes.byref(w))
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 2, 7, 1 << 30, need - 1, ctypes.byref(o), None) == b.SV_EWORKSPACE
    need = lib.sv_workspace_bytes(b.SV_MODE_PROPOSE, 15, 0, ctypes.byref(w))
    assert lib.spec_draft_propose(ctypes.byref(w), P, P, 1.0, 15, 1 << 30, need - 1, P, None, None) == b.SV_EWORKSPACE
    # misaligned workspace
    assert lib.spec_verify_greedy(ctypes.byref(w), P, P, 2, 7, (1 << 30) + 16, 1 << 40, ctypes.byref(o),
                                  None) == b.SV_EINVAL


def _w8(**kw):
    w = _w(**{k: v for k, v in kw.items() if k in ("d", "d_ff", "V", "mlp")})
    w.wtype = b.SV_WEIGHTS_FP8_E4M3
    z = 1 << 22
    w.s_lm = 5 * z
    if w.d_ff:
        w.s_gate, w.s_up, w.s_down = 6 * z, 7 * z, 8 * z
    for k, v in kw.items():
        if k.startswith("s_") or k == "wtype":
            setattr(w, k, v)
    return w


def test_fp8_weights_workspace_rules(lib):
    # one 16-token block streams every product: supported
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(_w8())) > 0
    assert lib.sv_workspace_bytes(b.SV_MODE_GREEDY, 1, 15, ctypes.byref(_w8())) > 0
    assert lib.sv_workspace_bytes(b.SV_MODE_PROPOSE, 15, 0, ctypes.byref(_w8())) > 0
    # batches past the streaming kernel's rows, missing scales, unknown weight types: rejected
    assert lib.sv_workspace_bytes(b.SV_MODE_GREEDY, 8, 7, ctypes.byref(_w8())) == 0
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(_w8(s_lm=None))) == 0
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(_w8(s_down=None))) == 0
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(_w8(wtype=7))) == 0
    # without an MLP only the LM-head scales are needed
    assert lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(_w8(mlp=False, d_ff=0))) > 0


def _cache(**kw):
    z = 1 << 20
    c = b.SvCache(kv=z, layer_stride=1 << 24, half_stride=1 << 23, n_layers=4, block_size=16, entry_bytes=2048,
                  max_blocks=64, n_blocks=1024, block_table=2 * z, seq_len=3 * z, rec_state=4 * z, rec_snap=5 * z,
                  rec_bytes=1 << 16)
    for k, v in kw.items():
        setattr(c, k, v)
    return c


@pytest.mark.parametrize("bad", [
    dict(seq_len=None), dict(entry_bytes=24), dict(entry_bytes=0), dict(block_size=0), dict(kv=(1 << 20) + 8),
    dict(block_table=None), dict(n_blocks=0), dict(layer_stride=(1 << 24) + 4), dict(rec_bytes=100),
    dict(rec_snap=None), dict(rec_state=(1 << 22) + 4), dict(n_layers=-1),
])
def test_commit_rejects_bad_cache(lib, bad):
    c = _cache(**bad)
    acc = 6 << 20
    assert lib.spec_commit(ctypes.byref(c), acc, None, None, 8, 15, None, None) == b.SV_EINVAL


@pytest.mark.parametrize("B,Kmax,acc", [(0, 15, 6 << 20), (8, -1, 6 << 20), (8, 64, 6 << 20), (8, 15, None)])
def test_commit_rejects_bad_sizes(lib, B, Kmax, acc):
    c = _cache()
    assert lib.spec_commit(ctypes.byref(c), acc, None, None, B, Kmax, None, None) == b.SV_EINVAL
    assert lib.spec_commit(None, 6 << 20, None, None, 8, 15, None, None) == b.SV_EINVAL


def test_noalloc_entry_rejects_before_touching_the_device(lib):
    """The allocation-free sampled call refuses sizes beyond its static scratch (and bad
    arguments) before any device call, so this runs without a GPU."""
    w, o = _w(), _outs()
    P = 1 << 28
    assert lib.sv_strerror(b.SV_ESCRATCH).startswith(b"sizes need more workspace")
    need = lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 1, 15, ctypes.byref(w))
    assert 0 < need <= b.SV_STATIC_SCRATCH_BYTES  # one 16-token block fits
    big = lib.sv_workspace_bytes(b.SV_MODE_SAMPLE, 8, 7, ctypes.byref(w))
    assert big > b.SV_STATIC_SCRATCH_BYTES
    assert lib.spec_verify_sample_noalloc(ctypes.byref(w), P, P, P, P, 1.0, 8, 7, ctypes.byref(o), None) == b.SV_ESCRATCH
    assert lib.spec_verify_sample_noalloc(ctypes.byref(w), P, P, P, P, 0.0, 1, 15, ctypes.byref(o), None) == b.SV_EINVAL
    assert lib.spec_verify_sample_noalloc(ctypes.byref(w), None, P, P, P, 1.0, 1, 15, ctypes.byref(o),
                                          None) == b.SV_EINVAL


def test_peak_probe_library_exports_its_header():
    from draft_block_verification_spec_amd import peaks
    if not os.path.exists(peaks.LIB_PATH):
        from draft_block_verification_spec_amd import build
        build.build()
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "sv_peaks.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(sv_probe_\w+)\s*\(", src))
    assert declared == set(peaks.EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", peaks.LIB_PATH], capture_output=True, text=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    assert {s for s in exported if s.startswith("sv_")} == declared
    lib = peaks.load()
    ms = ctypes.c_float()
    assert lib.sv_probe_read(None, 1 << 20, 1 << 24, None, ctypes.byref(ms)) == -1  # rejected before any launch
    assert lib.sv_probe_read(1 << 28, 100, 1 << 24, None, ctypes.byref(ms)) == -1
