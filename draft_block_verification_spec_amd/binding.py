"""ctypes binding of libspecverify (include/spec_verify.h).

Argument marshalling only: every step of the verification runs in the HIP
kernels of the shared library.  PyTorch supplies device memory and the stream.
The functions carry the C names; each checks dtypes/devices, allocates the
outputs and workspace it is not given, and raises ``SpecVerifyError`` on a
non-zero return code.  There is no fallback: without the built library every
call fails.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libspecverify.so")

SV_OK, SV_EINVAL, SV_EWORKSPACE, SV_EHIP, SV_ESCRATCH = 0, -1, -2, -3, -4
SV_MAX_K = 8190  # largest K (Kmax) of a greedy, sampled or scheduled call
SV_STATIC_SCRATCH_BYTES = 32 << 20
SV_DEV_OK, SV_DEV_BAD_TOKEN, SV_DEV_NONFINITE, SV_DEV_BAD_COMMIT, SV_DEV_BAD_TREE, SV_DEV_TIMEOUT = 0, 1, 2, 3, 4, 5
SV_MODE_GREEDY, SV_MODE_SAMPLE, SV_MODE_SCHEDULED, SV_MODE_PROPOSE = 0, 1, 2, 3
SV_DIAG_COLS = 8

EXPORTS = ("sv_workspace_bytes", "spec_verify_greedy", "spec_verify_sample", "spec_verify_sample_noalloc",
           "spec_verify_scheduled",
           "spec_draft_propose", "spec_verify_tree", "spec_commit", "sv_version", "sv_strerror",
           "sv_last_hip_error")


class SpecVerifyError(RuntimeError):
    pass


SV_WEIGHTS_BF16, SV_WEIGHTS_FP8_E4M3 = 0, 1


class SvWeights(ctypes.Structure):
    _fields_ = [("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
                ("w_lm", ctypes.c_void_p), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("V", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("s_down", ctypes.c_void_p), ("s_lm", ctypes.c_void_p)]


class SvOutputs(ctypes.Structure):
    _fields_ = [("accepted_len", ctypes.c_void_p), ("emitted", ctypes.c_void_p), ("verify_len", ctypes.c_void_p),
                ("tau", ctypes.c_void_p), ("counters", ctypes.c_void_p), ("dev_status", ctypes.c_void_p),
                ("diag", ctypes.c_void_p), ("logits", ctypes.c_void_p), ("hidden", ctypes.c_void_p),
                ("ev_lm_begin", ctypes.c_void_p), ("ev_lm_end", ctypes.c_void_p)]


class SvCache(ctypes.Structure):
    _fields_ = [("kv", ctypes.c_void_p), ("layer_stride", ctypes.c_int64), ("half_stride", ctypes.c_int64),
                ("n_layers", ctypes.c_int32), ("block_size", ctypes.c_int32), ("entry_bytes", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("n_blocks", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("seq_len", ctypes.c_void_p), ("rec_state", ctypes.c_void_p), ("rec_snap", ctypes.c_void_p),
                ("rec_bytes", ctypes.c_int64)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise SpecVerifyError(f"{p} not found: build it with `python -m draft_block_verification_spec_amd.build`")
    lib = ctypes.CDLL(p)
    vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.sv_workspace_bytes.restype = sz
    lib.sv_workspace_bytes.argtypes = [i32, i32, i32, ctypes.POINTER(SvWeights)]
    lib.spec_verify_greedy.restype = i32
    lib.spec_verify_greedy.argtypes = [ctypes.POINTER(SvWeights), vp, vp, i32, i32, vp, sz,
                                       ctypes.POINTER(SvOutputs), vp]
    lib.spec_verify_sample.restype = i32
    lib.spec_verify_sample.argtypes = [ctypes.POINTER(SvWeights), vp, vp, vp, vp, f32, i32, i32, vp, sz,
                                       ctypes.POINTER(SvOutputs), vp]
    lib.spec_verify_sample_noalloc.restype = i32
    lib.spec_verify_sample_noalloc.argtypes = [ctypes.POINTER(SvWeights), vp, vp, vp, vp, f32, i32, i32,
                                               ctypes.POINTER(SvOutputs), vp]
    lib.spec_verify_scheduled.restype = i32
    lib.spec_verify_scheduled.argtypes = [ctypes.POINTER(SvWeights), vp, vp, vp, vp, f32, f32, i32, i32, i32, vp,
                                          sz, ctypes.POINTER(SvOutputs), vp]
    lib.spec_draft_propose.restype = i32
    lib.spec_draft_propose.argtypes = [ctypes.POINTER(SvWeights), vp, vp, f32, i32, vp, sz, vp, vp, vp]
    lib.spec_verify_tree.restype = i32
    lib.spec_verify_tree.argtypes = [ctypes.POINTER(SvWeights), vp, vp, vp, vp, vp, f32, i32, i32, vp, sz,
                                     ctypes.POINTER(SvOutputs), vp, i32, vp]
    lib.spec_commit.restype = i32
    lib.spec_commit.argtypes = [ctypes.POINTER(SvCache), vp, vp, vp, i32, i32, vp, vp]
    lib.sv_version.restype = ctypes.c_char_p
    lib.sv_strerror.restype = ctypes.c_char_p
    lib.sv_strerror.argtypes = [i32]
    lib.sv_last_hip_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _check_dev(t, dtype, name):
    if t is None:
        return
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SpecVerifyError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise SpecVerifyError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise SpecVerifyError(f"{name} must be contiguous")


def _shape(t, shape, name):
    """The C ABI takes bare pointers: a tensor of the wrong size would send the kernels
    past its end, so every shape is checked here, before the call."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise SpecVerifyError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _room(t, n, dtype, name):
    """An output the kernels write n elements of (any shape, contiguous)."""
    if t is None:
        return
    if t.dtype != dtype:
        raise SpecVerifyError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() < n:
        raise SpecVerifyError(f"{name} must be contiguous with at least {n} elements, got {t.numel()}")


def _check_weight_shapes(w_lm, w_gate, w_up, w_down, s_lm=None, s_gate=None, s_up=None, s_down=None):
    if w_lm.dim() != 2:
        raise SpecVerifyError(f"w_lm must be [V, d], got {tuple(w_lm.shape)}")
    V, d = w_lm.shape
    if (w_gate is None) != (w_up is None) or (w_gate is None) != (w_down is None):
        raise SpecVerifyError("w_gate, w_up and w_down go together")
    if w_gate is not None:
        if w_gate.dim() != 2:
            raise SpecVerifyError(f"w_gate must be [d_ff, d], got {tuple(w_gate.shape)}")
        d_ff = w_gate.shape[0]
        _shape(w_gate, (d_ff, d), "w_gate")
        _shape(w_up, (d_ff, d), "w_up")
        _shape(w_down, (d, d_ff), "w_down")
        _shape(s_gate, (d_ff,), "s_gate")
        _shape(s_up, (d_ff,), "s_up")
        _shape(s_down, (d,), "s_down")
    _shape(s_lm, (V,), "s_lm")


def _check_call_shapes(w, h, *, draft=None, h_draft=None, u=None, out=None, mode=None):
    """h [B, K+1, d] with the weights' d; draft [B, K]; h_draft [B, K, d]; u [B, K+1]; and
    room in every output the call writes.  Returns (B, K)."""
    if h.dim() != 3 or h.shape[-1] != w.d:
        raise SpecVerifyError(f"h must be [B, K+1, {w.d}], got {tuple(h.shape)}")
    B, K = h.shape[0], h.shape[1] - 1
    _shape(draft, (B, K), "draft")
    _shape(h_draft, (B, K, w.d), "h_draft")
    _shape(u, (B, K + 1), "u")
    if out is not None:
        rows_t = B * (K + 1)
        rows = rows_t + (0 if mode == SV_MODE_GREEDY else B * K)
        i32, f32 = torch.int32, torch.float32
        _room(out.accepted_len, B, i32, "accepted_len")
        _room(out.emitted, rows_t, i32, "emitted")
        _room(out.tau, 1, f32, "tau")
        _room(out.counters, 3, torch.int64, "counters")
        _room(out.dev_status, 1, i32, "dev_status")
        _room(out.diag, rows * SV_DIAG_COLS, f32, "diag")
        _room(out.logits, rows * w.V, f32, "logits")
        _room(out.hidden, rows_t * w.d, torch.bfloat16, "hidden")
        if mode == SV_MODE_SCHEDULED:
            _room(out.verify_len, B, i32, "verify_len")
        _room(out.path, rows_t, i32, "path")
    return B, K


@dataclass
class Weights:
    """Device weights, row-major [out, in], and the C struct that points at them.

    bf16 tensors, or (FP8) uint8 E4M3 codes with the fp32 scale of every output row in
    ``s_lm``, ``s_gate``, ``s_up``, ``s_down``."""

    w_lm: torch.Tensor
    w_gate: torch.Tensor | None = None
    w_up: torch.Tensor | None = None
    w_down: torch.Tensor | None = None
    s_lm: torch.Tensor | None = None
    s_gate: torch.Tensor | None = None
    s_up: torch.Tensor | None = None
    s_down: torch.Tensor | None = None
    c: SvWeights = field(init=False)

    def __post_init__(self):
        fp8 = self.w_lm.dtype == torch.uint8
        for n in ("w_lm", "w_gate", "w_up", "w_down"):
            _check_dev(getattr(self, n), torch.uint8 if fp8 else torch.bfloat16, n)
        if fp8:
            for n in ("s_lm",) + (("s_gate", "s_up", "s_down") if self.w_gate is not None else ()):
                if getattr(self, n) is None:
                    raise SpecVerifyError(f"{n}: FP8 weights need their row scales")
                _check_dev(getattr(self, n), torch.float32, n)
        _check_weight_shapes(self.w_lm, self.w_gate, self.w_up, self.w_down, self.s_lm if fp8 else None,
                             self.s_gate if fp8 else None, self.s_up if fp8 else None, self.s_down if fp8 else None)
        V, d = self.w_lm.shape
        d_ff = 0 if self.w_gate is None else self.w_gate.shape[0]
        self.c = SvWeights(_ptr(self.w_gate), _ptr(self.w_up), _ptr(self.w_down), _ptr(self.w_lm), d, d_ff, V,
                           SV_WEIGHTS_FP8_E4M3 if fp8 else SV_WEIGHTS_BF16,
                           _ptr(self.s_gate) if fp8 else None, _ptr(self.s_up) if fp8 else None,
                           _ptr(self.s_down) if fp8 else None, _ptr(self.s_lm) if fp8 else None)

    @property
    def d(self):
        return self.c.d

    @property
    def V(self):
        return self.c.V

    @property
    def d_ff(self):
        return self.c.d_ff


@dataclass
class Outputs:
    """Output tensors of one verification call (device)."""

    accepted_len: torch.Tensor
    emitted: torch.Tensor
    tau: torch.Tensor
    counters: torch.Tensor
    dev_status: torch.Tensor
    verify_len: torch.Tensor | None = None
    diag: torch.Tensor | None = None
    logits: torch.Tensor | None = None
    hidden: torch.Tensor | None = None
    ev_lm: tuple | None = None  # (torch.cuda.Event, torch.cuda.Event) around the LM-head GEMM
    path: torch.Tensor | None = None  # tree verification: node at each depth

    def c(self) -> SvOutputs:
        ev0 = ev1 = None
        if self.ev_lm is not None:
            ev0, ev1 = (e.cuda_event for e in self.ev_lm)
        return SvOutputs(_ptr(self.accepted_len), _ptr(self.emitted), _ptr(self.verify_len), _ptr(self.tau),
                         _ptr(self.counters), _ptr(self.dev_status), _ptr(self.diag), _ptr(self.logits),
                         _ptr(self.hidden), ev0, ev1)


def make_outputs(B: int, K: int, device, *, mode: int, V: int = 0, d: int = 0, diag=False, logits=False,
                 hidden=False) -> Outputs:
    i32 = dict(dtype=torch.int32, device=device)
    rows_t, rows_d = B * (K + 1), (0 if mode == SV_MODE_GREEDY else B * K)
    return Outputs(
        accepted_len=torch.empty(B, **i32), emitted=torch.empty(B, K + 1, **i32),
        tau=torch.empty(1, dtype=torch.float32, device=device),
        counters=torch.empty(3, dtype=torch.int64, device=device), dev_status=torch.empty(1, **i32),
        verify_len=torch.empty(B, **i32) if mode == SV_MODE_SCHEDULED else None,
        diag=torch.full((rows_t + rows_d, SV_DIAG_COLS), float("nan"), dtype=torch.float32, device=device)
        if diag else None,
        logits=torch.full((rows_t + rows_d, V), float("nan"), dtype=torch.float32, device=device) if logits else None,
        hidden=torch.zeros(rows_t, d, dtype=torch.bfloat16, device=device) if hidden else None)


def sv_workspace_bytes(mode: int, B: int, K: int, w: Weights) -> int:
    return int(load().sv_workspace_bytes(mode, B, K, ctypes.byref(w.c)))


def workspace(mode: int, B: int, K: int, w: Weights, device=None) -> torch.Tensor:
    n = sv_workspace_bytes(mode, B, K, w)
    if n == 0:
        raise SpecVerifyError("invalid sizes for the workspace")
    return torch.empty(n, dtype=torch.uint8, device=device or w.w_lm.device)


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _used_on(stream, *tensors) -> None:
    """Buffers allocated here (on torch's current stream) for a call enqueued on another
    stream are recorded as used there, so torch's caching allocator does not hand their
    memory out again before that stream has passed the call."""
    if stream is None:
        return
    s = stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(_stream(stream))
    if s.cuda_stream == torch.cuda.current_stream().cuda_stream:
        return
    for t in tensors:
        if isinstance(t, torch.Tensor):
            t.record_stream(s)


def _tensors(out: "Outputs") -> list:
    return [v for v in vars(out).values() if isinstance(v, torch.Tensor)]


def _raise(rc: int, what: str):
    if rc != SV_OK:
        msg = load().sv_strerror(rc).decode()
        if rc == SV_EHIP:
            msg += ": " + load().sv_last_hip_error().decode()
        raise SpecVerifyError(f"{what} failed: {msg} ({rc})")


def spec_verify_greedy(w: Weights, h, draft, *, out: Outputs | None = None, ws=None, stream=None, diag=False,
                       logits=False, hidden=False) -> Outputs:
    _check_dev(h, torch.bfloat16, "h")
    _check_dev(draft, torch.int32, "draft")
    B, K = _check_call_shapes(w, h, draft=draft, out=out, mode=SV_MODE_GREEDY)
    mine = ([] if out is not None else ["out"]) + ([] if ws is not None else ["ws"])
    out = out or make_outputs(B, K, h.device, mode=SV_MODE_GREEDY, V=w.V, d=w.d, diag=diag, logits=logits,
                              hidden=hidden)
    ws = ws if ws is not None else workspace(SV_MODE_GREEDY, B, K, w, h.device)
    oc = out.c()
    rc = load().spec_verify_greedy(ctypes.byref(w.c), _ptr(h), _ptr(draft), B, K, _ptr(ws), ws.numel(),
                                   ctypes.byref(oc), _stream(stream))
    _raise(rc, "spec_verify_greedy")
    _used_on(stream, *(_tensors(out) if "out" in mine else []), *([ws] if "ws" in mine else []))
    return out


def spec_verify_sample(w: Weights, h, h_draft, draft, u, T: float, *, out: Outputs | None = None, ws=None,
                       stream=None, diag=False, logits=False, hidden=False) -> Outputs:
    _check_dev(h, torch.bfloat16, "h")
    _check_dev(h_draft, torch.bfloat16, "h_draft")
    _check_dev(draft, torch.int32, "draft")
    _check_dev(u, torch.float32, "u")
    B, K = _check_call_shapes(w, h, draft=draft, h_draft=h_draft, u=u, out=out, mode=SV_MODE_SAMPLE)
    mine = ([] if out is not None else ["out"]) + ([] if ws is not None else ["ws"])
    out = out or make_outputs(B, K, h.device, mode=SV_MODE_SAMPLE, V=w.V, d=w.d, diag=diag, logits=logits,
                              hidden=hidden)
    ws = ws if ws is not None else workspace(SV_MODE_SAMPLE, B, K, w, h.device)
    oc = out.c()
    rc = load().spec_verify_sample(ctypes.byref(w.c), _ptr(h), _ptr(h_draft), _ptr(draft), _ptr(u), float(T), B, K,
                                   _ptr(ws), ws.numel(), ctypes.byref(oc), _stream(stream))
    _raise(rc, "spec_verify_sample")
    _used_on(stream, *(_tensors(out) if "out" in mine else []), *([ws] if "ws" in mine else []))
    return out


def spec_verify_sample_noalloc(w: Weights, h, h_draft, draft, u, T: float, *, out: Outputs | None = None,
                               stream=None, diag=False, logits=False, hidden=False) -> Outputs:
    """spec_verify_sample with the library's static per-GPU scratch as the workspace (no
    workspace argument); raises on sizes beyond SV_STATIC_SCRATCH_BYTES."""
    _check_dev(h, torch.bfloat16, "h")
    _check_dev(h_draft, torch.bfloat16, "h_draft")
    _check_dev(draft, torch.int32, "draft")
    _check_dev(u, torch.float32, "u")
    B, K = _check_call_shapes(w, h, draft=draft, h_draft=h_draft, u=u, out=out, mode=SV_MODE_SAMPLE)
    mine = out is None
    out = out or make_outputs(B, K, h.device, mode=SV_MODE_SAMPLE, V=w.V, d=w.d, diag=diag, logits=logits,
                              hidden=hidden)
    oc = out.c()
    rc = load().spec_verify_sample_noalloc(ctypes.byref(w.c), _ptr(h), _ptr(h_draft), _ptr(draft), _ptr(u),
                                           float(T), B, K, ctypes.byref(oc), _stream(stream))
    _raise(rc, "spec_verify_sample_noalloc")
    if mine:
        _used_on(stream, *_tensors(out))
    return out


def spec_verify_scheduled(w: Weights, h, h_draft, draft, u, T: float, survival_threshold: float, budget_rows: int,
                          *, out: Outputs | None = None, ws=None, stream=None, diag=False, logits=False,
                          hidden=False) -> Outputs:
    _check_dev(h, torch.bfloat16, "h")
    _check_dev(h_draft, torch.bfloat16, "h_draft")
    _check_dev(draft, torch.int32, "draft")
    _check_dev(u, torch.float32, "u")
    B, K = _check_call_shapes(w, h, draft=draft, h_draft=h_draft, u=u, out=out, mode=SV_MODE_SCHEDULED)
    mine = ([] if out is not None else ["out"]) + ([] if ws is not None else ["ws"])
    out = out or make_outputs(B, K, h.device, mode=SV_MODE_SCHEDULED, V=w.V, d=w.d, diag=diag, logits=logits,
                              hidden=hidden)
    ws = ws if ws is not None else workspace(SV_MODE_SCHEDULED, B, K, w, h.device)
    oc = out.c()
    rc = load().spec_verify_scheduled(ctypes.byref(w.c), _ptr(h), _ptr(h_draft), _ptr(draft), _ptr(u), float(T),
                                      float(survival_threshold), int(budget_rows), B, K, _ptr(ws), ws.numel(),
                                      ctypes.byref(oc), _stream(stream))
    _raise(rc, "spec_verify_scheduled")
    _used_on(stream, *(_tensors(out) if "out" in mine else []), *([ws] if "ws" in mine else []))
    return out


def spec_draft_propose(w: Weights, h_draft, coins, T: float, *, draft_out=None, conf_out=None, ws=None,
                       stream=None):
    """Returns (draft ids int32 [rows], top-1 confidences fp32 [rows]) for h_draft [rows, d] (or [B, K, d])."""
    _check_dev(h_draft, torch.bfloat16, "h_draft")
    if h_draft.dim() < 1 or h_draft.shape[-1] != w.d:
        raise SpecVerifyError(f"h_draft must be [..., {w.d}], got {tuple(h_draft.shape)}")
    rows = h_draft.numel() // h_draft.shape[-1]
    if coins is not None:
        _check_dev(coins, torch.float32, "coins")
        if coins.numel() != rows:
            raise SpecVerifyError(f"coins must hold one coin per draft row ({rows}), got {coins.numel()}")
    _room(draft_out, rows, torch.int32, "draft_out")
    _room(conf_out, rows, torch.float32, "conf_out")
    dev = h_draft.device
    mine = [t is None for t in (draft_out, conf_out, ws)]
    draft_out = draft_out if draft_out is not None else torch.empty(rows, dtype=torch.int32, device=dev)
    conf_out = conf_out if conf_out is not None else torch.empty(rows, dtype=torch.float32, device=dev)
    ws = ws if ws is not None else workspace(SV_MODE_PROPOSE, rows, 0, w, dev)
    rc = load().spec_draft_propose(ctypes.byref(w.c), _ptr(h_draft), _ptr(coins), float(T), rows, _ptr(ws),
                                   ws.numel(), _ptr(draft_out), _ptr(conf_out), _stream(stream))
    _raise(rc, "spec_draft_propose")
    _used_on(stream, *[t for t, m in zip((draft_out, conf_out, ws), mine) if m])
    return draft_out.view(h_draft.shape[:-1]), conf_out.view(h_draft.shape[:-1])


def spec_verify_tree(w: Weights, h, h_draft, tokens, parent, u, T: float, *, out: Outputs | None = None, ws=None,
                     stream=None, diag=False, logits=False, hidden=False, wait_polls: int = -1) -> Outputs:
    """Tree verification of B trees of K+1 nodes: h [B, K+1, d]; h_draft [B, K, d] (T > 0);
    tokens / parent [B, K] (node j+1); u [B, K+1] (T > 0).  T == 0 is greedy.  The output
    carries ``path`` [B, K+1] (node at each depth, -1 beyond the accepted depth).  ``wait_polls``
    bounds a workgroup's wait for the others of its request per meeting (< 0: the default)."""
    greedy = float(T) == 0.0
    _check_dev(h, torch.bfloat16, "h")
    _check_dev(tokens, torch.int32, "tokens")
    _check_dev(parent, torch.int32, "parent")
    if not greedy:
        _check_dev(h_draft, torch.bfloat16, "h_draft")
        _check_dev(u, torch.float32, "u")
    mode = SV_MODE_GREEDY if greedy else SV_MODE_SAMPLE
    B, K = _check_call_shapes(w, h, draft=tokens, h_draft=None if greedy else h_draft, u=None if greedy else u,
                              out=out, mode=mode)
    _shape(parent, (B, K), "parent")
    mine = ([] if out is not None else ["out"]) + ([] if ws is not None else ["ws"])
    out = out or make_outputs(B, K, h.device, mode=mode, V=w.V, d=w.d, diag=diag, logits=logits, hidden=hidden)
    if out.path is None:
        out.path = torch.empty(B, K + 1, dtype=torch.int32, device=h.device)
        mine.append("path")
    ws = ws if ws is not None else workspace(mode, B, K, w, h.device)
    oc = out.c()
    rc = load().spec_verify_tree(ctypes.byref(w.c), _ptr(h), None if greedy else _ptr(h_draft), _ptr(tokens),
                                 _ptr(parent), None if greedy else _ptr(u), float(T), B, K, _ptr(ws), ws.numel(),
                                 ctypes.byref(oc), _ptr(out.path), int(wait_polls), _stream(stream))
    _raise(rc, "spec_verify_tree")
    _used_on(stream, *(_tensors(out) if "out" in mine else [out.path] if "path" in mine else []),
             *([ws] if "ws" in mine else []))
    return out


def spec_commit(accepted_len, seq_len, *, Kmax: int, kv=None, block_table=None, rec_state=None, rec_snap=None,
                verify_len=None, path=None, dev_status=None, stream=None) -> None:
    """Commit the accepted prefix of the last verify block (in place).

    kv: uint8 [n_layers, 2, n_blocks, block_size, entry_bytes] paged cache (or None);
    block_table: int32 [B, max_blocks]; seq_len: int32 [B] (advanced); rec_state: uint8
    [B, rec_bytes] and rec_snap: uint8 [B, Kmax+1, rec_bytes] (or both None);
    accepted_len / verify_len: int32 [B]; path: int32 [B, Kmax+1] for a tree (or None)."""
    _check_dev(accepted_len, torch.int32, "accepted_len")
    _check_dev(seq_len, torch.int32, "seq_len")
    for t, n in ((verify_len, "verify_len"), (path, "path"), (block_table, "block_table"), (dev_status, "dev_status")):
        _check_dev(t, torch.int32, n)
    for t, n in ((kv, "kv"), (rec_state, "rec_state"), (rec_snap, "rec_snap")):
        _check_dev(t, torch.uint8, n)
    B = seq_len.numel()
    _shape(accepted_len, (B,), "accepted_len")
    _shape(verify_len, (B,), "verify_len")
    _shape(path, (B, Kmax + 1), "path")
    _room(dev_status, 1, torch.int32, "dev_status")
    if block_table is not None and (block_table.dim() != 2 or block_table.shape[0] != B):
        raise SpecVerifyError(f"block_table must be [{B}, max_blocks], got {tuple(block_table.shape)}")
    if rec_state is not None and (rec_state.dim() != 2 or rec_state.shape[0] != B):
        raise SpecVerifyError(f"rec_state must be [{B}, n], got {tuple(rec_state.shape)}")
    c = SvCache()
    c.seq_len = _ptr(seq_len)
    if kv is not None:
        if kv.dim() != 5 or kv.shape[1] != 2 or block_table is None:
            raise SpecVerifyError("kv must be [n_layers, 2, n_blocks, block_size, entry_bytes] with a block_table")
        L_, _, nb, bs, eb = kv.shape
        c.kv, c.n_layers, c.n_blocks, c.block_size, c.entry_bytes = _ptr(kv), L_, nb, bs, eb
        c.layer_stride, c.half_stride = kv.stride(0), kv.stride(1)
        c.block_table, c.max_blocks = _ptr(block_table), block_table.shape[-1]
    if rec_state is not None or rec_snap is not None:
        if rec_state is None or rec_snap is None or tuple(rec_snap.shape) != (B, Kmax + 1, rec_state.shape[-1]):
            raise SpecVerifyError("rec_state [B, n] and rec_snap [B, Kmax+1, n] go together")
        c.rec_state, c.rec_snap, c.rec_bytes = _ptr(rec_state), _ptr(rec_snap), rec_state.shape[-1]
    rc = load().spec_commit(ctypes.byref(c), _ptr(accepted_len), _ptr(verify_len), _ptr(path), B, int(Kmax),
                            _ptr(dev_status), _stream(stream))
    _raise(rc, "spec_commit")


def version() -> str:
    return load().sv_version().decode()
