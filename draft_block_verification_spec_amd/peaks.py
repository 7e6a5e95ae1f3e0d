"""ctypes binding of libsvpeaks.so (include/sv_peaks.h): the achievable HBM read rate and
dense bf16 MFMA rate of the GPU, measured by two probe kernels and reported beside the
vendor peaks.  Argument marshalling only; torch supplies the device buffers."""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsvpeaks.so")
EXPORTS = ("sv_probe_read", "sv_probe_mfma")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not found: build it with `python -m draft_block_verification_spec_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp = ctypes.c_void_p
        lib.sv_probe_read.restype = ctypes.c_int
        lib.sv_probe_read.argtypes = [vp, ctypes.c_size_t, vp, vp, ctypes.POINTER(ctypes.c_float)]
        lib.sv_probe_mfma.restype = ctypes.c_int
        lib.sv_probe_mfma.argtypes = [ctypes.c_int, vp, vp, ctypes.POINTER(ctypes.c_float),
                                      ctypes.POINTER(ctypes.c_double)]
        _lib = lib
    return _lib


def measure(device, read_bytes: int = 2 << 30, repeats: int = 5, mfma_iters: int = 20000) -> dict:
    """Best of `repeats` launches of each probe: HBM read GB/s over a `read_bytes` buffer and
    dense bf16 MFMA TFLOP/s."""
    lib = load()
    buf = torch.ones(read_bytes // 2, dtype=torch.int16, device=device)
    out = torch.zeros(1024, dtype=torch.int32, device=device)
    outf = torch.zeros(1024, dtype=torch.float32, device=device)
    st = torch.cuda.current_stream(device).cuda_stream
    ms = ctypes.c_float()
    fl = ctypes.c_double()
    rd, mf = [], []
    for _ in range(repeats):
        if lib.sv_probe_read(buf.data_ptr(), read_bytes, out.data_ptr(), st, ctypes.byref(ms)) != 0:
            raise RuntimeError("sv_probe_read failed")
        rd.append(read_bytes / (ms.value * 1e-3) / 1e9)
        if lib.sv_probe_mfma(mfma_iters, outf.data_ptr(), st, ctypes.byref(ms), ctypes.byref(fl)) != 0:
            raise RuntimeError("sv_probe_mfma failed")
        mf.append(fl.value / (ms.value * 1e-3) / 1e12)
    del buf
    return {"hbm_read_GBps": max(rd), "mfma_bf16_TFLOPs": max(mf),
            "probe": f"best of {repeats}: one read of {read_bytes >> 20} MiB with 16-byte nontemporal loads; "
                     f"{mfma_iters} x 8 independent v_mfma_f32_32x32x16_bf16 per wave, one wave per SIMD"}
