"""Binding of the machine-rate probes of libmoe (include/moe_probe.h):
argument marshalling and event timing only.

hbm_read_rate() and mfma_rate() give, on the GPU at hand, the HBM read rate
through the global -> LDS copies the expert GEMMs use and the MFMA rate of a
register-resident loop of their instruction; the harness reports achieved
rates against these as well as against the published peaks.
"""
import ctypes

import torch

from . import MOE_BF16, MOE_FP8_E4M3, MoeError, lib

_bound = False


def _lib():
    global _bound
    L = lib()
    if not _bound:
        L.moe_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_void_p]
        L.moe_probe_hbm_read.restype = ctypes.c_int
        L.moe_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.moe_probe_mfma.restype = ctypes.c_int
        _bound = True
    return L


def _check(code):
    if code != 0:
        raise MoeError(code, lib().moe_last_error().decode())


def _time(launch, reps):
    s = torch.cuda.current_stream()
    launch(s)  # warm-up
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    for _ in range(reps):
        launch(s)
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


def hbm_read_rate(nbytes=4 << 30, blocks=2048, reps=5):
    """Bytes per second read from HBM by the global -> LDS copy probe."""
    L = _lib()
    unit = blocks * 65536
    nbytes = max(unit, nbytes // unit * unit)
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    t = _time(lambda s: _check(L.moe_probe_hbm_read(buf.data_ptr(), nbytes, blocks, sink.data_ptr(),
                                                    s.cuda_stream)), reps)
    del buf
    return nbytes / t


def mfma_rate(dtype="bf16", iters=4000, blocks=256, reps=3):
    """Flop per second of the register-resident MFMA probe ("bf16" or "fp8")."""
    L = _lib()
    dt = MOE_BF16 if dtype == "bf16" else MOE_FP8_E4M3
    flop_each = 32768 if dtype == "bf16" else 131072
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    t = _time(lambda s: _check(L.moe_probe_mfma(dt, iters, blocks, sink.data_ptr(), s.cuda_stream)),
              reps)
    return blocks * 8 * iters * 10 * flop_each / t
