"""The bench's matrix-core probe (csrc/mfma_peak.hip, built as libmfma_peak.so): times
back-to-back independent MFMAs on every SIMD with HIP events on the current stream and
returns the sustained TFLOP/s, the measured ceiling that attention rates are compared
with beside the spec sheet's peak."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmfma_peak.so")
FLOP_PER_MFMA = {"bf16": 2 * 32 * 32 * 16, "fp8": 2 * 32 * 32 * 64}
KIND = {"bf16": 0, "fp8": 1}


def measure(dtype: str = "bf16", workgroups: int = 2048, iters: int = 20000,
            reps: int = 5) -> dict:
    """Best and median of ``reps`` timed launches (after one warm-up launch) of
    ``workgroups`` x 4 waves, each wave issuing 4 * ``iters`` MFMAs of ``dtype``."""
    import torch
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build with "
                           "`python -m exact_io_aware_46_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.mfma_peak_launch.restype = ctypes.c_int
    lib.mfma_peak_launch.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                     ctypes.c_void_p]
    chains = int(lib.mfma_peak_chains())
    out = torch.empty(workgroups * 256, dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream()

    def launch():
        rc = lib.mfma_peak_launch(KIND[dtype], out.data_ptr(), workgroups, iters, s.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"mfma_peak_launch failed ({rc})")

    launch()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        launch()
        e1.record(s)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    flop = workgroups * 4 * iters * chains * FLOP_PER_MFMA[dtype]
    ms.sort()
    return {"dtype": dtype, "tflops": round(flop / (ms[0] * 1e-3) / 1e12, 1),
            "tflops_median": round(flop / (ms[len(ms) // 2] * 1e-3) / 1e12, 1),
            "ms": round(ms[0], 3), "waves": workgroups * 4, "mfma_per_wave": iters * chains}


if __name__ == "__main__":
    import json
    for dt in ("bf16", "fp8"):
        print(json.dumps(measure(dt)), flush=True)
