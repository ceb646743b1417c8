"""ctypes binding of ``libts_probe.so`` (``include/ts_probe.h``): measurement
probes of what this GPU sustains -- the bf16 matrix-core rate, vector-ALU issue
rates, LDS read bandwidth and a plain HBM streaming read. The benchmark reports the hot-path
kernels against these next to the published peaks. Not part of the hot path.
"""
from __future__ import annotations

import ctypes
import os
import statistics

import torch

_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libts_probe.so")
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_PATH):
            raise RuntimeError(f"{_PATH} is missing: build it with `python -m long_context_kv_ts_amd.build`")
        l = ctypes.CDLL(_PATH)
        l.ts_probe_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        l.ts_probe_mfma_bf16.restype = ctypes.c_int
        l.ts_probe_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
        l.ts_probe_mfma_bf16_flops.restype = ctypes.c_double
        l.ts_probe_valu.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        l.ts_probe_valu.restype = ctypes.c_int
        l.ts_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]
        l.ts_probe_stream_read.restype = ctypes.c_int
        l.ts_probe_lds_read.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        l.ts_probe_lds_read.restype = ctypes.c_int
        l.ts_probe_lds_read_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        l.ts_probe_lds_read_bytes.restype = ctypes.c_double
        _lib = l
    return _lib


def _ok(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what}: launch failed (hipError {rc})")


def _timed(launch, reps: int):
    """Per-launch microseconds of `reps` back-to-back launches (HIP events on the current stream)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record()
    for i in range(reps):
        launch()
        ev[i + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps)]


def mfma_bf16_peak(dev, seconds: float = 0.4, waves_per_simd: int = 2, toggle: bool = True, iters: int = 20000):
    """Sustained dense bf16 matrix-core rate (TFLOP/s): launches back to back
    for about `seconds`, so that the clock settles under load; the median over
    the second half of the launches, and the best launch (the first
    milliseconds, before the power limit). `toggle`: changing operand data."""
    sink = torch.empty(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    launch = lambda: _ok(lib().ts_probe_mfma_bf16(waves_per_simd, int(toggle), iters, sink.data_ptr(), stream),
                         "mfma probe")
    one = _timed(launch, 2)[-1]
    reps = max(10, int(seconds * 1e6 / max(one, 1.0)))
    us = _timed(launch, reps)
    flops = lib().ts_probe_mfma_bf16_flops(waves_per_simd, iters)
    rates = [flops / (t * 1e-6) / 1e12 for t in us]
    tail = rates[len(rates) // 2:]
    return {"sustained_tflops": round(statistics.median(tail), 1), "best_tflops": round(max(rates), 1),
            "launch_us": round(statistics.median(us[len(us) // 2:]), 2), "launches": reps,
            "waves_per_simd": waves_per_simd, "toggling_operands": bool(toggle)}


def valu_issue(dev, op: int, iters: int = 4096, reps: int = 20):
    """Nanoseconds per wave instruction per SIMD (2 waves per SIMD, 16 independent chains):
    op 0 = v_fma_f32, 1 = v_exp_f32; median over `reps` launches."""
    sink = torch.empty(256, dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    launch = lambda: _ok(lib().ts_probe_valu(op, iters, sink.data_ptr(), stream), "valu probe")
    _timed(launch, 3)
    us = statistics.median(_timed(launch, reps))
    return round(us * 1e3 / (2 * 16 * iters), 3)


def stream_read(dev, nbytes: int = 209_715_200, copies: int = 4, reps: int = 40):
    """Plain streaming read from HBM (GB/s): `copies` buffers of `nbytes` read in
    turn, so that the 256 MB last-level cache holds none of the one being read;
    median over `reps` launches."""
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(i + 1) for i in range(copies)]
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    state = {"i": 0}

    def launch():
        b = bufs[state["i"] % copies]
        state["i"] += 1
        _ok(lib().ts_probe_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), stream), "stream read probe")

    _timed(launch, copies)
    us = _timed(launch, reps)
    med = statistics.median(us)
    del bufs
    return {"GBs": round(nbytes / (med * 1e-6) / 1e9, 1), "bytes": nbytes, "launch_us": round(med, 2),
            "buffers": copies}


def lds_read(dev, transposed: bool, iters: int = 4000, reps: int = 10):
    """LDS read bandwidth over all CUs (TB/s) with ds_read_b128 or, transposed,
    ds_read_b64_tr_b16; median over `reps` launches."""
    sink = torch.empty(256, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    launch = lambda: _ok(lib().ts_probe_lds_read(int(transposed), iters, sink.data_ptr(), stream), "lds probe")
    _timed(launch, 2)
    us = statistics.median(_timed(launch, reps))
    nbytes = lib().ts_probe_lds_read_bytes(int(transposed), iters)
    return {"TBs": round(nbytes / (us * 1e-6) / 1e12, 2), "per_cu_GBs": round(nbytes / (us * 1e-6) / 1e9 / 256, 1),
            "launch_us": round(us, 2), "instruction": "ds_read_b64_tr_b16" if transposed else "ds_read_b128"}


def measure_all(dev) -> dict:
    """Every probe once: what the benchmark reports as the measured ceilings."""
    return {"mfma_bf16": mfma_bf16_peak(dev),
            "mfma_bf16_constant_operands": mfma_bf16_peak(dev, toggle=False, seconds=0.2),
            "mfma_bf16_1wave": mfma_bf16_peak(dev, waves_per_simd=1, seconds=0.2),
            "hbm_stream_read": stream_read(dev),
            "lds_read_b128": lds_read(dev, False),
            "lds_read_tr_b64": lds_read(dev, True),
            "ns_per_wave_instr_per_simd": {"v_fma_f32": valu_issue(dev, 0), "v_exp_f32": valu_issue(dev, 1)}}


if __name__ == "__main__":
    import json

    print(json.dumps(measure_all(torch.device("cuda:0")), indent=1))
