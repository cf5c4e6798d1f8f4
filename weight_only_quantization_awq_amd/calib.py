"""Roofline calibration on the GPU: HBM copy bandwidth and MFMA issue rate.

    python -m weight_only_quantization_awq_amd.calib            # both, JSON line
    python -m weight_only_quantization_awq_amd.calib copy --bytes 1073741824 --reps 3

The copy run is also the reference kernel for turning rocprofv3 FETCH_SIZE /
WRITE_SIZE counter readings into bytes (it moves exactly `bytes` each way).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_lib = None

MFMA_FLOP = {0: 8 * 16384, 1: 4 * 32768, 2: 8 * 2048, 3: 16 * 32768, 4: 16 * 32768,
             5: 16 * 32768}   # per wave per iteration
MFMA_NAME = {0: "v_mfma_f32_16x16x32_f16", 1: "v_mfma_f32_32x32x16_f16", 2: "v_mfma_f32_16x16x4_f32",
             3: "v_mfma_f32_32x32x16_f16, 16 accumulators, random operands",
             4: "v_mfma_f32_32x32x16_f16, 16 accumulators, zero operands",
             5: "v_mfma_f32_32x32x16_bf16, 16 accumulators, random operands"}


def load():
    global _lib
    if _lib is None:
        path = os.path.join(_PKG, "libawq_calib.so")
        if not os.path.exists(path):
            raise ImportError(f"{path} missing: run the build first")
        lib = ctypes.CDLL(path)
        lib.awq_calib_copy.restype = ctypes.c_int
        lib.awq_calib_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.awq_calib_stream.restype = ctypes.c_int
        lib.awq_calib_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.c_void_p]
        lib.awq_calib_mfma.restype = ctypes.c_int
        lib.awq_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _lib = lib
    return _lib


def copy_gbs(nbytes: int = 1 << 30, reps: int = 5) -> dict:
    lib = load()
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.awq_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, st) == 0
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        lib.awq_calib_copy(src.data_ptr(), dst.data_ptr(), nbytes, st)
        e1.record()
    torch.cuda.synchronize()
    ms = min(e0.elapsed_time(e1) for e0, e1 in evs)
    return {"bytes_each_way": nbytes, "ms": ms, "GB_s": 2 * nbytes / (ms * 1e-3) / 1e9}


def stream_gbs(mode: int, nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """mode 0: write-only fill, mode 1: read-only stream, mode 2: fill with streaming stores."""
    lib = load()
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.awq_calib_stream(buf.data_ptr(), nbytes, mode, sink.data_ptr(), st) == 0
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in evs:
        e0.record()
        lib.awq_calib_stream(buf.data_ptr(), nbytes, mode, sink.data_ptr(), st)
        e1.record()
    torch.cuda.synchronize()
    ms = min(e0.elapsed_time(e1) for e0, e1 in evs)
    return {"mode": {0: "write", 1: "read", 2: "write_streaming"}[mode], "bytes": nbytes, "ms": ms, "GB_s": nbytes / (ms * 1e-3) / 1e9}


def mfma_tflops(kind: int, iters: int = 4096, blocks: int = 1024) -> dict:
    lib = load()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    assert lib.awq_calib_mfma(out.data_ptr(), kind, blocks, 64, st) == 0
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    lib.awq_calib_mfma(out.data_ptr(), kind, blocks, iters, st)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    flop = blocks * 4 * iters * MFMA_FLOP[kind]
    return {"instr": MFMA_NAME[kind], "ms": ms, "TFLOP_s": flop / (ms * 1e-3) / 1e12}


def main():
    p = argparse.ArgumentParser()
    p.add_argument("what", nargs="?", default="all", choices=["all", "copy", "stream", "mfma"])
    p.add_argument("--bytes", type=int, default=1 << 30)
    p.add_argument("--reps", type=int, default=5)
    a = p.parse_args()
    res = {}
    if a.what in ("all", "copy"):
        res["copy"] = copy_gbs(a.bytes, a.reps)
    if a.what in ("all", "stream"):
        res["write"] = stream_gbs(0, a.bytes, a.reps)
        res["read"] = stream_gbs(1, a.bytes, a.reps)
        res["write_streaming"] = stream_gbs(2, a.bytes, a.reps)
    if a.what in ("all", "mfma"):
        res["mfma"] = [mfma_tflops(k) for k in (0, 1, 2)] + [mfma_tflops(k, iters=4096) for k in (3, 4, 5, 3, 4, 5)]
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
