"""Measured peaks of the device, reported by the benchmark beside the
published ones: an LDS-fed f16 MFMA stream on pseudo-random operands and a
large streaming read; and floors of one launch: an empty kernel, and a
kernel that moves a row-wise selection's bytes without selecting.
Measurement helpers only, in their own library (``libpeak_probe.so``, built
from ``csrc/peak_probe.hip``); not part of the indexer or its C-ABI.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpeak_probe.so")

_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sparse_attention_lightning_indexer_amd.build`")
    lib = ctypes.CDLL(path)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.peak_probe_sink_floats.argtypes = []
    lib.peak_probe_sink_floats.restype = i32
    lib.peak_probe_mfma.argtypes = [i32, p, p, p]
    lib.peak_probe_mfma.restype = ctypes.c_int
    lib.peak_probe_read.argtypes = [p, sz, p, p]
    lib.peak_probe_read.restype = ctypes.c_int
    lib.peak_probe_empty.argtypes = [i32, i32, p]
    lib.peak_probe_empty.restype = ctypes.c_int
    lib.peak_probe_rows.argtypes = [p, ctypes.c_int64, p, i32, i32, i32, p, p, p]
    lib.peak_probe_rows.restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = lib
    return lib


def _ok(status: int, what: str):
    if status != 0:
        raise RuntimeError(f"{what} failed with status {status}")


def probe_peaks(device=None, mfma_iters: int = 4000, read_bytes: int = 4 << 30, repeats: int = 3):
    """Sustained f16 MFMA TFLOP/s with B operands from LDS, and streaming-read
    GB/s over `read_bytes`.  Each is the best of `repeats` timed launches
    after one untimed launch, timed with events on torch's current stream
    (the stream the probes are launched on)."""
    import torch
    lib = load_library()
    dev = device or torch.device("cuda", torch.cuda.current_device())
    sink = torch.empty(lib.peak_probe_sink_floats(), dtype=torch.float32, device=dev)
    buf = torch.zeros(read_bytes // 4, dtype=torch.float32, device=dev)
    flops = ctypes.c_double(0.0)
    s = torch.cuda.current_stream(dev).cuda_stream

    def timed(fn):
        fn()
        best = None
        for _ in range(repeats):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize(dev)
            ms = a.elapsed_time(b)
            best = ms if best is None else min(best, ms)
        return best

    ms_m = timed(lambda: _ok(lib.peak_probe_mfma(mfma_iters, sink.data_ptr(), ctypes.byref(flops), s), "mfma probe"))
    ms_r = timed(lambda: _ok(lib.peak_probe_read(buf.data_ptr(), read_bytes, sink.data_ptr(), s), "read probe"))
    del buf
    return {"mfma_f16_tflops": flops.value / (ms_m * 1e-3) / 1e12, "read_gbs": read_bytes / (ms_r * 1e-3) / 1e9,
            "mfma_ms": ms_m, "read_ms": ms_r}


def empty(blocks: int, threads: int):
    """Launch the empty kernel on torch's current stream."""
    import torch
    _ok(load_library().peak_probe_empty(blocks, threads, torch.cuda.current_stream().cuda_stream), "empty probe")


def rows(scores, lens, k: int, val, idx):
    """Launch the row probe on torch's current stream: scores [n_rows][n]
    f32, lens int32 [n_rows] or None, val/idx [n_rows][k]."""
    import torch
    n_rows, n = scores.shape
    assert scores.dtype == torch.float32 and scores.stride(1) == 1
    assert val.shape == (n_rows, k) and idx.shape == (n_rows, k) and val.is_contiguous() and idx.is_contiguous()
    assert lens is None or (lens.dtype == torch.int32 and lens.numel() == n_rows and lens.is_contiguous())
    _ok(load_library().peak_probe_rows(scores.data_ptr(), scores.stride(0), None if lens is None else lens.data_ptr(),
                                       n_rows, n, k, val.data_ptr(), idx.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream), "rows probe")


def read(buf, sink):
    """Launch the streaming-read probe over the whole of `buf` (a device
    tensor of a multiple of 16 bytes) on torch's current stream."""
    import torch
    _ok(load_library().peak_probe_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                       torch.cuda.current_stream().cuda_stream), "read probe")


def sink_for(device):
    """The device buffer the read and MFMA probes take."""
    import torch
    return torch.empty(load_library().peak_probe_sink_floats(), dtype=torch.float32, device=device)
