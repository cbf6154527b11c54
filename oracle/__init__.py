"""Lightning-indexer oracle (CPU, fp64).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the HIP library or its
Python binding.  It shares no code with them.

``indexer_oracle.c`` holds the arithmetic (plain loops in double); this module
only builds it with gcc, loads it with ctypes and marshals numpy arrays.
``materialize.py`` holds an independent NumPy formulation of the same score
(the per-head "materialise then sum" scheme) used as a cross-check.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "indexer_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
           "-Wall", "-Wextra", *extra_flags, "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def load(path: Optional[str] = None):
    """Load (building first if nothing is built) and declare signatures."""
    global _lib
    if path is None:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB):
            build()
        path = LIB
    lib = ctypes.CDLL(path)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.oracle_score_prefill.argtypes = [p, i64, i64, p, i64, p, p, i64, p,
                                         i32, i32, i32, i32, p, i64]
    lib.oracle_score_prefill.restype = None
    lib.oracle_score_decode.argtypes = [p, i64, i64, p, i32, p, i64, p,
                                        i32, i32, i32, p, p, i64, i32, i32, p, i64]
    lib.oracle_score_decode.restype = None
    lib.oracle_topk_f64.argtypes = [p, i64, i32, i32, p, i32, p, p]
    lib.oracle_topk_f64.restype = None
    lib.oracle_topk_f32.argtypes = [p, i64, i32, i32, p, i32, p, p]
    lib.oracle_topk_f32.restype = None
    lib.oracle_topk_blocks_f32.argtypes = [p, i64, i32, i32, p, i32, i32, i32, p, p]
    lib.oracle_topk_blocks_f32.restype = None
    lib.oracle_topk_blocks_f64.argtypes = [p, i64, i32, i32, p, i32, i32, i32, p, p]
    lib.oracle_topk_blocks_f64.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = i32
    if path == LIB:
        _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _f16(a):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float16
    return a.view(np.uint16)


def num_threads(lib=None) -> int:
    return (lib or load()).oracle_num_threads()


def score_prefill(q, k, w, mask=None, vis_len=None, lib=None) -> np.ndarray:
    """q f16 [T][H][d], k f16 [P][d], w f32 [H], mask f16 [T][P] or None,
    vis_len i32 [T] or None  ->  f64 [T][P]."""
    lib = lib or load()
    qh, kh = _f16(q), _f16(k)
    T, H, d = qh.shape
    P = kh.shape[0]
    w = np.ascontiguousarray(w, dtype=np.float32)
    mh = None if mask is None else _f16(mask)
    vl = None if vis_len is None else np.ascontiguousarray(vis_len, dtype=np.int32)
    out = np.empty((T, P), dtype=np.float64)
    lib.oracle_score_prefill(_ptr(qh), H * d, d, _ptr(kh), d, _ptr(w),
                             _ptr(mh), P, _ptr(vl), T, P, H, d, _ptr(out), P)
    return out


def score_decode(q, k_cache, block_table, seq_lens, Q, max_seq_len, w,
                 mask=None, lib=None) -> np.ndarray:
    """Paged score; returns f64 [R*Q][max_seq_len]."""
    lib = lib or load()
    qh, kc = _f16(q), _f16(k_cache)
    RQ, H, d = qh.shape
    bs = kc.shape[1]
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    R = sl.shape[0]
    assert RQ == R * Q
    w = np.ascontiguousarray(w, dtype=np.float32)
    mh = None if mask is None else _f16(mask)
    out = np.empty((RQ, max_seq_len), dtype=np.float64)
    lib.oracle_score_decode(_ptr(qh), H * d, d, _ptr(kc), bs, _ptr(bt), bt.shape[1],
                            _ptr(sl), R, Q, max_seq_len, _ptr(w), _ptr(mh),
                            max_seq_len, H, d, _ptr(out), max_seq_len)
    return out


def topk(score: np.ndarray, k_top: int, row_len=None, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row top-k of f64 or f32 scores [n_rows][n_cols].
    Returns (idx i32 [n_rows][k_top], val of the input dtype)."""
    lib = lib or load()
    score = np.ascontiguousarray(score)
    n_rows, n_cols = score.shape
    rl = None if row_len is None else np.ascontiguousarray(row_len, dtype=np.int32)
    idx = np.empty((n_rows, k_top), dtype=np.int32)
    if score.dtype == np.float64:
        val = np.empty((n_rows, k_top), dtype=np.float64)
        lib.oracle_topk_f64(_ptr(score), n_cols, n_rows, n_cols, _ptr(rl), k_top,
                            _ptr(idx), _ptr(val))
    elif score.dtype == np.float32:
        val = np.empty((n_rows, k_top), dtype=np.float32)
        lib.oracle_topk_f32(_ptr(score), n_cols, n_rows, n_cols, _ptr(rl), k_top,
                            _ptr(idx), _ptr(val))
    else:
        raise TypeError(score.dtype)
    return idx, val


def topk_blocks(score: np.ndarray, k_top: int, init_blocks: int, local_blocks: int,
                row_len=None, lib=None) -> Tuple[np.ndarray, np.ndarray]:
    """Block ranking: per row, the first init_blocks and last local_blocks
    candidates forced (by index), then the rest by score; f32 or f64 rows."""
    lib = lib or load()
    score = np.ascontiguousarray(score)
    n_rows, n_cols = score.shape
    rl = None if row_len is None else np.ascontiguousarray(row_len, dtype=np.int32)
    idx = np.empty((n_rows, k_top), dtype=np.int32)
    if score.dtype == np.float64:
        val = np.empty((n_rows, k_top), dtype=np.float64)
        lib.oracle_topk_blocks_f64(_ptr(score), n_cols, n_rows, n_cols, _ptr(rl), init_blocks,
                                   local_blocks, k_top, _ptr(idx), _ptr(val))
    elif score.dtype == np.float32:
        val = np.empty((n_rows, k_top), dtype=np.float32)
        lib.oracle_topk_blocks_f32(_ptr(score), n_cols, n_rows, n_cols, _ptr(rl), init_blocks,
                                   local_blocks, k_top, _ptr(idx), _ptr(val))
    else:
        raise TypeError(score.dtype)
    return idx, val


def decode_row_len(seq_lens, Q, max_seq_len) -> np.ndarray:
    """Visible keys of each paged decode row r*Q + j: seq_len - Q + 1 + j,
    clipped to [0, max_seq_len]."""
    sl = np.asarray(seq_lens, dtype=np.int64)
    vis = (sl[:, None] - Q + 1 + np.arange(Q)[None, :]).reshape(-1)
    return np.clip(vis, 0, max_seq_len).astype(np.int32)


def score_inputs(inp, lib=None) -> np.ndarray:
    """Score a ``workloads`` input bundle (prefill or paged)."""
    if hasattr(inp, "k_cache"):
        return score_decode(inp.q, inp.k_cache, inp.block_table, inp.seq_lens,
                            inp.Q, inp.max_seq_len, inp.w, inp.mask, lib=lib)
    return score_prefill(inp.q, inp.k, inp.w, inp.mask, inp.vis_len, lib=lib)


def score_rows(inp, rows, lib=None) -> np.ndarray:
    """Oracle scores for a subset of query rows only (whole key range)."""
    rows = np.asarray(rows, dtype=np.int64)
    if hasattr(inp, "k_cache"):
        # score each request touched once, then pick its rows
        out = np.empty((len(rows), inp.max_seq_len))
        for r in sorted(set(int(t) // inp.Q for t in rows)):
            q = inp.q[r * inp.Q:(r + 1) * inp.Q]
            m = None if inp.mask is None else inp.mask[r * inp.Q:(r + 1) * inp.Q]
            full = score_decode(q, inp.k_cache, inp.block_table[r:r + 1],
                                inp.seq_lens[r:r + 1], inp.Q, inp.max_seq_len,
                                inp.w, m, lib=lib)
            for i, t in enumerate(rows):
                if int(t) // inp.Q == r:
                    out[i] = full[int(t) % inp.Q]
        return out
    mask = None if inp.mask is None else inp.mask[rows]
    vis = None if inp.vis_len is None else inp.vis_len[rows]
    return score_prefill(inp.q[rows], inp.k, inp.w, mask, vis, lib=lib)
