"""Lightning-indexer score and top-k on AMD Instinct MI355X (gfx950).

A thin binding over the C-ABI library ``libindexer.so`` (declared in
``include/indexer.h``).  Every function here only checks and marshals
arguments (torch tensors -> device pointers, strides, the current HIP stream)
and calls the library; all computation runs in the library's HIP kernels.
There is no CPU fallback: if the library is missing, the functions raise.

    score[t, s] = sum_h w[h] * relu(q[t, h, :] . k[s, :]) + mask[t, s]

then the k_top best keys per row (score descending, ties to the lower key
index, -inf never selected, short rows padded with index -1 / value -inf).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libindexer.so")

OK, EINVAL, ENOTSUP, EWORKSPACE, EHIP = range(5)
OP_TOPK, OP_FUSED_PREFILL, OP_FUSED_DECODE, OP_STREAM_PREFILL = range(4)
MAX_K_TOP = 2048

EXPORTS = (
    "indexer_abi_version", "indexer_status_string", "indexer_last_error",
    "indexer_score_prefill", "indexer_score_decode", "indexer_topk",
    "indexer_score_topk_fused_prefill", "indexer_score_topk_fused_decode",
    "indexer_workspace_bytes", "indexer_score_topk_fused_decode_noalloc",
    "indexer_topk_blocks", "indexer_score_topk_fused_decode_blocks", "indexer_pool_keys",
    "indexer_score_topk_stream_prefill",
)
NOALLOC_SCRATCH_BYTES = 16 << 20


class IndexerError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load the HIP library and declare its signatures.  Loading needs no
    GPU; raises if the library has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m sparse_attention_lightning_indexer_amd.build` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    st = ctypes.c_int
    lib.indexer_abi_version.argtypes = []
    lib.indexer_abi_version.restype = ctypes.c_int
    lib.indexer_status_string.argtypes = [ctypes.c_int]
    lib.indexer_status_string.restype = ctypes.c_char_p
    lib.indexer_last_error.argtypes = []
    lib.indexer_last_error.restype = ctypes.c_char_p
    lib.indexer_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i32]
    lib.indexer_workspace_bytes.restype = sz
    lib.indexer_score_prefill.argtypes = [p, i64, i64, p, i64, p, p, i64, p,
                                          i32, i32, i32, i32, p, i64, p]
    lib.indexer_score_prefill.restype = st
    lib.indexer_score_decode.argtypes = [p, i64, i64, p, i32, i64, p, i64, p,
                                         i32, i32, i32, p, p, i64, i32, i32, p, i64, p]
    lib.indexer_score_decode.restype = st
    lib.indexer_topk.argtypes = [p, i64, i32, i32, p, i32, p, p, i64, p, sz, p]
    lib.indexer_topk.restype = st
    lib.indexer_score_topk_fused_prefill.argtypes = [p, i64, i64, p, i64, p, p, i64, p,
                                                     i32, i32, i32, i32, i32, p, p, i64,
                                                     p, sz, p]
    lib.indexer_score_topk_fused_prefill.restype = st
    lib.indexer_score_topk_fused_decode.argtypes = [p, i64, i64, p, i32, i64, p, i64, p,
                                                    i32, i32, i32, p, p, i64, i32, i32,
                                                    i32, p, p, i64, p, sz, p]
    lib.indexer_score_topk_fused_decode.restype = st
    lib.indexer_score_topk_stream_prefill.argtypes = [p, i64, i64, p, i64, p, p, i64, p,
                                                      i32, i32, i32, i32, i32, p, p, i64,
                                                      p, sz, p]
    lib.indexer_score_topk_stream_prefill.restype = st
    lib.indexer_pool_keys.argtypes = [p, i64, i32, i32, i32, p, i64, p]
    lib.indexer_pool_keys.restype = st
    lib.indexer_topk_blocks.argtypes = [p, i64, i32, i32, p, i32, i32, i32, p, p, i64, p, sz, p]
    lib.indexer_topk_blocks.restype = st
    lib.indexer_score_topk_fused_decode_blocks.argtypes = [p, i64, i64, p, i32, i64, p, i64, p,
                                                           i32, i32, i32, p, p, i64, i32, i32,
                                                           i32, i32, i32, p, p, i64, p, sz, p]
    lib.indexer_score_topk_fused_decode_blocks.restype = st
    lib.indexer_score_topk_fused_decode_noalloc.argtypes = [p, i64, i64, p, i32, i64, p, i64, p,
                                                            i32, i32, i32, p, p, i64, i32, i32,
                                                            i32, p, p, i64, p]
    lib.indexer_score_topk_fused_decode_noalloc.restype = st
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status: int):
    if status != OK:
        msg = load_library().indexer_last_error().decode()
        raise IndexerError(status, msg)


# ---------------------------------------------------------------- torch glue

def _torch():
    import torch
    return torch


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _need(t, name, dtype, device, dims=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dims is not None and t.dim() != dims:
        raise ValueError(f"{name} must have {dims} dims, got {t.dim()}")


def _lengths(t, name, n, device):
    """An i32 vector of one entry per row (lengths), made contiguous."""
    _need(t, name, _torch().int32, device, 1)
    if t.shape[0] != n:
        raise ValueError(f"{name} must have one entry per row ({n}), got {t.shape[0]}")
    return t.contiguous()


def _rows_out(out, name, dtype, n_rows, n_cols, device):
    """An output of n_rows rows of n_cols contiguous entries (any row stride
    the library accepts)."""
    _need(out, name, dtype, device, 2)
    if tuple(out.shape) != (n_rows, n_cols) or (n_rows > 0 and n_cols > 1 and out.stride(1) != 1):
        raise ValueError(f"{name} must be [{n_rows}, {n_cols}] with contiguous rows, got "
                         f"{tuple(out.shape)} with strides {tuple(out.stride())}")


def _topk_outputs(idx, val, n_rows, k_top, with_values, device):
    """The (idx, val) outputs of a selection: given ones are checked, missing
    ones allocated; both contiguous [n_rows, k_top]."""
    torch = _torch()
    if idx is None:
        idx = torch.empty((n_rows, k_top), dtype=torch.int32, device=device)
    _need(idx, "idx", torch.int32, device, 2)
    if val is None and with_values:
        val = torch.empty((n_rows, k_top), dtype=torch.float32, device=device)
    if val is not None:
        _need(val, "val", torch.float32, device, 2)
    for o in (idx, val):
        if o is not None and (tuple(o.shape) != (n_rows, k_top) or not o.is_contiguous()):
            raise ValueError(f"outputs must be contiguous [{n_rows}, {k_top}]")
    return idx, val


def _q_checks(q, w):
    torch = _torch()
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    dev = q.device
    _need(q, "q", torch.float16, dev, 3)
    _need(w, "w", torch.float32, dev, 1)
    if q.stride(2) != 1:
        raise ValueError("q's head_dim must be contiguous")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous")
    if w.shape[0] != q.shape[1]:
        raise ValueError(f"w must hold one weight per head ({q.shape[1]}), got {w.shape[0]}")
    return dev


def _keys(k, d, device):
    _need(k, "k", _torch().float16, device, 2)
    if k.stride(1) != 1:
        raise ValueError("k's head_dim must be contiguous")
    if k.shape[1] != d:
        raise ValueError(f"k must be [P, {d}] (q's head_dim), got {tuple(k.shape)}")


def workspace_bytes(op: int, n_rows: int, n_cols: int, k_top: int) -> int:
    return int(load_library().indexer_workspace_bytes(op, n_rows, n_cols, k_top))


def score_prefill(q, k, w, mask=None, vis_len=None, out=None):
    """q f16 [T,H,d], k f16 [P,d], w f32 [H], mask f16 [T,P] or None,
    vis_len i32 [T] or None -> f32 [T,P] scores (invisible = -inf)."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    T, H, d = q.shape
    _keys(k, d, dev)
    P = k.shape[0]
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (T, P):
            raise ValueError("mask must be [T, P] with contiguous rows")
    if vis_len is not None:
        vis_len = _lengths(vis_len, "vis_len", T, dev)
    if out is None:
        out = torch.empty((T, P), dtype=torch.float32, device=dev)
    _rows_out(out, "out", torch.float32, T, P, dev)
    if T == 0 or P == 0:  # nothing to compute (and empty tensors have no address)
        return out
    _check(lib.indexer_score_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), _ptr(w),
        _ptr(mask), mask.stride(0) if mask is not None else 0, _ptr(vis_len),
        T, P, H, d, _ptr(out), out.stride(0), _stream(dev)))
    return out


def _paged_checks(q, k_cache, block_table, seq_lens, dev, max_seq_len):
    torch = _torch()
    _need(k_cache, "k_cache", torch.float16, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(seq_lens, "seq_lens", torch.int32, dev, 1)
    bs = k_cache.shape[1]
    if k_cache.shape[2] != q.shape[2]:
        raise ValueError(f"k_cache must be [n_blocks, block_size, {q.shape[2]}] (q's head_dim), "
                         f"got {tuple(k_cache.shape)}")
    if k_cache.stride(2) != 1 or k_cache.stride(0) != bs * k_cache.stride(1):
        raise ValueError("k_cache must be [n_blocks, block_size, d] with contiguous slots")
    if block_table.stride(1) != 1:
        raise ValueError("block_table rows must be contiguous")
    need = -(-max_seq_len // bs) if bs > 0 else 0
    if block_table.shape[0] < seq_lens.shape[0] or block_table.shape[1] < need:
        raise ValueError(f"block_table must be at least [n_requests, ceil(max_seq_len/block_size)] = "
                         f"[{seq_lens.shape[0]}, {need}], got {tuple(block_table.shape)}")
    if not seq_lens.is_contiguous():
        raise ValueError("seq_lens must be contiguous")
    return bs


def score_decode(q, k_cache, block_table, seq_lens, query_len: int,
                 max_seq_len: int, w, mask=None, out=None):
    """Paged decode / speculative decode.  q f16 [R*Q,H,d] (row r*Q+j is query
    j of request r), k_cache f16 [n_blocks, block_size, d], block_table i32
    [R, max_blocks], seq_lens i32 [R] -> f32 [R*Q, max_seq_len]."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    RQ, H, d = q.shape
    bs = _paged_checks(q, k_cache, block_table, seq_lens, dev, max_seq_len)
    R = seq_lens.shape[0]
    if RQ != R * query_len:
        raise ValueError(f"q has {RQ} rows, expected n_requests*query_len = {R * query_len}")
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (RQ, max_seq_len):
            raise ValueError("mask must be [R*Q, max_seq_len] with contiguous rows")
    if out is None:
        out = torch.empty((RQ, max_seq_len), dtype=torch.float32, device=dev)
    _rows_out(out, "out", torch.float32, RQ, max_seq_len, dev)
    if RQ == 0 or max_seq_len == 0:  # nothing to compute
        return out
    _check(lib.indexer_score_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), bs, k_cache.stride(1),
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), R, query_len,
        max_seq_len, _ptr(w), _ptr(mask), mask.stride(0) if mask is not None else 0,
        H, d, _ptr(out), out.stride(0), _stream(dev)))
    return out


def topk(score, k_top: int, row_len=None, with_values: bool = True,
         idx=None, val=None) -> Tuple:
    """Per-row top-k of f32 scores [n_rows, n_cols] -> (idx i32 [n_rows,k],
    val f32 [n_rows,k] or None)."""
    torch = _torch()
    lib = load_library()
    if not score.is_cuda:
        raise ValueError("score must be a GPU tensor")
    dev = score.device
    _need(score, "score", torch.float32, dev, 2)
    if score.stride(1) != 1:
        raise ValueError("score rows must be contiguous")
    n_rows, n_cols = score.shape
    if row_len is not None:
        row_len = _lengths(row_len, "row_len", n_rows, dev)
    idx, val = _topk_outputs(idx, val, n_rows, k_top, with_values, dev)
    ws_n = workspace_bytes(OP_TOPK, n_rows, n_cols, k_top)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev) if ws_n else None
    if n_rows == 0:  # nothing to select
        return idx, val
    _check(lib.indexer_topk(
        _ptr(score), score.stride(0), n_rows, n_cols, _ptr(row_len), k_top,
        _ptr(idx), _ptr(val), idx.stride(0), _ptr(ws), ws_n, _stream(dev)))
    return idx, val


def topk_blocks(score, k_top: int, init_blocks: int, local_blocks: int, row_len=None,
                with_values: bool = True, idx=None, val=None) -> Tuple:
    """Block ranking over f32 score rows: the first init_blocks and last
    local_blocks candidates of each row always selected (by index), then the
    best of the rest -> (idx i32 [n_rows,k], val f32 [n_rows,k] or None)."""
    torch = _torch()
    lib = load_library()
    if not score.is_cuda:
        raise ValueError("score must be a GPU tensor")
    dev = score.device
    _need(score, "score", torch.float32, dev, 2)
    if score.stride(1) != 1:
        raise ValueError("score rows must be contiguous")
    n_rows, n_cols = score.shape
    if row_len is not None:
        row_len = _lengths(row_len, "row_len", n_rows, dev)
    idx, val = _topk_outputs(idx, val, n_rows, k_top, with_values, dev)
    ws_n = workspace_bytes(OP_TOPK, n_rows, n_cols, k_top)
    ws = torch.empty(max(ws_n, 1), dtype=torch.uint8, device=dev) if ws_n else None
    if n_rows == 0:
        return idx, val
    _check(lib.indexer_topk_blocks(
        _ptr(score), score.stride(0), n_rows, n_cols, _ptr(row_len), init_blocks, local_blocks, k_top,
        _ptr(idx), _ptr(val), idx.stride(0), _ptr(ws), ws_n, _stream(dev)))
    return idx, val


def pool_keys(k, pool_size: int, out=None):
    """Mean-pool consecutive windows of pool_size keys: f16 [n_keys, d] ->
    f16 [ceil(n_keys / pool_size), d] (a short last window averages what it
    holds; exact sum, one rounding of the mean to f16)."""
    torch = _torch()
    lib = load_library()
    if not k.is_cuda:
        raise ValueError("k must be a GPU tensor")
    dev = k.device
    _need(k, "k", torch.float16, dev, 2)
    if k.stride(1) != 1:
        raise ValueError("k's head_dim must be contiguous")
    n, d = k.shape
    if pool_size < 1:
        raise ValueError("pool_size must be >= 1")
    n_pool = -(-n // pool_size)
    if out is None:
        out = torch.empty((n_pool, d), dtype=torch.float16, device=dev)
    _need(out, "out", torch.float16, dev, 2)
    if tuple(out.shape) != (n_pool, d) or out.stride(1) != 1:
        raise ValueError(f"out must be [{n_pool}, {d}] with contiguous rows")
    if n == 0:
        return out
    _check(lib.indexer_pool_keys(_ptr(k), k.stride(0), n, d, pool_size, _ptr(out), out.stride(0), _stream(dev)))
    return out


def _workspace(op, n_rows, n_cols, k_top, dev, workspace):
    torch = _torch()
    need = workspace_bytes(op, n_rows, n_cols, k_top)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, dev, 1)  # its size in bytes is its numel
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return workspace, need


def score_topk_fused_prefill(q, k, w, k_top: int, mask=None, vis_len=None,
                             with_values: bool = True, workspace=None, idx=None, val=None):
    """indexer_score_prefill + indexer_topk with scores kept in a workspace.
    `idx` / `val` may be given as outputs ([n_tokens, k_top], contiguous)."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    T, H, d = q.shape
    _keys(k, d, dev)
    P = k.shape[0]
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (T, P):
            raise ValueError("mask must be [T, P] with contiguous rows")
    if vis_len is not None:
        vis_len = _lengths(vis_len, "vis_len", T, dev)
    idx, val = _topk_outputs(idx, val, T, k_top, with_values, dev)
    if T == 0:  # nothing to compute
        return idx, val
    ws, need = _workspace(OP_FUSED_PREFILL, T, P, k_top, dev, workspace)
    _check(lib.indexer_score_topk_fused_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), _ptr(w),
        _ptr(mask), mask.stride(0) if mask is not None else 0, _ptr(vis_len),
        T, P, H, d, k_top, _ptr(idx), _ptr(val), k_top, _ptr(ws),
        ws.numel(), _stream(dev)))
    return idx, val


def score_topk_stream_prefill(q, k, w, k_top: int, mask=None, vis_len=None,
                              with_values: bool = True, workspace=None, idx=None, val=None):
    """The result of score_topk_fused_prefill without a score buffer: per
    row and key chunk candidate lists (about 128 KiB per row at k_top 2048),
    merged into the ordered top-k."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    T, H, d = q.shape
    _keys(k, d, dev)
    P = k.shape[0]
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (T, P):
            raise ValueError("mask must be [T, P] with contiguous rows")
    if vis_len is not None:
        vis_len = _lengths(vis_len, "vis_len", T, dev)
    idx, val = _topk_outputs(idx, val, T, k_top, with_values, dev)
    if T == 0:
        return idx, val
    ws, need = _workspace(OP_STREAM_PREFILL, T, P, k_top, dev, workspace)
    _check(lib.indexer_score_topk_stream_prefill(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k), k.stride(0), _ptr(w),
        _ptr(mask), mask.stride(0) if mask is not None else 0, _ptr(vis_len),
        T, P, H, d, k_top, _ptr(idx), _ptr(val), k_top, _ptr(ws), ws.numel(), _stream(dev)))
    return idx, val


def score_topk_fused_decode(q, k_cache, block_table, seq_lens, query_len: int,
                            max_seq_len: int, w, k_top: int, mask=None,
                            with_values: bool = True, workspace=None, idx=None, val=None):
    """indexer_score_decode + indexer_topk with scores kept in a workspace.
    `idx` / `val` may be given as [rows, k_top] outputs."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    RQ, H, d = q.shape
    bs = _paged_checks(q, k_cache, block_table, seq_lens, dev, max_seq_len)
    R = seq_lens.shape[0]
    if RQ != R * query_len:
        raise ValueError(f"q has {RQ} rows, expected n_requests*query_len = {R * query_len}")
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (RQ, max_seq_len):
            raise ValueError("mask must be [R*Q, max_seq_len] with contiguous rows")
    idx, val = _topk_outputs(idx, val, RQ, k_top, with_values, dev)
    if RQ == 0:  # nothing to compute
        return idx, val
    ws, need = _workspace(OP_FUSED_DECODE, RQ, max_seq_len, k_top, dev, workspace)
    _check(lib.indexer_score_topk_fused_decode(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), bs, k_cache.stride(1),
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), R, query_len,
        max_seq_len, _ptr(w), _ptr(mask), mask.stride(0) if mask is not None else 0,
        H, d, k_top, _ptr(idx), _ptr(val), k_top, _ptr(ws), ws.numel(), _stream(dev)))
    return idx, val


def score_topk_fused_decode_blocks(q, k_cache, block_table, seq_lens, query_len: int,
                                   max_seq_len: int, w, k_top: int, init_blocks: int, local_blocks: int,
                                   mask=None, with_values: bool = True, workspace=None, idx=None, val=None):
    """score_topk_fused_decode with block ranking: each row's first
    init_blocks and last local_blocks visible keys are always selected."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    RQ, H, d = q.shape
    bs = _paged_checks(q, k_cache, block_table, seq_lens, dev, max_seq_len)
    R = seq_lens.shape[0]
    if RQ != R * query_len:
        raise ValueError(f"q has {RQ} rows, expected n_requests*query_len = {R * query_len}")
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (RQ, max_seq_len):
            raise ValueError("mask must be [R*Q, max_seq_len] with contiguous rows")
    idx, val = _topk_outputs(idx, val, RQ, k_top, with_values, dev)
    if RQ == 0:
        return idx, val
    ws, need = _workspace(OP_FUSED_DECODE, RQ, max_seq_len, k_top, dev, workspace)
    _check(lib.indexer_score_topk_fused_decode_blocks(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), bs, k_cache.stride(1),
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), R, query_len,
        max_seq_len, _ptr(w), _ptr(mask), mask.stride(0) if mask is not None else 0,
        H, d, init_blocks, local_blocks, k_top, _ptr(idx), _ptr(val), k_top, _ptr(ws), ws.numel(),
        _stream(dev)))
    return idx, val


def score_topk_fused_decode_noalloc(q, k_cache, block_table, seq_lens, query_len: int,
                                    max_seq_len: int, w, k_top: int, mask=None, idx=None, val=None):
    """score_topk_fused_decode without a workspace: the library keeps the
    score rows in its static per-GPU scratch (at most NOALLOC_SCRATCH_BYTES;
    larger calls raise).  Calls that overlap on one GPU race.  `idx` (and
    `val`, or None for no values) must be given when the caller cannot
    allocate; otherwise they are allocated here."""
    torch = _torch()
    lib = load_library()
    dev = _q_checks(q, w)
    RQ, H, d = q.shape
    bs = _paged_checks(q, k_cache, block_table, seq_lens, dev, max_seq_len)
    R = seq_lens.shape[0]
    if RQ != R * query_len:
        raise ValueError(f"q has {RQ} rows, expected n_requests*query_len = {R * query_len}")
    if mask is not None:
        _need(mask, "mask", torch.float16, dev, 2)
        if mask.stride(1) != 1 or tuple(mask.shape) != (RQ, max_seq_len):
            raise ValueError("mask must be [R*Q, max_seq_len] with contiguous rows")
    # values come with indices allocated here, or when an output is given for them
    idx, val = _topk_outputs(idx, val, RQ, k_top, idx is None, dev)
    if RQ == 0:
        return idx, val
    _check(lib.indexer_score_topk_fused_decode_noalloc(
        _ptr(q), q.stride(0), q.stride(1), _ptr(k_cache), bs, k_cache.stride(1),
        _ptr(block_table), block_table.stride(0), _ptr(seq_lens), R, query_len,
        max_seq_len, _ptr(w), _ptr(mask), mask.stride(0) if mask is not None else 0,
        H, d, k_top, _ptr(idx), _ptr(val), k_top, _stream(dev)))
    return idx, val


__all__ = [
    "score_prefill", "score_decode", "topk", "score_topk_fused_prefill",
    "score_topk_fused_decode", "score_topk_fused_decode_noalloc", "score_topk_fused_decode_blocks",
    "topk_blocks", "pool_keys", "score_topk_stream_prefill", "workspace_bytes", "load_library", "IndexerError",
    "EXPORTS", "MAX_K_TOP",
]
