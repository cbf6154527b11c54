"""The no-allocation fused decode entry point against the workspace one,
through the C-ABI: two calls in a row (the second smaller, so the static
scratch still holds the first call's larger rows), each bit for bit equal to
indexer_score_topk_fused_decode on the same inputs, and the top-k equal to
the oracle's ranking of the GPU's own scores; a call whose rows exceed the
scratch is refused before anything is enqueued."""
import ctypes

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_lightning_indexer_amd as li  # noqa: E402
from gpu_helpers import DEV, check_topk_exact, dev, gpu_score  # noqa: E402


def _noalloc(lib, inp, idx, val):
    q, kc, bt, sl, w = (dev(x) for x in (inp.q, inp.k_cache, inp.block_table, inp.seq_lens, inp.w))
    m = dev(inp.mask)
    st = lib.indexer_score_topk_fused_decode_noalloc(
        q.data_ptr(), q.stride(0), q.stride(1), kc.data_ptr(), inp.block_size, kc.stride(1),
        bt.data_ptr(), bt.stride(0), sl.data_ptr(), inp.R, inp.Q, inp.max_seq_len, w.data_ptr(),
        None if m is None else m.data_ptr(), 0 if m is None else m.stride(0), inp.H, inp.d,
        inp.k_top, idx.data_ptr(), val.data_ptr(), inp.k_top, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return st, (q, kc, bt, sl, w, m)


def test_noalloc_matches_workspace_entry_point():
    lib = li.load_library()
    big = W.random_decode(31, 32, 4, 64, 128, 64, 3000, 16000, 256, w_kind="uniform", max_seq_len=16000)
    small = W.random_decode(32, 5, 1, 16, 64, 16, 1, 300, 24, w_kind="signed", max_seq_len=304,
                            mask_kind="bias")
    for inp in (big, small):
        rows = inp.R * inp.Q
        need = li.workspace_bytes(li.OP_FUSED_DECODE, rows, inp.max_seq_len, inp.k_top)
        assert need <= li.NOALLOC_SCRATCH_BYTES
        idx = torch.full((rows, inp.k_top), -7, dtype=torch.int32, device=DEV)
        val = torch.full((rows, inp.k_top), 7.0, dtype=torch.float32, device=DEV)
        st, keep = _noalloc(lib, inp, idx, val)
        assert st == li.OK, lib.indexer_last_error()
        ref_i, ref_v = li.score_topk_fused_decode(dev(inp.q), dev(inp.k_cache), dev(inp.block_table),
                                                  dev(inp.seq_lens), inp.Q, inp.max_seq_len, dev(inp.w),
                                                  inp.k_top, dev(inp.mask))
        torch.cuda.synchronize()
        assert torch.equal(idx, ref_i), f"{inp.name}: indices differ from the workspace entry point"
        assert torch.equal(val.view(torch.int32), ref_v.view(torch.int32)), f"{inp.name}: values differ"
        g = gpu_score(inp).cpu().numpy()
        check_topk_exact(idx.cpu().numpy(), val.cpu().numpy(), g, inp.k_top, where=inp.name)


def test_noalloc_refuses_rows_beyond_its_scratch():
    lib = li.load_library()
    inp = W.random_decode(33, 2, 1, 64, 128, 64, 10, 20, 8)
    cols = li.NOALLOC_SCRATCH_BYTES // (4 * 2) + 4   # two rows of this many keys do not fit
    idx = torch.empty((2, 8), dtype=torch.int32, device=DEV)
    val = torch.empty((2, 8), dtype=torch.float32, device=DEV)
    q, kc, sl, w = dev(inp.q), dev(inp.k_cache), dev(inp.seq_lens), dev(inp.w)
    bt = torch.zeros((2, (cols + 63) // 64), dtype=torch.int32, device=DEV)
    st = lib.indexer_score_topk_fused_decode_noalloc(
        q.data_ptr(), q.stride(0), q.stride(1), kc.data_ptr(), 64, kc.stride(1), bt.data_ptr(),
        bt.stride(0), sl.data_ptr(), 2, 1, cols, w.data_ptr(), None, 0, 64, 128, 8, idx.data_ptr(),
        val.data_ptr(), 8, torch.cuda.current_stream().cuda_stream)
    assert st == li.EWORKSPACE
    assert b"INDEXER_NOALLOC_SCRATCH_BYTES" in lib.indexer_last_error()
