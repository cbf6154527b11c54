"""The C-ABI library on the host: it loads without a GPU, exports every
symbol include/indexer.h declares, and rejects bad arguments before it would
enqueue anything (none of these calls reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

import sparse_attention_lightning_indexer_amd as li

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "indexer.h")

A = 0x10000        # a fake, 256-byte aligned "device" address; never dereferenced
B = 0x20000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(indexer_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return li.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 14, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(li.EXPORTS)


def test_version_and_status_strings(lib):
    v = int(re.search(r"#define INDEXER_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.indexer_abi_version() == v
    assert lib.indexer_status_string(0) == b"INDEXER_OK"
    for s in range(1, 5):
        assert lib.indexer_status_string(s).startswith(b"INDEXER_E")
    assert lib.indexer_status_string(99) == b"unknown indexer status"


def test_workspace_bytes(lib):
    assert lib.indexer_workspace_bytes(li.OP_TOPK, 10, 100, 8) == 0
    # fused: scores [rows][round_up(cols, 4)] f32, rounded up to 256 bytes
    assert lib.indexer_workspace_bytes(li.OP_FUSED_PREFILL, 3, 5, 2) == 256
    assert lib.indexer_workspace_bytes(li.OP_FUSED_PREFILL, 8192, 8192, 2048) == 8192 * 8192 * 4
    assert lib.indexer_workspace_bytes(li.OP_FUSED_DECODE, 128, 16383, 2048) == 128 * 16384 * 4
    assert lib.indexer_workspace_bytes(7, 1, 1, 1) == ctypes.c_size_t(-1).value
    assert lib.indexer_workspace_bytes(li.OP_TOPK, -1, 1, 1) == ctypes.c_size_t(-1).value


def prefill(lib, **kw):
    a = dict(q=A, qst=64 * 128, qsh=128, k=B, kss=128, w=A, mask=None, mst=0, vis=None,
             T=4, P=16, H=64, d=128, score=A, sst=16, stream=None)
    a.update(kw)
    return lib.indexer_score_prefill(a["q"], a["qst"], a["qsh"], a["k"], a["kss"], a["w"], a["mask"],
                                     a["mst"], a["vis"], a["T"], a["P"], a["H"], a["d"], a["score"],
                                     a["sst"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(H=0), li.ENOTSUP, b"n_heads=0"),
    (dict(H=1025), li.ENOTSUP, b"n_heads=1025"),
    (dict(H=-3), li.ENOTSUP, b"not supported"),
    (dict(d=100, qsh=104, qst=104 * 64, kss=104), li.ENOTSUP, b"head_dim=100"),
    (dict(d=264, qsh=264, qst=264 * 64, kss=264), li.ENOTSUP, b"head_dim=264"),
    (dict(d=0, qsh=8, qst=8 * 64, kss=8), li.ENOTSUP, b"head_dim=0"),
    (dict(q=None), li.EINVAL, b"q is NULL"),
    (dict(k=None), li.EINVAL, b"k is NULL"),
    (dict(w=None), li.EINVAL, b"w is NULL"),
    (dict(score=None), li.EINVAL, b"score is NULL"),
    (dict(q=A + 2), li.EINVAL, b"q must be 16-byte aligned"),
    (dict(k=B + 8), li.EINVAL, b"k must be 16-byte aligned"),
    (dict(qsh=100), li.EINVAL, b"q_stride_h"),
    (dict(qsh=64), li.EINVAL, b"q_stride_h"),
    (dict(kss=120), li.EINVAL, b"k_stride_s"),
    (dict(mask=A, mst=8), li.EINVAL, b"mask_stride_t"),
    (dict(sst=8), li.EINVAL, b"score_stride_t"),
    (dict(T=-1), li.EINVAL, b"n_tokens=-1"),
])
def test_prefill_rejects(lib, kw, status, msg):
    assert prefill(lib, **kw) == status
    assert msg in lib.indexer_last_error()


def test_empty_prefill_is_a_no_op(lib):
    assert prefill(lib, T=0) == li.OK
    assert prefill(lib, P=0, sst=0) == li.OK
    assert lib.indexer_last_error() == b""


def decode(lib, **kw):
    a = dict(q=A, qst=64 * 128, qsh=128, kc=B, bs=64, kss=128, bt=A, bts=128, sl=A, R=2, Q=4,
             L=8192, w=A, mask=None, mst=0, H=64, d=128, score=A, sst=8192, stream=None)
    a.update(kw)
    return lib.indexer_score_decode(a["q"], a["qst"], a["qsh"], a["kc"], a["bs"], a["kss"], a["bt"],
                                    a["bts"], a["sl"], a["R"], a["Q"], a["L"], a["w"], a["mask"],
                                    a["mst"], a["H"], a["d"], a["score"], a["sst"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(bts=127), li.EINVAL, b"bt_stride"),
    (dict(bs=0), li.EINVAL, b"block_size"),
    (dict(Q=0), li.EINVAL, b"query_len"),
    (dict(bt=None), li.EINVAL, b"block_table is NULL"),
    (dict(sl=None), li.EINVAL, b"seq_lens is NULL"),
    (dict(kc=None), li.EINVAL, b"k_cache is NULL"),
    (dict(H=2000), li.ENOTSUP, b"n_heads=2000"),
    (dict(sst=100), li.EINVAL, b"score_stride_t"),
    (dict(R=70000, Q=70000), li.EINVAL, b"int32"),
])
def test_decode_rejects(lib, kw, status, msg):
    assert decode(lib, **kw) == status
    assert msg in lib.indexer_last_error()


def test_empty_decode_is_a_no_op(lib):
    assert decode(lib, R=0) == li.OK
    assert decode(lib, L=0, sst=0, bts=0) == li.OK


def topk(lib, **kw):
    a = dict(score=A, sst=100, n=4, c=100, rl=None, k=8, idx=B, val=None, ost=8, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.indexer_topk(a["score"], a["sst"], a["n"], a["c"], a["rl"], a["k"], a["idx"], a["val"],
                            a["ost"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,status,msg", [
    (dict(k=0), li.EINVAL, b"k_top=0"),
    (dict(k=4096, ost=4096), li.ENOTSUP, b"INDEXER_MAX_K_TOP"),
    (dict(idx=None), li.EINVAL, b"idx is NULL"),
    (dict(ost=4), li.EINVAL, b"out_stride"),
    (dict(sst=50), li.EINVAL, b"score_stride_t"),
    (dict(score=None), li.EINVAL, b"score is NULL"),
    (dict(n=-2), li.EINVAL, b"n_rows=-2"),
    (dict(idx=B + 2), li.EINVAL, b"aligned"),
])
def test_topk_rejects(lib, kw, status, msg):
    assert topk(lib, **kw) == status
    assert msg in lib.indexer_last_error()


def test_fused_workspace_checks(lib):
    st = lib.indexer_score_topk_fused_prefill(A, 64 * 128, 128, B, 128, A, None, 0, None, 4, 16, 64, 128,
                                              8, B, None, 8, None, 0, None)
    assert st == li.EWORKSPACE and b"workspace" in lib.indexer_last_error()
    st = lib.indexer_score_topk_fused_prefill(A, 64 * 128, 128, B, 128, A, None, 0, None, 4, 16, 64, 128,
                                              8, B, None, 8, A + 64, 1 << 20, None)
    assert st == li.EWORKSPACE   # misaligned workspace
    st = lib.indexer_score_topk_fused_decode(A, 64 * 128, 128, B, 64, 128, A, 2, A, 2, 1, 128, A, None, 0,
                                             64, 128, 8, B, None, 8, A, 16, None)
    assert st == li.EWORKSPACE


def test_probe_argument_checks():
    """The measured-peak probes (their own library, not the indexer's ABI)
    validate before launching (no GPU needed)."""
    from sparse_attention_lightning_indexer_amd import peak_probe
    pl = peak_probe.load_library()
    d = ctypes.c_double(0.0)
    assert pl.peak_probe_mfma(0, A, ctypes.byref(d), None) == 1
    assert pl.peak_probe_mfma(10, None, ctypes.byref(d), None) == 1
    assert pl.peak_probe_read(None, 1 << 20, A, None) == 1
    assert pl.peak_probe_read(A + 4, 1 << 20, A, None) == 1
    assert pl.peak_probe_read(A, 17, A, None) == 1
    assert pl.peak_probe_empty(0, 64, None) == 1
    assert pl.peak_probe_empty(1, 1025, None) == 1
    I = ctypes.c_void_p(16)
    assert pl.peak_probe_rows(None, 64, None, 1, 64, 8, A, I, None) == 1
    assert pl.peak_probe_rows(A, 32, None, 1, 64, 8, A, I, None) == 1      # stride < row_len
    assert pl.peak_probe_rows(A, 1 << 15, None, 1, 16385, 8, A, I, None) == 1
    assert pl.peak_probe_rows(A, 64, None, 1, 64, 16385, A, I, None) == 1
    assert pl.peak_probe_rows(A, 64, None, 0, 64, 8, A, I, None) == 1
    lib = li.load_library()
    assert not any(hasattr(lib, n) for n in ("indexer_probe_mfma", "indexer_probe_read"))


def test_block_ranking_argument_checks(lib):
    """Negative window sizes are refused before anything is enqueued."""
    st = lib.indexer_topk_blocks(A, 100, 4, 100, None, -1, 0, 8, B, None, 8, None, 0, None)
    assert st == li.EINVAL and b"init_blocks" in lib.indexer_last_error()
    st = lib.indexer_topk_blocks(A, 100, 4, 100, None, 0, -2, 8, B, None, 8, None, 0, None)
    assert st == li.EINVAL
    st = lib.indexer_topk_blocks(A, 100, 4, 100, None, 1, 2, 0, B, None, 8, None, 0, None)
    assert st == li.EINVAL   # k_top
    st = lib.indexer_score_topk_fused_decode_blocks(A, 64 * 128, 128, B, 64, 128, A, 2, A, 2, 1, 128, A, None, 0,
                                                    64, 128, 3, -1, 8, B, None, 8, A, 1 << 20, None)
    assert st == li.EINVAL and b"local_blocks" in lib.indexer_last_error()


@pytest.mark.parametrize("kw,status,msg", [
    (dict(n=-1), li.EINVAL, b"n_keys"),
    (dict(d=12, ks=16, ps=16), li.ENOTSUP, b"head_dim=12"),
    (dict(d=2048, ks=2048, ps=2048), li.ENOTSUP, b"head_dim=2048"),
    (dict(pool=0), li.EINVAL, b"pool_size=0"),
    (dict(pool=8193), li.ENOTSUP, b"pool_size=8193"),
    (dict(k=None), li.EINVAL, b"NULL"),
    (dict(out=B + 8), li.EINVAL, b"aligned"),
    (dict(ks=120), li.EINVAL, b"k_stride_s"),
    (dict(ps=64), li.EINVAL, b"pool_stride_s"),
])
def test_pool_rejects(lib, kw, status, msg):
    a = dict(k=A, ks=128, n=100, d=128, pool=4, out=B, ps=128)
    a.update(kw)
    assert lib.indexer_pool_keys(a["k"], a["ks"], a["n"], a["d"], a["pool"], a["out"], a["ps"], None) == status
    assert msg in lib.indexer_last_error()


def test_stream_workspace_and_checks(lib):
    """The streaming prefill's workspace holds candidate lists, not score
    rows: it does not grow with the row length past 4 chunks of 32768 keys;
    more heads than one pass are refused before any launch."""
    ws = lib.indexer_workspace_bytes(li.OP_STREAM_PREFILL, 1024, 131072, 2048)
    assert ws == 1024 * 4 * 4096 * 8 + 1024 * 4 * 4
    assert lib.indexer_workspace_bytes(li.OP_STREAM_PREFILL, 1024, 1 << 20, 2048) == ws
    assert ws < lib.indexer_workspace_bytes(li.OP_FUSED_PREFILL, 1024, 131072, 2048) // 3
    assert lib.indexer_workspace_bytes(li.OP_STREAM_PREFILL, 16, 256, 32) == 16 * 2304 * 8 + 256
    st = lib.indexer_score_topk_stream_prefill(A, 65 * 128, 128, B, 128, A, None, 0, None, 4, 1000, 65, 128,
                                               8, B, None, 8, A, 1 << 30, None)
    assert st == li.ENOTSUP and b"one pass" in lib.indexer_last_error()
    st = lib.indexer_score_topk_stream_prefill(A, 64 * 128, 128, B, 128, A, None, 0, None, 4, 1000, 64, 128,
                                               8, B, None, 8, A, 100, None)
    assert st == li.EWORKSPACE
