"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the
same seeded inputs.  See gpu_helpers.py for the comparison bars."""
import dataclasses
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
from oracle import pooling
import workloads as W

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import sparse_attention_lightning_indexer_amd as li  # noqa: E402
from gpu_helpers import (DEV, check_scores, check_topk_exact, check_topk_vs_f64,  # noqa: E402
                         denominators, dev, gpu_fused, gpu_score, gpu_topk)


def _full_check(inp, where, check_f64_topk=True):
    g_t = gpu_score(inp)
    g = g_t.cpu().numpy()
    o = oracle.score_inputs(inp)
    den = denominators(inp)
    err = check_scores(g, o, den, where=where)
    gi, gv = gpu_topk(g_t, inp.k_top)
    check_topk_exact(gi, gv, g, inp.k_top, where=where)
    if check_f64_topk:
        check_topk_vs_f64(gi, o, den, inp.k_top, where=where)
    fi, fv = gpu_fused(inp)
    assert np.array_equal(fi, gi) and np.array_equal(fv.view(np.uint32), gv.view(np.uint32)), f"{where}: fused differs"
    return err


# ----------------------------------------------------------------- tiny

def test_tiny_reference_case():
    inp = W.tiny()
    err = _full_check(inp, "tiny")
    print(f"tiny max scaled error {err:.2e}")


# ------------------------------------------------------------ random prefill

PREFILL_CASES = [
    # T, P, H, d, k_top, mask, w, vis
    (37, 301, 4, 64, 16, "random", "uniform", "none"),
    (5, 96, 4, 128, 96, "none", "equal", "none"),
    (19, 257, 8, 64, 40, "bias", "signed", "none"),
    (33, 130, 8, 128, 7, "causal", "uniform", "random"),
    (9, 200, 16, 64, 64, "random", "pow2", "none"),
    (17, 513, 16, 128, 100, "zero", "signed", "random"),
    (6, 77, 32, 64, 80, "bias", "uniform", "none"),
    (23, 333, 32, 128, 33, "causal", "signed", "none"),
    (3, 65, 64, 64, 5, "random", "uniform", "none"),
    (41, 700, 64, 128, 128, "causal", "equal", "none"),
    (11, 1000, 64, 128, 300, "none", "signed", "random"),
    (2, 31, 64, 128, 64, "random", "uniform", "none"),
    (8, 64, 64, 128, 2048, "causal", "uniform", "none"),
    (4, 40, 64, 128, 8, "all_inf", "uniform", "none"),
]


@pytest.mark.parametrize("T,P,H,d,k_top,mask,wk,vis", PREFILL_CASES,
                         ids=[f"T{c[0]}P{c[1]}H{c[2]}d{c[3]}k{c[4]}-{c[5]}-{c[6]}-{c[7]}" for c in PREFILL_CASES])
def test_random_prefill(T, P, H, d, k_top, mask, wk, vis):
    inp = W.random_prefill(1000 + T + P + H + d, T, P, H, d, k_top, mask_kind=mask, w_kind=wk, vis_kind=vis)
    _full_check(inp, inp.name)


@pytest.mark.parametrize("H,d", [(4, 64), (8, 128), (16, 64), (32, 128), (64, 128), (64, 64)])
def test_integer_inputs_bit_exact(H, d):
    """Exact-arithmetic inputs: every partial sum is representable in f32, so
    the GPU must equal the oracle bit for bit, and so must the top-k (which
    is full of exact ties)."""
    inp = W.integer_prefill(77 + H + d, 29, 389, H, d, 50, mask_kind="random")
    g_t = gpu_score(inp)
    g = g_t.cpu().numpy()
    o = oracle.score_inputs(inp)
    assert np.array_equal(g.astype(np.float64), o)
    gi, gv = gpu_topk(g_t, inp.k_top)
    oi, ov = oracle.topk(o, inp.k_top)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.astype(np.float64), ov)


# ------------------------------------------------------------ paged decode

DECODE_CASES = [
    # R, Q, H, d, block_size, len_lo, len_hi, k_top
    (5, 1, 64, 128, 64, 1, 300, 32),
    (3, 4, 64, 128, 64, 3, 700, 64),
    (4, 2, 16, 64, 16, 0, 90, 20),
    (6, 3, 8, 128, 32, 1, 129, 50),
    (2, 5, 64, 128, 64, 4, 260, 64),
    (3, 8, 32, 64, 64, 8, 200, 16),
    (2, 9, 64, 128, 64, 9, 300, 40),
    (3, 16, 4, 64, 16, 16, 100, 10),
    (4, 1, 64, 128, 37, 1, 250, 30),
    (2, 4, 64, 128, 64, 0, 3, 8),
]


@pytest.mark.parametrize("R,Q,H,d,bs,lo,hi,k_top", DECODE_CASES,
                         ids=[f"R{c[0]}Q{c[1]}H{c[2]}d{c[3]}bs{c[4]}L{c[5]}-{c[6]}k{c[7]}" for c in DECODE_CASES])
def test_random_decode(R, Q, H, d, bs, lo, hi, k_top):
    inp = W.random_decode(500 + R * Q + H + bs, R, Q, H, d, bs, lo, hi, k_top, w_kind="uniform")
    _full_check(inp, inp.name)


# Larger cases for the persistent decode kernel: each workgroup gets many
# key tiles spanning several row groups; the last two shapes take the chunked
# kernel instead (block size below 4, more than 1536 row groups).
STREAM_CASES = [
    # R, Q, H, d, block_size, len_lo, len_hi, k_top
    (700, 1, 64, 128, 64, 1, 1500, 64),      # many short requests per workgroup
    (48, 1, 64, 128, 64, 9000, 14000, 128),  # > 16 tiles per workgroup
    (300, 4, 64, 128, 16, 4, 1200, 32),      # four query rows per group: each consumer loads its row's q per row group
    (200, 2, 32, 64, 37, 1, 3000, 40),       # block size not a power of two
    (100, 3, 8, 128, 4, 1, 2000, 20),        # smallest block size of the persistent kernel
    (40, 16, 4, 64, 16, 100, 3000, 24),      # 16 rows per group, several row groups per tile stream
    (60, 9, 64, 128, 64, 9, 2500, 16),       # two row groups per request
    (1500, 1, 64, 128, 64, 1, 400, 16),      # 1500 row groups: near the persistent kernel's 1536
    (50, 1, 16, 64, 2, 1, 800, 10),          # block size 2: chunked kernel
    (2100, 1, 4, 64, 16, 1, 200, 8),         # 2100 row groups: chunked kernel
]


@pytest.mark.parametrize("R,Q,H,d,bs,lo,hi,k_top", STREAM_CASES,
                         ids=[f"R{c[0]}Q{c[1]}H{c[2]}d{c[3]}bs{c[4]}L{c[5]}-{c[6]}k{c[7]}" for c in STREAM_CASES])
def test_stream_decode(R, Q, H, d, bs, lo, hi, k_top):
    inp = W.random_decode(900 + R + Q + H + bs, R, Q, H, d, bs, lo, hi, k_top, w_kind="uniform")
    _full_check(inp, inp.name)


def test_fused_decode_reuses_workspace():
    """The fused paged entry point: three calls on one workspace filled with
    random bytes, with a request that has no key and rows that see none; each
    result must equal the score kernel + top-k kernel result bit for bit and
    the oracle's ranking of the GPU's own scores."""
    torch = pytest.importorskip("torch")
    a = W.random_decode(77, 40, 2, 64, 128, 64, 1, 3000, 50)
    sl = a.seq_lens.copy()
    sl[5], sl[6] = 0, 1
    a = dataclasses.replace(a, seq_lens=sl)
    b = W.random_decode(78, 70, 1, 64, 128, 64, 1, 7000, 64)
    need = max(li.workspace_bytes(li.OP_FUSED_DECODE, x.R * x.Q, x.max_seq_len, x.k_top) for x in (a, b))
    gen = torch.Generator(device=DEV).manual_seed(5)
    ws = torch.randint(0, 256, (need,), dtype=torch.uint8, device=DEV, generator=gen)
    for inp in (a, b, a):
        fi, fv = li.score_topk_fused_decode(dev(inp.q), dev(inp.k_cache), dev(inp.block_table),
                                            dev(inp.seq_lens), inp.Q, inp.max_seq_len, dev(inp.w),
                                            inp.k_top, workspace=ws)
        torch.cuda.synchronize()
        fi, fv = fi.cpu().numpy(), fv.cpu().numpy()
        g_t = gpu_score(inp)
        gi, gv = gpu_topk(g_t, inp.k_top)
        assert np.array_equal(fi, gi), f"{inp.name}: fused indices differ"
        assert np.array_equal(fv.view(np.uint32), gv.view(np.uint32)), f"{inp.name}: values differ"
        check_topk_exact(fi, fv, g_t.cpu().numpy(), inp.k_top, where=inp.name)


# head counts the kernels are not compiled for: the last head tile is
# zero-filled (extra heads weigh 0); every path, with the oracle on the real heads
ODD_HEAD_CASES = [
    # kind, H, d, (prefill T, P) or (decode R, Q, lo, hi)
    ("prefill", 1, 64, (9, 130)),
    ("prefill", 3, 128, (21, 333)),
    ("prefill", 12, 64, (17, 257)),
    ("prefill", 24, 128, (33, 400)),
    ("prefill", 48, 128, (40, 700)),
    ("prefill", 63, 64, (11, 300)),
    ("decode", 5, 128, (40, 1, 1, 700)),
    ("decode", 20, 64, (30, 3, 1, 900)),
    ("decode", 40, 128, (50, 1, 1, 1500)),
    ("decode", 56, 128, (20, 4, 4, 1000)),
]


@pytest.mark.parametrize("kind,H,d,shape", ODD_HEAD_CASES,
                         ids=[f"{c[0]}-H{c[1]}-d{c[2]}" for c in ODD_HEAD_CASES])
def test_any_head_count(kind, H, d, shape):
    if kind == "prefill":
        T, P = shape
        inp = W.random_prefill(300 + H, T, P, H, d, 24, mask_kind="random", w_kind="signed")
    else:
        R, Q, lo, hi = shape
        inp = W.random_decode(400 + H, R, Q, H, d, 64, lo, hi, 24, w_kind="signed")
    _full_check(inp, f"{kind} H={H} d={d}")


# Head dimensions off the compiled tile widths (run zero-padded to 64, 128 or
# 256) and head counts past one pass (64 heads, or 32 at 256 dimensions: the
# passes add their head groups' sums into the same score rows, the last one
# adds the mask).
WIDE_CASES = [
    # kind, H, d, (prefill T, P) or (decode R, Q, lo, hi), mask
    ("prefill", 4, 8, (9, 130), "random"),
    ("prefill", 16, 48, (21, 333), "bias"),
    ("prefill", 64, 96, (17, 257), "causal"),
    ("prefill", 8, 136, (13, 300), "random"),
    ("prefill", 32, 192, (19, 400), "bias"),
    ("prefill", 20, 256, (11, 270), "random"),
    ("prefill", 64, 256, (9, 300), "bias"),      # two passes of 32 heads at 256
    ("prefill", 65, 128, (15, 333), "bias"),     # two passes: 64 + 1
    ("prefill", 128, 64, (12, 250), "causal"),
    ("prefill", 200, 80, (7, 180), "bias"),      # four passes, padded dimension
    ("decode", 64, 96, (20, 1, 1, 700), "none"),
    ("decode", 32, 256, (10, 4, 4, 600), "bias"),
    ("decode", 96, 128, (12, 2, 2, 900), "bias"),
    ("decode", 130, 40, (8, 3, 3, 500), "random"),
    ("decode", 8, 200, (16, 1, 1, 300), "none"),
    ("prefill", 1024, 256, (5, 97), "bias"),     # the largest supported shape: 32 passes of 32 heads
    ("prefill", 1024, 64, (6, 140), "causal"),   # 16 passes of 64 heads
    ("decode", 1024, 128, (3, 2, 2, 150), "bias"),
]


@pytest.mark.parametrize("kind,H,d,shape,mk", WIDE_CASES,
                         ids=[f"{c[0]}-H{c[1]}-d{c[2]}-{c[4]}" for c in WIDE_CASES])
def test_any_head_dim_and_many_heads(kind, H, d, shape, mk):
    if kind == "prefill":
        T, P = shape
        inp = W.random_prefill(600 + H + d, T, P, H, d, 24, mask_kind=mk, w_kind="signed")
    else:
        R, Q, lo, hi = shape
        width = hi + (-hi) % 8
        inp = W.random_decode(700 + H + d, R, Q, H, d, 64, lo, hi, 24, w_kind="signed",
                              max_seq_len=width, mask_kind=mk)
    _full_check(inp, f"{kind} H={H} d={d} mask={mk}")


@pytest.mark.parametrize("H,d", [(96, 256), (100, 72), (40, 200)])
def test_integer_inputs_bit_exact_wide(H, d):
    """Exact-arithmetic inputs at padded head dimensions and over several
    head passes: every partial sum is representable in f32, so the GPU equals
    the oracle bit for bit whatever the summation order, on both layouts."""
    inp = W.integer_prefill(55 + H + d, 11, 301, H, d, 30, mask_kind="random")
    g = gpu_score(inp).cpu().numpy()
    o = oracle.score_inputs(inp)
    assert np.array_equal(g.astype(np.float64), o)
    paged = W.paged_from_prefill(dataclasses.replace(inp, mask=None), 16)
    gp = gpu_score(paged).cpu().numpy()
    assert np.array_equal(gp.astype(np.float64), oracle.score_inputs(paged))


def test_rows_with_nothing_visible():
    """Degenerate rows through every entry point: prefill rows hidden by a
    zero visible prefix or by an all -inf mask row, decode requests of length
    0 and rows that see no key, and k_top above the row length; scores must
    be -inf exactly there and the selections all padding."""
    base = W.random_prefill(21, 6, 300, 64, 128, 40, mask_kind="random", w_kind="signed")
    vis = np.array([0, 1, 300, 150, 299, 77], np.int32)
    mask = base.mask.copy()
    mask[3, :] = np.float16(-np.inf)
    pre = dataclasses.replace(base, vis_len=vis, mask=mask)
    _full_check(pre, "prefill with hidden rows")
    g = gpu_score(pre).cpu().numpy()
    assert np.all(np.isneginf(g[0])) and np.all(np.isneginf(g[3]))
    fi, fv = gpu_fused(pre)
    assert np.all(fi[0] == -1) and np.all(fi[3] == -1) and np.all(np.isneginf(fv[0]))

    dec = W.random_decode(22, 5, 3, 64, 128, 64, 1, 200, 16)
    sl = dec.seq_lens.copy()
    sl[[0, 2]] = 0
    sl[4] = 2          # query 0 of request 4 sees no key, query 2 sees two
    dec = dataclasses.replace(dec, seq_lens=sl)
    _full_check(dec, "decode with empty requests")
    gi, _ = gpu_fused(dec)
    assert np.all(gi[0:3] == -1) and np.all(gi[6:9] == -1) and np.all(gi[12] == -1)

    wide = dataclasses.replace(W.random_prefill(23, 3, 40, 16, 64, 16), k_top=100)
    gi, gv = gpu_fused(wide)
    assert gi.shape == (3, 100) and np.all(gi[:, 40:] == -1) and np.all(np.isneginf(gv[:, 40:]))
    _full_check(wide, "k_top above the row length")


def test_binding_rejects_mismatched_tensors():
    """The binding checks every tensor's length and shape against the
    problem before calling the library (a short weight, length or output
    tensor would otherwise be read or written past its end): each call
    below raises (ValueError, or TypeError for a wrong dtype) and launches
    nothing; explicit outputs of the
    right shape are used as given."""
    d = DEV
    T, P, H, D = 5, 64, 8, 64
    q = torch.zeros((T, H, D), dtype=torch.float16, device=d)
    k = torch.zeros((P, D), dtype=torch.float16, device=d)
    w = torch.ones(H, device=d)
    vis = torch.full((T,), P, dtype=torch.int32, device=d)
    bad = [
        lambda: li.score_prefill(q, k, torch.ones(H - 1, device=d)),                    # short w
        lambda: li.score_prefill(q, torch.zeros((P, D + 8), dtype=torch.float16, device=d), w),  # k width
        lambda: li.score_prefill(q, k, w, vis_len=vis[:T - 1]),                          # short vis_len
        lambda: li.score_prefill(q, k, w, out=torch.empty((T - 1, P), device=d)),       # short out
        lambda: li.score_topk_fused_prefill(q, k, w, 8, vis_len=vis[:2]),
        lambda: li.score_topk_stream_prefill(q, k, w, 8, val=torch.empty((T, 8), dtype=torch.float16, device=d)),
        lambda: li.topk(torch.zeros((T, P), device=d), 8, row_len=vis[:3]),
        lambda: li.topk(torch.zeros((T, P), device=d), 8, idx=torch.empty((T, 4), dtype=torch.int32, device=d)),
        lambda: li.topk(torch.zeros((T, P), device=d), 8, idx=torch.empty((T, 8), dtype=torch.int64, device=d)),
        lambda: li.topk_blocks(torch.zeros((T, P), device=d), 8, 1, 1, val=torch.empty((T, 8, 1), device=d)),
    ]
    kc = torch.zeros((4, 16, D), dtype=torch.float16, device=d)
    bt = torch.zeros((T, 4), dtype=torch.int32, device=d)
    sl = torch.full((T,), 60, dtype=torch.int32, device=d)
    bad += [
        lambda: li.score_decode(q, torch.zeros((4, 16, D - 8), dtype=torch.float16, device=d), bt, sl, 1, 64, w),
        lambda: li.score_decode(q, kc, bt, sl, 1, 64, w, out=torch.empty((T, 32), device=d)),
        lambda: li.score_topk_fused_decode(q, kc, bt, sl, 1, 64, torch.ones(2 * H, device=d), 8),
        lambda: li.score_topk_fused_decode_blocks(q, kc, bt, sl, 1, 64, w, 8, 1, 1,
                                                  idx=torch.empty((T, 8), dtype=torch.int32, device=d)[:, ::2]),
        lambda: li.score_topk_fused_decode_noalloc(q, kc, bt, sl, 1, 64, w, 8,
                                                   idx=torch.empty((T + 1, 8), dtype=torch.int32, device=d)),
    ]
    for i, call in enumerate(bad):
        with pytest.raises((ValueError, TypeError)):
            call()
            pytest.fail(f"case {i} was accepted")
    idx = torch.full((T, 8), -7, dtype=torch.int32, device=d)
    val = torch.empty((T, 8), device=d)
    s = torch.arange(T * P, dtype=torch.float32, device=d).reshape(T, P)
    gi, gv = li.topk(s, 8, row_len=vis, idx=idx, val=val)
    torch.cuda.synchronize()
    assert gi is idx and gv is val
    assert np.array_equal(idx.cpu().numpy(), np.tile(np.arange(P - 1, P - 9, -1), (T, 1)))


def test_zero_rows_are_a_no_op():
    """Zero query rows (prefill), zero requests (decode) and zero score rows
    (top-k) return empty results without launching anything."""
    d = DEV
    w = torch.ones(64, device=d)
    q0 = torch.empty((0, 64, 128), dtype=torch.float16, device=d)
    k = torch.zeros((128, 128), dtype=torch.float16, device=d)
    assert li.score_prefill(q0, k, w).shape == (0, 128)
    idx, val = li.score_topk_fused_prefill(q0, k, w, 8)
    assert idx.shape == (0, 8)
    kc = torch.zeros((2, 64, 128), dtype=torch.float16, device=d)
    bt = torch.zeros((0, 2), dtype=torch.int32, device=d)
    sl = torch.zeros((0,), dtype=torch.int32, device=d)
    assert li.score_decode(q0, kc, bt, sl, 1, 128, w).shape == (0, 128)
    idx, val = li.topk(torch.empty((0, 50), device=d), 8)
    assert idx.shape == (0, 8)
    torch.cuda.synchronize()


def test_decode_with_mask_and_signed_weights():
    """Row width 321 (not a multiple of 8): the chunked kernel's mask path."""
    inp = W.random_decode(42, 4, 4, 64, 128, 64, 50, 400, 32, w_kind="signed", mask_kind="bias",
                          max_seq_len=321)
    _full_check(inp, inp.name)


# Masked calls the persistent kernel takes (row width a multiple of 8, block
# size >= 4): the mask travels with the key tiles through its LDS ring.
MASKED_STREAM_CASES = [
    # R, Q, H, d, block_size, len_lo, len_hi, max_seq_len, k_top, mask
    (40, 1, 64, 128, 64, 1, 3000, 3008, 64, "bias"),     # split mapping, one query row
    (200, 1, 64, 128, 64, 1, 1000, 1024, 32, "random"),  # split mapping, many row groups per CU
    (32, 4, 64, 128, 64, 4, 5000, 5000, 128, "bias"),    # spec-decode shape, four rows a group
    (24, 4, 64, 128, 16, 4, 2000, 2048, 40, "random"),   # block size 16
    (30, 16, 16, 64, 16, 16, 1500, 1504, 24, "bias"),    # general mapping, two row groups per request
    (50, 3, 8, 128, 4, 3, 900, 904, 20, "random"),       # general mapping, block size 4
    (20, 9, 64, 128, 64, 9, 2500, 2504, 16, "bias"),     # split mapping, three row groups per request
    (60, 2, 4, 64, 37, 2, 700, 704, 12, "random"),       # 4 heads, block size not a power of two
]


@pytest.mark.parametrize("R,Q,H,d,bs,lo,hi,width,k_top,mk", MASKED_STREAM_CASES,
                         ids=[f"R{c[0]}Q{c[1]}H{c[2]}d{c[3]}bs{c[4]}L{c[5]}-{c[6]}w{c[7]}-{c[9]}"
                              for c in MASKED_STREAM_CASES])
def test_masked_stream_decode(R, Q, H, d, bs, lo, hi, width, k_top, mk):
    inp = W.random_decode(1300 + R + Q + H + bs, R, Q, H, d, bs, lo, hi, k_top, w_kind="signed",
                          max_seq_len=width, mask_kind=mk)
    _full_check(inp, inp.name)
    # masked keys are never selected
    gi, _ = gpu_fused(inp)
    picked = np.take_along_axis(inp.mask, np.where(gi >= 0, gi, 0), axis=1).astype(np.float32)
    assert not np.any(np.isneginf(picked) & (gi >= 0))


@pytest.mark.parametrize("permute", [True, False], ids=["permuted", "identity"])
@pytest.mark.parametrize("H,d,bs", [(64, 128, 64), (16, 64, 16), (4, 128, 8)])
def test_integer_inputs_paged_bit_exact(H, d, bs, permute):
    """Exact-arithmetic inputs through the paged path: the same keys laid out
    in blocks through a permuted or an in-order block table, query j of the
    T rows seeing the first P - T + 1 + j keys.  Every partial sum is
    representable in f32, so the GPU equals the oracle bit for bit, and its
    top-k equals the oracle's top-k of the exact scores."""
    base = W.integer_prefill(88 + H + d + bs, 13, 777, H, d, 40, mask_kind="none")
    paged = W.paged_from_prefill(base, bs, permute=permute)
    g_t = gpu_score(paged)
    g = g_t.cpu().numpy()
    o = oracle.score_inputs(paged)
    assert np.array_equal(g.astype(np.float64), o)
    gi, gv = gpu_topk(g_t, paged.k_top)
    oi, ov = oracle.topk(o, paged.k_top)
    assert np.array_equal(gi, oi)
    assert np.array_equal(gv.astype(np.float64), ov)
    fi, fv = gpu_fused(paged)
    assert np.array_equal(fi, oi)


def test_decode_wider_rows_than_lengths():
    """max_seq_len larger than every request: the extra columns are -inf."""
    inp = W.random_decode(43, 3, 2, 64, 128, 64, 10, 100, 16, max_seq_len=333)
    _full_check(inp, inp.name)


def test_decode_block_table_width():
    """A block table with spare columns (row stride past ceil(max_seq_len /
    block_size)) gives the same scores bit for bit; one narrower than that
    is refused by the binding before any kernel runs (the kernel may load
    any entry of those columns)."""
    inp = W.random_decode(44, 5, 1, 64, 128, 16, 30, 300, 16)
    ref = gpu_score(inp).cpu().numpy()
    bt = inp.block_table
    wide = np.full((bt.shape[0], bt.shape[1] + 7), 12345, np.int32)
    wide[:, : bt.shape[1]] = bt
    q, kc, sl, w = dev(inp.q), dev(inp.k_cache), dev(inp.seq_lens), dev(inp.w)
    got = li.score_decode(q, kc, dev(wide), sl, inp.Q, inp.max_seq_len, w).cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    narrow = dev(np.ascontiguousarray(bt[:, :-1]))
    with pytest.raises(ValueError, match="block_table"):
        li.score_decode(q, kc, narrow, sl, inp.Q, inp.max_seq_len, w)
    with pytest.raises(ValueError, match="block_table"):
        li.score_topk_fused_decode(q, kc, narrow, sl, inp.Q, inp.max_seq_len, w, inp.k_top)


def test_paged_equals_contiguous():
    """The same keys through a permuted and an in-order block table give
    bit-identical scores, and agree with the contiguous layout (query j
    seeing the first P - T + 1 + j keys) within the score bar."""
    base = W.random_prefill(7, 4, 500, 64, 128, 16, mask_kind="none", w_kind="uniform")
    vis = np.array([500 - 4 + 1 + j for j in range(4)], np.int32)
    contig = dataclasses.replace(base, vis_len=vis)
    permuted = W.paged_from_prefill(base, 64)
    in_order = W.paged_from_prefill(base, 64, permute=False)
    a = gpu_score(contig).cpu().numpy()
    b = gpu_score(permuted).cpu().numpy()
    c = gpu_score(in_order).cpu().numpy()
    assert np.array_equal(b.view(np.uint32), c.view(np.uint32))
    check_scores(b, oracle.score_inputs(contig), denominators(contig), where="paged vs oracle")
    check_scores(a, b.astype(np.float64), denominators(contig), where="contiguous vs paged")


# ------------------------------------------------------------ metamorphic

def test_weight_scaling_is_exact():
    inp = W.random_prefill(3, 21, 450, 64, 128, 40, mask_kind="zero", w_kind="uniform")
    a = gpu_score(inp).cpu().numpy()
    b = gpu_score(dataclasses.replace(inp, w=(inp.w * 4).astype(np.float32))).cpu().numpy()
    assert np.array_equal(b, a * 4)
    ia, _ = gpu_fused(inp)
    ib, _ = gpu_fused(dataclasses.replace(inp, w=(inp.w * 4).astype(np.float32)))
    assert np.array_equal(ia, ib)


def test_zero_query_gives_mask():
    inp = W.random_prefill(4, 9, 300, 64, 128, 16, mask_kind="bias")
    g = gpu_score(dataclasses.replace(inp, q=np.zeros_like(inp.q))).cpu().numpy()
    assert np.array_equal(g, inp.mask.astype(np.float32))


def test_runs_are_bit_identical():
    inp = W.random_decode(5, 4, 4, 64, 128, 64, 100, 900, 64)
    a = gpu_score(inp).cpu().numpy()
    b = gpu_score(inp).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_graph_replays_match_eager():
    """The fused entry points captured into a HIP graph (as the benchmark
    times them): every replay, with eager calls on other inputs into the
    same buffers and synchronisations between replays, gives the eager
    results bit for bit."""
    dec = W.random_decode(6, 5, 2, 64, 128, 64, 100, 900, 64)
    pre = W.random_prefill(8, 40, 700, 64, 128, 32, mask_kind="causal", w_kind="uniform")
    other = W.random_decode(9, 5, 2, 64, 128, 64, 100, 900, 64)
    d_in = [dev(x) for x in (dec.q, dec.k_cache, dec.block_table, dec.seq_lens, dec.w)]
    o_in = [dev(x) for x in (other.q, other.k_cache, other.block_table, other.seq_lens, other.w)]
    p_in = [dev(x) for x in (pre.q, pre.k, pre.w, pre.mask, pre.vis_len)]
    R = dec.R * dec.Q
    d_idx = torch.empty((R, dec.k_top), dtype=torch.int32, device=DEV)
    d_val = torch.empty((R, dec.k_top), dtype=torch.float32, device=DEV)
    p_idx = torch.empty((pre.T, pre.k_top), dtype=torch.int32, device=DEV)
    p_val = torch.empty((pre.T, pre.k_top), dtype=torch.float32, device=DEV)
    max_sl = max(dec.max_seq_len, other.max_seq_len)
    d_ws = torch.empty(li.workspace_bytes(li.OP_FUSED_DECODE, R, max_sl, dec.k_top), dtype=torch.uint8, device=DEV)
    p_ws = torch.empty(li.workspace_bytes(li.OP_FUSED_PREFILL, pre.T, pre.P, pre.k_top), dtype=torch.uint8, device=DEV)

    def run_dec(x, sl_max):
        q, kc, bt, sl, w = x
        li.score_topk_fused_decode(q, kc, bt, sl, dec.Q, sl_max, w, dec.k_top, workspace=d_ws, idx=d_idx, val=d_val)

    def run_pre():
        q, k, w, m, v = p_in
        li.score_topk_fused_prefill(q, k, w, pre.k_top, m, v, workspace=p_ws, idx=p_idx, val=p_val)

    def both():
        run_dec(d_in, dec.max_seq_len)
        run_pre()

    both()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (d_idx, d_val, p_idx, p_val)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            both()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(4):
        run_dec(o_in, other.max_seq_len)  # eager work on other inputs into the same buffers
        p_idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip((d_idx, d_val, p_idx, p_val), ref):
            assert torch.equal(got.view(torch.int32), want.view(torch.int32)), f"replay {rep} differs"


def test_graph_replays_of_the_other_entry_points():
    """The streaming prefill, the block-ranking decode, the pooled-key
    producer and the no-allocation decode captured into one HIP graph (all
    buffers allocated beforehand): every replay, with eager calls on other
    inputs into the same buffers between replays, equals the eager results
    bit for bit."""
    pre = W.random_prefill(11, 30, 40000, 64, 128, 512, mask_kind="causal", w_kind="signed")
    other_pre = W.random_prefill(12, 30, 40000, 64, 128, 512, mask_kind="random", w_kind="uniform")
    dec = W.random_decode(13, 6, 4, 64, 128, 64, 100, 3000, 128, max_seq_len=3000)
    keys = np.random.default_rng(14).standard_normal((5000, 128)).astype(np.float16)
    p_in = [dev(x) for x in (pre.q, pre.k, pre.w, pre.mask)]
    o_in = [dev(x) for x in (other_pre.q, other_pre.k, other_pre.w, other_pre.mask)]
    d_in = [dev(x) for x in (dec.q, dec.k_cache, dec.block_table, dec.seq_lens, dec.w)]
    k_in = dev(keys)
    R = dec.R * dec.Q
    s_idx = torch.empty((pre.T, pre.k_top), dtype=torch.int32, device=DEV)
    s_val = torch.empty((pre.T, pre.k_top), dtype=torch.float32, device=DEV)
    s_ws = torch.empty(li.workspace_bytes(li.OP_STREAM_PREFILL, pre.T, pre.P, pre.k_top), dtype=torch.uint8, device=DEV)
    b_idx = torch.empty((R, dec.k_top), dtype=torch.int32, device=DEV)
    b_val = torch.empty((R, dec.k_top), dtype=torch.float32, device=DEV)
    b_ws = torch.empty(li.workspace_bytes(li.OP_FUSED_DECODE, R, dec.max_seq_len, dec.k_top), dtype=torch.uint8, device=DEV)
    n_idx = torch.empty((R, dec.k_top), dtype=torch.int32, device=DEV)
    n_val = torch.empty((R, dec.k_top), dtype=torch.float32, device=DEV)
    pooled = torch.empty((1250, 128), dtype=torch.float16, device=DEV)

    def run_pre(x):
        q, k, w, m = x
        li.score_topk_stream_prefill(q, k, w, pre.k_top, m, workspace=s_ws, idx=s_idx, val=s_val)

    def all_calls():
        run_pre(p_in)
        q, kc, bt, sl, w = d_in
        li.score_topk_fused_decode_blocks(q, kc, bt, sl, dec.Q, dec.max_seq_len, w, dec.k_top, 2, 32,
                                          workspace=b_ws, idx=b_idx, val=b_val)
        li.pool_keys(k_in, 4, out=pooled)
        li.score_topk_fused_decode_noalloc(q, kc, bt, sl, dec.Q, dec.max_seq_len, w, dec.k_top,
                                           idx=n_idx, val=n_val)

    outs = (s_idx, s_val, b_idx, b_val, pooled, n_idx, n_val)
    all_calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            all_calls()
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    for rep in range(3):
        run_pre(o_in)                      # eager work on other inputs into the same buffers
        b_idx.fill_(-5)
        pooled.fill_(3.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got.view(torch.int16 if got.dtype == torch.float16 else torch.int32),
                               want.view(torch.int16 if want.dtype == torch.float16 else torch.int32)), \
                f"replay {rep} differs"


def test_heads_major_query_layout():
    """q given as a [H, T, d] tensor viewed as [T, H, d] (strides T*d... ) is
    read through its strides."""
    inp = W.random_prefill(8, 12, 222, 64, 128, 16, mask_kind="random")
    qh = torch.from_numpy(np.ascontiguousarray(inp.q.transpose(1, 0, 2))).to(DEV)
    q_view = qh.permute(1, 0, 2)
    g = li.score_prefill(q_view, dev(inp.k), dev(inp.w), dev(inp.mask)).cpu().numpy()
    o = oracle.score_inputs(inp)
    check_scores(g, o, denominators(inp), where="heads-major")


def test_topk_row_len_and_short_rows():
    rng = np.random.default_rng(0)
    s = rng.integers(-20, 20, size=(50, 3000)).astype(np.float32)
    s[rng.random(s.shape) < 0.3] = -np.inf
    s[rng.random(s.shape) < 0.01] = np.nan
    s[rng.random(s.shape) < 0.02] = -0.0
    row_len = rng.integers(0, 3000, size=50).astype(np.int32)
    for k in (1, 17, 512, 2048):
        gi, gv = gpu_topk(dev(s), k, dev(row_len))
        check_topk_exact(gi, gv, s, k, row_len, where=f"row_len k={k}")


@pytest.mark.parametrize("n_cols", [1, 255, 1024, 1025, 2048, 4096, 5000, 8192, 12000, 16384, 16385,
                                    40000, 65535, 65536, 100003, 131072, 262144, 1000003])
def test_topk_row_lengths(n_cols):
    rng = np.random.default_rng(n_cols)
    rows = 8
    s = (rng.standard_normal((rows, n_cols)) * 10).astype(np.float32)
    s[:, ::7] = np.round(s[:, ::7])           # exact ties
    s[0, :] = 1.0                              # a row of equal scores
    s[1, rng.random(n_cols) < 0.5] = -np.inf
    s[2] = 24.0 + rng.random(n_cols).astype(np.float32)   # narrow: one binade
    s[3] = -np.abs(s[3])                       # all negative
    s[4, rng.random(n_cols) < 0.9] = 0.0       # mostly exact zeros (and -0)
    s[4, rng.random(n_cols) < 0.3] = -0.0
    s[5, :] = -np.inf                          # nothing selectable
    s[6, rng.random(n_cols) < 0.05] = np.nan
    for k in (1, 31, 64, 512, 2048):
        gi, gv = gpu_topk(dev(s), k)
        check_topk_exact(gi, gv, s, k, where=f"n_cols={n_cols} k={k}")


@pytest.mark.parametrize("n_cols", [700, 5000, 16384, 70000, 131072])
def test_topk_key_edge_values(n_cols):
    """Rows that mix the scores the order-preserving key treats specially:
    +-0, subnormals of both signs, +-FLT_MAX, +inf (tied), -inf and NaN
    payloads with either sign bit; row kernels and the long-row kernel
    equal the oracle bit for bit."""
    rng = np.random.default_rng(n_cols + 5)
    fmax = np.finfo(np.float32).max
    sub = np.array([0x00000001, 0x00000002, 0x007fffff, 0x80000001, 0x80000002, 0x807fffff],
                   dtype=np.uint32).view(np.float32)
    nans = np.array([0x7fc00000, 0xffc00000, 0x7f800001, 0xff800001, 0xffffffff],
                    dtype=np.uint32).view(np.float32)
    specials = np.concatenate([sub, nans, np.array([0.0, -0.0, fmax, -fmax, np.inf, -np.inf,
                                                    np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny],
                                                   dtype=np.float32)])
    rows = 5
    s = rng.standard_normal((rows, n_cols)).astype(np.float32)
    for r in range(rows):
        pos = rng.choice(n_cols, size=min(n_cols, 40 * len(specials)), replace=False)
        s[r, pos] = np.resize(specials, pos.size)
    with np.errstate(invalid="ignore"):           # the signaling NaN payloads
        s[1] *= np.float32(1e-39)                # the normal values pushed into the subnormal range
    s[2] = np.where(rng.random(n_cols) < 0.5, -0.0, 0.0).astype(np.float32)
    s[2, rng.random(n_cols) < 0.2] = sub[3]      # -0, +0 and the largest negative subnormal
    s[3, rng.random(n_cols) < 0.3] = np.inf      # many ties at +inf
    s[4] = -np.abs(s[4])                         # all negative, with -FLT_MAX and negative NaNs
    s[4, rng.random(n_cols) < 0.1] = nans[1]
    for k in (1, 64, 512, 2048):
        gi, gv = gpu_topk(dev(s), k)
        check_topk_exact(gi, gv, s, k, where=f"edge values n_cols={n_cols} k={k}")


def test_topk_long_rows_with_periodic_structure():
    """Long rows whose large scores sit in evenly spaced blocks of 256 keys,
    or everywhere but in them (a structure a sampled estimate of the k-th
    score would misjudge both ways), and rows with a few large values: equal
    bit for bit to the oracle's selection of the same f32 scores."""
    rng = np.random.default_rng(17)
    n = 131072
    s = rng.standard_normal((6, n)).astype(np.float32)
    blocks = np.zeros(n, dtype=bool)
    for j in range(32):
        b0 = j * (n - 256) // 31
        blocks[b0:b0 + 256] = True
    s[0, blocks] += 100.0          # large values only in the blocks
    s[1, ~blocks] += 100.0         # large values everywhere else
    s[2, blocks] = -np.inf         # the blocks hold nothing selectable
    s[3, rng.permutation(n)[:1500]] += 50.0   # fewer large values than k
    s[4, blocks] = 7.0             # the blocks tie on one value
    s[5, ::3] = np.round(s[5, ::3] * 4) / 4   # many ties near every score
    row_len = np.array([n, n, n, n, n - 1000, 70001], dtype=np.int32)
    for k in (64, 2048):
        for rl in (None, row_len):
            gi, gv = gpu_topk(dev(s), k, None if rl is None else dev(rl))
            check_topk_exact(gi, gv, s, k, rl, where=f"periodic k={k} row_len={rl is not None}")


def test_topk_long_rows_straddling_a_power_of_two():
    """Long rows whose best few thousand scores lie just either side of 2.0
    (whose float exponent bits all differ from those just below it), or of
    0, or on a few values only: the gathered set is ordered by bins of key
    distance, equal bit for bit to the oracle's selection."""
    rng = np.random.default_rng(23)
    n = 131072
    s = rng.uniform(0.0, 1.9, size=(4, n)).astype(np.float32)
    top = rng.permutation(n)[:4000]
    s[0, top] = rng.uniform(1.95, 2.05, size=4000).astype(np.float32)
    s[1, top] = rng.uniform(-0.01, 0.01, size=4000).astype(np.float32) + 3.0 * (rng.random(4000) < 0.3)
    s[2] = -s[2]
    s[2, top] = rng.uniform(-0.05, 0.05, size=4000).astype(np.float32)   # around zero, both signs
    s[3, top] = np.round(rng.uniform(1.95, 2.05, size=4000) * 64).astype(np.float32) / 64   # few values, ties
    for k in (100, 2048):
        gi, gv = gpu_topk(dev(s), k)
        check_topk_exact(gi, gv, s, k, where=f"straddle k={k}")


@pytest.mark.parametrize("n_rows", [8, 600])
def test_topk_rows_straddling_a_power_of_two(n_rows):
    """Register-resident rows (one per 1024 or per 512 threads) whose scores
    lie around 2.0, around 0 with both signs, or around 2.0 on a few values:
    the histogram bins are key distances, and the result is bit for bit the
    oracle's selection."""
    rng = np.random.default_rng(29 + n_rows)
    n = 5000
    s = (2.0 + 0.3 * rng.standard_normal((n_rows, n))).astype(np.float32)
    s[1::3] = (0.05 * rng.standard_normal((len(s[1::3]), n))).astype(np.float32)
    s[2::3] = np.round(s[2::3] * 32) / 32
    row_len = rng.integers(1, n + 1, size=n_rows).astype(np.int32)
    for k in (64, 512, 2048):
        for rl in (None, row_len):
            gi, gv = gpu_topk(dev(s), k, None if rl is None else dev(rl))
            check_topk_exact(gi, gv, s, k, rl, where=f"straddle rows={n_rows} k={k}")


@pytest.mark.parametrize("n_rows", [4, 520])
def test_topk_selection_ends_at_a_bin_edge(n_rows):
    """Rows whose best keys fill the top histogram bins exactly (k = 8, 15),
    or stop inside a bin of equal keys (k = 10), on the one-row-per-1024-
    threads and the two-rows-per-CU launch shapes."""
    rng = np.random.default_rng(5)
    n = 3000
    s = rng.uniform(1.0, 2.0, size=(n_rows, n)).astype(np.float32)
    for r in range(n_rows):
        pos = rng.permutation(n)[:15]
        s[r, pos[:3]] = 100.0
        s[r, pos[3:8]] = 50.0
        s[r, pos[8:15]] = 25.0
    for k in (8, 10, 15, 16):
        gi, gv = gpu_topk(dev(s), k)
        check_topk_exact(gi, gv, s, k, where=f"bin edge rows={n_rows} k={k}")



def test_topk_many_rows_heavy_ties():
    """Enough rows for the 512-thread launch shape (four rows per CU), with
    scores drawn from a few values: crowded bins take the general path,
    whose ordering of more than 512 selected keys is the bitonic sort, and
    equal scores are ordered by index."""
    rng = np.random.default_rng(11)
    n_rows, n = 600, 5000
    s = rng.integers(0, 7, size=(n_rows, n)).astype(np.float32)
    s[rng.random(s.shape) < 0.1] = -np.inf
    s[:4] = 3.0                                   # rows of one value
    for k in (100, 600, 2048):
        gi, gv = gpu_topk(dev(s), k)
        check_topk_exact(gi, gv, s, k, where=f"heavy ties rows={n_rows} k={k}")


# ------------------------------------------------------------ block ranking

@pytest.mark.parametrize("n_cols", [300, 5000, 16384, 40000, 131072])
def test_topk_blocks_rows(n_cols):
    """Block ranking on every top-k kernel (row kernels of 512 and 1024
    threads, the streaming long-row kernel): ties, -inf, NaN, row lengths
    and windows that cover the row, equal bit for bit to the oracle's
    ranking of the same f32 scores."""
    rng = np.random.default_rng(n_cols + 1)
    for rows in (6, 600) if n_cols <= 16384 else (6,):
        s = rng.integers(-30, 30, size=(rows, n_cols)).astype(np.float32)
        s[rng.random(s.shape) < 0.2] = -np.inf
        s[rng.random(s.shape) < 0.01] = np.nan
        s[0, :] = 2.0                                   # one value everywhere
        row_len = rng.integers(0, n_cols, size=rows, endpoint=True).astype(np.int32)
        row_len[1] = n_cols
        for init, local, k in [(1, 16, 64), (4, 0, 512), (0, 64, 100), (3000, 0, 2048), (2, 20000, 40)]:
            gi, gv = li.topk_blocks(dev(s), k, init, local, dev(row_len))
            torch.cuda.synchronize()
            oi, ov = oracle.topk_blocks(s, k, init, local, row_len)
            assert np.array_equal(gi.cpu().numpy(), oi), f"n_cols={n_cols} rows={rows} {init},{local},{k}"
            assert np.array_equal(gv.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("R,Q,H,lo,hi,init,local,k_top,mk", [
    (32, 1, 64, 1, 8192, 1, 64, 512, "none"),      # the decode shape, sink block + local window
    (8, 4, 64, 4, 16384, 4, 256, 2048, "none"),    # spec-decode: each query row's own local window
    (12, 2, 16, 1, 900, 2, 8, 30, "bias"),         # masked keys inside the windows are not selected
])
def test_fused_decode_blocks(R, Q, H, lo, hi, init, local, k_top, mk):
    width = hi + (-hi) % 8
    inp = W.random_decode(1400 + R + Q + H, R, Q, H, 128, 64, lo, hi, k_top, w_kind="uniform",
                          max_seq_len=width, mask_kind=mk)
    g = gpu_score(inp).cpu().numpy()
    gi, gv = li.score_topk_fused_decode_blocks(dev(inp.q), dev(inp.k_cache), dev(inp.block_table),
                                               dev(inp.seq_lens), inp.Q, inp.max_seq_len, dev(inp.w),
                                               k_top, init, local, dev(inp.mask))
    torch.cuda.synchronize()
    rl = oracle.decode_row_len(inp.seq_lens, inp.Q, inp.max_seq_len)
    oi, ov = oracle.topk_blocks(g, k_top, init, local, rl)
    assert np.array_equal(gi.cpu().numpy(), oi)
    assert np.array_equal(gv.cpu().numpy().view(np.uint32), ov.view(np.uint32))
    # the forced windows are present in every row that can hold them
    gi = gi.cpu().numpy()
    for t in range(gi.shape[0]):
        n = int(rl[t])
        forced = [s for s in list(range(min(init, n))) + list(range(max(n - local, 0), n))
                  if np.isfinite(g[t, s])]
        if len(set(forced)) <= k_top:
            assert set(forced) <= set(gi[t].tolist())


# ------------------------------------------------------------ streaming score + top-k

def _stream_vs_fused(inp, where):
    """The streaming entry point against the fused one (score rows in a
    workspace, then the top-k kernel), bit for bit."""
    fi, fv = gpu_fused(inp)
    si, sv = li.score_topk_stream_prefill(dev(inp.q), dev(inp.k), dev(inp.w), inp.k_top, dev(inp.mask),
                                          dev(inp.vis_len))
    torch.cuda.synchronize()
    si, sv = si.cpu().numpy(), sv.cpu().numpy()
    if not np.array_equal(si, fi):
        r = int(np.argwhere((si != fi).any(axis=1))[0, 0])
        c = int(np.argwhere(si[r] != fi[r])[0, 0])
        raise AssertionError(f"{where}: streaming index differs at row {r} pos {c}: {si[r, c-2:c+3]} vs {fi[r, c-2:c+3]}")
    assert np.array_equal(sv.view(np.uint32), fv.view(np.uint32)), f"{where}: streaming values differ"
    return si, sv


@pytest.mark.parametrize("T,P,H,d,k_top,mask,wk,vis", PREFILL_CASES,
                         ids=[f"T{c[0]}P{c[1]}H{c[2]}d{c[3]}k{c[4]}-{c[5]}-{c[6]}-{c[7]}" for c in PREFILL_CASES])
def test_stream_random_prefill(T, P, H, d, k_top, mask, wk, vis):
    inp = W.random_prefill(1000 + T + P + H + d, T, P, H, d, k_top, mask_kind=mask, w_kind=wk, vis_kind=vis)
    _stream_vs_fused(inp, inp.name)


@pytest.mark.parametrize("T,P,H,d,k_top,mask,wk", [
    (37, 40000, 64, 128, 2048, "random", "signed"),    # two key chunks, lists compacted many times
    (20, 100000, 64, 128, 512, "bias", "uniform"),     # four chunks
    (9, 131072, 16, 64, 2048, "causal", "signed"),
    (5, 70001, 48, 96, 100, "random", "signed"),       # padded heads and head dimension
    (6, 50000, 20, 256, 1, "none", "uniform"),         # head dimension 256, k_top = 1
    (64, 33000, 4, 64, 2000, "zero", "signed"),        # four heads: 32 rows a workgroup
])
def test_stream_long_rows(T, P, H, d, k_top, mask, wk):
    inp = W.random_prefill(2000 + T + H + d, T, P, H, d, k_top, mask_kind=mask, w_kind=wk)
    _stream_vs_fused(inp, inp.name)


def test_stream_adversarial_rows():
    """Rows whose every score ties (q = 0: only the index decides, so the
    bound search resolves entries to the last digit), rows whose scores rise
    along the keys (every key joins its list; compactions all the way), rows
    with fewer visible keys than k_top and rows with none."""
    T, P, H, d = 12, 70000, 4, 64
    base = W.random_prefill(31, T, P, H, d, 2048, mask_kind="bias", w_kind="uniform")
    ties = dataclasses.replace(base, q=np.zeros_like(base.q), mask=np.zeros((T, P), np.float16))
    si, _ = _stream_vs_fused(ties, "all scores equal")
    assert np.array_equal(si, np.tile(np.arange(2048, dtype=np.int32), (T, 1)))
    q = np.zeros((T, H, d), np.float16)
    q[:, :, 0] = 1
    k = np.zeros((P, d), np.float16)
    k[:, 0] = (np.arange(P) * (8.0 / P)).astype(np.float16)       # scores rise with the key
    rising = dataclasses.replace(base, q=q, k=k, w=np.full(H, 0.125, np.float32), mask=None)
    _stream_vs_fused(rising, "rising scores")
    vis = np.array([0, 1, 5, 2047, 2048, 2049, 40000, 69999, 70000, 3, 0, 12345], np.int32)
    few = dataclasses.replace(base, vis_len=vis)
    si, _ = _stream_vs_fused(few, "short rows")
    assert np.all(si[0] == -1) and np.all(si[10] == -1)


@pytest.mark.parametrize("name", ["tiny", "prefill_causal", "long_chunk"])
def test_stream_workloads(name):
    """The streaming path on the contiguous workloads equals the fused path
    bit for bit, and never selects a masked key."""
    inp = getattr(W, name)()
    si, _ = _stream_vs_fused(inp, name)
    sel = np.where(si >= 0, si, 0)
    picked = np.take_along_axis(inp.mask, sel, axis=1).astype(np.float32)
    assert not np.any(np.isneginf(picked) & (si >= 0))


# ------------------------------------------------------------ pooled keys

@pytest.mark.parametrize("n,d,pool,kind", [
    (1, 8, 1, "normal"), (7, 64, 3, "normal"), (1000, 128, 4, "normal"), (4099, 128, 64, "normal"),
    (513, 136, 7, "bits"), (2048, 256, 2, "bits"), (3000, 64, 513, "normal"), (97, 128, 100, "bits"),
    (20000, 128, 8192, "normal"),
])
def test_pool_keys_bit_exact(n, d, pool, kind):
    """Mean pooling on the GPU equals the oracle bit for bit: N(0,1) keys,
    and keys of random finite f16 bit patterns (subnormals, values near
    65504, both signs); full and short last windows."""
    rng = np.random.default_rng(n + d + pool)
    if kind == "normal":
        k = rng.standard_normal((n, d)).astype(np.float16)
    else:
        raw = rng.integers(0, 0x10000, size=(n, d)).astype(np.uint16)
        raw[(raw & 0x7c00) == 0x7c00] &= 0x3fff
        k = raw.view(np.float16)
    got = li.pool_keys(dev(k), pool).cpu().numpy()
    want = pooling.pool_keys(k, pool)
    assert np.array_equal(got.view(np.uint16), want.view(np.uint16))


def test_pool_keys_strided_and_scored():
    """Row strides past head_dim on both sides, and the pooled keys fed to
    the score: pooled on the GPU then scored equals the oracle's pooled keys
    scored by the oracle."""
    rng = np.random.default_rng(3)
    raw = rng.standard_normal((1200, 160)).astype(np.float16)
    k_view = dev(raw)[:, :128]                        # row stride 160
    out = torch.empty((300, 136), dtype=torch.float16, device=DEV)[:, :128]
    got = li.pool_keys(k_view, 4, out=out)
    torch.cuda.synchronize()
    want = pooling.pool_keys(raw[:, :128], 4)
    assert np.array_equal(got.cpu().numpy().view(np.uint16), want.view(np.uint16))
    inp = W.random_prefill(5, 9, 300, 64, 128, 16, mask_kind="random", w_kind="uniform")
    inp = dataclasses.replace(inp, k=want)
    g = li.score_prefill(dev(inp.q), got.contiguous(), dev(inp.w), dev(inp.mask)).cpu().numpy()
    check_scores(g, oracle.score_inputs(inp), denominators(inp), where="pooled keys scored")


# ------------------------------------------------------------ full workloads

def _sampled_check(inp, rows, where):
    g_t = gpu_score(inp)
    g = g_t.cpu().numpy()
    o = oracle.score_rows(inp, rows)
    den = denominators(inp, rows)
    err = check_scores(g[rows], o, den, where=where)
    gi, gv = gpu_topk(g_t, inp.k_top)
    check_topk_exact(gi, gv, g, inp.k_top, where=where)
    check_topk_vs_f64(gi[rows], o, den, inp.k_top, where=where)
    fi, fv = gpu_fused(inp)
    assert np.array_equal(fi, gi), f"{where}: fused indices differ from score + top-k"
    # masked keys are never selected; visible-count padding is exact
    if inp.mask is not None:
        m = inp.mask
        sel = np.where(gi >= 0, gi, 0)
        picked = np.take_along_axis(m, sel, axis=1)
        assert not np.any(np.isneginf(picked.astype(np.float32)) & (gi >= 0))
    print(f"{where}: max scaled error {err:.2e} over {len(rows)} sampled rows")
    return g


def test_workload_decode():
    inp = W.decode()
    rows = np.arange(inp.R * inp.Q)
    _sampled_check(inp, rows, "decode")


def test_workload_spec_decode():
    """Every one of the 128 rows against the oracle."""
    inp = W.spec_decode()
    rows = np.arange(inp.R * inp.Q)
    _sampled_check(inp, rows, "spec_decode")


def test_workload_prefill_causal():
    """64 rows in contiguous stripes: every row slot of the kernel's row
    groups (8 rows each), the first rows (one key chunk), rows around the
    k_top = 2048 visible-key boundary, and the last rows (every key chunk)."""
    inp = W.prefill_causal()
    rows = np.concatenate([np.arange(0, 16), np.arange(2040, 2056), np.arange(5000, 5016),
                           np.arange(8176, 8192)])
    g = _sampled_check(inp, rows, "prefill_causal")
    # causal: row t has exactly t+1 finite entries
    finite = np.isfinite(g).sum(axis=1)
    assert np.array_equal(finite, np.arange(1, 8193))


def test_workload_long_chunk():
    """64 rows in contiguous stripes at the start, middle and end of the
    chunk (every row slot of the kernel's row groups; every row spans every
    key chunk)."""
    inp = W.long_chunk()
    rows = np.concatenate([np.arange(0, 24), np.arange(504, 520), np.arange(1000, 1024)])
    _sampled_check(inp, rows, "long_chunk")


def test_peak_probes_measure_something():
    """The measured-peak probes run and report plausible rates (well above a
    tenth and below twice the published 2.5 PFLOP/s and 8 TB/s)."""
    from sparse_attention_lightning_indexer_amd.peak_probe import probe_peaks
    r = probe_peaks(DEV, mfma_iters=200, read_bytes=256 << 20, repeats=1)
    assert 250.0 < r["mfma_f16_tflops"] < 5000.0, r
    assert 800.0 < r["read_gbs"] < 16000.0, r


def test_floor_probes():
    """The launch-floor probes run; the row probe writes each row's first k
    entries of its visible prefix (-inf past it) and their indices."""
    from sparse_attention_lightning_indexer_amd import peak_probe as pp
    pp.empty(3, 1024)
    g = torch.Generator().manual_seed(5)
    sc = torch.randn((6, 3000), generator=g).to(DEV)
    lens = torch.tensor([3000, 0, 1, 700, 2999, 64], dtype=torch.int32).to(DEV)
    k = 1100
    v = torch.empty((6, k), dtype=torch.float32, device=DEV)
    i = torch.empty((6, k), dtype=torch.int32, device=DEV)
    pp.rows(sc, lens, k, v, i)
    torch.cuda.synchronize()
    want = sc[:, :k].clone()
    for r, n in enumerate(lens.tolist()):
        want[r, n:] = -math.inf
    assert torch.equal(v, want)
    assert torch.equal(i.cpu(), torch.arange(k, dtype=torch.int32).expand(6, k))
    buf = torch.zeros(1 << 20, dtype=torch.float32, device=DEV)
    pp.read(buf, pp.sink_for(DEV))
    torch.cuda.synchronize()


@pytest.mark.parametrize("seed", range(40))
def test_topk_randomized_sweep(seed):
    """Seeded random shapes through every top-k kernel (register rows of 512
    and 1024 threads, the long-row kernel with and without its sampled pass,
    block ranking): row lengths around the kernels' limits, k from 1 to
    2048, and score mixes of ties, -inf, NaN, both signs and narrow ranges;
    bit for bit the oracle's selection of the same f32 scores."""
    rng = np.random.default_rng(1000 + seed)
    n_cols = int(rng.choice([3000, 9000, 16384, 16385, 40000, 65535, 65536, 70001, 131072]))
    n_rows = int(rng.choice([3, 8, 600])) if n_cols <= 16384 else int(rng.choice([3, 8]))
    k = int(rng.choice([1, 7, 64, 333, 512, 1024, 2048]))
    kind = seed % 4
    if kind == 0:
        s = rng.standard_normal((n_rows, n_cols)) * rng.uniform(0.1, 100.0)
    elif kind == 1:
        s = rng.integers(-50, 50, size=(n_rows, n_cols)).astype(np.float64)   # heavy ties
    elif kind == 2:
        s = 2.0 + rng.standard_normal((n_rows, n_cols)) * 0.02                  # narrow, around 2.0
    else:
        s = np.exp(rng.standard_normal((n_rows, n_cols)) * 3.0) * np.sign(rng.standard_normal((n_rows, n_cols)))
    s = s.astype(np.float32)
    s[rng.random(s.shape) < rng.uniform(0.0, 0.5)] = -np.inf
    s[rng.random(s.shape) < 0.001] = np.nan
    row_len = rng.integers(0, n_cols + 1, size=n_rows).astype(np.int32)
    row_len[0] = n_cols
    gi, gv = gpu_topk(dev(s), k, dev(row_len))
    check_topk_exact(gi, gv, s, k, row_len, where=f"sweep seed={seed} n={n_cols} rows={n_rows} k={k} kind={kind}")
    if seed % 3 == 0:
        init, local = int(rng.integers(0, 300)), int(rng.integers(0, 300))
        bi, bv = li.topk_blocks(dev(s), k, init, local, dev(row_len))
        torch.cuda.synchronize()
        oi, ov = oracle.topk_blocks(s, k, init, local, row_len)
        assert np.array_equal(bi.cpu().numpy(), oi), f"sweep blocks seed={seed}"
        assert np.array_equal(bv.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("seed", range(64))
def test_score_randomized_sweep(seed):
    """Seeded random shapes through the score kernels and the fused paths:
    prefill and paged decode, head counts from 1 to 100 (compiled, padded
    and in passes), head dimensions from 8 to 256, every mask and weight
    kind, visible prefixes, query lengths and block sizes; scores against
    the fp64 oracle, top-k bit for bit, fused equal to score then top-k,
    and (prefill, one pass over the heads) the streaming path equal to the
    fused one."""
    rng = np.random.default_rng(2000 + seed)
    H = int(rng.choice([1, 3, 4, 8, 12, 16, 32, 48, 64, 100]))
    d = int(rng.choice([8, 24, 64, 72, 128, 200, 256]))
    w_kind = str(rng.choice(["uniform", "equal", "signed", "pow2"]))
    if seed % 2 == 0:
        T, P = int(rng.integers(1, 40)), int(rng.integers(1, 700))
        k_top = int(rng.integers(1, min(P, 2048) + 1))
        mask_kind = str(rng.choice(["none", "zero", "random", "causal", "bias", "all_inf"]))
        vis_kind = str(rng.choice(["none", "random"]))
        inp = W.random_prefill(3000 + seed, T, P, H, d, k_top, mask_kind=mask_kind, w_kind=w_kind, vis_kind=vis_kind)
        where = f"sweep prefill seed={seed} T={T} P={P} H={H} d={d} k={k_top} {mask_kind}/{w_kind}/{vis_kind}"
        if H <= (32 if d > 128 else 64):
            fi, fv = gpu_fused(inp)
            si, sv = li.score_topk_stream_prefill(dev(inp.q), dev(inp.k), dev(inp.w), k_top, dev(inp.mask),
                                                  dev(inp.vis_len))
            torch.cuda.synchronize()
            assert np.array_equal(si.cpu().numpy(), fi), f"{where}: streaming indices differ"
            assert np.array_equal(sv.cpu().numpy().view(np.uint32), fv.view(np.uint32)), f"{where}: streaming values differ"
    else:
        R, Q = int(rng.integers(1, 9)), int(rng.choice([1, 2, 4]))
        bs = int(rng.choice([1, 4, 16, 64]))
        lo = int(rng.integers(0, 300))
        hi = lo + int(rng.integers(0, 500))
        k_top = int(rng.integers(1, 257))
        mask_kind = str(rng.choice(["none", "random", "bias"]))
        inp = W.random_decode(3000 + seed, R, Q, H, d, bs, lo, hi, k_top, w_kind=w_kind, mask_kind=mask_kind)
        where = f"sweep decode seed={seed} R={R} Q={Q} H={H} d={d} bs={bs} len={lo}..{hi} k={k_top} {mask_kind}/{w_kind}"
    _full_check(inp, where)
