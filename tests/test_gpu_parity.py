"""GPU parity: the HIP path (through the C-ABI) against the CPU oracle on the
same seeded inputs.  See gpu_helpers.py for the comparison bars."""
import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
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
# key tiles spanning several row groups (and, with one query row, more tiles
# than its score staging area holds); the last two shapes take the chunked
# kernel instead (block size below 4, more than 2048 row groups).
STREAM_CASES = [
    # R, Q, H, d, block_size, len_lo, len_hi, k_top
    (700, 1, 64, 128, 64, 1, 1500, 64),      # many short requests per workgroup
    (48, 1, 64, 128, 64, 9000, 14000, 128),  # > 16 tiles per workgroup: staging flushes
    (300, 4, 64, 128, 16, 4, 1200, 32),      # general mapping: q reloaded per row group
    (200, 2, 32, 64, 37, 1, 3000, 40),       # block size not a power of two
    (100, 3, 8, 128, 4, 1, 2000, 20),        # smallest block size of the persistent kernel
    (40, 16, 4, 64, 16, 100, 3000, 24),      # 16 rows per group: a flush every 2 tiles
    (60, 9, 64, 128, 64, 9, 2500, 16),       # two row groups per request
    (50, 1, 16, 64, 2, 1, 800, 10),          # block size 2: chunked kernel
    (2100, 1, 4, 64, 16, 1, 200, 8),         # 2100 row groups: per-group words fill much of the LDS
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
    inp = W.random_decode(42, 4, 4, 64, 128, 64, 50, 400, 32, w_kind="signed", mask_kind="bias")
    _full_check(inp, inp.name)


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
                                    40000, 131072])
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
    inp = W.spec_decode()
    rows = np.array([0, 1, 2, 3, 37, 38, 64, 127])
    _sampled_check(inp, rows, "spec_decode")


def test_workload_prefill_causal():
    inp = W.prefill_causal()
    rows = np.array([0, 1, 7, 8, 100, 2046, 2047, 2048, 4095, 5000, 8190, 8191])
    g = _sampled_check(inp, rows, "prefill_causal")
    # causal: row t has exactly t+1 finite entries
    finite = np.isfinite(g).sum(axis=1)
    assert np.array_equal(finite, np.arange(1, 8193))


def test_workload_long_chunk():
    inp = W.long_chunk()
    rows = np.array([0, 1, 511, 1022, 1023])
    _sampled_check(inp, rows, "long_chunk")


def test_peak_probes_measure_something():
    """The measured-peak probes run and report plausible rates (well above a
    tenth and below twice the published 2.5 PFLOP/s and 8 TB/s)."""
    r = li.probe_peaks(DEV, mfma_iters=200, read_bytes=256 << 20, repeats=1)
    assert 250.0 < r["mfma_f16_tflops"] < 5000.0, r
    assert 800.0 < r["read_gbs"] < 16000.0, r
