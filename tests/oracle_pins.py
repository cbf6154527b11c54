"""Pins for the CPU oracle: checks against what the pages and mathematics fix,
not against the oracle itself.

Each ``pin_*`` takes a loaded oracle library (ctypes handle) and raises
AssertionError on a mismatch.  ``test_oracle_pins.py`` runs them on the real
oracle; ``test_oracle_mutants.py`` runs them on oracle builds with a planted
mistake and expects at least one of them to fail for every mutant.
"""
from __future__ import annotations

import numpy as np

import oracle
from oracle import materialize, pooling
import workloads as W
from conftest import golden_array, load_golden


def _close(a, b, rtol=1e-12, atol=1e-12):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    ia, ib = np.isneginf(a), np.isneginf(b)
    assert np.array_equal(ia, ib), "different -inf sets"
    fa, fb = a[~ia], b[~ib]
    assert np.all(np.isfinite(fa)) and np.all(np.isfinite(fb)), "non-finite visible score"
    err = np.abs(fa - fb) - (atol + rtol * np.abs(fb))
    assert np.all(err <= 0), f"max abs diff {np.max(np.abs(fa - fb)) if fa.size else 0}"


# ------------------------------------------------------------ worked examples

def pin_worked_example_score(lib):
    g = load_golden("score_worked_example.json")
    q = golden_array(g["q"]).astype(np.float16)
    k = golden_array(g["k"]).astype(np.float16)
    w = golden_array(g["w"]).astype(np.float32)
    mask = golden_array(g["mask"]).astype(np.float16)
    got = oracle.score_prefill(q, k, w, mask, lib=lib)
    want = golden_array(g["score"])
    assert np.array_equal(got, want), (got, want)


def pin_worked_example_topk(lib):
    g = load_golden("score_worked_example.json")
    score = golden_array(g["score"])
    for kk, exp in g["topk"].items():
        idx, val = oracle.topk(score, int(kk), lib=lib)
        assert np.array_equal(idx, np.array(exp["idx"])), (kk, idx)
        assert np.array_equal(val, golden_array(exp["val"])), (kk, val)
        idx32, val32 = oracle.topk(score.astype(np.float32), int(kk), lib=lib)
        assert np.array_equal(idx32, idx)
        assert np.array_equal(val32, val.astype(np.float32))


def pin_topk_ties(lib):
    g = load_golden("topk_ties.json")
    row = golden_array(g["row"])[None, :]
    for kk, exp in g["cases"].items():
        for dt in (np.float64, np.float32):
            idx, val = oracle.topk(row.astype(dt), int(kk), lib=lib)
            assert idx.tolist() == [exp["idx"]], (kk, dt, idx)
            want = golden_array(exp["val"]).astype(dt)
            assert np.array_equal(val[0], want), (kk, dt, val)
            # the sign of zero is reported as stored
            assert np.array_equal(np.signbit(val[0]), np.signbit(want))


def pin_decode_mask_example(lib):
    """Masked paged decode worked by hand: the mask row is the query row
    r*Q + j, finite entries are biases added after the head sum (outside the
    rectifier), -inf hides a key, and keys past the visible length ignore
    the mask."""
    g = load_golden("decode_mask_example.json")
    q = golden_array(g["q"]).astype(np.float16)
    kc = golden_array(g["k_cache"]).astype(np.float16)
    bt = np.array(g["block_table"], dtype=np.int32)
    sl = np.array(g["seq_lens"], dtype=np.int32)
    w = golden_array(g["w"]).astype(np.float32)
    mask = golden_array(g["mask"]).astype(np.float16)
    got = oracle.score_decode(q, kc, bt, sl, g["Q"], g["max_seq_len"], w, mask, lib=lib)
    assert np.array_equal(got, golden_array(g["score"])), got


def pin_decode_visibility_example(lib):
    g = load_golden("decode_visibility_example.json")
    q = golden_array(g["q"]).astype(np.float16)
    kc = golden_array(g["k_cache"]).astype(np.float16)
    bt = np.array(g["block_table"], dtype=np.int32)
    sl = np.array(g["seq_lens"], dtype=np.int32)
    w = golden_array(g["w"]).astype(np.float32)
    got = oracle.score_decode(q, kc, bt, sl, g["Q"], g["max_seq_len"], w, lib=lib)
    assert np.array_equal(got, golden_array(g["score"])), got


# ------------------------------------------------------------ f16 decoding

def pin_every_f16_through_relu(lib):
    """H=1, d=1, k=1, w=1: score = max(x, 0) for every one of the 65536 f16
    bit patterns x (compared with numpy's own f16 -> f64 widening)."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = bits.view(np.float16)
    finite = np.isfinite(x)
    x = x[finite]
    q = x.reshape(-1, 1, 1)
    k = np.ones((1, 1), dtype=np.float16)
    got = oracle.score_prefill(q, k, np.ones(1, np.float32), lib=lib)[:, 0]
    want = np.maximum(x.astype(np.float64), 0.0)
    assert np.array_equal(got, want)
    # and through the key side with a negative weight: -1 * max(-x, 0)
    kq = x.reshape(-1, 1)
    got2 = oracle.score_prefill(-np.ones((1, 1, 1), np.float16), kq,
                                -np.ones(1, np.float32), lib=lib)[0]
    assert np.array_equal(got2, -np.maximum(-x.astype(np.float64), 0.0))


# ------------------------------------------------------------ closed forms

def pin_sign_flip_identity(lib):
    """ReLU(x) - ReLU(-x) = x, so score(q) - score(-q) = sum_h w_h (q_h . k):
    a plain matrix product, for any weights (mask-free)."""
    for seed, (T, P, H, d) in enumerate([(3, 7, 4, 16), (5, 9, 3, 8), (2, 33, 64, 128)]):
        inp = W.random_prefill(seed, T, P, H, d, 4, mask_kind="none", w_kind="signed")
        a = oracle.score_prefill(inp.q, inp.k, inp.w, lib=lib)
        b = oracle.score_prefill(-inp.q, inp.k, inp.w, lib=lib)
        qw = np.einsum("thd,h->td", inp.q.astype(np.float64), inp.w.astype(np.float64))
        lin = qw @ inp.k.astype(np.float64).T
        _close(a - b, lin, rtol=1e-10, atol=1e-10)


def pin_scale_identity(lib):
    """Every head weight 1/sqrt(d) equals 1/sqrt(d) times the unweighted sum of
    rectified heads (the b11372 note on the lightning indexer).  At d = 64 the
    scale is 2^-3, so the two agree bit for bit."""
    for d in (64, 128):
        inp = W.random_prefill(7, 6, 40, 8, d, 4, mask_kind="random")
        s = np.float32(1.0 / np.sqrt(d))
        a = oracle.score_prefill(inp.q, inp.k, np.full(8, s, np.float32), inp.mask, lib=lib)
        b = oracle.score_prefill(inp.q, inp.k, np.ones(8, np.float32), inp.mask, lib=lib)
        m = np.where(np.isneginf(inp.mask), 0, inp.mask).astype(np.float64)
        if d == 64:
            assert np.array_equal(a - m, (b - m) * float(s))
        else:
            _close(a - m, (b - m) * float(s), rtol=1e-14, atol=1e-14)


def pin_zero_cases(lib):
    """q = 0, k = 0 or w = 0 leave score = mask on visible entries."""
    inp = W.random_prefill(3, 5, 21, 4, 16, 4, mask_kind="bias", w_kind="signed")
    want = inp.mask.astype(np.float64)
    for q, k, w in [(np.zeros_like(inp.q), inp.k, inp.w),
                    (inp.q, np.zeros_like(inp.k), inp.w),
                    (inp.q, inp.k, np.zeros_like(inp.w))]:
        got = oracle.score_prefill(q, k, w, inp.mask, lib=lib)
        assert np.array_equal(got, want)


def pin_single_head_single_dim(lib):
    """H = 1, d = 1: score = w * max(q k, 0) + mask."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((7, 1, 1)).astype(np.float16)
    k = rng.standard_normal((11, 1)).astype(np.float16)
    w = np.array([0.75], np.float32)
    mask = (rng.standard_normal((7, 11)) * 3).astype(np.float16)
    got = oracle.score_prefill(q, k, w, mask, lib=lib)
    want = 0.75 * np.maximum(q[:, 0, 0].astype(np.float64)[:, None] * k[:, 0].astype(np.float64)[None, :], 0) + mask
    assert np.array_equal(got, want)


def pin_rectify_each_head_before_sum(lib):
    """Head A scores +a, head B scores -b with b > a, w = 1: the score is a
    (rectify, then sum), not ReLU(a - b) = 0."""
    q = np.array([[[3.0, 0.0], [-5.0, 0.0]]], np.float16)   # heads A, B
    k = np.array([[1.0, 0.0]], np.float16)
    got = oracle.score_prefill(q, k, np.ones(2, np.float32), lib=lib)
    assert got[0, 0] == 3.0


def pin_one_hot_heads(lib):
    """One-hot q per head and one-hot keys: score[t][s] = sum of w_h over the
    heads whose hot coordinate matches the key's, times the product of the
    two hot values when positive."""
    H, d = 6, 8
    rng = np.random.default_rng(11)
    hot_q = rng.integers(0, d, size=(4, H))
    val_q = rng.choice([-2.0, -1.0, 0.5, 1.0, 2.0], size=(4, H))
    hot_k = rng.integers(0, d, size=9)
    val_k = rng.choice([-1.0, 1.0, 3.0], size=9)
    q = np.zeros((4, H, d), np.float16)
    for t in range(4):
        for h in range(H):
            q[t, h, hot_q[t, h]] = val_q[t, h]
    k = np.zeros((9, d), np.float16)
    k[np.arange(9), hot_k] = val_k
    w = np.arange(1, H + 1, dtype=np.float32) / 4
    got = oracle.score_prefill(q, k, w, lib=lib)
    want = np.zeros((4, 9))
    for t in range(4):
        for s in range(9):
            for h in range(H):
                if hot_q[t, h] == hot_k[s]:
                    want[t, s] += w[h] * max(val_q[t, h] * val_k[s], 0.0)
    assert np.array_equal(got, want)


# ------------------------------------------------------------ cross-checks

def pin_materialise_then_sum(lib):
    """The per-head 'materialise then sum' scheme the pages replaced (a
    library matmul over token-head rows) gives the same scores."""
    cases = [
        W.random_prefill(1, 9, 37, 4, 64, 8, mask_kind="random", w_kind="uniform"),
        W.random_prefill(2, 5, 50, 64, 128, 8, mask_kind="bias", w_kind="signed", vis_kind="random"),
        W.random_prefill(3, 4, 31, 3, 16, 8, mask_kind="causal", w_kind="pow2"),
        W.tiny(),
    ]
    for inp in cases:
        a = oracle.score_prefill(inp.q, inp.k, inp.w, inp.mask, inp.vis_len, lib=lib)
        b = materialize.score_prefill(inp.q, inp.k, inp.w, inp.mask, inp.vis_len)
        _close(a, b, rtol=1e-12, atol=1e-12)


def pin_invariants(lib):
    """With every w_h >= 0: score >= mask on visible entries; -inf exactly
    where the mask is -inf; raising one weight never lowers a score."""
    inp = W.random_prefill(4, 12, 45, 8, 32, 8, mask_kind="bias", w_kind="uniform")
    a = oracle.score_prefill(inp.q, inp.k, inp.w, inp.mask, lib=lib)
    m = inp.mask.astype(np.float64)
    vis = ~np.isneginf(m)
    assert np.array_equal(np.isneginf(a), ~vis)
    assert np.all(a[vis] >= m[vis])
    w2 = inp.w.copy()
    w2[3] += 0.5
    b = oracle.score_prefill(inp.q, inp.k, w2, inp.mask, lib=lib)
    assert np.all(b[vis] >= a[vis])


def pin_exact_integer_inputs(lib):
    """Integer q, k in {-2..2} and power-of-two weights make every term exact,
    so the oracle must equal exact integer arithmetic (numpy int64)."""
    inp = W.integer_prefill(9, 6, 40, 64, 128, 8, mask_kind="random")
    got = oracle.score_prefill(inp.q, inp.k, inp.w, inp.mask, lib=lib)
    qi = inp.q.astype(np.int64)
    ki = inp.k.astype(np.int64)
    dots = np.einsum("thd,sd->ths", qi, ki)                   # exact integers
    e = (-np.log2(inp.w)).astype(np.int64)                    # w_h = 2^-e_h
    scaled = np.maximum(dots, 0) << (7 - e)[None, :, None]    # units of 2^-7
    want = scaled.sum(axis=1).astype(np.float64) / 128.0
    want[np.isneginf(inp.mask.astype(np.float64))] = -np.inf
    assert np.array_equal(got, want)


def pin_key_permutation(lib):
    """Permuting the keys permutes the score columns (bit for bit)."""
    inp = W.random_prefill(12, 5, 29, 4, 16, 4, mask_kind="bias")
    perm = np.random.default_rng(0).permutation(29)
    a = oracle.score_prefill(inp.q, inp.k, inp.w, inp.mask, lib=lib)
    b = oracle.score_prefill(inp.q, inp.k[perm], inp.w, inp.mask[:, perm], lib=lib)
    assert np.array_equal(a[:, perm], b)


def pin_decode_matches_materialise(lib):
    """Paged decode through a permuted block table vs gathering each
    request's keys and scoring them with the materialised scheme; the cache
    slots no request owns are NaN, so a stray read would show."""
    cases = [(3, 1, 4, 16, 8, 5, 40, "none"),
             (2, 4, 8, 32, 16, 3, 50, "none"),
             (4, 3, 64, 128, 64, 1, 130, "none"),
             # masks: finite biases with some -inf, and 0 / -inf; the mask row
             # of query j of request r is row r*Q + j
             (3, 2, 4, 16, 8, 5, 40, "bias"),
             (4, 3, 8, 32, 16, 2, 60, "random"),
             (3, 4, 64, 128, 64, 4, 100, "bias")]
    for seed, (R, Q, H, d, bs, lo, hi, mk) in enumerate(cases):
        inp = W.random_decode(seed, R, Q, H, d, bs, lo, hi, 8, w_kind="signed", mask_kind=mk)
        a = oracle.score_decode(inp.q, inp.k_cache, inp.block_table, inp.seq_lens,
                                inp.Q, inp.max_seq_len, inp.w, inp.mask, lib=lib)
        b = materialize.score_decode(inp.q, inp.k_cache, inp.block_table, inp.seq_lens,
                                     inp.Q, inp.max_seq_len, inp.w, inp.mask)
        _close(a, b, rtol=1e-12, atol=1e-12)


def pin_decode_equals_prefill_layout(lib):
    """One request's keys paged through a permuted table give bit-identical
    scores to the same keys stored contiguously, with query j seeing the
    first P - T + 1 + j keys."""
    inp = W.random_prefill(21, 4, 70, 8, 32, 8, mask_kind="none", w_kind="uniform")
    paged = W.paged_from_prefill(inp, 16)
    a = oracle.score_decode(paged.q, paged.k_cache, paged.block_table, paged.seq_lens,
                            paged.Q, paged.max_seq_len, paged.w, lib=lib)
    vis = np.array([70 - 4 + 1 + j for j in range(4)], np.int32)
    b = oracle.score_prefill(inp.q, inp.k, inp.w, None, vis, lib=lib)
    assert np.array_equal(a, b)


def pin_topk_against_library_sort(lib):
    """Top-k equals a numpy lexsort by (score desc, index asc) over the
    selectable entries, on rows with heavy ties, -inf, NaN and row lengths."""
    rng = np.random.default_rng(3)
    n_rows, n_cols = 40, 300
    s = rng.integers(-6, 6, size=(n_rows, n_cols)).astype(np.float64)
    s[rng.random(s.shape) < 0.15] = -np.inf
    s[rng.random(s.shape) < 0.02] = np.nan
    s[rng.random(s.shape) < 0.05] = -0.0
    row_len = rng.integers(0, n_cols, size=n_rows, endpoint=True).astype(np.int32)
    for k_top in (1, 7, 64, 299, 300, 400):
        for dt in (np.float64, np.float32):
            idx, val = oracle.topk(s.astype(dt), k_top, row_len, lib=lib)
            for t in range(n_rows):
                row = s[t, : row_len[t]]
                ok = np.nonzero(~np.isnan(row) & ~np.isneginf(row))[0]
                order = ok[np.lexsort((ok, -row[ok]))][:k_top]
                want = np.full(k_top, -1)
                want[: len(order)] = order
                assert np.array_equal(idx[t], want), (k_top, dt, t)
                wv = np.full(k_top, -np.inf)
                wv[: len(order)] = row[order]
                assert np.array_equal(val[t], wv.astype(dt))


def pin_topk_blocks_example(lib):
    g = load_golden("topk_blocks_example.json")
    row = golden_array(g["row"])[None, :]
    for c in g["cases"]:
        for dt in (np.float64, np.float32):
            idx, val = oracle.topk_blocks(row.astype(dt), c["k"], c["init"], c["local"],
                                          np.array([c["row_len"]], np.int32), lib=lib)
            assert idx.tolist() == [c["idx"]], (c, dt, idx)
            assert np.array_equal(val[0], golden_array(c["val"]).astype(dt)), (c, dt, val)


def pin_topk_blocks_against_library_sort(lib):
    """Block ranking equals a numpy lexsort by (not forced, -score for the
    unforced, index) over the selectable candidates, on rows with heavy
    ties, -inf, NaN and row lengths, for windows wider than the rows too."""
    rng = np.random.default_rng(8)
    n_rows, n_cols = 30, 200
    s = rng.integers(-5, 5, size=(n_rows, n_cols)).astype(np.float64)
    s[rng.random(s.shape) < 0.15] = -np.inf
    s[rng.random(s.shape) < 0.03] = np.nan
    row_len = rng.integers(0, n_cols, size=n_rows, endpoint=True).astype(np.int32)
    for init, local, k_top in [(0, 0, 17), (3, 0, 10), (0, 5, 10), (4, 6, 8), (4, 6, 40), (250, 0, 64),
                               (0, 300, 5), (1, 1, 200)]:
        for dt in (np.float64, np.float32):
            idx, val = oracle.topk_blocks(s.astype(dt), k_top, init, local, row_len, lib=lib)
            for t in range(n_rows):
                n = int(row_len[t])
                row = s[t, :n]
                ok = np.nonzero(~np.isnan(row) & ~np.isneginf(row))[0]
                forced = (ok < init) | ((local > 0) & (ok >= n - local))
                primary = np.where(forced, 0.0, -row[ok])   # forced keys tie on 0 and go by index
                order = ok[np.lexsort((ok, primary, ~forced))][:k_top]
                want = np.full(k_top, -1)
                want[: len(order)] = order
                assert np.array_equal(idx[t], want), (init, local, k_top, dt, t)
                wv = np.full(k_top, -np.inf)
                wv[: len(order)] = row[order]
                assert np.array_equal(val[t], wv.astype(dt))


def pin_topk_blocks_without_windows_is_topk(lib):
    """No forced keys: block ranking is the plain top-k (pinned above)."""
    rng = np.random.default_rng(9)
    s = rng.standard_normal((12, 90)).astype(np.float32)
    s[rng.random(s.shape) < 0.2] = -np.inf
    for k_top in (1, 9, 90, 120):
        a = oracle.topk_blocks(s, k_top, 0, 0, lib=lib)
        b = oracle.topk(s, k_top, lib=lib)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------------------ pooled keys

def pin_pool_keys_example(lib):
    g = load_golden("pool_keys_example.json")
    k = golden_array(g["k"]).astype(np.float16)
    for c in g["cases"]:
        got = pooling.pool_keys(k, c["pool"])
        assert np.array_equal(got.astype(np.float64), golden_array(c["pooled"])), (c["pool"], got)
    for c in g["extra"]:
        got = pooling.pool_keys(golden_array(c["k"]).astype(np.float16), c["pool"])
        assert np.array_equal(got.astype(np.float64), golden_array(c["pooled"])), got


def _nearest_f16(x):
    """The f16 nearest a Python float (ties to the even bit pattern), by
    search over every finite f16 with exact rational distances."""
    from fractions import Fraction
    bits = np.arange(0, 0x7c00, dtype=np.uint32).astype(np.uint16)   # +0 .. 65504
    mags = bits.view(np.float16).astype(np.float64)
    a = abs(x)
    if a >= 65520.0:
        return np.float16(np.inf if x > 0 else -np.inf)
    i = int(np.searchsorted(mags, a))
    cands = [j for j in (i - 1, i) if 0 <= j < len(mags)]
    fa = Fraction(a)
    best = min(cands, key=lambda j: (abs(Fraction(float(mags[j])) - fa), int(bits[j]) & 1))
    v = np.float16(mags[best])
    return -v if (x < 0 or (x == 0 and np.signbit(x))) else v


def pin_pool_keys_brute_force(lib):
    """Tiny windows of random finite f16 bit patterns (subnormals, large
    values, both signs): every pooled element equals the f16 nearest the
    f64 rounding of the exact rational mean, found by exhaustive search."""
    from fractions import Fraction
    rng = np.random.default_rng(4)
    for trial in range(6):
        n, d, pool = int(rng.integers(1, 10)), 3, int(rng.integers(1, 5))
        raw = rng.integers(0, 0x10000, size=(n, d)).astype(np.uint16)
        raw[(raw & 0x7c00) == 0x7c00] &= 0x3fff          # no inf / NaN
        k = raw.view(np.float16)
        got = pooling.pool_keys(k, pool)
        for p in range(got.shape[0]):
            rows = k[p * pool: min((p + 1) * pool, n)]
            for i in range(d):
                exact = sum(Fraction(float(v)) for v in rows[:, i]) / rows.shape[0]
                want = _nearest_f16(float(exact))
                assert got[p, i].view(np.uint16) == want.view(np.uint16) or (got[p, i] == 0 and want == 0), \
                    (trial, p, i, got[p, i], want)


def pin_pool_keys_properties(lib):
    """Windows of one key are the keys; one window over every key is the
    column mean; equal keys pool to themselves; reordering keys inside a
    window changes nothing; doubling normal-range keys doubles the result."""
    rng = np.random.default_rng(6)
    k = rng.standard_normal((37, 16)).astype(np.float16)
    assert np.array_equal(pooling.pool_keys(k, 1), k)
    whole = pooling.pool_keys(k, 64)
    assert whole.shape == (1, 16)
    assert np.array_equal(whole[0], (k.astype(np.float64).sum(0) / 37).astype(np.float16))
    c = np.full((10, 8), np.float16(0.3), np.float16)
    assert np.array_equal(pooling.pool_keys(c, 3), np.full((4, 8), np.float16(0.3), np.float16))
    perm = np.concatenate([rng.permutation(np.arange(w, min(w + 5, 37))) for w in range(0, 37, 5)])
    assert np.array_equal(pooling.pool_keys(k[perm], 5), pooling.pool_keys(k, 5))
    big = (rng.uniform(1, 2, size=(20, 8)) * np.where(rng.random((20, 8)) < 0.5, -1, 1)).astype(np.float16)
    assert np.array_equal(pooling.pool_keys(big * np.float16(2), 3), pooling.pool_keys(big, 3) * np.float16(2))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
