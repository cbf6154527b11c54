"""Shared helpers of the GPU parity tests: run the HIP path through the C-ABI
binding and compare with the CPU oracle on the same seeded inputs.

Score bar (fp32 accumulation of f16 products): for every visible entry
    |gpu - oracle| <= 2e-3 * (sum_h |w_h| * relu(dot_h) + |mask|
                              + 1e-2 * sum_h |w_h| * sum_i |q_hi * k_i|)
with -inf at exactly the same entries.  The first two terms make it a plain
relative error when w >= 0 and the mask is 0.  The last term is a floor for
dot products that nearly cancel: every f16 x f16 product is exact in f32, so
the accumulation error of one head's dot product is at most
gamma_{d-1} * sum_i |q_hi k_i| (the standard forward error bound of
floating-point summation), about 7.6e-6 * sum_i |q_hi k_i| for d = 128 --
below the floor's 2e-5 with a margin of 2.6, yet a hundred times below what
a dropped head or a wrong key would cost.  Top-k bar: the GPU's indices equal, bit for bit, the oracle's
top-k of the GPU's own f32 scores; against the oracle's fp64 ranking, each
position's score agrees within the same tolerance, padding sits at the same
positions, and the selected sets are equal wherever the gap between the k-th
and (k+1)-th oracle scores exceeds the tolerance.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

import oracle
import sparse_attention_lightning_indexer_amd as li

TOL = 2e-3
DEV = torch.device("cuda:0")


def dev(a):
    return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def gpu_score(inp):
    if hasattr(inp, "k_cache"):
        out = li.score_decode(dev(inp.q), dev(inp.k_cache), dev(inp.block_table),
                              dev(inp.seq_lens), inp.Q, inp.max_seq_len, dev(inp.w),
                              dev(inp.mask))
    else:
        out = li.score_prefill(dev(inp.q), dev(inp.k), dev(inp.w), dev(inp.mask),
                               dev(inp.vis_len))
    torch.cuda.synchronize()
    return out


def gpu_fused(inp, k_top=None):
    k_top = k_top or inp.k_top
    if hasattr(inp, "k_cache"):
        idx, val = li.score_topk_fused_decode(dev(inp.q), dev(inp.k_cache), dev(inp.block_table),
                                              dev(inp.seq_lens), inp.Q, inp.max_seq_len,
                                              dev(inp.w), k_top, dev(inp.mask))
    else:
        idx, val = li.score_topk_fused_prefill(dev(inp.q), dev(inp.k), dev(inp.w), k_top,
                                               dev(inp.mask), dev(inp.vis_len))
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def gpu_topk(score_t, k_top, row_len=None):
    idx, val = li.topk(score_t, k_top, row_len)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), val.cpu().numpy()


def abs_weights(inp):
    return dataclasses.replace(inp, w=np.abs(inp.w).astype(np.float32))


ABS_FLOOR = 1e-2


def _oracle_rows(inp, rows):
    s = oracle.score_inputs(inp) if rows is None else oracle.score_rows(inp, rows)
    return np.where(np.isneginf(s), 0.0, s)      # columns past a row's visible keys


def denominator_parts(inp, rows=None):
    """(main, floor) for every entry of the given rows: main is
    sum_h |w_h| relu(dot_h) + |mask| (the plain relative-error denominator when
    w >= 0 and the mask is 0), floor is ABS_FLOOR * sum_h |w_h| sum_i |q_hi k_i|."""
    ia = dataclasses.replace(abs_weights(inp), mask=None)
    if hasattr(ia, "vis_len"):
        ia = dataclasses.replace(ia, vis_len=None)
    main = _oracle_rows(ia, rows)
    # with |q| and |k| every dot product is the sum of the absolute products
    if hasattr(ia, "k_cache"):
        ib = dataclasses.replace(ia, q=np.abs(ia.q), k_cache=np.abs(ia.k_cache))
    else:
        ib = dataclasses.replace(ia, q=np.abs(ia.q), k=np.abs(ia.k))
    floor = ABS_FLOOR * _oracle_rows(ib, rows)
    if inp.mask is not None:
        m = inp.mask if rows is None else inp.mask[np.asarray(rows)]
        m = m.astype(np.float64)
        main = main + np.where(np.isneginf(m), 0.0, np.abs(m))
    return main, floor


class Den(np.ndarray):
    """The score bar's denominator (main + floor), carrying the floor-free
    part so that check_scores can report the error without the floor."""


def denominators(inp, rows=None):
    main, floor = denominator_parts(inp, rows)
    den = (main + floor).view(Den)
    den.main = main
    return den


# per-workload summary of the unfloored error, printed by the tests (-s)
UNFLOORED = {}


def check_scores(g, o, den, tol=TOL, where=""):
    g = np.asarray(g, dtype=np.float64)
    assert g.shape == o.shape, (g.shape, o.shape)
    inv_o, inv_g = np.isneginf(o), np.isneginf(g)
    bad = np.argwhere(inv_o != inv_g)
    assert bad.size == 0, f"{where}: -inf sets differ at {bad[:5].tolist()} (gpu {g[tuple(bad[0])]}, oracle {o[tuple(bad[0])]})"
    vis = ~inv_o
    assert np.all(np.isfinite(g[vis])), f"{where}: non-finite visible GPU score"
    diff = np.abs(g[vis] - o[vis])
    err = diff / (np.asarray(den)[vis] + 1e-30)
    if err.size:
        i = int(np.argmax(err))
        assert err[i] <= tol, f"{where}: max scaled error {err[i]:.3e} (gpu {g[vis][i]}, oracle {o[vis][i]})"
    main = getattr(den, "main", None)
    if main is not None and err.size:
        # the same error without the cancellation floor: plain relative error
        # (w >= 0, mask 0) or its signed-weight form
        raw = diff / (main[vis] + 1e-30)
        needed = int(np.count_nonzero(raw > tol))
        UNFLOORED[where] = (float(raw.max()), needed, int(raw.size))
        print(f"{where}: max error {err.max():.2e} with the floor, {raw.max():.2e} without it; "
              f"{needed} of {raw.size} entries need the floor")
    return float(err.max()) if err.size else 0.0


def check_topk_exact(g_idx, g_val, g_score_np, k_top, row_len=None, where=""):
    """GPU top-k == oracle top-k of the GPU's own f32 scores, bit for bit."""
    oi, ov = oracle.topk(np.ascontiguousarray(g_score_np, dtype=np.float32), k_top, row_len)
    if not np.array_equal(g_idx, oi):
        r = int(np.argwhere((g_idx != oi).any(axis=1))[0, 0])
        c = int(np.argwhere(g_idx[r] != oi[r])[0, 0])
        raise AssertionError(f"{where}: top-k index mismatch row {r} pos {c}: gpu {g_idx[r, c-2:c+3]} oracle {oi[r, c-2:c+3]}")
    if g_val is not None:
        assert np.array_equal(g_val.view(np.uint32), ov.view(np.uint32)), f"{where}: top-k values differ"


def check_topk_vs_f64(g_idx, o_rows, den_rows, k_top, tol=TOL, where=""):
    """Against the oracle's fp64 ranking of the same rows (o_rows, f64)."""
    oi, ov = oracle.topk(o_rows, min(k_top + 1, o_rows.shape[1]) if o_rows.shape[1] > k_top else k_top)
    for r in range(o_rows.shape[0]):
        gi = g_idx[r]
        oik, ovk = oi[r, :k_top], ov[r, :k_top]
        assert np.array_equal(gi == -1, oik == -1), f"{where}: padding differs in row {r}"
        v = oik != -1
        og = o_rows[r, gi[v]]
        assert np.all(np.isfinite(og)), f"{where}: row {r} selected an invisible key"
        lim = tol * den_rows[r, oik[v]] + 1e-30
        d = np.abs(og - ovk[v])
        assert np.all(d <= lim), f"{where}: row {r} position {int(np.argmax(d - lim))} score off by {d.max():.3e}"
        if v.sum() == k_top and oi.shape[1] > k_top and oi[r, k_top] != -1:
            gap = ovk[-1] - ov[r, k_top]
            if gap > tol * den_rows[r, oik[-1]]:
                assert set(gi.tolist()) == set(oik.tolist()), f"{where}: row {r} selected set differs"
        else:
            assert set(gi[gi != -1].tolist()) == set(oik[v].tolist()), f"{where}: row {r} set differs"
