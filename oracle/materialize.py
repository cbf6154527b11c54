"""Independent NumPy cross-check of the oracle (fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

This is the scheme the llama.cpp b11372 notes ("qwen4exp: halve the indexer
score memory") describe as the *old* graph: score every head in one product,
keeping the whole per-head tensor [n_pool, n_idx_h, n_tokens], rectify it,
then weight and reduce over heads.  It spends the memory the method avoids,
which is why it serves only as a small-shape cross-check of the oracle's
rectify-each-head-then-sum loop.  The product here is a library matmul over
flattened token-head rows, a different formulation from the oracle's loops.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def score_prefill(q, k, w, mask=None, vis_len=None) -> np.ndarray:
    """f64 [T][P]; same conventions as the oracle."""
    T, H, d = q.shape
    P = k.shape[0]
    # whole per-head product at once: [T*H, d] x [d, P] -> [T, H, P]
    per_head = (_f64(q).reshape(T * H, d) @ _f64(k).T).reshape(T, H, P)
    rectified = np.maximum(per_head, 0.0)
    out = np.einsum("thp,h->tp", rectified, _f64(w))
    invisible = np.zeros((T, P), dtype=bool)
    if mask is not None:
        m = _f64(mask)
        invisible |= np.isneginf(m)
        out = out + np.where(np.isneginf(m), 0.0, m)
    if vis_len is not None:
        invisible |= np.arange(P)[None, :] >= np.asarray(vis_len)[:, None]
    out[invisible] = -np.inf
    return out


def score_decode(q, k_cache, block_table, seq_lens, Q, max_seq_len, w,
                 mask=None) -> np.ndarray:
    """Gather each request's keys into a contiguous [seq_len][d] array, then
    score its Q rows with ``score_prefill``."""
    R = len(seq_lens)
    RQ, H, d = q.shape
    bs = k_cache.shape[1]
    out = np.full((RQ, max_seq_len), -np.inf)
    for r in range(R):
        L = min(int(seq_lens[r]), max_seq_len)
        if L <= 0:
            continue
        pos = np.arange(L)
        keys = k_cache[block_table[r, pos // bs], pos % bs]
        # query j sees s < seq_len - Q + 1 + j, cut to the stored row width
        vis = np.array([int(seq_lens[r]) - Q + 1 + j for j in range(Q)])
        vis = np.clip(vis, 0, L)
        m = None if mask is None else mask[r * Q:(r + 1) * Q, :L]
        out[r * Q:(r + 1) * Q, :L] = score_prefill(q[r * Q:(r + 1) * Q], keys, w, m, vis)
    return out
