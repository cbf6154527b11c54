"""Mean pooling of keys (CPU, fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): imported by the tests,
never by the HIP library or its binding; it shares no code with them.

The llama.cpp b11372 notes ("qwen4exp: compute the indexer score with the
lightning indexer") run the lightning indexer on pooled keys without saying
how the keys are pooled.  The reading this oracle follows: pooled key p of
n keys is the element-wise mean of keys [p * pool, min((p + 1) * pool, n)),
a short last window averaging the keys it holds; the sum is exact (at most
8192 f16 values fit the 53-bit f64 significand), the mean is one f64
division, and the result is that f64 rounded to the nearest f16 (ties to
even).
"""
from __future__ import annotations

import numpy as np


def pool_keys(k, pool: int) -> np.ndarray:
    """f16 [n, d] -> f16 [ceil(n / pool), d]."""
    k = np.asarray(k, dtype=np.float16)
    n, d = k.shape
    n_pool = -(-n // pool)
    out = np.empty((n_pool, d), dtype=np.float16)
    for p in range(n_pool):
        window = k[p * pool: min((p + 1) * pool, n)].astype(np.float64)
        total = window.sum(axis=0)            # exact for these magnitudes
        mean = total / window.shape[0]        # one correctly rounded division
        out[p] = mean.astype(np.float16)      # nearest f16, ties to even
    return out
