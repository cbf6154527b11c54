"""Seeded synthetic inputs for the lightning-indexer score and top-k.

This module is shared by the oracle tests, the GPU parity tests and the
benchmark.  It only draws random numbers and lays them out in the shapes the
indexer consumes; it holds none of the method's arithmetic (no dot products,
no rectification, no head sums, no visibility rule, no selection).

Recipe (fixed, so every consumer sees identical bytes for a given seed):
  * ``rng = numpy.random.default_rng(seed)``; every float is drawn in float32
    and rounded to f16 with numpy's round-to-nearest-even ``astype``.
  * Contiguous (prefill) inputs are drawn in the order q, k, w, mask.
  * Paged (decode) inputs are drawn in the order seq_lens, q, k_cache, w,
    block permutation.  Physical block ids are a seeded permutation, so the
    block table is never the identity.  Cache slots that no request owns
    (the tail of each request's last block, plus a few spare blocks) are
    filled with f16 NaN when ``poison`` is set, so any read of them shows up
    in the scores; unused block-table entries are -1.

The five named workloads follow the shapes and distributions of the pages'
settings: the tiny four-head reference case, decode with one query token per
request, speculative decode with four query tokens per request, causal
prefill, and a long-context chunked prefill.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

F16 = np.float16
NEG_INF_F16 = np.float16(-np.inf)
NAN_F16 = np.float16(np.nan)


@dataclass
class PrefillInputs:
    """Contiguous inputs: q [T][H][d] f16, k [P][d] f16, w [H] f32,
    mask [T][P] f16 (0 or -inf, or None), vis_len [T] i32 (or None)."""
    name: str
    q: np.ndarray
    k: np.ndarray
    w: np.ndarray
    mask: Optional[np.ndarray]
    vis_len: Optional[np.ndarray]
    k_top: int
    info: dict = field(default_factory=dict)

    @property
    def T(self) -> int:
        return self.q.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def d(self) -> int:
        return self.q.shape[2]

    @property
    def P(self) -> int:
        return self.k.shape[0]


@dataclass
class DecodeInputs:
    """Paged inputs: q [R*Q][H][d] f16 (row r*Q+j is query j of request r),
    k_cache [n_blocks][block_size][d] f16, block_table [R][max_blocks] i32,
    seq_lens [R] i32, w [H] f32, optional mask [R*Q][max_seq_len] f16."""
    name: str
    q: np.ndarray
    k_cache: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray
    Q: int
    max_seq_len: int
    w: np.ndarray
    mask: Optional[np.ndarray]
    k_top: int
    info: dict = field(default_factory=dict)

    @property
    def R(self) -> int:
        return self.seq_lens.shape[0]

    @property
    def H(self) -> int:
        return self.q.shape[1]

    @property
    def d(self) -> int:
        return self.q.shape[2]

    @property
    def block_size(self) -> int:
        return self.k_cache.shape[1]


def _normal_f16(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x.astype(F16)


def _causal_mask(T: int, P: int, first_pos: int) -> np.ndarray:
    """f16 [T][P]: 0 where key s <= first_pos + t, -inf elsewhere."""
    m = np.full((T, P), NEG_INF_F16, dtype=F16)
    for t in range(T):
        m[t, : min(P, first_pos + t + 1)] = 0
    return m


# --------------------------------------------------------------------------
# Contiguous (prefill-style) inputs
# --------------------------------------------------------------------------

def tiny(seed: int = 0) -> PrefillInputs:
    """16 tokens, 256 pooled keys, 4 heads, head_dim 64; every head weight is
    1/sqrt(64); 26 of the 256 key columns (10%, seeded) are -inf for every
    token; top-32."""
    rng = np.random.default_rng(seed)
    T, P, H, d = 16, 256, 4, 64
    q = _normal_f16(rng, (T, H, d))
    k = _normal_f16(rng, (P, d))
    w = np.full(H, 1.0 / 8.0, dtype=np.float32)
    cols = rng.permutation(P)[: int(round(0.1 * P))]
    mask = np.zeros((T, P), dtype=F16)
    mask[:, cols] = NEG_INF_F16
    return PrefillInputs("tiny", q, k, w, mask, None, 32,
                         {"masked_cols": np.sort(cols)})


def prefill_causal(seed: int = 0, T: int = 8192, H: int = 64, d: int = 128,
                   k_top: int = 2048) -> PrefillInputs:
    """Causal prefill: T tokens against P=T keys, key s visible to token t
    iff s <= t (f16 0/-inf mask, and the visible-prefix hint t + 1); every
    head weight 1/sqrt(d)."""
    rng = np.random.default_rng(seed)
    P = T
    q = _normal_f16(rng, (T, H, d))
    k = _normal_f16(rng, (P, d))
    w = np.full(H, 1.0 / np.sqrt(d), dtype=np.float32)
    mask = _causal_mask(T, P, 0)
    vis = np.arange(1, T + 1, dtype=np.int32)          # the optional visible-prefix hint, t + 1
    return PrefillInputs("prefill_causal", q, k, w, mask, vis, k_top)


def long_chunk(seed: int = 0, T: int = 1024, P: int = 131072, H: int = 64,
               d: int = 128, k_top: int = 2048) -> PrefillInputs:
    """Chunked prefill at long context: a chunk of T tokens at positions
    P-T .. P-1 against P pooled keys, causal; q, k ~ N(0, 0.5^2);
    w ~ N(0,1)/sqrt(d), signed."""
    rng = np.random.default_rng(seed)
    q = _normal_f16(rng, (T, H, d), std=0.5)
    k = _normal_f16(rng, (P, d), std=0.5)
    w = (rng.standard_normal(H, dtype=np.float32) / np.float32(np.sqrt(d))).astype(np.float32)
    mask = _causal_mask(T, P, P - T)
    vis = np.arange(P - T + 1, P + 1, dtype=np.int32)  # visible prefix of token t: P - T + 1 + t
    return PrefillInputs("long_chunk", q, k, w, mask, vis, k_top,
                         {"first_pos": P - T})


def random_prefill(seed: int, T: int, P: int, H: int, d: int, k_top: int,
                   mask_kind: str = "random", w_kind: str = "uniform",
                   vis_kind: str = "none", std: float = 1.0) -> PrefillInputs:
    """Small random prefill case for parity tests.

    mask_kind: "none" | "zero" | "random" (about 20% -inf) | "causal" |
               "bias" (finite f16 biases plus some -inf) | "all_inf"
    w_kind:    "uniform" (U(0,1)) | "equal" (1/sqrt(d)) | "signed" (N(0,1)) |
               "pow2" (powers of two 2^-7..2^0)
    vis_kind:  "none" | "random" (per-token prefix length in [0, P])
    """
    rng = np.random.default_rng(seed)
    q = _normal_f16(rng, (T, H, d), std)
    k = _normal_f16(rng, (P, d), std)
    w = _weights(rng, H, d, w_kind)
    mask = _mask(rng, T, P, mask_kind)
    vis = None
    if vis_kind == "random":
        vis = rng.integers(0, P, size=T, endpoint=True).astype(np.int32)
    return PrefillInputs(f"rand_T{T}_P{P}_H{H}_d{d}", q, k, w, mask, vis, k_top)


def integer_prefill(seed: int, T: int, P: int, H: int, d: int, k_top: int,
                    mask_kind: str = "random") -> PrefillInputs:
    """Exact-arithmetic inputs: q, k entries in {-2..2}, w powers of two in
    2^-7 .. 2^0.  Every product, dot, weighted term and partial sum is then
    exactly representable in f32, so any summation order gives identical bits
    (and there are many exact ties)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-2, 2, size=(T, H, d), endpoint=True).astype(F16)
    k = rng.integers(-2, 2, size=(P, d), endpoint=True).astype(F16)
    w = np.ldexp(np.float32(1.0), -rng.integers(0, 7, size=H, endpoint=True)).astype(np.float32)
    mask = _mask(rng, T, P, mask_kind)
    return PrefillInputs(f"int_T{T}_P{P}_H{H}_d{d}", q, k, w, mask, None, k_top)


def _weights(rng, H, d, kind):
    if kind == "uniform":
        return rng.random(H, dtype=np.float32)
    if kind == "uniform_scaled":
        return (rng.random(H, dtype=np.float32) / np.float32(np.sqrt(d))).astype(np.float32)
    if kind == "equal":
        return np.full(H, 1.0 / np.sqrt(d), dtype=np.float32)
    if kind == "signed":
        return rng.standard_normal(H, dtype=np.float32)
    if kind == "pow2":
        return np.ldexp(np.float32(1.0), -rng.integers(0, 7, size=H, endpoint=True)).astype(np.float32)
    if kind == "zero":
        return np.zeros(H, dtype=np.float32)
    raise ValueError(kind)


def _mask(rng, T, P, kind):
    if kind == "none":
        return None
    if kind == "zero":
        return np.zeros((T, P), dtype=F16)
    if kind == "random":
        m = np.zeros((T, P), dtype=F16)
        m[rng.random((T, P)) < 0.2] = NEG_INF_F16
        return m
    if kind == "causal":
        return _causal_mask(T, P, max(0, P - T))
    if kind == "bias":
        m = (rng.standard_normal((T, P), dtype=np.float32) * 4).astype(F16)
        m[rng.random((T, P)) < 0.1] = NEG_INF_F16
        return m
    if kind == "all_inf":
        return np.full((T, P), NEG_INF_F16, dtype=F16)
    raise ValueError(kind)


# --------------------------------------------------------------------------
# Paged (decode-style) inputs
# --------------------------------------------------------------------------

def _paged(rng, name, seq_lens, Q, H, d, block_size, w_kind, k_top, std=1.0,
           poison=True, spare_blocks=3, max_seq_len=None, mask_kind="none"):
    R = len(seq_lens)
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max()) if R else 0
    q = _normal_f16(rng, (R * Q, H, d), std)
    nblk = [(int(L) + block_size - 1) // block_size for L in seq_lens]
    n_used = int(sum(nblk))
    n_phys = n_used + spare_blocks
    k_cache = _normal_f16(rng, (n_phys, block_size, d), std)
    w = _weights(rng, H, d, w_kind)
    perm = rng.permutation(n_phys).astype(np.int32)
    max_blocks = max(1, (max_seq_len + block_size - 1) // block_size)
    bt = np.full((R, max_blocks), -1, dtype=np.int32)
    off = 0
    for r in range(R):
        bt[r, : nblk[r]] = perm[off: off + nblk[r]]
        off += nblk[r]
    if poison:
        spare = perm[n_used:]
        k_cache[spare] = NAN_F16
        for r in range(R):
            L = int(seq_lens[r])
            if nblk[r] and L % block_size:
                k_cache[bt[r, nblk[r] - 1], L % block_size:] = NAN_F16
    mask = _mask(rng, R * Q, max_seq_len, mask_kind)
    return DecodeInputs(name, q, k_cache, bt, seq_lens, Q, max_seq_len, w,
                        mask, k_top)


def decode(seed: int = 0, poison: bool = True) -> DecodeInputs:
    """32 requests, one query token each, seq_len ~ U{1024..8192}, 64-key
    pages; 64 heads of dim 128; w ~ U(0,1)/sqrt(128); top-512."""
    rng = np.random.default_rng(seed)
    seq_lens = rng.integers(1024, 8192, size=32, endpoint=True)
    return _paged(rng, "decode", seq_lens, 1, 64, 128, 64, "uniform_scaled", 512,
                  poison=poison)


def spec_decode(seed: int = 0, poison: bool = True) -> DecodeInputs:
    """32 requests, four query tokens each (one plus three speculative),
    16384 keys each in 64-key pages; 64 heads of dim 128; w ~ U(0,1);
    top-2048."""
    rng = np.random.default_rng(seed)
    seq_lens = np.full(32, 16384)
    return _paged(rng, "spec_decode", seq_lens, 4, 64, 128, 64, "uniform", 2048,
                  poison=poison)


def random_decode(seed: int, R: int, Q: int, H: int, d: int, block_size: int,
                  len_lo: int, len_hi: int, k_top: int, w_kind: str = "uniform",
                  poison: bool = True, max_seq_len: Optional[int] = None,
                  mask_kind: str = "none") -> DecodeInputs:
    """Small random paged case for parity tests; seq_len ~ U{len_lo..len_hi}."""
    rng = np.random.default_rng(seed)
    seq_lens = rng.integers(len_lo, len_hi, size=R, endpoint=True)
    return _paged(rng, f"rdec_R{R}_Q{Q}_H{H}_d{d}_bs{block_size}", seq_lens, Q,
                  H, d, block_size, w_kind, k_top, poison=poison,
                  max_seq_len=max_seq_len, mask_kind=mask_kind)


def paged_from_prefill(inp: PrefillInputs, block_size: int, seed: int = 1,
                       permute: bool = True) -> DecodeInputs:
    """Re-lay a one-request prefill case as a paged cache (Q = T, seq_len =
    P), for layout-equivalence tests: blocks placed by a seeded permutation,
    or in order with `permute=False`."""
    rng = np.random.default_rng(seed)
    P, d = inp.k.shape
    nb = (P + block_size - 1) // block_size
    perm = (rng.permutation(nb + 2) if permute else np.arange(nb + 2)).astype(np.int32)
    k_cache = np.full((nb + 2, block_size, d), NAN_F16, dtype=F16)
    for b in range(nb):
        rows = inp.k[b * block_size: (b + 1) * block_size]
        k_cache[perm[b], : rows.shape[0]] = rows
    bt = perm[:nb][None, :].copy()
    return DecodeInputs(inp.name + "_paged", inp.q, k_cache, bt,
                        np.array([P], dtype=np.int32), inp.T, P, inp.w,
                        None, inp.k_top)


CONFIGS = {
    "tiny": tiny,
    "decode": decode,
    "spec_decode": spec_decode,
    "prefill_causal": prefill_causal,
    "long_chunk": long_chunk,
}
