"""The seeded generators: shapes, determinism, and the poisoning of cache
slots that no request owns."""
import numpy as np

import workloads as W


def test_tiny_shapes_and_mask():
    a, b = W.tiny(), W.tiny()
    assert a.q.shape == (16, 4, 64) and a.k.shape == (256, 64)
    assert np.array_equal(a.q.view(np.uint16), b.q.view(np.uint16))
    assert a.w.dtype == np.float32 and np.all(a.w == 0.125)
    cols = np.isneginf(a.mask.astype(np.float32)).all(axis=0)
    assert cols.sum() == 26
    assert np.all(np.isneginf(a.mask.astype(np.float32)).any(axis=0) == cols)


def test_decode_layout():
    d = W.decode()
    assert d.R == 32 and d.Q == 1 and d.H == 64 and d.d == 128 and d.block_size == 64
    assert d.seq_lens.min() >= 1024 and d.seq_lens.max() <= 8192
    assert d.max_seq_len == d.seq_lens.max()
    used = set()
    for r in range(d.R):
        nb = -(-int(d.seq_lens[r]) // 64)
        ids = d.block_table[r, :nb]
        assert np.all(ids >= 0) and np.all(d.block_table[r, nb:] == -1)
        used.update(ids.tolist())
        L = int(d.seq_lens[r])
        last = d.k_cache[ids[-1]]
        tail = L - (nb - 1) * 64
        assert not np.isnan(last[:tail].astype(np.float32)).any()
        assert np.isnan(last[tail:].astype(np.float32)).all()
    assert len(used) == sum(-(-int(L) // 64) for L in d.seq_lens)
    spare = sorted(set(range(d.k_cache.shape[0])) - used)
    assert spare and np.isnan(d.k_cache[spare].astype(np.float32)).all()


def test_spec_decode_layout():
    s = W.spec_decode()
    assert s.R == 32 and s.Q == 4 and s.q.shape == (128, 64, 128)
    assert np.all(s.seq_lens == 16384) and s.max_seq_len == 16384
    assert s.k_top == 2048


def test_random_prefill_reproducible():
    a = W.random_prefill(5, 7, 33, 8, 64, 4, mask_kind="bias", vis_kind="random")
    b = W.random_prefill(5, 7, 33, 8, 64, 4, mask_kind="bias", vis_kind="random")
    assert np.array_equal(a.q.view(np.uint16), b.q.view(np.uint16))
    assert np.array_equal(a.mask.view(np.uint16), b.mask.view(np.uint16))
    assert np.array_equal(a.vis_len, b.vis_len)
