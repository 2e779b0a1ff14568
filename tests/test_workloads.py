"""Host-side metadata of the five workloads (CPU only): block tables, slot
mappings, cu_seqlens, reference counts and poison placement."""
import numpy as np
import pytest

import oracle
import workloads as W


def _check_common(w):
    bs = w.block_size
    # slots: distinct, inside the pool, and equal to the oracle's slot-of-position definition
    sm = w.slot_mapping
    assert len(set(sm.tolist())) == len(sm)
    assert sm.min() >= 0 and sm.max() < w.num_blocks * bs
    expect = []
    if w.cu_seqlens_q is not None:
        for b in range(len(w.cu_seqlens_q) - 1):
            lq = int(w.cu_seqlens_q[b + 1] - w.cu_seqlens_q[b])
            lk = int(w.cu_seqlens_k[b + 1] - w.cu_seqlens_k[b])
            expect += [oracle.slot_of(w.pre_block_tables[b], p, bs) for p in range(lk - lq, lk)]
    if w.dec_context_lens is not None:
        for b, L in enumerate(w.dec_context_lens.tolist()):
            expect.append(oracle.slot_of(w.dec_block_tables[b], L - 1, bs))
    assert np.array_equal(sm, np.asarray(expect, dtype=np.int32))
    # the step never writes a shared block
    written_blocks = set((sm // bs).tolist())
    assert not written_blocks & set(w.shared_blocks)
    assert all(w.refcount[b] == 1 for b in written_blocks)
    # every slot the step writes holds poison before the store
    flat_k = W.to_float32(w.k_cache.reshape(-1, w.num_kv_heads, w.head_dim), w.dtype)
    assert np.isnan(flat_k[sm]).all()
    # the poison block is NaN everywhere and is where table padding points
    assert np.isnan(W.to_float32(w.k_cache[w.poison_block], w.dtype)).all()
    for bt, lens in ((w.dec_block_tables, w.dec_context_lens),
                     (w.pre_block_tables, None if w.cu_seqlens_k is None else np.diff(w.cu_seqlens_k))):
        if bt is None:
            continue
        for b, L in enumerate(lens.tolist()):
            used = -(-L // bs)
            assert (bt[b, used:] == w.poison_block).all()
            assert (bt[b, :used] != w.poison_block).all()
            # resident tokens are finite
            resident = L - (1 if bt is w.dec_block_tables else int(np.diff(w.cu_seqlens_q)[b]))
            rows = oracle.gather(w.k_cache, bt[b], resident, bs)
            assert np.isfinite(W.to_float32(rows, w.dtype)).all()


@pytest.mark.parametrize("i", [1, 2, 4, 6])
def test_config_metadata(i):
    w = W.make_config(i)
    _check_common(w)


def test_config1_shape_and_pool():
    w = W.make_config(1)
    assert (w.num_blocks, w.block_size, w.num_q_heads, w.num_kv_heads, w.head_dim) == (64, 16, 4, 2, 64)
    assert w.dec_block_tables.shape == (4, 7)
    assert 1 <= w.dec_context_lens.min() and w.dec_context_lens.max() <= 100
    assert w.dtype == "f32" and abs(w.scale - 0.125) < 1e-15


def test_config4_prefix_sharing():
    w = W.make_config(4)
    assert len(w.shared_blocks) == 2
    assert (w.refcount[w.shared_blocks] == 16).all()
    assert (w.pre_block_tables[:, :2] == np.asarray(w.shared_blocks)).all()
    lq = np.diff(w.cu_seqlens_q)
    lk = np.diff(w.cu_seqlens_k)
    assert (lk - lq == 512).all() and lq.min() >= 128 and lq.max() <= 2048
    assert len(w.slot_mapping) == int(lq.sum())


def test_seed_determinism():
    a = W.make_config(2)
    b = W.make_config(2)
    assert np.array_equal(a.k_cache, b.k_cache) and np.array_equal(a.dec_q, b.dec_q)
    assert np.array_equal(a.dec_block_tables, b.dec_block_tables)
    c = W.make_config(2, seed=7)
    assert not np.array_equal(a.dec_context_lens, c.dec_context_lens)


def test_fill_normal_independent_of_threads(monkeypatch):
    a = W.fill_normal((3, 1 << 21), "bf16", 3, 1)
    monkeypatch.setattr(W, "_workers", lambda: 1)
    b = W.fill_normal((3, 1 << 21), "bf16", 3, 1)
    assert np.array_equal(a, b)
    x = W.to_float32(a, "bf16")
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01


def test_bf16_rounding_ties_to_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, np.nan], dtype=np.float32)
    bits = W.f32_to_bf16_bits(x)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82 and bits[3] == 0xC020
    assert np.isnan(W.to_float32(bits[4:], "bf16")).all()


def test_pool_refcounts_and_exhaustion():
    p = W.BlockPool([2, 0, 1])
    a = p.alloc(2)
    assert a == [2, 0]
    p.share([2])
    assert p.refcount[2] == 2
    p.release([2])
    p.release([2])
    assert 2 in p.free
    with pytest.raises(W.PoolExhausted):
        p.alloc(3)


def test_small_mixed_step_layout():
    # the mixed-step recipe at a size that builds in milliseconds
    seqs = [W.SeqSpec("prefill", 700, 512), W.SeqSpec("prefill", 512, 512)]
    seqs += [W.SeqSpec("decode", L, 1, shared=4 if j % 2 else 0) for j, L in enumerate([1100, 1500, 1025, 2000])]
    w = W.build("mini-mixed", 3, "bf16", 8, 2, 64, 256, seqs, shared_prefix_blocks=4)
    _check_common(w)
    assert len(w.slot_mapping) == 512 + 512 + 4
    assert (w.refcount[w.shared_blocks] == 2).all()


def test_config6_shared_prompt_and_cascade_groups():
    w = W.make_config(6)
    assert len(w.shared_blocks) == 64 and (w.refcount[w.shared_blocks] == 64).all()
    assert (w.dec_block_tables[:, :64] == np.asarray(w.shared_blocks)).all()
    shared, offsets, seqs, gmax, smax, own = w.cascade_groups()
    assert own == int((w.dec_context_lens - 16384).max())
    assert (shared == 64 * 256).all() and list(offsets) == [0, 64] and sorted(seqs) == list(range(64))
    assert (gmax, smax) == (64, 16384)
    suffix = w.dec_context_lens - 16384
    assert suffix.min() >= 1 and suffix.max() <= 512
    # unique bytes: the prompt once plus every sequence's own tokens
    row = 2 * w.num_kv_heads * w.head_dim * 2
    assert w.decode_kv_bytes_unique() == (16384 + int(suffix.sum())) * row
    assert w.decode_kv_bytes() == int(w.dec_context_lens.sum()) * row
    capped = w.cascade_groups(group_cap=10)
    assert list(capped[1]) == [0, 10, 20, 30, 40, 50, 60, 64] and capped[3] == 10


def test_cascade_groups_of_config5():
    w = W.make_config(5)
    shared, offsets, seqs, gmax, smax, own = w.cascade_groups()
    assert own == int(w.dec_context_lens.max())  # the longest context has no shared prefix
    assert list(offsets) == [0, 50] and sorted(seqs) == w.notes["sharers"] and smax == 4096
    assert (shared[seqs] == 4096).all() and (np.delete(shared, seqs) == 0).all()
