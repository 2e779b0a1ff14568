"""Fused rotary embedding + cache write on the GPU against the fp64 oracle.

Bar (derived from the arithmetic, since the pages state no tolerance for this
step): the kernel reduces angles in fp64 and rotates in fp32, an error below
2^-19 of the pair's norm; rounding the result to the storage type adds half a
unit in its last place, at most 2^-8 (bf16) or 2^-24 (fp32) of the value.  So
each rotated element must lie within 2^-8 |exact| + 2^-19 |pair| (bf16) or
2^-23 |exact| + 2^-19 |pair| (fp32) of the oracle.  v and every cache slot not
named in the slot mapping must be bit-exact; position 0 must return q and k
bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import bits, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _pair_norm(x, interleaved):
    """|pair| for every element of x [N, H, D] (float64)."""
    a, b = oracle.rope_pairs(x.shape[-1], interleaved)
    n = np.sqrt(x[..., a] ** 2 + x[..., b] ** 2)
    out = np.empty_like(x)
    out[..., a] = n
    out[..., b] = n
    return out


def _within(got, exact, interleaved, dtype):
    rel = 2.0 ** -8 if dtype == W.BF16 else 2.0 ** -23
    tol = rel * np.abs(exact) + 2.0 ** -19 * _pair_norm(exact, interleaved) + 1e-30
    err = np.abs(oracle.widen(got, dtype) - exact)
    ratio = float(np.max(err / tol)) if err.size else 0.0
    return ratio


def _case(dtype, N, Hq, Hkv, D, bs, nb, seed, neg_every=7, max_pos=40000):
    rng = np.random.default_rng(seed)
    q = W.fill_normal((N, Hq, D), dtype, seed, 31)
    k = W.fill_normal((N, Hkv, D), dtype, seed, 32)
    v = W.fill_normal((N, Hkv, D), dtype, seed, 33)
    kc = W.fill_normal((nb, bs, Hkv, D), dtype, seed, 34)
    vc = W.fill_normal((nb, bs, Hkv, D), dtype, seed, 35)
    slots = rng.choice(nb * bs, size=N, replace=False).astype(np.int32)
    if neg_every:
        slots[1::neg_every] = -1  # token 0 keeps its slot
    pos = rng.integers(0, max_pos, size=N).astype(np.int32)
    pos[:1] = 0
    return q, k, v, pos, kc, vc, slots


def _run(q, k, v, pos, kc, vc, slots, theta, interleaved, dtype):
    dq, dk, dv = to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype)
    dkc, dvc = to_dev(kc, dtype), to_dev(vc, dtype)
    pkv.rope_kv_store(dq, dk, dv, to_dev(pos), dkc, dvc, to_dev(slots), theta, interleaved)
    torch.cuda.synchronize()
    return to_host(dq, dtype), to_host(dkc, dtype), to_host(dvc, dtype)


def _check(q, k, v, pos, kc, vc, slots, theta, interleaved, dtype, got_q, got_kc, got_vc):
    q_rot, kc_exact, vc_exact = oracle.rope_kv_store(q, k, v, pos, kc, vc, slots, kc.shape[1], theta,
                                                     interleaved, dtype)
    r_q = _within(got_q, q_rot, interleaved, dtype)
    assert r_q <= 1.0, f"q off by {r_q} of the tolerance"
    # v: bit-exact over the whole pool
    assert np.array_equal(bits(got_vc), bits(vc_exact))
    # k cache: untouched slots bit-exact, written slots within tolerance
    flat_got = got_kc.reshape(-1, *got_kc.shape[2:])
    flat_in = kc.reshape(-1, *kc.shape[2:])
    written = np.zeros(flat_in.shape[0], dtype=bool)
    written[slots[slots >= 0]] = True
    assert np.array_equal(bits(flat_got[~written]), bits(flat_in[~written]))
    live = slots >= 0
    k_exact = kc_exact.reshape(-1, *kc_exact.shape[2:])[slots[live]]
    r_k = _within(flat_got[slots[live]], k_exact, interleaved, dtype)
    assert r_k <= 1.0, f"k off by {r_k} of the tolerance"
    # position 0 leaves q and k as they were, bit for bit
    for i in np.flatnonzero(np.asarray(pos) == 0):
        assert np.array_equal(bits(got_q[i]), bits(q[i]))
        if slots[i] >= 0:
            assert np.array_equal(bits(flat_got[slots[i]]), bits(k[i]))
    return r_q, r_k


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("heads,N", [((32, 8), 37), ((16, 8), 5), ((6, 2), 300), ((8, 8), 1)])
def test_rope_kv_store_sweep(dtype, D, interleaved, heads, N):
    Hq, Hkv = heads
    bs, nb = 16, max(4, -(-N // 16) + 3)
    theta = 1e6 if D == 128 else 1e4
    case = _case(dtype, N, Hq, Hkv, D, bs, nb, seed=N + D + Hq)
    log(f"rope_kv_store {dtype} D={D} interleaved={interleaved} heads={heads} N={N}")
    got = _run(*case, theta, interleaved, dtype)
    r_q, r_k = _check(*case, theta, interleaved, dtype, *got)
    log(f"  max error / tolerance: q {r_q:.3f} k {r_k:.3f}")


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_kv_store_mixed_step_tokens(interleaved):
    """The 2,248 new tokens of the mixed continuous-batching step (4 x 512 chunk
    tokens, then 200 decode tokens) at their own positions and slots, in the
    full-size pool: every rotated element against the oracle, v and the rest of
    the pool bit-exact (the pool compare runs on the device)."""
    w = W.make_config(5)
    dtype, hkv, d = w.dtype, w.num_kv_heads, w.head_dim
    q = np.concatenate([w.pre_q, w.dec_q], axis=0)
    assert q.shape[0] == w.new_k.shape[0]
    pos = np.asarray(w.store_positions, dtype=np.int32)
    log(f"rope_kv_store mixed step: {q.shape[0]} tokens, interleaved={interleaved}")
    dq, dk, dv = to_dev(q, dtype), to_dev(w.new_k, dtype), to_dev(w.new_v, dtype)
    dkc, dvc = to_dev(w.k_cache, dtype), to_dev(w.v_cache, dtype)
    k_before, v_before = dkc.clone(), dvc.clone()
    slots = to_dev(w.slot_mapping)
    pkv.rope_kv_store(dq, dk, dv, to_dev(pos), dkc, dvc, slots, 1e6, interleaved)
    torch.cuda.synchronize()
    idx = slots.long()
    k_rows = dkc.view(-1, hkv, d)[idx]
    assert torch.equal(dvc.view(-1, hkv, d)[idx].view(torch.int16), dv.view(torch.int16))
    for before, after in ((k_before, dkc), (v_before, dvc)):
        expect = before.view(-1, hkv, d)
        expect[idx] = after.view(-1, hkv, d)[idx]
        assert torch.equal(expect.view(torch.int16), after.view(-1, hkv, d).view(torch.int16))
    del k_before, v_before, expect
    r_q = _within(to_host(dq, dtype), oracle.rope(oracle.widen(q, dtype), pos, 1e6, interleaved), interleaved, dtype)
    r_k = _within(to_host(k_rows, dtype), oracle.rope(oracle.widen(w.new_k, dtype), pos, 1e6, interleaved),
                  interleaved, dtype)
    log(f"  max error / tolerance: q {r_q:.3f} k {r_k:.3f}")
    assert r_q <= 1.0 and r_k <= 1.0, (r_q, r_k)


def test_rope_kv_store_zero_tokens_is_a_no_op():
    dtype = "bf16"
    q, k, v, pos, kc, vc, slots = _case(dtype, 0, 4, 2, 64, 16, 4, seed=1, neg_every=0)
    got = _run(q, k, v, pos, kc, vc, slots, 1e4, False, dtype)
    assert np.array_equal(bits(got[1]), bits(kc)) and np.array_equal(bits(got[2]), bits(vc))


def test_rope_kv_store_large_positions_stay_accurate():
    """Positions near 2^20, where an fp32 angle would have lost its fraction."""
    dtype = "f32"
    case = list(_case(dtype, 64, 8, 8, 128, 16, 8, seed=9, neg_every=0, max_pos=1 << 20))
    case[3] = (np.arange(64, dtype=np.int32) + (1 << 20) - 64)
    got = _run(*case, 1e4, False, dtype)
    r_q, r_k = _check(*case, 1e4, False, dtype, *got)
    log(f"  large positions: q {r_q:.3f} k {r_k:.3f} of the tolerance")
