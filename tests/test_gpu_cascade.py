"""Shared-prefix ("cascade") decode on the GPU against the fp64 oracle.

The result must be plain decode's (same definition), so the bar is the decode
bar: max abs error <= 2e-2 for bf16.  With no groups the call must give plain
decode's bits (same kernels, same path).
"""
import numpy as np
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, log, max_abs, oracle_caches, oracle_decode, to_dev, to_host, tol

pytestmark = pytest.mark.gpu


def cascade_meta(w, group_cap=None):
    return w.cascade_groups(group_cap)


def run_cascade(step, meta, split_tokens=0):
    w = step.w
    shared, offsets, seqs, gmax, smax, own = meta
    out = torch.empty_like(step.dec_q)
    pkv.cascade_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, step.dec_cl, to_dev(shared),
                            to_dev(offsets), to_dev(seqs), w.scale, out, max_context_len=w.max_context_len,
                            max_group_size=gmax, max_shared_len=smax, max_own_len=own, split_tokens=split_tokens)
    torch.cuda.synchronize()
    return out


def _shared_case(hq, hkv, d, bs, n, prefix_blocks, seed, big_group=False):
    rng = np.random.default_rng(seed)
    seqs = []
    for j in range(n):
        if big_group or j % 3 == 0:
            sh = prefix_blocks
        elif j % 3 == 1:
            sh = prefix_blocks // 2
        else:
            sh = 0
        L = sh * bs + int(rng.integers(1, 5 * bs))
        if j % 7 == 5:
            L = sh * bs + 1  # only the newest token is the sequence's own
        seqs.append(W.SeqSpec("decode", L, 1, shared=sh))
    return W.build(f"cascade-{hq}-{hkv}-{d}-{bs}", seed, "bf16", hq, hkv, d, bs, seqs,
                   shared_prefix_blocks=prefix_blocks, perm_rng=rng)


SHAPES = [(32, 8, 128, 16), (16, 8, 128, 256), (8, 1, 128, 32), (16, 2, 64, 8), (4, 4, 64, 16), (64, 8, 128, 64),
          (16, 4, 64, 32)]


@pytest.mark.parametrize("split", [0, 64, pkv.SPLIT_BALANCED])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_cascade_sweep(shape, split):
    hq, hkv, d, bs = shape
    prefix = max(2, 1024 // bs) if bs <= 64 else 4
    w = _shared_case(hq, hkv, d, bs, 40, prefix, seed=hq + d + bs)
    log(f"cascade sweep {shape} split={split} prefix={prefix} blocks")
    step = DeviceStep(w)
    step.store()
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    out = run_cascade(step, cascade_meta(w), split)
    err = max_abs(to_host(out, "bf16"), oracle_decode(w, kc, vc), "bf16")
    log(f"  max abs error {err:.3g}")
    assert err <= tol("bf16"), err


@pytest.mark.parametrize("hq,hkv", [(32, 8), (16, 8), (64, 8)])
def test_cascade_groups_larger_than_a_workgroup(hq, hkv):
    """100 members in one group (several member tiles), also cut into groups of 7."""
    w = _shared_case(hq, hkv, 128, 16, 100, 20, seed=hq, big_group=True)
    step = DeviceStep(w)
    step.store()
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    ref = oracle_decode(w, kc, vc)
    for cap in (None, 7):
        out = run_cascade(step, cascade_meta(w, cap))
        err = max_abs(to_host(out, "bf16"), ref, "bf16")
        log(f"cascade 100 members {hq}/{hkv} groups of {cap or 100}: max abs error {err:.3g}")
        assert err <= tol("bf16"), err


def test_cascade_without_groups_is_plain_decode_bitwise():
    w = _shared_case(32, 8, 128, 16, 30, 8, seed=5)
    step = DeviceStep(w)
    step.store()
    step.decode(split_tokens=64)
    torch.cuda.synchronize()
    plain = to_host(step.dec_out, "bf16").copy()
    empty = (np.zeros(len(plain), np.int32), np.zeros(1, np.int32), np.zeros(1, np.int32), 0, 0, 0)
    out = run_cascade(step, empty, 64)
    assert np.array_equal(to_host(out, "bf16"), plain)


def test_cascade_argument_errors():
    w = _shared_case(32, 8, 128, 16, 6, 4, seed=6)
    step = DeviceStep(w)
    shared, offsets, seqs, gmax, smax, own = cascade_meta(w)
    with pytest.raises(pkv.PkvError):  # shared length not a whole number of blocks
        run_cascade(step, (shared, offsets, seqs, gmax, smax + 3, own))
    w32 = W.build("cascade-f32", 6, "f32", 32, 8, 128, 16, w.seqs, shared_prefix_blocks=4)
    step32 = DeviceStep(w32)
    with pytest.raises(pkv.PkvError, match="bf16"):
        run_cascade(step32, cascade_meta(w32))


@pytest.mark.parametrize("shape", [(32, 8, 128, 16), (16, 4, 64, 16)], ids=lambda s: "-".join(map(str, s)))
def test_cascade_prefix_not_a_whole_tile(shape):
    """A 144-key shared prefix (9 blocks of 16): the group pass's only chunk ends
    16 keys into its second 128-key tile, so its tail keys are masked."""
    hq, hkv, d, bs = shape
    w = _shared_case(hq, hkv, d, bs, 24, 9, seed=17)
    step = DeviceStep(w)
    step.store()
    torch.cuda.synchronize()
    meta = cascade_meta(w)
    assert meta[4] == 144
    kc, vc = oracle_caches(w)
    out = run_cascade(step, meta)
    err = max_abs(to_host(out, "bf16"), oracle_decode(w, kc, vc), "bf16")
    log(f"cascade 144-key prefix {shape}: max abs error {err:.3g}")
    assert err <= tol("bf16"), err


def test_cascade_rejects_non_positive_scale():
    w = _shared_case(32, 8, 128, 16, 12, 9, seed=18)
    step = DeviceStep(w)
    shared, offsets, seqs, gmax, smax, own = cascade_meta(w)
    for scale in (0.0, -0.088):
        out = torch.empty_like(step.dec_q)
        with pytest.raises(pkv.PkvError, match="scale"):
            pkv.cascade_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, step.dec_cl, to_dev(shared),
                                    to_dev(offsets), to_dev(seqs), scale, out, max_context_len=w.max_context_len,
                                    max_group_size=gmax, max_shared_len=smax, max_own_len=own)


def test_config6_shared_prompt_cascade():
    """64 sequences behind one 16,384-token prompt: every row against plain GPU
    decode and against the oracle.  (The mixed step's batch is checked row by row
    in test_gpu_full_size.py.)"""
    w = W.make_config(6)
    step = DeviceStep(w)
    step.store()
    step.decode()
    torch.cuda.synchronize()
    plain = to_host(step.dec_out, w.dtype).copy()
    out = to_host(run_cascade(step, cascade_meta(w)), w.dtype)
    diff = float(np.max(np.abs(W.to_float32(out, w.dtype) - W.to_float32(plain, w.dtype))))
    log(f"config 6 cascade vs plain decode: max abs difference {diff:.3g}")
    assert diff <= tol(w.dtype)
    kc, vc = oracle_caches(w)
    err = max_abs(out, oracle_decode(w, kc, vc), w.dtype)
    log(f"config 6 cascade, all rows: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err
