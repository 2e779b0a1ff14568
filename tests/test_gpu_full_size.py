"""The prefix-cached prefill and mixed-step workloads at full size, every output
row against the fp64 oracle (GPU).

* kv_store: both pools compared bit for bit with the oracle's, so the rows
  written and every row left alone are checked.
* attention: every query row of every sequence, element by element, within
  2e-2 (bf16 inputs, fp32 accumulation).
* shared prefix blocks: reading a block that several sequences share gives
  the same bits as reading a private copy of it placed elsewhere in the pool
  (blocks of a common prefix are reused by reference counting, "Nano-vLLM
  Architecture and Performance", Key Features, "Paged KV Cache"; a kernel only
  sees block ids, so sharing must not change any result).
* decode at the mixed step's context lengths (up to 32,768 keys) with fp32
  values at 1e-5: at that length one dropped or repeated key moves an output
  by about 1/L, which 2e-2 cannot see.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, bits, log, max_abs, oracle_caches, oracle_decode, to_dev, to_host, tol

pytestmark = pytest.mark.gpu


class Ran:
    """A workload after one step on the GPU, with the oracle's caches."""

    def __init__(self, w):
        self.w = w
        self.step = DeviceStep(w)
        self.step.step()
        self.kc, self.vc = oracle_caches(w)


@pytest.fixture(scope="module")
def c4():
    w = W.make_config(4)
    log("prefix-cached prefill workload built")
    r = Ran(w)
    yield r
    del r.step
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def c5():
    w = W.make_config(5)
    log("mixed-step workload built")
    r = Ran(w)
    yield r
    del r.step
    torch.cuda.empty_cache()


def _pools_bitwise(r):
    w = r.w
    for name, dev, ref in (("k_cache", r.step.k_cache, r.kc), ("v_cache", r.step.v_cache, r.vc)):
        got = to_host(dev, w.dtype)
        assert np.array_equal(bits(got), bits(ref)), f"{name} differs from the oracle's"


def _oracle_prefill(r):
    w = r.w
    if getattr(r, "pre_ref", None) is None:
        r.pre_ref = oracle.prefill(w.pre_q, r.kc, r.vc, w.cu_seqlens_q, w.cu_seqlens_k, w.pre_block_tables, w.scale,
                                   w.dtype, w.block_size)
    return r.pre_ref


def _one_launch_prefill(r):
    """The same prefill through the one-launch kernel (no workspace)."""
    s, w = r.step, r.w
    out = torch.empty_like(s.pre_out)
    pkv.paged_prefill_attn(s.pre_q, s.k_cache, s.v_cache, s.cu_q, s.cu_k, s.pre_bt, out, max_seqlen_q=w.max_seqlen_q,
                           max_seqlen_k=w.max_seqlen_k, scale=w.scale, planned=False)
    torch.cuda.synchronize()
    return out


def _with_private_copies(step, tables, rows, shared_ids):
    """Pools extended by one private copy of the shared blocks per listed table
    row, and tables whose listed rows point at their own copies instead."""
    nb = step.k_cache.shape[0]
    ids = torch.tensor(shared_ids, dtype=torch.long, device="cuda")
    reps = len(rows)
    k2 = torch.cat([step.k_cache, step.k_cache[ids].repeat(reps, 1, 1, 1)]).contiguous()
    v2 = torch.cat([step.v_cache, step.v_cache[ids].repeat(reps, 1, 1, 1)]).contiguous()
    t2 = tables.copy()
    n = len(shared_ids)
    for j, row in enumerate(rows):
        assert list(t2[row, :n]) == list(shared_ids)
        t2[row, :n] = nb + j * n + np.arange(n)
    return k2, v2, t2


# ------------------------------------------------------------------ prefix-cached prefill


def test_prefix_cached_prefill_store_bitwise(c4):
    _pools_bitwise(c4)
    # the two shared blocks hold the cached prefix and are never written
    for b in c4.w.shared_blocks:
        assert np.array_equal(bits(c4.kc[b]), bits(c4.w.k_cache[b]))
        assert np.array_equal(bits(c4.vc[b]), bits(c4.w.v_cache[b]))


def test_prefix_cached_prefill_every_row(c4):
    w = c4.w
    ref = _oracle_prefill(c4)
    got = to_host(c4.step.pre_out, w.dtype)
    err = max_abs(got, ref, w.dtype)
    log(f"prefix-cached prefill, all {got.shape[0]} query rows x {w.num_q_heads} heads: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_prefix_cached_prefill_one_launch_kernel_same_bits(c4):
    """No query tile here has more key tiles than the piece cap, so the planned
    kernel computes every tile exactly as the one-launch kernel does."""
    out = _one_launch_prefill(c4)
    assert torch.equal(out.view(torch.int16), c4.step.pre_out.view(torch.int16))


def test_prefix_cached_prefill_shared_equals_private_bitwise(c4):
    w, s = c4.w, c4.step
    rows = list(range(len(w.cu_seqlens_q) - 1))
    k2, v2, t2 = _with_private_copies(s, w.pre_block_tables, rows, w.shared_blocks)
    out2 = torch.empty_like(s.pre_out)
    pkv.paged_prefill_attn(s.pre_q, k2, v2, s.cu_q, s.cu_k, to_dev(t2), out2, max_seqlen_q=w.max_seqlen_q,
                           max_seqlen_k=w.max_seqlen_k, scale=w.scale, planned=True)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), s.pre_out.view(torch.int16))


# ------------------------------------------------------------------ mixed step


def test_mixed_step_store_bitwise(c5):
    _pools_bitwise(c5)
    for b in c5.w.shared_blocks:
        assert np.array_equal(bits(c5.kc[b]), bits(c5.w.k_cache[b]))
        assert np.array_equal(bits(c5.vc[b]), bits(c5.w.v_cache[b]))


def test_mixed_step_decode_every_row(c5):
    w = c5.w
    ref = oracle_decode(w, c5.kc, c5.vc)
    got = to_host(c5.step.dec_out, w.dtype)
    err = max_abs(got, ref, w.dtype)
    log(f"mixed step decode, all {got.shape[0]} sequences: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_mixed_step_prefill_every_row(c5):
    w = c5.w
    ref = _oracle_prefill(c5)
    got = to_host(c5.step.pre_out, w.dtype)
    err = max_abs(got, ref, w.dtype)
    log(f"mixed step prefill, all {got.shape[0]} chunk rows: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_mixed_step_prefill_one_launch_kernel_every_row(c5):
    """The chunks' query tiles are cut into pieces by the planned path; the
    one-launch kernel computes them whole.  Both against the oracle."""
    w = c5.w
    got = to_host(_one_launch_prefill(c5), w.dtype)
    err = max_abs(got, _oracle_prefill(c5), w.dtype)
    log(f"mixed step prefill, one-launch kernel, all rows: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_mixed_step_prefill_repeats_bitwise(c5):
    s = c5.step
    first = s.pre_out.clone()
    s.prefill()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), s.pre_out.view(torch.int16))


def test_mixed_step_decode_shared_equals_private_bitwise(c5):
    w, s = c5.w, c5.step
    sharers = w.notes["sharers"]
    k2, v2, t2 = _with_private_copies(s, w.dec_block_tables, sharers, w.shared_blocks)
    out2 = torch.empty_like(s.dec_out)
    pkv.paged_decode_attn(s.dec_q, k2, v2, to_dev(t2), s.dec_cl, w.scale, out2, max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), s.dec_out.view(torch.int16))


def test_mixed_step_cascade_every_row(c5):
    """Shared-prefix decode of the step's 200 sequences (50 behind one
    16-block prefix), every row against the oracle."""
    w, s = c5.w, c5.step
    shared, offsets, seqs, gmax, smax, own = w.cascade_groups()
    out = torch.empty_like(s.dec_q)
    pkv.cascade_decode_attn(s.dec_q, s.k_cache, s.v_cache, s.dec_bt, s.dec_cl, to_dev(shared), to_dev(offsets),
                            to_dev(seqs), w.scale, out, max_context_len=w.max_context_len, max_group_size=gmax,
                            max_shared_len=smax, max_own_len=own)
    torch.cuda.synchronize()
    err = max_abs(to_host(out, w.dtype), oracle_decode(w, c5.kc, c5.vc), w.dtype)
    log(f"mixed step shared-prefix decode, all rows: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


# ------------------------------------------------------------------ long contexts in fp32


def _long_fp32_case():
    """The mixed step's decode lengths in fp32 on a subset of sequences that keeps
    the pool small: the 8 longest, the shortest, and 4 of the sequences behind the
    shared 16-block prefix (with the prefix shared as in the mixed step)."""
    w5 = W.make_config(5)
    lens = w5.dec_context_lens
    sharers = set(w5.notes["sharers"])
    order = list(np.argsort(-lens, kind="stable"))
    pick = order[:8] + [int(np.argmin(lens))]
    pick += [j for j in sorted(sharers) if j not in pick][:4]
    seqs = [W.SeqSpec("decode", int(lens[j]), 1, shared=16 if j in sharers else 0) for j in pick]
    del w5
    return W.build("mixed-step-decode-lengths-f32", 55, W.F32, 32, 8, 128, 256, seqs, shared_prefix_blocks=16)


@pytest.fixture(scope="module")
def long_f32():
    w = _long_fp32_case()
    log(f"fp32 long-context case built: contexts {w.dec_context_lens.tolist()}")
    s = DeviceStep(w)
    s.store()
    torch.cuda.synchronize()
    kc, vc = oracle_caches(w)
    ref = oracle_decode(w, kc, vc)
    yield w, s, ref
    del s
    torch.cuda.empty_cache()


@pytest.mark.parametrize("split", [0, 2048, 512, pkv.SPLIT_BALANCED])
def test_long_context_decode_fp32(long_f32, split):
    w, s, ref = long_f32
    assert int(w.dec_context_lens.max()) > 30000
    s.decode(split_tokens=split)
    torch.cuda.synchronize()
    err = max_abs(to_host(s.dec_out, w.dtype), ref, w.dtype)
    log(f"fp32 decode up to {w.max_context_len} keys, split {split}: max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_long_context_decode_fp32_shared_equals_private(long_f32):
    w, s, _ = long_f32
    s.decode()
    torch.cuda.synchronize()
    rows = [i for i, q in enumerate([x for x in w.seqs if x.kind == "decode"]) if q.shared]
    k2, v2, t2 = _with_private_copies(s, w.dec_block_tables, rows, w.shared_blocks)
    out2 = torch.empty_like(s.dec_out)
    pkv.paged_decode_attn(s.dec_q, k2, v2, to_dev(t2), s.dec_cl, w.scale, out2, max_context_len=w.max_context_len)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int32), s.dec_out.view(torch.int32))
