"""Device-side precondition checks: zero counts on every workload's metadata,
the right counter for each kind of planted violation, and the binding's debug
mode refusing a call before it launches.  The check kernels read metadata
only; the one test that reaches an attention call gives the caches slack
blocks past `num_blocks`, so even a missed check could not read outside them."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, log, to_dev

pytestmark = pytest.mark.gpu

ZERO = {n: 0 for n in pkv.CHECK_NAMES}


def _only(counts, name, at_least=1):
    assert counts[name] >= at_least, counts
    assert all(v == 0 for k, v in counts.items() if k != name), counts


@pytest.mark.parametrize("i", [1, 2, 3, 4, 5, 6])
def test_every_workload_passes(i):
    w = W.make_config(i)
    log(f"checks on workload {i}")
    nb, bs = w.num_blocks, w.block_size
    assert pkv.check_slots(to_dev(w.slot_mapping), nb, bs) == ZERO
    if w.dec_q is not None:
        bt, cl = to_dev(w.dec_block_tables), to_dev(w.dec_context_lens)
        assert pkv.check_decode_inputs(bt, cl, w.max_context_len, nb, bs) == ZERO
        sh, go, gs, gm, sm, own = w.cascade_groups()
        if len(go) > 1:
            assert pkv.check_cascade_inputs(bt, cl, to_dev(sh), to_dev(go), to_dev(gs), gm, sm, bs) == ZERO
    if w.pre_q is not None:
        assert pkv.check_prefill_inputs(to_dev(w.cu_seqlens_q), to_dev(w.cu_seqlens_k), to_dev(w.pre_block_tables),
                                        w.max_seqlen_q, w.max_seqlen_k, nb, bs) == ZERO
        # packed k/v: no table
        assert pkv.check_prefill_inputs(to_dev(w.cu_seqlens_q), to_dev(w.cu_seqlens_k), None, w.max_seqlen_q,
                                        w.max_seqlen_k, int(w.cu_seqlens_k[-1]), 1) == ZERO


def _decode_meta():
    w = W.make_config(2)
    return w, w.dec_block_tables.copy(), w.dec_context_lens.copy()


def test_decode_violations():
    w, bt, cl = _decode_meta()
    nb, bs, L = w.num_blocks, w.block_size, w.max_context_len

    def run(bt_, cl_, maxL=L):
        return pkv.check_decode_inputs(to_dev(bt_), to_dev(cl_), maxL, nb, bs)

    b = int(np.argmax(cl))
    used = -(-int(cl[b]) // bs)
    bad = bt.copy()
    bad[b, used - 1] = nb                   # one past the pool, in a used position
    _only(run(bad, cl), "block_id", 1)
    bad = bt.copy()
    bad[3, 0] = -7
    bad[5, 0] = nb + 100
    _only(run(bad, cl), "block_id", 2)
    unused = bt.copy()
    short = int(np.argmin(cl))
    if -(-int(cl[short]) // bs) < bt.shape[1]:
        unused[short, -1] = -1                  # past the sequence's used blocks: not read, not a violation
        assert run(unused, cl) == ZERO
    badl = cl.copy()
    badl[0] = L + 1
    badl[1] = -2
    _only(run(bt, badl), "length", 2)
    # a context that needs more blocks than a table row holds
    badl = cl.copy()
    badl[2] = bt.shape[1] * bs + 1
    _only(run(bt, badl, maxL=bt.shape[1] * bs + 1), "length", 1)


def test_prefill_violations():
    w = W.make_config(4)
    cq, ck, bt = w.cu_seqlens_q.copy(), w.cu_seqlens_k.copy(), w.pre_block_tables.copy()
    nb, bs = w.num_blocks, w.block_size

    def run(cq_, ck_, bt_=bt, mq=w.max_seqlen_q, mk=w.max_seqlen_k):
        return pkv.check_prefill_inputs(to_dev(cq_), to_dev(ck_), None if bt_ is None else to_dev(bt_), mq, mk,
                                        nb, bs)

    bad = cq.copy()
    bad[3] = bad[2] - 1                         # decreasing
    assert run(bad, ck)["cu_seqlens"] >= 1
    bad = cq.copy()
    bad[1:] += 600                              # sequence 0 gets 600 more queries than keys
    assert run(bad, ck)["cu_seqlens"] >= 1
    assert run(cq, ck, mq=w.max_seqlen_q - 1)["cu_seqlens"] >= 1
    assert run(cq, ck, mk=w.max_seqlen_k - 1)["cu_seqlens"] >= 1
    bad = cq.copy()
    bad += 1                                    # does not start at 0
    assert run(bad, ck)["cu_seqlens"] >= 1
    badt = bt.copy()
    badt[7, 1] = nb
    _only(run(cq, ck, badt), "block_id", 1)


def test_slot_violations():
    w = W.make_config(5)
    sl = w.slot_mapping.copy()
    nb, bs = w.num_blocks, w.block_size
    bad = sl.copy()
    bad[10] = nb * bs
    bad[11] = nb * bs + 12345
    _only(pkv.check_slots(to_dev(bad), nb, bs), "slot", 2)
    dup = sl.copy()
    dup[100] = dup[2000]
    dup[5] = dup[6]
    _only(pkv.check_slots(to_dev(dup), nb, bs), "duplicate_slot", 2)
    assert pkv.check_slots(to_dev(dup), nb, bs, duplicates=False) == ZERO
    skip = sl.copy()
    skip[::7] = -1
    assert pkv.check_slots(to_dev(skip), nb, bs) == ZERO


def test_cascade_violations():
    w = W.make_config(5)
    bt, cl = w.dec_block_tables.copy(), w.dec_context_lens.copy()
    sh, go, gs, gm, sm, own = w.cascade_groups()
    bs = w.block_size

    def run(bt_=bt, sh_=sh, go_=go, gs_=gs, gm_=gm, sm_=sm):
        return pkv.check_cascade_inputs(to_dev(bt_), to_dev(cl), to_dev(sh_), to_dev(go_), to_dev(gs_), gm_, sm_, bs)

    member = int(gs[7])
    bad = bt.copy()
    bad[member, 3] = bad[member, 20]            # a member whose 4th shared block differs
    _only(run(bt_=bad), "shared_prefix", 1)
    bads = sh.copy()
    bads[member] = sh[member] - bs              # shared length differs from its group's
    _only(run(sh_=bads), "shared_prefix", 1)
    bads = sh.copy()
    bads[gs] = sh[gs] - 3                       # not whole blocks
    assert run(sh_=bads, sm_=sm)["shared_prefix"] >= len(gs)
    outsider = int(np.flatnonzero(sh == 0)[0])
    bads = sh.copy()
    bads[outsider] = sh[member]                 # a sharer that no group names
    _only(run(sh_=bads), "group", 1)
    go2 = np.array([0, len(gs), 2 * len(gs)], np.int32)
    gs2 = np.concatenate([gs, gs]).astype(np.int32)  # every member in two groups
    assert run(go_=go2, gs_=gs2)["group"] >= len(gs)
    goff = go.copy()
    goff[-1] = len(gs) + 5                      # offsets past the member list
    assert run(go_=goff, gm_=gm + 5)["group"] >= 1
    assert run(gm_=gm - 1)["group"] >= 1        # group larger than max_group_size


def test_debug_mode_refuses_before_launch(monkeypatch):
    """A block id one past num_blocks: the call raises before any attention
    kernel runs (the caches have 4 slack blocks, so nothing could be read
    outside them regardless)."""
    w = W.make_config(2)
    step = DeviceStep(w)
    nb = w.num_blocks
    hkv, d, bs = w.num_kv_heads, w.head_dim, w.block_size
    kc = torch.zeros((nb + 4, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    bt = w.dec_block_tables.copy()
    b = int(np.argmax(w.dec_context_lens))
    bt[b, 0] = nb
    monkeypatch.setattr(pkv, "DEBUG_CHECKS", True)
    with pytest.raises(pkv.PkvError, match="block_id"):
        pkv.paged_decode_attn(step.dec_q, kc[:nb], vc[:nb], to_dev(bt), step.dec_cl, w.scale, step.dec_out,
                              max_context_len=w.max_context_len)
    # a valid call still runs in debug mode
    pkv.paged_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, step.dec_cl, w.scale, step.dec_out,
                          max_context_len=w.max_context_len)
    torch.cuda.synchronize()
