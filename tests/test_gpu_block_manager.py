"""The block manager's tables and slots driving the kernels: prompts are
stored through their slots (tokens found in the prefix cache are not stored
again), one token is appended per sequence, and decode runs over the tables;
caches are compared bitwise and outputs against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import bits, log, max_abs, to_dev, to_host

pytestmark = pytest.mark.gpu


def _rows(tokens, hkv, d, stream):
    # K (stream 1) or V (stream 2) rows as a function of the token and its prefix
    out = np.empty((len(tokens), hkv, d), dtype=np.uint16)
    for p in range(len(tokens)):
        seed = hash((tuple(tokens[:p + 1]),)) & 0x7FFFFFFF
        out[p] = W.fill_normal((hkv, d), "bf16", seed, stream)
    return out


def test_block_manager_drives_store_and_decode():
    rng = np.random.default_rng(5)
    bs, nb, hq, hkv, d = 16, 96, 16, 4, 128
    bm = pkv.BlockManager(nb, bs)
    shared = list(rng.integers(0, 1000, size=2 * bs))
    prompts = [shared + list(rng.integers(0, 1000, size=n)) for n in (5, 17, 40)]
    prompts += [list(rng.integers(0, 1000, size=n)) for n in (1, 33, 70)]
    kc = W.fill_normal((nb, bs, hkv, d), "bf16", 1, 1)
    vc = W.fill_normal((nb, bs, hkv, d), "bf16", 1, 2)
    kc[:] = 0x7FC0  # poison everything; only stored rows become finite
    vc[:] = 0x7FC0
    host_k, host_v = kc.copy(), vc.copy()
    dk, dv = to_dev(kc, "bf16"), to_dev(vc, "bf16")
    cached = []
    for sid, toks in enumerate(prompts):
        c = bm.allocate(sid, toks)
        cached.append(c)
        new = toks[c:]
        slots = bm.slot_mapping(sid, c, len(new))
        k_rows = _rows(toks, hkv, d, 1)[c:]
        v_rows = _rows(toks, hkv, d, 2)[c:]
        if len(new):
            pkv.kv_store(to_dev(k_rows, "bf16"), to_dev(v_rows, "bf16"), dk, dv, to_dev(slots))
            host_k, host_v = oracle.kv_store(host_k, host_v, k_rows, v_rows, slots, bs)
    assert cached[:3] == [0, 2 * bs, 2 * bs] and cached[3:] == [0, 0, 0]
    # one decode step: append a token to every sequence, store it, attend
    new_tok = [int(t) for t in rng.integers(0, 1000, size=len(prompts))]
    slots = np.asarray([bm.append(sid, t) for sid, t in enumerate(new_tok)], dtype=np.int32)
    full = [p + [t] for p, t in zip(prompts, new_tok)]
    k_new = np.stack([_rows(f, hkv, d, 1)[-1] for f in full])
    v_new = np.stack([_rows(f, hkv, d, 2)[-1] for f in full])
    pkv.kv_store(to_dev(k_new, "bf16"), to_dev(v_new, "bf16"), dk, dv, to_dev(slots))
    host_k, host_v = oracle.kv_store(host_k, host_v, k_new, v_new, slots, bs)
    width = max(-(-len(f) // bs) for f in full)
    pad = int(np.flatnonzero([bm.refcount(b) == 0 for b in range(nb)])[0])
    tables = np.stack([bm.block_table(sid, width=width, pad=pad) for sid in range(len(full))])
    lens = np.asarray([bm.seq_len(sid) for sid in range(len(full))], dtype=np.int32)
    q = W.fill_normal((len(full), hq, d), "bf16", 9, 5)
    out = torch.empty((len(full), hq, d), dtype=torch.bfloat16, device="cuda")
    log("decode over block-manager tables")
    pkv.paged_decode_attn(to_dev(q, "bf16"), dk, dv, to_dev(tables), to_dev(lens), 0.088, out,
                          max_context_len=int(lens.max()), split_tokens=64)
    torch.cuda.synchronize()
    assert np.array_equal(bits(to_host(dk, "bf16")), bits(host_k))
    assert np.array_equal(bits(to_host(dv, "bf16")), bits(host_v))
    ref = oracle.decode(q, host_k, host_v, tables, lens, 0.088, "bf16", bs)
    err = max_abs(to_host(out, "bf16"), ref, "bf16")
    assert err <= 2e-2, err
    assert np.isfinite(W.to_float32(to_host(out, "bf16"), "bf16")).all()
