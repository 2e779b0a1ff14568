"""Decode with the newest token's cache write fused in: outputs and the whole
cache pool must be bit-identical to kv_store followed by decode (the path the
other tests pin to the oracle), on the decode shapes, both split choices and
the decode workloads at full size."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, bits, log, max_abs, oracle_caches, oracle_decode, to_host, tol

pytestmark = pytest.mark.gpu

SHAPES = [
    ("f32", 4, 2, 64, 16), ("f32", 32, 8, 128, 256), ("bf16", 16, 8, 128, 256), ("bf16", 32, 8, 128, 16),
    ("bf16", 8, 1, 128, 32), ("bf16", 16, 2, 64, 8), ("bf16", 64, 8, 128, 64), ("bf16", 4, 4, 64, 16),
    ("bf16", 16, 4, 64, 32),
]


def _both(w, split=0):
    """(outputs, k_cache, v_cache) of the two-call path and of the fused call."""
    a = DeviceStep(w)
    a.store()
    a.decode(split_tokens=split)
    b = DeviceStep(w)
    out = torch.empty_like(b.dec_q)
    pkv.paged_decode_store_attn(b.dec_q, b.new_k, b.new_v, b.k_cache, b.v_cache, b.dec_bt, b.dec_cl, w.scale, out,
                                max_context_len=w.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    dt = w.dtype
    return ((to_host(a.dec_out, dt), to_host(a.k_cache, dt), to_host(a.v_cache, dt)),
            (to_host(out, dt), to_host(b.k_cache, dt), to_host(b.v_cache, dt)))


def _same(x, y):
    for p, q in zip(x, y):
        assert np.array_equal(bits(p), bits(q))


@pytest.mark.parametrize("split", [0, 64, pkv.SPLIT_BALANCED])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_fused_store_matches_two_calls_bitwise(shape, split):
    dtype, hq, hkv, d, bs = shape
    lens = [1, 2, bs - 1, bs, bs + 1, 3 * bs + 1, 63, 64, 65, 200, 517, 1]
    seqs = [W.SeqSpec("decode", int(L), 1) for L in lens]
    w = W.build(f"fused-{dtype}-{hq}-{hkv}-{d}-{bs}", hq + d + bs, dtype, hq, hkv, d, bs, seqs)
    log(f"fused store {shape} split={split}")
    two, fused = _both(w, split)
    _same(two, fused)
    # and against the oracle directly
    kc, vc = oracle_caches(w)
    assert max_abs(fused[0], oracle_decode(w, kc, vc), dtype) <= tol(dtype)


@pytest.mark.parametrize("i,dtype", [(1, None), (2, None), (3, None), (2, "f32")])
def test_fused_store_decode_workloads(i, dtype):
    w = W.make_config(i, dtype=dtype)
    log(f"fused store on workload {i} {w.dtype}")
    two, fused = _both(w)
    _same(two, fused)


def test_fused_store_single_token_contexts_return_v():
    """Every context is just the new token: the output is that token's V (exact)."""
    seqs = [W.SeqSpec("decode", 1, 1) for _ in range(9)]
    w = W.build("fused-one", 3, "bf16", 32, 8, 128, 16, seqs)
    two, fused = _both(w)
    _same(two, fused)
    G = w.num_q_heads // w.num_kv_heads
    expect = np.repeat(w.new_v, G, axis=1)
    assert np.array_equal(fused[0], expect)
