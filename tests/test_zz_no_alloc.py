"""The allocation-free decode entry point against the workspace one (GPU).

pkv_paged_decode_attn_noalloc runs the same kernels as pkv_paged_decode_attn
with the split states in the library's per-GPU scratch, so with the same
split length its outputs must be bit-identical.  Two calls in a row, the
second on a smaller input: the scratch keeps the first call's states, which
the second must not see.
"""
import numpy as np
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, log

pytestmark = pytest.mark.gpu


def _run_both(w, split):
    step = DeviceStep(w)
    step.store()
    ref = torch.empty_like(step.dec_q)
    pkv.paged_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, step.dec_cl, w.scale, ref,
                          max_context_len=w.max_context_len, split_tokens=split)
    got = torch.full_like(step.dec_q, float("nan"))
    pkv.paged_decode_attn_noalloc(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, step.dec_cl, w.scale, got,
                                  max_context_len=w.max_context_len, split_tokens=split)
    torch.cuda.synchronize()
    return ref, got


def _same_bits(a, b):
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def test_noalloc_decode_equals_workspace_decode_twice():
    big = W.make_config(3)  # 64 sequences of 2048-8192 keys, block 16, split-K with merge
    log(f"noalloc decode, first call: {big.name}")
    ref, got = _run_both(big, 0)
    assert _same_bits(ref, got)
    del ref, got
    seqs = [W.SeqSpec("decode", L, 1) for L in (1, 17, 300, 1000, 2049)]
    small = W.build("noalloc-small-f32", 7, W.F32, 8, 2, 64, 16, seqs)
    log("noalloc decode, second call: 5 sequences, fp32, 8/2 heads, D 64")
    ref, got = _run_both(small, 64)
    assert _same_bits(ref, got)
    assert np.isfinite(got.cpu().numpy()).all()


def test_noalloc_decode_rejects_states_above_the_scratch():
    limit = pkv.noalloc_scratch_bytes()
    assert limit == 64 << 20
    B, hq, hkv, d, bs = 256, 32, 8, 128, 16
    L = 65536
    need = pkv.decode_workspace_bytes(B, hq, d, L, 64)
    assert need > limit
    q = torch.zeros((B, hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, bs, hkv, d), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((B, L // bs), dtype=torch.int32, device="cuda")
    cl = torch.ones((B,), dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    with pytest.raises(pkv.PkvError, match="scratch"):
        pkv.paged_decode_attn_noalloc(q, kc, kc, bt, cl, 0.088, out, max_context_len=L, split_tokens=64)
