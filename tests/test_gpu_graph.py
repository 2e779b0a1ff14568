"""The whole step (kv_store, prefill, decode split + reduce) captured once in a
HIP graph and replayed: every replay must give the eager result bit for bit
(the kernels are deterministic and the library neither allocates nor
synchronizes, so capture needs nothing else).  Between replays the program
does its own eager work and synchronizes."""
import numpy as np
import pytest
import torch

import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, log, to_dev, to_host

pytestmark = pytest.mark.gpu


def _capture_inputs(w, split):
    st = DeviceStep(w)
    B, Hq, D = st.dec_q.shape
    ws = torch.empty(max(pkv.decode_workspace_bytes(B, Hq, D, w.max_context_len, split), 16), dtype=torch.uint8,
                     device="cuda")
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()

    def step():
        pkv.kv_store(st.new_k, st.new_v, st.k_cache, st.v_cache, st.slots)
        pkv.paged_prefill_attn(st.pre_q, st.k_cache, st.v_cache, st.cu_q, st.cu_k, st.pre_bt, st.pre_out,
                               max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, scale=w.scale)
        pkv.paged_decode_attn(st.dec_q, st.k_cache, st.v_cache, st.dec_bt, st.dec_cl, w.scale, st.dec_out,
                              max_context_len=w.max_context_len, split_tokens=split, workspace=ws)

    return st, step, k0, v0


@pytest.mark.parametrize("split", [256, pkv.SPLIT_BALANCED])
def test_graph_replays_match_eager_bitwise(split):
    seqs = [W.SeqSpec("prefill", 900, 300), W.SeqSpec("prefill", 130, 130)]
    seqs += [W.SeqSpec("decode", L, 1) for L in (1, 40, 700, 1500, 3000)]
    w = W.build("graph-step", 21, "bf16", 32, 8, 128, 64, seqs)
    st, step, k0, v0 = _capture_inputs(w, split)
    log("eager step")
    step()
    torch.cuda.synchronize()
    ref_dec, ref_pre = st.dec_out.clone(), st.pre_out.clone()
    ref_k = st.k_cache.clone()

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    log("capture")
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(4):
        # the program's own eager work between replays: clobber outputs, restore the caches
        st.dec_out.fill_(7.0)
        st.pre_out.fill_(-3.0)
        st.k_cache.copy_(k0)
        st.v_cache.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"replay {r}")
        assert torch.equal(st.dec_out.view(torch.int16), ref_dec.view(torch.int16)), f"decode differs on replay {r}"
        assert torch.equal(st.pre_out.view(torch.int16), ref_pre.view(torch.int16)), f"prefill differs on replay {r}"
        assert torch.equal(st.k_cache.view(torch.int16), ref_k.view(torch.int16)), f"kv_store differs on replay {r}"


def test_graph_replay_sees_new_inputs():
    # a replay reads the current contents of the captured buffers: new queries give new outputs
    seqs = [W.SeqSpec("decode", L, 1) for L in (5, 300, 1000)]
    w = W.build("graph-inputs", 22, "bf16", 16, 8, 128, 16, seqs)
    st = DeviceStep(w)
    st.store()
    out = torch.empty_like(st.dec_q)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ws = torch.empty(max(pkv.decode_workspace_bytes(3, 16, 128, 1000, 256), 16), dtype=torch.uint8, device="cuda")

    def dec():
        pkv.paged_decode_attn(st.dec_q, st.k_cache, st.v_cache, st.dec_bt, st.dec_cl, w.scale, out,
                              max_context_len=1000, split_tokens=256, workspace=ws)

    with torch.cuda.stream(s):
        dec()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        dec()
    for seed in (1, 2):
        q = W.fill_normal(tuple(st.dec_q.shape), "bf16", 100 + seed, 5)
        st.dec_q.copy_(to_dev(q, "bf16"))
        g.replay()
        torch.cuda.synchronize()
        got = to_host(out, "bf16").copy()
        dec()
        torch.cuda.synchronize()
        assert np.array_equal(got, to_host(out, "bf16"))


@pytest.mark.parametrize("split", [512, pkv.SPLIT_BALANCED])
def test_graph_fused_store_decode_step_matches_eager(split):
    """The decode step with the cache write fused in (one launch plus the merge)
    captured and replayed: outputs and caches equal the eager two-call step."""
    seqs = [W.SeqSpec("decode", L, 1) for L in (1, 17, 256, 257, 1000, 4000)]
    w = W.build("graph-fused", 23, "bf16", 32, 8, 128, 16, seqs)
    ref = DeviceStep(w)
    ref.store()
    ref.decode(split_tokens=split)
    torch.cuda.synchronize()
    st = DeviceStep(w)
    B, Hq, D = st.dec_q.shape
    ws = torch.empty(max(pkv.decode_workspace_bytes(B, Hq, D, w.max_context_len, split), 16), dtype=torch.uint8,
                     device="cuda")
    k0, v0 = st.k_cache.clone(), st.v_cache.clone()
    out = torch.empty_like(st.dec_q)

    def step():
        pkv.paged_decode_store_attn(st.dec_q, st.new_k, st.new_v, st.k_cache, st.v_cache, st.dec_bt, st.dec_cl,
                                    w.scale, out, max_context_len=w.max_context_len, split_tokens=split, workspace=ws)

    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        out.fill_(5.0)
        st.k_cache.copy_(k0)
        st.v_cache.copy_(v0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        log(f"fused replay {r}")
        assert torch.equal(out.view(torch.int16), ref.dec_out.view(torch.int16))
        assert torch.equal(st.k_cache.view(torch.int16), ref.k_cache.view(torch.int16))
        assert torch.equal(st.v_cache.view(torch.int16), ref.v_cache.view(torch.int16))
