"""Helpers for the GPU tests: move a workload to the device, run one step of
the HIP path through the Python binding, and run the same step through the
fp64 oracle on the host."""
from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import paged_kv_gqa_mapping_amd as pkv
import workloads as W

BF16_TOL = 2e-2
F32_TOL = 1e-5


def log(msg: str) -> None:
    print(f"[{time.strftime('%H:%M:%S')}] {msg}", flush=True)
    sys.stdout.flush()


def tol(dtype: str) -> float:
    return BF16_TOL if dtype == W.BF16 else F32_TOL


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """Host array -> device tensor; uint16 bf16 bit patterns become torch.bfloat16."""
    if a is None:
        return None
    if dtype == W.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def to_host(t: torch.Tensor, dtype: str) -> np.ndarray:
    """Device tensor -> host array in the oracle's storage format."""
    t = t.detach().cpu().contiguous()
    if dtype == W.BF16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def bits(a: np.ndarray) -> np.ndarray:
    """Raw bit view for bitwise comparisons (NaN payloads included)."""
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


class DeviceStep:
    """A workload's tensors on the GPU plus the calls of one step."""

    def __init__(self, w: W.Workload):
        self.w = w
        dt = w.dtype
        self.k_cache = to_dev(w.k_cache, dt)
        self.v_cache = to_dev(w.v_cache, dt)
        self.new_k = to_dev(w.new_k, dt)
        self.new_v = to_dev(w.new_v, dt)
        self.slots = to_dev(w.slot_mapping)
        self.dec = w.dec_q is not None
        self.pre = w.pre_q is not None
        if self.dec:
            self.dec_q = to_dev(w.dec_q, dt)
            self.dec_bt = to_dev(w.dec_block_tables)
            self.dec_cl = to_dev(w.dec_context_lens)
            self.dec_out = torch.empty_like(self.dec_q)
        if self.pre:
            self.pre_q = to_dev(w.pre_q, dt)
            self.pre_bt = to_dev(w.pre_block_tables)
            self.cu_q = to_dev(w.cu_seqlens_q)
            self.cu_k = to_dev(w.cu_seqlens_k)
            self.pre_out = torch.empty_like(self.pre_q)

    def store(self):
        pkv.kv_store(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slots)

    def decode(self, split_tokens: int = 0):
        w = self.w
        pkv.paged_decode_attn(self.dec_q, self.k_cache, self.v_cache, self.dec_bt, self.dec_cl, w.scale, self.dec_out,
                              max_context_len=w.max_context_len, split_tokens=split_tokens)

    def prefill(self, planned: bool = True):
        """planned: the device-planned work lists (the binding allocates their workspace)."""
        w = self.w
        pkv.paged_prefill_attn(self.pre_q, self.k_cache, self.v_cache, self.cu_q, self.cu_k, self.pre_bt,
                               self.pre_out, max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k, scale=w.scale,
                               planned=planned)

    def step(self, split_tokens: int = 0, planned: bool = True):
        self.store()
        if self.pre:
            self.prefill(planned)
        if self.dec:
            self.decode(split_tokens)
        torch.cuda.synchronize()


def oracle_caches(w: W.Workload):
    return oracle.kv_store(w.k_cache, w.v_cache, w.new_k, w.new_v, w.slot_mapping, w.block_size)


def oracle_decode(w: W.Workload, kc, vc, rows=None):
    """fp64 decode output for all sequences, or only the listed ones."""
    idx = np.arange(len(w.dec_context_lens)) if rows is None else np.asarray(rows)
    return oracle.decode(w.dec_q[idx], kc, vc, w.dec_block_tables[idx], w.dec_context_lens[idx], w.scale, w.dtype,
                         w.block_size)


def max_abs(gpu: np.ndarray, ref: np.ndarray, dtype: str) -> float:
    return float(np.max(np.abs(W.to_float32(gpu, dtype).astype(np.float64) - ref))) if ref.size else 0.0
