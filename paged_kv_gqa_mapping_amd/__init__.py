"""Paged-KV GQA attention for AMD MI355X (gfx950): Python binding of libpkv.so.

The binding only marshals arguments: it checks tensor shapes, dtypes and
devices, derives the sizes, and calls the C ABI (include/pkv.h) with raw
device pointers and the current HIP stream.  Every step of the computation
runs in the library's HIP kernels.  There is no fallback: if libpkv.so has not
been built (``python -m paged_kv_gqa_mapping_amd.build``) every call raises.

Entry points (names follow the operations of a nano-vLLM style engine):

* ``kv_store(k, v, k_cache, v_cache, slot_mapping)``
* ``paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, scale, out)``
* ``paged_prefill_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, block_tables, out)``
* ``paged_gather(k_cache, v_cache, block_tables, cu_seqlens_k)``
* ``rope_kv_store(q, k, v, positions, k_cache, v_cache, slot_mapping, rope_theta)``
* ``cascade_decode_attn(q, k_cache, v_cache, block_tables, context_lens, shared_lens,
  group_offsets, group_seqs, scale, out)``
* ``check_decode_inputs``, ``check_prefill_inputs``, ``check_slots``,
  ``check_cascade_inputs``: device-side precondition checks (counts per kind).
  With the environment variable ``PKV_DEBUG_CHECKS=1`` every call runs the
  matching checks first and raises ``PkvError`` on a violation (this
  synchronizes, so it is for debugging, not for graph capture).

Tensors: caches ``[num_blocks, block_size, num_kv_heads, head_dim]``;
``torch.bfloat16`` or ``torch.float32``; metadata ``torch.int32``; all on the
GPU and contiguous.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "kv_store",
    "paged_decode_attn",
    "paged_decode_attn_noalloc",
    "noalloc_scratch_bytes",
    "paged_decode_split",
    "paged_decode_reduce",
    "paged_prefill_attn",
    "prefill_workspace_bytes",
    "paged_gather",
    "rope_kv_store",
    "cascade_decode_attn",
    "paged_decode_store_attn",
    "cascade_workspace_bytes",
    "check_decode_inputs",
    "check_prefill_inputs",
    "check_slots",
    "check_cascade_inputs",
    "decode_split_tokens",
    "decode_workspace_bytes",
    "lib",
    "library_path",
    "PkvError",
    "OutOfBlocks",
    "BlockManager",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1
# split_tokens value for token-balanced decode pieces (PKV_SPLIT_BALANCED)
SPLIT_BALANCED = -1

_lib = None

# Run the device-side precondition checks before every call (debugging aid).
DEBUG_CHECKS = os.environ.get("PKV_DEBUG_CHECKS", "") not in ("", "0")
CHECK_NAMES = ("length", "block_id", "cu_seqlens", "slot", "duplicate_slot", "shared_prefix", "group")
_NUM_FLAGS = 8


class PkvError(RuntimeError):
    """A non-OK status from libpkv.so (message from pkv_last_error)."""


class OutOfBlocks(PkvError):
    """The block manager has too few free blocks (nothing was changed)."""


def lib() -> ctypes.CDLL:
    """The loaded libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise PkvError(f"{library_path} is missing: build it with `python -m paged_kv_gqa_mapping_amd.build`")
    L = ctypes.CDLL(library_path)
    P, I32, I64, F, V = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p
    L.pkv_version.restype = ctypes.c_int
    L.pkv_status_string.restype = ctypes.c_char_p
    L.pkv_status_string.argtypes = [ctypes.c_int]
    L.pkv_last_error.restype = ctypes.c_char_p
    L.pkv_kv_store.argtypes = [P, P, P, P, P, I64, I32, I32, I64, I32, I32, V]
    L.pkv_kv_store.restype = ctypes.c_int
    L.pkv_rope_kv_store.argtypes = [P, P, P, P, P, P, P, I64, I32, I32, I32, I64, I32, ctypes.c_double, I32, I32, V]
    L.pkv_rope_kv_store.restype = ctypes.c_int
    L.pkv_paged_decode_store_attn.argtypes = [P, P, P, P, P, P, I32, P, I32, F, P, I32, I32, I32, I32, I64, I32, I32,
                                              I32, P, I64, V]
    L.pkv_paged_decode_store_attn.restype = ctypes.c_int
    L.pkv_cascade_decode_attn.argtypes = [P, P, P, P, I32, P, I32, P, P, P, I32, I32, I32, I32, F, P, I32, I32, I32,
                                          I32, I64, I32, I32, I32, P, I64, V]
    L.pkv_cascade_decode_attn.restype = ctypes.c_int
    L.pkv_cascade_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, I32, I32]
    L.pkv_cascade_workspace_bytes.restype = I64
    L.pkv_check_decode_inputs.argtypes = [P, I32, P, I32, I32, I64, I32, P, V]
    L.pkv_check_prefill_inputs.argtypes = [P, P, P, I32, I32, I32, I32, I64, I32, P, V]
    L.pkv_check_slots.argtypes = [P, I64, I64, I32, P, P, V]
    L.pkv_check_cascade_inputs.argtypes = [P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, V]
    for name in ("pkv_check_decode_inputs", "pkv_check_prefill_inputs", "pkv_check_slots",
                 "pkv_check_cascade_inputs"):
        getattr(L, name).restype = ctypes.c_int
    L.pkv_decode_split_tokens.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    L.pkv_decode_split_tokens.restype = I32
    L.pkv_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    L.pkv_decode_workspace_bytes.restype = I64
    dec = [P, P, P, P, I32, P, I32, F, P, I32, I32, I32, I32, I64, I32, I32, I32, P, I64, V]
    for name in ("pkv_paged_decode_attn", "pkv_paged_decode_split", "pkv_paged_decode_reduce"):
        getattr(L, name).argtypes = dec
        getattr(L, name).restype = ctypes.c_int
    L.pkv_paged_decode_attn_noalloc.argtypes = dec[:-3] + [V]
    L.pkv_paged_decode_attn_noalloc.restype = ctypes.c_int
    L.pkv_noalloc_scratch_bytes.argtypes = []
    L.pkv_noalloc_scratch_bytes.restype = I64
    L.pkv_paged_prefill_attn.argtypes = [P, P, P, P, P, P, I32, P, F, I32, I64, I32, I32, I32, I32, I32, I64, I32,
                                         I32, P, I64, V]
    L.pkv_paged_prefill_attn.restype = ctypes.c_int
    L.pkv_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32]
    L.pkv_prefill_workspace_bytes.restype = I64
    L.pkv_paged_gather.argtypes = [P, P, P, I32, P, I32, I32, P, P, I32, I32, I64, I32, I32, V]
    L.pkv_paged_gather.restype = ctypes.c_int
    L.pkv_bm_create.argtypes = [I64, I32, I32]
    L.pkv_bm_create.restype = P
    L.pkv_bm_destroy.argtypes = [P]
    L.pkv_bm_destroy.restype = None
    L.pkv_bm_last_error.restype = ctypes.c_char_p
    L.pkv_bm_num_free_blocks.argtypes = [P]
    L.pkv_bm_num_free_blocks.restype = I64
    L.pkv_bm_block_refcount.argtypes = [P, I32]
    L.pkv_bm_block_refcount.restype = I32
    L.pkv_bm_can_allocate.argtypes = [P, P, I64]
    L.pkv_bm_can_allocate.restype = ctypes.c_int
    L.pkv_bm_allocate.argtypes = [P, I64, P, I64, ctypes.POINTER(I64)]
    L.pkv_bm_allocate.restype = ctypes.c_int
    L.pkv_bm_append.argtypes = [P, I64, I32, ctypes.POINTER(I32)]
    L.pkv_bm_append.restype = ctypes.c_int
    L.pkv_bm_free.argtypes = [P, I64]
    L.pkv_bm_free.restype = ctypes.c_int
    L.pkv_bm_preempt.argtypes = [P, ctypes.POINTER(I64), ctypes.POINTER(I64)]
    L.pkv_bm_preempt.restype = ctypes.c_int
    L.pkv_bm_seq_len.argtypes = [P, I64]
    L.pkv_bm_seq_len.restype = I64
    L.pkv_bm_block_table.argtypes = [P, I64, P, I32, I32]
    L.pkv_bm_block_table.restype = I32
    L.pkv_bm_slot_mapping.argtypes = [P, I64, I64, I64, P]
    L.pkv_bm_slot_mapping.restype = ctypes.c_int
    _lib = L
    return L


def _check(status: int) -> None:
    if status != 0:
        L = lib()
        raise PkvError(f"{L.pkv_status_string(status).decode()}: {L.pkv_last_error().decode()}")


def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _dev(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    return t


def _stream() -> int:
    return _torch().cuda.current_stream().cuda_stream


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def kv_store(k, v, k_cache, v_cache, slot_mapping) -> None:
    """Write token i's K/V rows ([N, Hkv, D]) to cache slot slot_mapping[i] (negative: skip)."""
    torch = _torch()
    _dev(k, "k", ndim=3)
    _dev(v, "v", k.dtype, 3)
    _dev(k_cache, "k_cache", k.dtype, 4)
    _dev(v_cache, "v_cache", k.dtype, 4)
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    N, Hkv, D = k.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if v.shape != k.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D) or slot_mapping.shape[0] != N:
        raise ValueError("shape mismatch among k, v, k_cache, v_cache, slot_mapping")
    if DEBUG_CHECKS:
        _require(check_slots(slot_mapping, NB, bs), "kv_store")
    _check(lib().pkv_kv_store(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping), N, Hkv, D, NB, bs,
                              _dtype_code(k), _stream()))


def rope_kv_store(q, k, v, positions, k_cache, v_cache, slot_mapping, rope_theta, interleaved=False) -> None:
    """Rotary embedding of q (in place, [N, Hq, D]) and k, then the cache write of the
    rotated k and of v at slot_mapping[i] (negative: no cache write)."""
    torch = _torch()
    _dev(q, "q", ndim=3)
    _dev(k, "k", q.dtype, 3)
    _dev(v, "v", q.dtype, 3)
    _dev(positions, "positions", torch.int32, 1)
    _dev(k_cache, "k_cache", q.dtype, 4)
    _dev(v_cache, "v_cache", q.dtype, 4)
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    N, Hq, D = q.shape
    _, Hkv, _ = k.shape
    NB, bs, Hkv2, D2 = k_cache.shape
    if (k.shape != (N, Hkv, D) or v.shape != k.shape or v_cache.shape != k_cache.shape or (Hkv2, D2) != (Hkv, D)
            or positions.shape[0] != N or slot_mapping.shape[0] != N):
        raise ValueError("shape mismatch among q, k, v, positions, k_cache, v_cache, slot_mapping")
    if DEBUG_CHECKS:
        _require(check_slots(slot_mapping, NB, bs), "rope_kv_store")
    _check(lib().pkv_rope_kv_store(_ptr(q), _ptr(k), _ptr(v), _ptr(positions), _ptr(k_cache), _ptr(v_cache),
                                   _ptr(slot_mapping), N, Hq, Hkv, D, NB, bs, float(rope_theta), int(bool(interleaved)),
                                   _dtype_code(q), _stream()))


def decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, block_size, dtype_code):
    return int(lib().pkv_decode_split_tokens(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                             block_size, dtype_code))


def decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, split_tokens) -> int:
    return int(lib().pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, split_tokens))


def _decode(fn_name, q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len, split_tokens,
            workspace, new_kv=None):
    torch = _torch()
    _dev(q, "q", ndim=3)
    _dev(k_cache, "k_cache", q.dtype, 4)
    _dev(v_cache, "v_cache", q.dtype, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(context_lens, "context_lens", torch.int32, 1)
    _dev(out, "out", q.dtype, 3)
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or D2 != D or out.shape != q.shape:
        raise ValueError("shape mismatch among q, k_cache, v_cache, out")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    code = _dtype_code(q)
    split = int(split_tokens) or decode_split_tokens(B, Hq, Hkv, D, max_context_len, bs, code)
    need = decode_workspace_bytes(B, Hq, D, max_context_len, split)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if DEBUG_CHECKS:
        _require(check_decode_inputs(block_tables, context_lens, max_context_len, NB, bs), fn_name)
    head = (_ptr(q),) if new_kv is None else (_ptr(q), _ptr(new_kv[0]), _ptr(new_kv[1]))
    _check(getattr(lib(), fn_name)(
        *head, _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(scale), _ptr(out), B, Hq, Hkv, D, NB, bs, code, split, _ptr(workspace), ws_bytes,
        _stream()))
    return out


def paged_decode_attn(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                      split_tokens=0, workspace=None):
    """Decode attention: q [B, Hq, D] over each sequence's context_lens[b] cached tokens -> out [B, Hq, D]."""
    return _decode("pkv_paged_decode_attn", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                   max_context_len, split_tokens, workspace)


def paged_decode_attn_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                              split_tokens=0):
    """paged_decode_attn with the split states in the library's per-GPU scratch
    (no workspace, nothing allocated); calls overlapping on one GPU race."""
    _dev(q, "q", ndim=3)
    _dev(k_cache, "k_cache", q.dtype, 4)
    _dev(v_cache, "v_cache", q.dtype, 4)
    _dev(block_tables, "block_tables", _torch().int32, 2)
    _dev(context_lens, "context_lens", _torch().int32, 1)
    _dev(out, "out", q.dtype, 3)
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if v_cache.shape != k_cache.shape or D2 != D or out.shape != q.shape:
        raise ValueError("shape mismatch among q, k_cache, v_cache, out")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables and context_lens need one row per sequence")
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    _check(lib().pkv_paged_decode_attn_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        int(max_context_len), float(scale), _ptr(out), B, Hq, Hkv, D, NB, bs, _dtype_code(q), int(split_tokens),
        _stream()))
    return out


def noalloc_scratch_bytes() -> int:
    return int(lib().pkv_noalloc_scratch_bytes())


def paged_decode_split(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                       split_tokens=0, workspace=None):
    """First pass of paged_decode_attn (per-split softmax states)."""
    return _decode("pkv_paged_decode_split", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                   max_context_len, split_tokens, workspace)


def paged_decode_reduce(q, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                        split_tokens=0, workspace=None):
    """Second pass of paged_decode_attn (merge of the split states); same arguments and workspace as the first."""
    return _decode("pkv_paged_decode_reduce", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                   max_context_len, split_tokens, workspace)


def paged_decode_store_attn(q, k, v, k_cache, v_cache, block_tables, context_lens, scale, out, max_context_len=None,
                            split_tokens=0, workspace=None):
    """kv_store of each sequence's newest token (k, v [B, Hkv, D], at position
    context_lens[b] - 1) fused into paged_decode_attn: one launch fewer, same bits."""
    torch = _torch()
    _dev(k, "k", q.dtype, 3)
    _dev(v, "v", q.dtype, 3)
    if k.shape != (q.shape[0], k_cache.shape[2], q.shape[2]) or v.shape != k.shape:
        raise ValueError("k and v must be [num_seqs, num_kv_heads, head_dim]")
    return _decode("pkv_paged_decode_store_attn", q, k_cache, v_cache, block_tables, context_lens, scale, out,
                   max_context_len, split_tokens, workspace, new_kv=(k, v))


def cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, max_own_len,
                            split_tokens, num_groups, max_group_size, max_shared_len) -> int:
    return int(lib().pkv_cascade_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                                 max_own_len, split_tokens, num_groups, max_group_size,
                                                 max_shared_len))


def cascade_decode_attn(q, k_cache, v_cache, block_tables, context_lens, shared_lens, group_offsets, group_seqs,
                        scale, out, max_context_len=None, max_group_size=None, max_shared_len=None, max_own_len=None,
                        split_tokens=0, workspace=None):
    """Shared-prefix decode: as paged_decode_attn, with groups of sequences whose first
    shared_lens[b] keys are the same blocks attended once per group.  Sizes left as None
    are read back from the device tensors (a synchronisation)."""
    torch = _torch()
    _dev(q, "q", ndim=3)
    _dev(k_cache, "k_cache", q.dtype, 4)
    _dev(v_cache, "v_cache", q.dtype, 4)
    for t, n in ((block_tables, "block_tables"), (context_lens, "context_lens"), (shared_lens, "shared_lens"),
                 (group_offsets, "group_offsets"), (group_seqs, "group_seqs")):
        _dev(t, n, torch.int32)
    _dev(out, "out", q.dtype, 3)
    B, Hq, D = q.shape
    NB, bs, Hkv, D2 = k_cache.shape
    if out.shape != q.shape or D2 != D or v_cache.shape != k_cache.shape or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("shape mismatch among q, k_cache, v_cache, block_tables")
    if context_lens.shape[0] != B or shared_lens.shape[0] != B:
        raise ValueError("context_lens and shared_lens need one entry per sequence")
    num_groups = group_offsets.shape[0] - 1
    if max_context_len is None:
        max_context_len = int(context_lens.max().item()) if B else 0
    if max_shared_len is None:
        max_shared_len = int(shared_lens.max().item()) if B else 0
    if max_group_size is None:
        max_group_size = int((group_offsets[1:] - group_offsets[:-1]).max().item()) if num_groups > 0 else 0
    if max_own_len is None:
        max_own_len = int((context_lens - shared_lens).max().item()) if B else 0
    split = int(split_tokens)
    need = cascade_workspace_bytes(B, Hq, Hkv, D, max_context_len, max_own_len, split, num_groups, max_group_size,
                                   max_shared_len)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if DEBUG_CHECKS:
        _require(check_decode_inputs(block_tables, context_lens, max_context_len, NB, bs), "cascade_decode_attn")
        if num_groups > 0:
            _require(check_cascade_inputs(block_tables, context_lens, shared_lens, group_offsets, group_seqs,
                                          max_group_size, max_shared_len, bs), "cascade_decode_attn")
    _check(lib().pkv_cascade_decode_attn(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        max_context_len, _ptr(shared_lens), _ptr(group_offsets), _ptr(group_seqs), num_groups, max_group_size,
        max_shared_len, max_own_len, float(scale), _ptr(out), B, Hq, Hkv, D, NB, bs, _dtype_code(q), split,
        _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream()))


def prefill_workspace_bytes(num_seqs, max_seqlen_q, num_q_heads, num_kv_heads, head_dim, dtype_code) -> int:
    return int(lib().pkv_prefill_workspace_bytes(num_seqs, max_seqlen_q, num_q_heads, num_kv_heads, head_dim,
                                                 dtype_code))


def paged_prefill_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, block_tables, out, max_seqlen_q=None,
                       max_seqlen_k=None, scale=None, workspace=None, planned=None):
    """Causal varlen prefill: q [sum Lq, Hq, D]; k, v the caches (block_tables given) or packed [sum Lk, Hkv, D].

    bf16: ``planned=True`` runs over device-planned work lists in ``workspace`` (allocated
    here when None): long query tiles cut into key pieces, one workgroup per planned item;
    otherwise the one-launch kernel.  The default (None) plans exactly when a workspace is
    passed."""
    torch = _torch()
    _dev(q, "q", ndim=3)
    _dev(out, "out", q.dtype, 3)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    Tq, Hq, D = q.shape
    B = cu_seqlens_q.shape[0] - 1
    if cu_seqlens_k.shape[0] != B + 1 or out.shape != q.shape:
        raise ValueError("cu_seqlens_q / cu_seqlens_k / out shape mismatch")
    if block_tables is not None:
        _dev(k, "k", q.dtype, 4)
        _dev(v, "v", q.dtype, 4)
        _dev(block_tables, "block_tables", torch.int32, 2)
        NB, bs, Hkv, D2 = k.shape
        W = block_tables.shape[1]
        if block_tables.shape[0] != B:
            raise ValueError("block_tables needs one row per sequence")
    else:
        _dev(k, "k", q.dtype, 3)
        _dev(v, "v", q.dtype, 3)
        NB, Hkv, D2 = k.shape
        bs, W = 0, 0
    if v.shape != k.shape or D2 != D:
        raise ValueError("shape mismatch among q, k, v")
    if max_seqlen_q is None or max_seqlen_k is None:
        cq = cu_seqlens_q.cpu()
        ck = cu_seqlens_k.cpu()
        max_seqlen_q = int((cq[1:] - cq[:-1]).max()) if B else 0
        max_seqlen_k = int((ck[1:] - ck[:-1]).max()) if B else 0
    sc = 0.0 if scale is None else float(scale)
    code = _dtype_code(q)
    if planned is None:
        planned = workspace is not None
    if not planned:
        workspace = None
    elif workspace is None:
        need = prefill_workspace_bytes(B, int(max_seqlen_q), Hq, Hkv, D, code)
        if need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if DEBUG_CHECKS:
        _require(check_prefill_inputs(cu_seqlens_q, cu_seqlens_k, block_tables, max_seqlen_q, max_seqlen_k, NB,
                                      bs if block_tables is not None else 1), "paged_prefill_attn")
    _check(lib().pkv_paged_prefill_attn(
        _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(block_tables), W, _ptr(out), sc, B,
        Tq, int(max_seqlen_q), int(max_seqlen_k), Hq, Hkv, D, NB, bs, code, _ptr(workspace), ws_bytes, _stream()))
    return out


# ---------------------------------------------------------------- precondition checks


def _flags(device):
    return _torch().zeros(_NUM_FLAGS, dtype=_torch().int32, device=device)


def _counts(flags) -> dict:
    vals = flags.cpu().tolist()  # synchronizes
    return {n: int(vals[i]) for i, n in enumerate(CHECK_NAMES)}


def _require(counts: dict, what: str) -> None:
    bad = {k: v for k, v in counts.items() if v}
    if bad:
        raise PkvError(f"{what}: device-side precondition violated: {bad}")


def check_decode_inputs(block_tables, context_lens, max_context_len, num_blocks, block_size) -> dict:
    """Violations (per kind) of decode's preconditions: context lengths within
    [0, max_context_len] and the block ids they use inside [0, num_blocks)."""
    torch = _torch()
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(context_lens, "context_lens", torch.int32, 1)
    f = _flags(block_tables.device)
    _check(lib().pkv_check_decode_inputs(_ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                         int(max_context_len), context_lens.shape[0], int(num_blocks), int(block_size),
                                         _ptr(f), _stream()))
    return _counts(f)


def check_prefill_inputs(cu_seqlens_q, cu_seqlens_k, block_tables, max_seqlen_q, max_seqlen_k, num_blocks,
                         block_size) -> dict:
    """Violations of prefill's preconditions (cu_seqlens from 0, ordered, Lq <= Lk, within
    the maxima; with block tables, the block ids holding each sequence's keys)."""
    torch = _torch()
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32, 1)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    W = 0
    if block_tables is not None:
        _dev(block_tables, "block_tables", torch.int32, 2)
        W = block_tables.shape[1]
    f = _flags(cu_seqlens_q.device)
    _check(lib().pkv_check_prefill_inputs(_ptr(cu_seqlens_q), _ptr(cu_seqlens_k), _ptr(block_tables), W,
                                          cu_seqlens_q.shape[0] - 1, int(max_seqlen_q), int(max_seqlen_k),
                                          int(num_blocks), int(block_size), _ptr(f), _stream()))
    return _counts(f)


def check_slots(slot_mapping, num_blocks, block_size, duplicates=True) -> dict:
    """Violations of kv_store's preconditions: slots inside the pool and (when
    ``duplicates``) no slot named twice."""
    torch = _torch()
    _dev(slot_mapping, "slot_mapping", torch.int32, 1)
    f = _flags(slot_mapping.device)
    bitmap = None
    if duplicates:
        bitmap = torch.empty((int(num_blocks) * int(block_size) + 31) // 32, dtype=torch.int32,
                             device=slot_mapping.device)
    _check(lib().pkv_check_slots(_ptr(slot_mapping), slot_mapping.shape[0], int(num_blocks), int(block_size),
                                 _ptr(bitmap), _ptr(f), _stream()))
    return _counts(f)


def check_cascade_inputs(block_tables, context_lens, shared_lens, group_offsets, group_seqs, max_group_size,
                         max_shared_len, block_size) -> dict:
    """Violations of the shared-prefix groups' preconditions (see pkv.h)."""
    torch = _torch()
    for t, n in ((context_lens, "context_lens"), (shared_lens, "shared_lens"), (group_offsets, "group_offsets"),
                 (group_seqs, "group_seqs")):
        _dev(t, n, torch.int32, 1)
    _dev(block_tables, "block_tables", torch.int32, 2)
    B = context_lens.shape[0]
    f = _flags(block_tables.device)
    seen = torch.empty(max(B, 1), dtype=torch.int32, device=block_tables.device)
    _check(lib().pkv_check_cascade_inputs(_ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
                                          _ptr(shared_lens), _ptr(group_offsets), _ptr(group_seqs),
                                          group_offsets.shape[0] - 1, group_seqs.shape[0], B, int(max_group_size),
                                          int(max_shared_len), int(block_size), _ptr(seen), _ptr(f), _stream()))
    return _counts(f)


def paged_gather(k_cache, v_cache, block_tables, cu_seqlens_k, max_seqlen_k=None, k_out=None, v_out=None):
    """Copy each sequence's logical K/V rows, read through its block table, to packed [sum Lk, Hkv, D] buffers."""
    torch = _torch()
    _dev(k_cache, "k_cache", ndim=4)
    _dev(v_cache, "v_cache", k_cache.dtype, 4)
    _dev(block_tables, "block_tables", torch.int32, 2)
    _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32, 1)
    NB, bs, Hkv, D = k_cache.shape
    B = cu_seqlens_k.shape[0] - 1
    ck = cu_seqlens_k.cpu()
    total = int(ck[-1]) if B >= 0 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int((ck[1:] - ck[:-1]).max()) if B else 0
    if k_out is None:
        k_out = torch.empty((total, Hkv, D), dtype=k_cache.dtype, device=k_cache.device)
    if v_out is None:
        v_out = torch.empty((total, Hkv, D), dtype=k_cache.dtype, device=k_cache.device)
    _dev(k_out, "k_out", k_cache.dtype, 3)
    _dev(v_out, "v_out", k_cache.dtype, 3)
    _check(lib().pkv_paged_gather(
        _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), block_tables.shape[1], _ptr(cu_seqlens_k), B,
        int(max_seqlen_k), _ptr(k_out), _ptr(v_out), Hkv, D, NB, bs, _dtype_code(k_cache), _stream()))
    return k_out, v_out


class BlockManager:
    """Host-side block manager of libpkv.so (allocation, reference counts, prefix reuse).

    ``tokens`` arguments are sequences of int token ids.  Methods raise
    :class:`OutOfBlocks` when the pool is short (the manager is unchanged) and
    :class:`PkvError` on bad arguments.
    """

    def __init__(self, num_blocks: int, block_size: int, prefix_cache: bool = True):
        L = lib()
        self._h = L.pkv_bm_create(int(num_blocks), int(block_size), 1 if prefix_cache else 0)
        if not self._h:
            raise PkvError(L.pkv_bm_last_error().decode())
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def __del__(self):
        h, self._h = getattr(self, "_h", None), None
        if h and _lib is not None:
            _lib.pkv_bm_destroy(h)

    def _check(self, st):
        if st < 0:
            msg = lib().pkv_bm_last_error().decode()
            raise (OutOfBlocks if st == -5 else PkvError)(msg)
        return st

    @staticmethod
    def _arr(tokens):
        import numpy as np

        a = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        return a, (a.ctypes.data_as(ctypes.c_void_p) if a.size else None)

    @property
    def num_free_blocks(self) -> int:
        return int(lib().pkv_bm_num_free_blocks(self._h))

    def refcount(self, block: int) -> int:
        return self._check(lib().pkv_bm_block_refcount(self._h, int(block)))

    def can_allocate(self, tokens) -> bool:
        a, p = self._arr(tokens)
        return bool(self._check(lib().pkv_bm_can_allocate(self._h, p, a.size)))

    def allocate(self, seq_id: int, tokens) -> int:
        """Blocks for a new sequence's prompt; returns how many leading tokens were cached."""
        a, p = self._arr(tokens)
        cached = ctypes.c_int64(0)
        self._check(lib().pkv_bm_allocate(self._h, int(seq_id), p, a.size, ctypes.byref(cached)))
        return int(cached.value)

    def append(self, seq_id: int, token: int) -> int:
        """Append one token; returns its slot."""
        slot = ctypes.c_int32(0)
        self._check(lib().pkv_bm_append(self._h, int(seq_id), int(token), ctypes.byref(slot)))
        return int(slot.value)

    def free(self, seq_id: int) -> None:
        self._check(lib().pkv_bm_free(self._h, int(seq_id)))

    def preempt(self):
        """Free the most recently allocated sequence; returns (seq_id, cached_tokens), the
        second being how many of its leading tokens the prefix cache still holds."""
        sid, cached = ctypes.c_int64(0), ctypes.c_int64(0)
        self._check(lib().pkv_bm_preempt(self._h, ctypes.byref(sid), ctypes.byref(cached)))
        return int(sid.value), int(cached.value)

    def seq_len(self, seq_id: int) -> int:
        return int(self._check(lib().pkv_bm_seq_len(self._h, int(seq_id))))

    def block_table(self, seq_id: int, width: int | None = None, pad: int = 0):
        import numpy as np

        n = -(-self.seq_len(seq_id) // self.block_size)
        width = n if width is None else int(width)
        out = np.empty(max(width, 0), dtype=np.int32)
        p = out.ctypes.data_as(ctypes.c_void_p) if out.size else None
        self._check(lib().pkv_bm_block_table(self._h, int(seq_id), p, width, int(pad)))
        return out

    def slot_mapping(self, seq_id: int, first_pos: int, count: int):
        import numpy as np

        out = np.empty(int(count), dtype=np.int32)
        p = out.ctypes.data_as(ctypes.c_void_p) if out.size else None
        self._check(lib().pkv_bm_slot_mapping(self._h, int(seq_id), int(first_pos), int(count), p))
        return out
