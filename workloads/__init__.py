"""Seeded synthetic inputs for the paged-KV attention path.

This module only *builds inputs*: sequence lengths, a reference-counted pool of
physical KV blocks, per-sequence block tables, slot mappings for the tokens a
step appends, cu_seqlens, and N(0,1) values for queries, new keys/values and
the tokens already resident in the cache.  It holds none of the attention
arithmetic, so the fp64 oracle (``oracle/``) and the HIP path both consume the
same arrays without sharing any of the computation.

Conventions (the pages fix none of them; each is stated where the inputs are
built):

* KV cache tensors are ``[num_blocks, block_size, num_kv_heads, head_dim]``,
  row-major, head_dim contiguous.  bf16 values are stored as ``uint16`` bit
  patterns, fp32 values as ``float32``.
* A token at absolute position ``p`` of a sequence lives in physical block
  ``table[p // block_size]`` at row ``p % block_size``; its *slot* is
  ``block * block_size + row`` ("PagedAttention" diagram of the nano-vllm
  README; the model runner builds slot mappings and block tables per step,
  "Nano-vLLM Architecture and Performance", section "How It Works End-to-End").
* Physical ids are a seeded permutation of the pool, dealt to sequences in
  order; table entries past a sequence's last block point at a poison block.
* Slots that hold no valid token (free blocks, the poison block, the tail of a
  sequence's last block, and the slots the step is about to write) are NaN, so
  a kernel that reads past a sequence shows it in its output.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

BF16 = "bf16"
F32 = "f32"

# Independent random streams (SeedSequence spawn keys) for each kind of value.
_STREAM_K_CACHE = 1
_STREAM_V_CACHE = 2
_STREAM_NEW_K = 3
_STREAM_NEW_V = 4
_STREAM_Q = 5

_CHUNK = 1 << 22  # elements per independently seeded chunk (thread-count independent)


def storage_dtype(dtype: str):
    if dtype == BF16:
        return np.uint16
    if dtype == F32:
        return np.float32
    raise ValueError(f"unknown dtype {dtype!r}")


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); returns uint16 bits.

    Input preparation only: inputs are drawn in float32 and stored in bf16.
    NaN stays NaN (quiet bit set).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = np.uint16(0x7FC0)
    return rounded


def nan_value(dtype: str):
    return np.uint16(0x7FC0) if dtype == BF16 else np.float32(np.nan)


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def fill_normal(shape, dtype: str, seed: int, stream: int) -> np.ndarray:
    """i.i.d. N(0,1) drawn in float32 (PCG64), stored in ``dtype``.

    The flat array is cut into fixed chunks, each with its own SeedSequence
    spawn key ``(stream, chunk)``, so the values do not depend on how many
    threads fill them.
    """
    n = int(np.prod(shape, dtype=np.int64))
    out = np.empty(n, dtype=storage_dtype(dtype))
    nchunks = (n + _CHUNK - 1) // _CHUNK

    def work(c):
        lo = c * _CHUNK
        hi = min(n, lo + _CHUNK)
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream, c))))
        if dtype == F32:
            g.standard_normal(out=out[lo:hi], dtype=np.float32)
        else:
            out[lo:hi] = f32_to_bf16_bits(g.standard_normal(hi - lo, dtype=np.float32))

    if nchunks <= 1:
        for c in range(nchunks):
            work(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(work, range(nchunks)))
    return out.reshape(shape)


class PoolExhausted(RuntimeError):
    pass


class BlockPool:
    """Reference-counted pool of physical KV blocks (host bookkeeping only).

    Blocks are handed out in the order of ``order`` (a seeded permutation), a
    shared block has its count raised once per extra owner, and a block goes
    back to the free list when its count reaches zero (blocks of a cached
    prefix are reused under reference counts: "Nano-vLLM Architecture and
    Performance", section "Paged KV Cache").
    """

    def __init__(self, order):
        order = [int(x) for x in order]
        self.num_blocks = len(order)
        if sorted(order) != list(range(self.num_blocks)):
            raise ValueError("order must be a permutation of range(num_blocks)")
        self.free = list(order)
        self.refcount = np.zeros(self.num_blocks, dtype=np.int32)

    def alloc(self, n: int) -> list:
        if n > len(self.free):
            raise PoolExhausted(f"need {n} blocks, {len(self.free)} free")
        ids, self.free = self.free[:n], self.free[n:]
        for b in ids:
            self.refcount[b] = 1
        return ids

    def share(self, ids) -> None:
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.refcount[b] += 1

    def release(self, ids) -> None:
        for b in ids:
            if self.refcount[b] <= 0:
                raise ValueError(f"block {b} is not allocated")
            self.refcount[b] -= 1
            if self.refcount[b] == 0:
                self.free.append(int(b))


@dataclass
class SeqSpec:
    """One sequence of a step: ``total`` tokens after the step, ``new`` of them appended now.

    ``kind`` is "decode" (one new token, one query) or "prefill" (``new``
    queries at positions ``total - new .. total - 1``).  ``shared`` is the
    number of leading full blocks it takes from the shared prefix.
    """

    kind: str
    total: int
    new: int
    shared: int = 0


@dataclass
class Workload:
    name: str
    seed: int
    dtype: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    poison_block: int
    refcount: np.ndarray
    shared_blocks: list
    k_cache: np.ndarray  # cache contents *before* the step's kv_store
    v_cache: np.ndarray
    # tokens the step appends (prefill tokens first, then decode tokens)
    new_k: np.ndarray
    new_v: np.ndarray
    slot_mapping: np.ndarray
    # position in its sequence of each appended token (same order as slot_mapping)
    store_positions: np.ndarray | None = None
    # decode part
    dec_q: np.ndarray | None = None
    dec_block_tables: np.ndarray | None = None
    dec_context_lens: np.ndarray | None = None
    # prefill part
    pre_q: np.ndarray | None = None
    pre_block_tables: np.ndarray | None = None
    cu_seqlens_q: np.ndarray | None = None
    cu_seqlens_k: np.ndarray | None = None
    seqs: list = field(default_factory=list)
    notes: dict = field(default_factory=dict)

    @property
    def group_size(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elt_bytes(self) -> int:
        return 2 if self.dtype == BF16 else 4

    @property
    def max_context_len(self) -> int:
        return int(self.dec_context_lens.max()) if self.dec_context_lens is not None and len(self.dec_context_lens) else 0

    @property
    def max_seqlen_q(self) -> int:
        if self.cu_seqlens_q is None or len(self.cu_seqlens_q) < 2:
            return 0
        return int(np.diff(self.cu_seqlens_q).max())

    @property
    def max_seqlen_k(self) -> int:
        if self.cu_seqlens_k is None or len(self.cu_seqlens_k) < 2:
            return 0
        return int(np.diff(self.cu_seqlens_k).max())

    # Algorithmic work (units stated in the measurement notes).
    def decode_kv_bytes(self) -> int:
        """K and V rows read once per (sequence, KV head), logical (shared blocks counted per sequence)."""
        if self.dec_context_lens is None:
            return 0
        return int(self.dec_context_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * self.elt_bytes

    def decode_kv_bytes_unique(self) -> int:
        """As decode_kv_bytes, with each decode sequence's shared prefix blocks counted once
        per distinct shared length (what shared-prefix decode reads)."""
        if self.dec_context_lens is None:
            return 0
        dec = [s for s in self.seqs if s.kind == "decode"]
        tokens = int(self.dec_context_lens.astype(np.int64).sum())
        shared = [s.shared * self.block_size for s in dec]
        tokens -= sum(shared)
        tokens += sum(set(x for x in shared if x > 0))
        return tokens * 2 * self.num_kv_heads * self.head_dim * self.elt_bytes

    def cascade_groups(self, group_cap: int | None = None):
        """Shared-prefix groups of the decode sequences (those taking the same number
        of leading shared blocks form a group, cut into groups of at most group_cap):
        (shared_lens [B] int32 in tokens, group_offsets int32, group_seqs int32,
        max_group_size, max_shared_len, max_own_len), the last being the longest
        context_len - shared_len."""
        dec = [s for s in self.seqs if s.kind == "decode"]
        shared = np.array([s.shared * self.block_size for s in dec], dtype=np.int32)
        groups = []
        for n in sorted(set(int(x) for x in shared if x > 0)):
            members = [j for j in range(len(dec)) if shared[j] == n]
            cap = group_cap or len(members)
            groups += [members[i:i + cap] for i in range(0, len(members), cap)]
        offsets = np.concatenate([[0], np.cumsum([len(g) for g in groups])]).astype(np.int32)
        seqs = np.array([j for g in groups for j in g], dtype=np.int32)
        own = int((self.dec_context_lens - shared).max(initial=0))
        return shared, offsets, seqs, max([len(g) for g in groups] + [0]), int(shared.max(initial=0)), own

    def decode_io_bytes(self) -> int:
        """q read + out written by the decode step."""
        if self.dec_q is None:
            return 0
        return 2 * self.dec_q.size * self.elt_bytes

    def prefill_flops(self) -> int:
        """4 * Hq * D per unmasked (query, key) pair (QK^T and PV, 2 flops per MAC)."""
        if self.cu_seqlens_q is None:
            return 0
        pairs = 0
        lq = np.diff(self.cu_seqlens_q).astype(np.int64)
        lk = np.diff(self.cu_seqlens_k).astype(np.int64)
        for a, b in zip(lq, lk):
            # query i sees (b - a + i + 1) keys, i = 0..a-1
            pairs += a * (b - a) + a * (a + 1) // 2
        return int(4 * self.num_q_heads * self.head_dim * pairs)

    def store_bytes(self) -> int:
        """kv_store moves N rows of K and V: read 2*N*Hkv*D*elt (+4N slot ids), write 2*N*Hkv*D*elt."""
        n = len(self.slot_mapping)
        row = self.num_kv_heads * self.head_dim * self.elt_bytes
        return 2 * (2 * n * row) + 4 * n


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def build(
    name: str,
    seed: int,
    dtype: str,
    num_q_heads: int,
    num_kv_heads: int,
    head_dim: int,
    block_size: int,
    seqs: list,
    *,
    shared_prefix_blocks: int = 0,
    num_blocks: int | None = None,
    table_width_decode: int | None = None,
    table_width_prefill: int | None = None,
    perm_rng: np.random.Generator | None = None,
    scale: float | None = None,
    poison: str = "nan",
) -> Workload:
    """Build one step's inputs.

    ``seqs`` lists prefill sequences first, then decode sequences (this is the
    order their new tokens appear in ``slot_mapping``).  Physical blocks are
    a permutation of ``num_blocks`` ids dealt in order: the shared prefix
    blocks first, then each sequence's private blocks, then the poison block.
    """
    if num_q_heads % num_kv_heads:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    if block_size & (block_size - 1):
        raise ValueError("block_size must be a power of two")
    rng = perm_rng if perm_rng is not None else np.random.default_rng(seed)
    bs = block_size
    for s in seqs:
        if s.kind not in ("decode", "prefill"):
            raise ValueError(s.kind)
        if s.kind == "decode" and s.new != 1:
            raise ValueError("a decode sequence appends exactly one token")
        if not (0 <= s.new <= s.total):
            raise ValueError("0 <= new <= total")
        if s.shared:
            if s.shared > shared_prefix_blocks:
                raise ValueError("sequence shares more blocks than the prefix has")
            # the step never writes into a shared block
            if s.total - s.new < s.shared * bs:
                raise ValueError("new tokens would land in a shared block")
    private = [_ceil_div(s.total, bs) - s.shared for s in seqs]
    need = shared_prefix_blocks + sum(private) + 1  # + poison
    nb = need if num_blocks is None else int(num_blocks)
    if nb < need:
        raise PoolExhausted(f"pool of {nb} blocks cannot hold {need}")

    order = rng.permutation(nb)
    pool = BlockPool(order)
    shared_ids = pool.alloc(shared_prefix_blocks) if shared_prefix_blocks else []
    seq_blocks = []
    for s, npriv in zip(seqs, private):
        ids = list(shared_ids[: s.shared])
        if s.shared:
            pool.share(shared_ids[: s.shared])
        ids += pool.alloc(npriv)
        seq_blocks.append(ids)
    if shared_ids:
        pool.release(shared_ids)  # the prefix's own (creator) reference
    poison_block = pool.alloc(1)[0]

    pre = [i for i, s in enumerate(seqs) if s.kind == "prefill"]
    dec = [i for i, s in enumerate(seqs) if s.kind == "decode"]

    def table(idx, width):
        width = max([len(seq_blocks[i]) for i in idx] + [1]) if width is None else width
        t = np.full((len(idx), width), poison_block, dtype=np.int32)
        for r, i in enumerate(idx):
            if len(seq_blocks[i]) > width:
                raise ValueError("table width too small")
            t[r, : len(seq_blocks[i])] = seq_blocks[i]
        return t

    # slot mapping of the appended tokens: prefill tokens first, then decode tokens
    slots, positions = [], []
    for i in pre + dec:
        s, ids = seqs[i], seq_blocks[i]
        for p in range(s.total - s.new, s.total):
            slots.append(ids[p // bs] * bs + p % bs)
            positions.append(p)
    slot_mapping = np.asarray(slots, dtype=np.int32)

    hkv, d = num_kv_heads, head_dim
    shape = (nb, bs, hkv, d)
    k_cache = fill_normal(shape, dtype, seed, _STREAM_K_CACHE)
    v_cache = fill_normal(shape, dtype, seed, _STREAM_V_CACHE)
    bad = nan_value(dtype) if poison == "nan" else storage_dtype(dtype)(0)
    # every slot not holding a resident token gets the poison value
    valid = np.zeros((nb, bs), dtype=bool)
    for s, ids in zip(seqs, seq_blocks):
        cached = s.total - s.new
        for j, b in enumerate(ids):
            lo, hi = j * bs, min(cached, (j + 1) * bs)
            if hi > lo:
                valid[b, : hi - lo] = True
    for b in range(nb):
        if valid[b].all():
            continue
        if not valid[b].any():
            k_cache[b] = bad
            v_cache[b] = bad
        else:
            k_cache[b, ~valid[b]] = bad
            v_cache[b, ~valid[b]] = bad

    n_new = len(slot_mapping)
    new_k = fill_normal((n_new, hkv, d), dtype, seed, _STREAM_NEW_K)
    new_v = fill_normal((n_new, hkv, d), dtype, seed, _STREAM_NEW_V)
    n_q = sum(seqs[i].new for i in pre) + len(dec)
    q_all = fill_normal((n_q, num_q_heads, d), dtype, seed, _STREAM_Q)
    n_pre_q = sum(seqs[i].new for i in pre)

    w = Workload(
        name=name, seed=seed, dtype=dtype, num_q_heads=num_q_heads, num_kv_heads=hkv, head_dim=d,
        block_size=bs, num_blocks=nb,
        scale=(1.0 / math.sqrt(d)) if scale is None else float(scale),
        poison_block=int(poison_block), refcount=pool.refcount.copy(), shared_blocks=list(shared_ids),
        k_cache=k_cache, v_cache=v_cache, new_k=new_k, new_v=new_v, slot_mapping=slot_mapping,
        store_positions=np.asarray(positions, dtype=np.int32), seqs=list(seqs),
    )
    if pre:
        w.pre_q = q_all[:n_pre_q]
        w.pre_block_tables = table(pre, table_width_prefill)
        w.cu_seqlens_q = np.concatenate([[0], np.cumsum([seqs[i].new for i in pre])]).astype(np.int32)
        w.cu_seqlens_k = np.concatenate([[0], np.cumsum([seqs[i].total for i in pre])]).astype(np.int32)
    if dec:
        w.dec_q = q_all[n_pre_q:]
        w.dec_block_tables = table(dec, table_width_decode)
        w.dec_context_lens = np.asarray([seqs[i].total for i in dec], dtype=np.int32)
    w.notes["seq_blocks"] = seq_blocks
    return w


# ---------------------------------------------------------------------------
# The five workloads.  Each draws, in order: lengths, offsets and sharing, the
# block permutation, cache contents, new k/v, then q.
# ---------------------------------------------------------------------------

CONFIG_NAMES = {
    1: "tiny-decode-f32",
    2: "qwen3-0.6b-decode-bf16",
    3: "llama8b-long-decode-splitk-bf16",
    4: "prefix-cached-varlen-prefill-bf16",
    5: "mixed-continuous-batching-step-bf16",
    6: "shared-prompt-decode-bf16",
}


def make_config(i: int, seed: int | None = None, poison: str = "nan", dtype: str | None = None) -> Workload:
    """Workload i (1..6).  ``dtype`` overrides the element type (the same shapes
    in fp32 let a 1e-5 tolerance see a single misplaced key at long context)."""
    seed = i if seed is None else seed
    rng = np.random.default_rng(seed)
    name = CONFIG_NAMES[i] if dtype is None else f"{CONFIG_NAMES[i]}-as-{dtype}"
    if i == 1:
        # 4 decode sequences, 4/2 heads, D=64, bs=16, a pool of exactly 64 blocks
        lens = rng.integers(1, 100, size=4, endpoint=True)
        seqs = [SeqSpec("decode", int(L), 1) for L in lens]
        return build(name, seed, dtype or F32, 4, 2, 64, 16, seqs, num_blocks=64, table_width_decode=7,
                     perm_rng=rng, poison=poison)
    dt = dtype or BF16
    if i == 2:
        lens = rng.integers(100, 1024, size=256, endpoint=True)
        seqs = [SeqSpec("decode", int(L), 1) for L in lens]
        return build(name, seed, dt, 16, 8, 128, 256, seqs, table_width_decode=4, perm_rng=rng, poison=poison)
    if i == 3:
        lens = rng.integers(2048, 8192, size=64, endpoint=True)
        seqs = [SeqSpec("decode", int(L), 1) for L in lens]
        return build(name, seed, dt, 32, 8, 128, 16, seqs, table_width_decode=512, perm_rng=rng, poison=poison)
    if i == 4:
        # suffix (new query) length s ~ U{128..2048}; context = 512-token shared prefix + s
        suffix = rng.integers(128, 2048, size=16, endpoint=True)
        seqs = [SeqSpec("prefill", 512 + int(s), int(s), shared=2) for s in suffix]
        w = build(name, seed, dt, 32, 8, 128, 256, seqs, shared_prefix_blocks=2, table_width_prefill=10,
                  perm_rng=rng, poison=poison)
        w.notes["reading"] = "suffix ~ U{128..2048} new queries after a 512-token shared prefix"
        return w
    if i == 5:
        offsets = rng.integers(0, 8192, size=4, endpoint=True)
        lens = rng.integers(1024, 32768, size=200, endpoint=True)
        eligible = np.flatnonzero(lens >= 4097)
        sharers = set(int(x) for x in rng.choice(eligible, size=50, replace=False))
        seqs = [SeqSpec("prefill", int(c) + 512, 512) for c in offsets]
        seqs += [SeqSpec("decode", int(L), 1, shared=16 if j in sharers else 0) for j, L in enumerate(lens)]
        w = build(name, seed, dt, 32, 8, 128, 256, seqs, shared_prefix_blocks=16, table_width_decode=128,
                  table_width_prefill=34, perm_rng=rng, poison=poison)
        w.notes["sharers"] = sorted(sharers)
        return w
    if i == 6:
        # shared-prefix decode: 64 sequences behind one cached 16,384-token prompt
        # (64 blocks of 256, refcount 64), each with U{1..512} tokens of its own
        suffix = rng.integers(1, 512, size=64, endpoint=True)
        seqs = [SeqSpec("decode", 64 * 256 + int(s), 1, shared=64) for s in suffix]
        w = build(name, seed, dt, 32, 8, 128, 256, seqs, shared_prefix_blocks=64, perm_rng=rng, poison=poison)
        w.notes["sharers"] = list(range(64))
        return w
    raise ValueError(f"no config {i}")


def to_float32(a: np.ndarray, dtype: str) -> np.ndarray:
    """Widen stored values to float32 (bf16 bits shifted into the high half)."""
    if dtype == F32:
        return a.astype(np.float32)
    return (a.astype(np.uint32) << np.uint32(16)).view(np.float32)
