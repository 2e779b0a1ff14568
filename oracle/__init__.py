"""Plain fp64 CPU oracle for the paged-KV attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (``paged_kv_gqa_mapping_amd``) never imports or calls it, and this
package imports nothing from the product path: the two share no code.

What it computes, step by step, is the plain definition of each operation,
written for a reader to check by eye; nothing is blocked, fused or reordered:

* ``kv_store`` — write each appended token's K and V row to the slot the slot
  mapping names (the store kernel that fills the paged cache blocks,
  "Nano-vLLM Architecture and Performance", section "FlashAttention
  Integration"; the store happens before attention, "Project overview and the
  four-layer architecture", section "Lifecycle of one request", step 4).
* ``gather`` — read a sequence's logical tokens back through its block table
  (the "PagedAttention: Allocate blocks on-demand" diagram of the nano-vllm
  README; blocks of a sequence need not be contiguous).
* ``decode`` / ``prefill`` — scaled dot-product attention ``softmax(q K^T *
  scale) V`` (the X-Ray mode panel "Compute Attention Scores" of the nano-vllm
  README divides the scores by the square root of the head dimension), with
  grouped-query head sharing (same panel: 32 query heads over 8 KV heads) and
  the causal rule that a token sees only earlier tokens and itself (the
  Self-Attention quiz of the README's tutorial mode).

Readings of points the pages leave open (each is also listed with its reason
in the design notes):

* R1  query head ``h`` reads KV head ``h // (Hq // Hkv)`` (contiguous groups).
* R2  caches are ``[num_blocks, block_size, Hkv, D]``, D contiguous.
* R3  ``slot = block * block_size + row``; a negative slot is skipped.
* R4  a decode sequence's ``context_len`` counts the token just stored.
* R5  prefill query ``i`` of a sequence with ``Lq`` new and ``Lk`` total tokens
      sits at position ``Lk - Lq + i`` and sees keys ``0 .. Lk - Lq + i``.
* R6  with block tables the prefill ``k, v`` are the caches; without them they
      are packed ``[sum Lk, Hkv, D]`` rows indexed by ``cu_seqlens_k``.
* R9  a context of length 0 gives an output row of zeros.

All floating point is float64.  bf16 inputs are ``uint16`` bit patterns and
are widened exactly (``bits << 16`` read as float32, then float64).
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
F32 = "f32"


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact widening of stored values to float64."""
    if dtype == BF16:
        a = np.asarray(a)
        if a.dtype != np.uint16:
            raise TypeError("bf16 values are stored as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == F32:
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def slot_of(table_row, position: int, block_size: int) -> int:
    """Slot of the token at ``position`` of a sequence whose block table row is ``table_row`` (R3)."""
    return int(table_row[position // block_size]) * block_size + position % block_size


def kv_store(k_cache, v_cache, k, v, slot_mapping, block_size: int):
    """Return copies of the caches with token ``i``'s K/V rows written at ``slot_mapping[i]``.

    Works on the stored bits (a pure copy).  A negative slot means "skip".
    Slots must be distinct and inside the pool (precondition, asserted).
    """
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    num_blocks = kc.shape[0]
    seen = set()
    for i, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        assert slot not in seen, "duplicate slot"
        seen.add(slot)
        block, row = divmod(slot, block_size)
        assert 0 <= block < num_blocks, "slot outside the pool"
        kc[block, row] = k[i]
        vc[block, row] = v[i]
    return kc, vc


def gather(cache, table_row, length: int, block_size: int):
    """The ``length`` logical tokens of one sequence, in order: ``[length, Hkv, D]`` (stored bits)."""
    out = np.empty((length,) + tuple(cache.shape[2:]), dtype=cache.dtype)
    for t in range(length):
        out[t] = cache[int(table_row[t // block_size]), t % block_size]
    return out


def attend(q, keys, values, scale: float):
    """softmax(scale * q K^T) V for one KV head.

    q: [G, D] query vectors of the heads that share this KV head;
    keys, values: [L, D].  Returns [G, D].  L = 0 gives zeros (R9).
    """
    if keys.shape[0] == 0:
        return np.zeros((q.shape[0], values.shape[1]), dtype=np.float64)
    scores = scale * (q @ keys.T)  # [G, L]
    m = scores.max(axis=1, keepdims=True)
    e = np.exp(scores - m)
    return (e @ values) / e.sum(axis=1, keepdims=True)


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, dtype: str, block_size: int):
    """Paged GQA decode attention.  q: [B, Hq, D] -> float64 [B, Hq, D].

    Sequence ``b`` attends all of its ``context_lens[b]`` tokens (R4), read
    through row ``b`` of the block tables.
    """
    q = widen(q, dtype)
    B, Hq, D = q.shape
    Hkv = k_cache.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(context_lens[b])
        K = widen(gather(k_cache, block_tables[b], L, block_size), dtype)
        V = widen(gather(v_cache, block_tables[b], L, block_size), dtype)
        for g in range(Hkv):
            heads = slice(g * G, (g + 1) * G)  # R1
            out[b, heads] = attend(q[b, heads], K[:, g], V[:, g], scale)
    return out


def prefill(q, k, v, cu_seqlens_q, cu_seqlens_k, block_tables, scale: float, dtype: str, block_size: int = 0):
    """Causal varlen prefill attention.  q: [sum Lq, Hq, D] -> float64 [sum Lq, Hq, D].

    Query ``i`` of sequence ``b`` sits at position ``p = Lk - Lq + i`` and sees
    keys ``0..p`` (R5).  Keys and values come through ``block_tables[b]`` from
    the caches ``k, v``, or, when ``block_tables`` is None, from the packed
    rows ``cu_seqlens_k[b] + t`` (R6).
    """
    q = widen(q, dtype)
    Tq, Hq, D = q.shape
    Hkv = k.shape[-2]
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    B = len(cu_seqlens_q) - 1
    for b in range(B):
        q0, q1 = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
        k0, k1 = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
        Lq, Lk = q1 - q0, k1 - k0
        assert 0 <= Lq <= Lk, "each sequence needs Lq <= Lk"
        if block_tables is None:
            K = widen(k[k0:k1], dtype)
            V = widen(v[k0:k1], dtype)
        else:
            K = widen(gather(k, block_tables[b], Lk, block_size), dtype)
            V = widen(gather(v, block_tables[b], Lk, block_size), dtype)
        for i in range(Lq):
            p = Lk - Lq + i
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                out[q0 + i, heads] = attend(q[q0 + i, heads], K[: p + 1, g], V[: p + 1, g], scale)
    return out


def partial_state(q, keys, values, scale: float):
    """Unnormalised softmax state of one chunk of keys: (m, l, o) with
    m = max score, l = sum exp(s - m), o = sum exp(s - m) v.  Test helper."""
    scores = scale * (q @ keys.T)
    m = scores.max(axis=1)
    e = np.exp(scores - m[:, None])
    return m, e.sum(axis=1), e @ values


def merge_states(states):
    """Combine chunk states (m_j, l_j, o_j) into the normalised output:
    M = max m_j, w_j = exp(m_j - M), out = sum w_j o_j / sum w_j l_j.  Test helper."""
    M = np.max(np.stack([s[0] for s in states]), axis=0)
    num = sum(np.exp(m - M)[:, None] * o for m, _, o in states)
    den = sum(np.exp(m - M) * l for m, l, _ in states)
    return num / den[:, None]


# ---------------------------------------------------------------- rotary embedding (next-row f2)
#
# The pages name a rotary position embedding layer that runs before the cache
# write ("Nano-vLLM Architecture and Performance", project layout, and the
# four-layer architecture page, layers/ listing) and a positions array that
# the model runner prepares per token (same page, "ModelRunner"), but print no
# formula.  The reading taken here is the rotary embedding as first published
# (RoFormer): dimension pair j of a head turns by the angle
# ``position * theta ** (-2 j / D)``, with the pair either (j, j + D/2)
# ("rotate-half", the layout of the Qwen3 model the pages serve) or (2j, 2j+1)
# ("interleaved").  theta is the caller's.


def rope_pairs(D: int, interleaved: bool):
    """Index arrays (first, second) of the D/2 rotated pairs of a head, pair j first."""
    j = np.arange(D // 2)
    if interleaved:
        return 2 * j, 2 * j + 1
    return j, j + D // 2


def rope(x, positions, theta: float, interleaved: bool = False):
    """Rotate every head of token ``i`` by its position.  x: float64 [N, H, D].

    For pair j = (a, b) of a head, with angle t = positions[i] * theta**(-2j/D):
    out[a] = x[a] cos t - x[b] sin t, out[b] = x[a] sin t + x[b] cos t
    (multiplication of x[a] + i x[b] by e^{it}).
    """
    x = np.asarray(x, dtype=np.float64)
    N, H, D = x.shape
    first, second = rope_pairs(D, interleaved)
    inv_freq = float(theta) ** (-2.0 * np.arange(D // 2) / D)
    angle = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]  # [N, D/2]
    c = np.cos(angle)[:, None, :]
    s = np.sin(angle)[:, None, :]
    out = np.empty_like(x)
    out[:, :, first] = x[:, :, first] * c - x[:, :, second] * s
    out[:, :, second] = x[:, :, first] * s + x[:, :, second] * c
    return out


def rope_kv_store(q, k, v, positions, k_cache, v_cache, slot_mapping, block_size: int,
                  theta: float, interleaved: bool, dtype: str):
    """Rotary embedding of q and k followed by the cache write of the rotated k and of v.

    Returns (q_rot, k_cache_out, v_cache_out): q_rot is float64 [N, Hq, D];
    k_cache_out is the widened (float64) K cache with the rotated k rows at
    their slots; v_cache_out holds the stored bits with v written as by
    ``kv_store``.  Tokens with a negative slot are rotated in q only.
    """
    q_rot = rope(widen(q, dtype), positions, theta, interleaved)
    k_rot = rope(widen(k, dtype), positions, theta, interleaved)
    kc, vc = kv_store(widen(k_cache, dtype), v_cache, k_rot, v, slot_mapping, block_size)
    return q_rot, kc, vc
