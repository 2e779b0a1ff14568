"""Pins of the fp64 oracle to things other than itself (CPU only).

Each pin is a function taking the implementation under check, so the
planted-mistake variants at the bottom (wrong head mapping, top-left causal
alignment, a dropped newest token, an off-by-one block, a wrong scale, a
transposed table) can be shown to fail at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


# ---------------------------------------------------------------- helpers


def _paged_case(seed, B, Hq, Hkv, D, bs, lens, dtype="f32", contiguous=False):
    """Random caches + block tables for decode-style checks (no kv_store)."""
    rng = np.random.default_rng(seed)
    nblk = [-(-L // bs) for L in lens]
    nb = sum(nblk) + 1
    order = np.arange(nb) if contiguous else rng.permutation(nb)
    W_ = max(nblk + [1])
    bt = np.full((B, W_), order[-1], dtype=np.int32)
    pos = 0
    for b in range(B):
        bt[b, : nblk[b]] = order[pos : pos + nblk[b]]
        pos += nblk[b]
    shape = (nb, bs, Hkv, D)
    kc = W.fill_normal(shape, dtype, seed, 11)
    vc = W.fill_normal(shape, dtype, seed, 12)
    q = W.fill_normal((B, Hq, D), dtype, seed, 13)
    return q, kc, vc, bt, np.asarray(lens, dtype=np.int32)


def _sdpa(q, k, v, scale, mask=None):
    """torch's fp64 scaled_dot_product_attention; q [H, Lq, D], k/v [H, Lk, D]."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        attn_mask=None if mask is None else torch.from_numpy(mask), scale=scale)
    return out[0].numpy()


def _contiguous_kv(cache, bt_row, L, bs, dtype):
    flat = cache.reshape((-1,) + cache.shape[2:])  # [NB*bs, Hkv, D]
    idx = np.asarray([int(bt_row[t // bs]) * bs + t % bs for t in range(L)], dtype=np.int64)
    return oracle.widen(flat[idx], dtype)


# ---------------------------------------------------------------- pins (functions of impl)


def pin_decode_vs_sdpa(decode_impl, seed=0, G=4, Hkv=2, D=32, bs=4, lens=(1, 5, 9, 17), dtype="f32"):
    """Decode == torch SDPA on the gathered K/V with each KV head repeated G times (R1)."""
    B = len(lens)
    q, kc, vc, bt, cl = _paged_case(seed, B, G * Hkv, Hkv, D, bs, lens, dtype)
    scale = 1.0 / math.sqrt(D)
    got = decode_impl(q, kc, vc, bt, cl, scale, dtype, bs)
    qd = oracle.widen(q, dtype)
    for b in range(B):
        K = _contiguous_kv(kc, bt[b], int(cl[b]), bs, dtype)  # [L, Hkv, D]
        V = _contiguous_kv(vc, bt[b], int(cl[b]), bs, dtype)
        Kh = np.repeat(K.transpose(1, 0, 2), G, axis=0)  # [Hq, L, D], head h -> KV head h // G
        Vh = np.repeat(V.transpose(1, 0, 2), G, axis=0)
        ref = _sdpa(qd[b][:, None, :], Kh, Vh, scale)[:, 0, :]
        if np.max(np.abs(got[b] - ref)) > TOL:
            return False
    return True


def pin_prefill_vs_sdpa(prefill_impl, seed=0, G=2, Hkv=2, D=16, bs=4, seqs=((3, 3), (2, 7), (5, 12), (1, 1)),
                        paged=True, dtype="f32"):
    """Prefill == torch SDPA with the bottom-right causal mask (R5); seqs are (Lq, Lk)."""
    rng = np.random.default_rng(seed)
    Hq = G * Hkv
    lq = [a for a, _ in seqs]
    lk = [b for _, b in seqs]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = W.fill_normal((int(cu_q[-1]), Hq, D), dtype, seed, 21)
    scale = 0.3 + rng.random()
    if paged:
        _, kc, vc, bt, _ = _paged_case(seed, len(seqs), Hq, Hkv, D, bs, lk, dtype)
        got = prefill_impl(q, kc, vc, cu_q, cu_k, bt, scale, dtype, bs)
    else:
        kc = W.fill_normal((int(cu_k[-1]), Hkv, D), dtype, seed, 22)
        vc = W.fill_normal((int(cu_k[-1]), Hkv, D), dtype, seed, 23)
        bt = None
        got = prefill_impl(q, kc, vc, cu_q, cu_k, None, scale, dtype, bs)
    qd = oracle.widen(q, dtype)
    for b, (Lq, Lk) in enumerate(seqs):
        if bt is not None:
            K = _contiguous_kv(kc, bt[b], Lk, bs, dtype)
            V = _contiguous_kv(vc, bt[b], Lk, bs, dtype)
        else:
            K = oracle.widen(kc[cu_k[b]:cu_k[b + 1]], dtype)
            V = oracle.widen(vc[cu_k[b]:cu_k[b + 1]], dtype)
        Kh = np.repeat(K.transpose(1, 0, 2), G, axis=0)
        Vh = np.repeat(V.transpose(1, 0, 2), G, axis=0)
        Q = qd[cu_q[b]:cu_q[b + 1]].transpose(1, 0, 2)  # [Hq, Lq, D]
        mask = np.arange(Lk)[None, :] <= (Lk - Lq + np.arange(Lq))[:, None]
        ref = _sdpa(Q, Kh, Vh, scale, mask).transpose(1, 0, 2)
        if Lq == Lk:  # the library's own causal flag agrees when nothing is cached
            ref2 = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q)[None], torch.from_numpy(Kh)[None], torch.from_numpy(Vh)[None],
                is_causal=True, scale=scale)[0].numpy().transpose(1, 0, 2)
            assert np.max(np.abs(ref - ref2)) < TOL
        if np.max(np.abs(got[cu_q[b]:cu_q[b + 1]] - ref)) > TOL:
            return False
    return True


def pin_prefill_equals_tokenwise_decode(prefill_impl, decode_impl, seed=1, bs=4, Lq=6, Lk=11, G=2, Hkv=2, D=16):
    """Cached attention equals recomputation: prefill row i == decode over the first p+1 tokens."""
    Hq = G * Hkv
    _, kc, vc, bt, _ = _paged_case(seed, 1, Hq, Hkv, D, bs, [Lk], "f32")
    q = W.fill_normal((Lq, Hq, D), "f32", seed, 31)
    scale = 1.0 / math.sqrt(D)
    pre = prefill_impl(q, kc, vc, np.array([0, Lq], np.int32), np.array([0, Lk], np.int32), bt, scale, "f32", bs)
    for i in range(Lq):
        p = Lk - Lq + i
        dec = decode_impl(q[i:i + 1], kc, vc, bt, np.array([p + 1], np.int32), scale, "f32", bs)
        if np.max(np.abs(pre[i] - dec[0])) > TOL:
            return False
    return True


def pin_context_one_is_v(decode_impl, dtype="bf16"):
    """L = 1: the single weight is exp(0)/1 = 1, so the output is that token's V exactly."""
    q, kc, vc, bt, _ = _paged_case(3, 3, 8, 2, 32, 16, [1, 1, 1], dtype)
    got = decode_impl(q, kc, vc, bt, np.array([1, 1, 1], np.int32), 0.17, dtype, 16)
    for b in range(3):
        v0 = oracle.widen(vc[bt[b, 0], 0], dtype)  # [Hkv, D]
        if not np.array_equal(got[b], np.repeat(v0, 4, axis=0)):
            return False
    return True


def pin_permutation_invariance(decode_impl, seed=4):
    """Moving blocks to other physical ids (data moves with them) leaves outputs bit-identical."""
    q, kc, vc, bt, cl = _paged_case(seed, 3, 4, 2, 16, 4, [7, 13, 2])
    scale = 0.25
    a = decode_impl(q, kc, vc, bt, cl, scale, "f32", 4)
    perm = np.random.default_rng(seed + 1).permutation(kc.shape[0])  # new id of old block j is perm[j]
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[perm] = kc
    vc2[perm] = vc
    b2 = decode_impl(q, kc2, vc2, perm[bt].astype(np.int32), cl, scale, "f32", 4)
    return np.array_equal(a, b2)


# ---------------------------------------------------------------- the pins, applied to the oracle


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,Hkv", [(1, 3), (2, 2), (4, 2), (8, 1)])
def test_decode_vs_sdpa(G, Hkv, dtype):
    assert pin_decode_vs_sdpa(oracle.decode, G=G, Hkv=Hkv, dtype=dtype)


def test_decode_vs_sdpa_contiguous_and_long():
    assert pin_decode_vs_sdpa(oracle.decode, lens=(64, 3, 100), bs=16, D=64)


@pytest.mark.parametrize("paged", [True, False])
@pytest.mark.parametrize("G", [1, 4])
def test_prefill_vs_sdpa(paged, G):
    assert pin_prefill_vs_sdpa(oracle.prefill, G=G, paged=paged)


def test_prefill_vs_sdpa_bf16():
    assert pin_prefill_vs_sdpa(oracle.prefill, dtype="bf16", seqs=((4, 9), (8, 8)))


def test_prefill_equals_tokenwise_decode():
    assert pin_prefill_equals_tokenwise_decode(oracle.prefill, oracle.decode)


def test_context_one_returns_v_exactly():
    assert pin_context_one_is_v(oracle.decode, "bf16")
    assert pin_context_one_is_v(oracle.decode, "f32")


def test_block_permutation_invariance_bitwise():
    assert pin_permutation_invariance(oracle.decode)


def test_zero_context_gives_zeros():
    q, kc, vc, bt, _ = _paged_case(5, 2, 4, 2, 16, 4, [3, 1])
    out = oracle.decode(q, kc, vc, bt, np.array([0, 1], np.int32), 0.5, "f32", 4)
    assert np.all(out[0] == 0.0)


def test_closed_form_scale_zero_is_mean_of_visible_values():
    q, kc, vc, bt, cl = _paged_case(6, 2, 4, 2, 16, 4, [5, 9])
    out = oracle.decode(q, kc, vc, bt, cl, 0.0, "f32", 4)
    for b in range(2):
        V = _contiguous_kv(vc, bt[b], int(cl[b]), 4, "f32")
        mean = V.mean(axis=0)  # [Hkv, D]
        assert np.max(np.abs(out[b] - np.repeat(mean, 2, axis=0))) < TOL


def test_closed_form_dominant_key():
    q, kc, vc, bt, cl = _paged_case(7, 1, 2, 1, 8, 4, [6])
    # make key 3 align with the query and dominate every other score by > 40
    qd = oracle.widen(q, "f32")
    kc = kc.copy()
    blk, row = int(bt[0, 3 // 4]), 3 % 4
    kc[blk, row, 0] = (qd[0, 0] / np.linalg.norm(qd[0, 0]) * 200.0).astype(np.float32)
    q2 = q.copy()
    q2[0, 1] = q2[0, 0]
    out = oracle.decode(q2, kc, vc, bt, cl, 1.0, "f32", 4)
    assert np.max(np.abs(out[0, 0] - oracle.widen(vc[blk, row, 0], "f32"))) < 1e-12


def test_closed_form_equal_heads_equal_outputs():
    q, kc, vc, bt, cl = _paged_case(8, 2, 8, 2, 16, 4, [10, 4])
    q = q.copy()
    q[:, 1:4] = q[:, 0:1]  # heads 0..3 form group 0 under R1
    out = oracle.decode(q, kc, vc, bt, cl, 0.3, "f32", 4)
    for h in range(1, 4):
        assert np.array_equal(out[:, h], out[:, 0])


@pytest.mark.parametrize("cuts", [[3], [1, 2, 3], [7, 8], [5, 9, 15]])
def test_split_merge_identity(cuts):
    rng = np.random.default_rng(9)
    L, G, D = 16, 3, 8
    q = rng.standard_normal((G, D))
    K = rng.standard_normal((L, D))
    V = rng.standard_normal((L, D))
    bounds = [0] + cuts + [L]
    states = [oracle.partial_state(q, K[a:b], V[a:b], 0.7) for a, b in zip(bounds[:-1], bounds[1:])]
    merged = oracle.merge_states(states)
    direct = oracle.attend(q, K, V, 0.7)
    assert np.max(np.abs(merged - direct)) < 1e-12 * max(1.0, np.max(np.abs(direct)))


def test_shared_prefix_states_merge_to_each_members_decode():
    """Cascade reading of shared-prefix decode: the states of a group's shared
    keys, taken once with all members' queries stacked, merged with each
    member's states of its own keys, give each member's plain decode output."""
    rng = np.random.default_rng(12)
    bs, P, G, Hkv, D = 4, 3, 2, 2, 8
    lens = [P * bs + 1, P * bs + 6, P * bs + 13]           # every member has keys beyond the prefix
    q, kc, vc, bt, cl = _paged_case(12, 3, G * Hkv, Hkv, D, bs, lens)
    bt[1, :P] = bt[0, :P]                                    # members 1 and 2 share member 0's prefix blocks
    bt[2, :P] = bt[0, :P]
    scale = 0.4
    direct = oracle.decode(q, kc, vc, bt, cl, scale, "f32", bs)
    qw = oracle.widen(q, "f32")
    K0 = oracle.widen(oracle.gather(kc, bt[0], P * bs, bs), "f32")
    V0 = oracle.widen(oracle.gather(vc, bt[0], P * bs, bs), "f32")
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        stacked = qw[:, heads].reshape(-1, D)                # every member's query heads of KV head g
        chunks = [oracle.partial_state(stacked, K0[a:a + 4, g], V0[a:a + 4, g], scale) for a in range(0, P * bs, 4)]
        for b in range(3):
            K = oracle.widen(oracle.gather(kc, bt[b], int(cl[b]), bs), "f32")[P * bs:, g]
            V = oracle.widen(oracle.gather(vc, bt[b], int(cl[b]), bs), "f32")[P * bs:, g]
            rows = slice(b * G, (b + 1) * G)
            mine = [(m[rows], l[rows], o[rows]) for m, l, o in chunks]
            merged = oracle.merge_states([oracle.partial_state(qw[b, heads], K, V, scale)] + mine)
            assert np.max(np.abs(merged - direct[b, heads])) < 1e-12


def test_kv_store_matches_flat_indexing_and_touches_nothing_else():
    rng = np.random.default_rng(10)
    nb, bs, hkv, d = 6, 4, 2, 8
    kc = W.fill_normal((nb, bs, hkv, d), "bf16", 10, 1)
    vc = W.fill_normal((nb, bs, hkv, d), "bf16", 10, 2)
    n = 9
    slots = rng.choice(nb * bs, size=n, replace=False).astype(np.int32)
    slots[4] = -1  # skipped
    k = W.fill_normal((n, hkv, d), "bf16", 10, 3)
    v = W.fill_normal((n, hkv, d), "bf16", 10, 4)
    k2, v2 = oracle.kv_store(kc, vc, k, v, slots, bs)
    ek = kc.reshape(nb * bs, hkv, d).copy()
    ev = vc.reshape(nb * bs, hkv, d).copy()
    keep = slots >= 0
    ek[slots[keep]] = k[keep]
    ev[slots[keep]] = v[keep]
    assert np.array_equal(k2.reshape(nb * bs, hkv, d), ek)
    assert np.array_equal(v2.reshape(nb * bs, hkv, d), ev)
    with pytest.raises(AssertionError):
        oracle.kv_store(kc, vc, k[:2], v[:2], np.array([3, 3], np.int32), bs)


def test_gather_matches_flat_indexing():
    _, kc, _, bt, cl = _paged_case(12, 3, 2, 2, 8, 4, [1, 9, 12], "bf16")
    for b in range(3):
        g = oracle.gather(kc, bt[b], int(cl[b]), 4)
        flat = kc.reshape(-1, 2, 8)
        idx = [int(bt[b, t // 4]) * 4 + t % 4 for t in range(int(cl[b]))]
        assert np.array_equal(g, flat[idx])


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F80, 0x4049, 0x0001], dtype=np.uint16)
    expect = [1.0, -1.0, 0.0, -0.0, np.inf, 3.140625, 2.0 ** -133]
    got = oracle.widen(bits, "bf16")
    assert np.array_equal(got, np.asarray(expect))


# ---------------------------------------------------------------- the pages' worked examples


def test_xray_panel_shapes_and_gqa_ratio():
    g = json.load(open(os.path.join(GOLDEN, "xray_gqa_shapes.json")))
    Hq, Hkv, D, T = g["num_q_heads"], g["num_kv_heads"], g["head_dim"], g["tokens"]
    assert Hq // Hkv == g["kv_cache_ratio"]
    assert abs(math.sqrt(D) - g["score_divisor"]) < 1e-12
    # a 5-token prompt read in one prefill through a single 256-token block
    bs = 256
    q = W.fill_normal((T, Hq, D), "bf16", 0, 41)
    kc = W.fill_normal((2, bs, Hkv, D), "bf16", 0, 42)
    vc = W.fill_normal((2, bs, Hkv, D), "bf16", 0, 43)
    bt = np.array([[1]], dtype=np.int32)
    out = oracle.prefill(q, kc, vc, np.array([0, T], np.int32), np.array([0, T], np.int32), bt,
                         1.0 / g["score_divisor"], "bf16", bs)
    assert out.shape == (T, Hq, D)
    # the score matrix of the panel: [1, Hq, T, T], causal
    qd = oracle.widen(q, "bf16").transpose(1, 0, 2)
    K = np.repeat(oracle.widen(kc[1, :T], "bf16").transpose(1, 0, 2), Hq // Hkv, axis=0)
    scores = (qd @ K.transpose(0, 2, 1)) / g["score_divisor"]
    assert (1,) + scores.shape == tuple(g["scores_shape"])
    # the first token sees only itself: its output is its own V for every head
    v0 = np.repeat(oracle.widen(vc[1, 0], "bf16"), Hq // Hkv, axis=0)
    assert np.array_equal(out[0], v0)
    # KV cache bytes per token: 8 heads instead of 32 is 4x less
    assert (Hq * D) / (Hkv * D) == g["kv_cache_ratio"]


def test_paged_blocks_diagram():
    g = json.load(open(os.path.join(GOLDEN, "paged_blocks_diagram.json")))
    nb, bs, hkv, d = g["num_blocks"], 4, 1, 8
    a, b = g["reading_seq_a"], g["reading_seq_b"]
    assert len(a) == g["seq_a_blocks"] and len(b) == g["seq_b_blocks"]
    assert sorted(a + b) == g["occupied"]
    assert sorted(set(range(nb)) - set(a + b)) == g["free"]
    kc = W.fill_normal((nb, bs, hkv, d), "f32", 1, 1)
    vc = W.fill_normal((nb, bs, hkv, d), "f32", 1, 2)
    kc[g["free"]] = np.nan  # free blocks never influence a result
    vc[g["free"]] = np.nan
    bt = np.array([a + [g["free"][0]], b], dtype=np.int32)
    cl = np.array([len(a) * bs, len(b) * bs - 1], dtype=np.int32)
    q = W.fill_normal((2, 2, d), "f32", 1, 3)
    out = oracle.decode(q, kc, vc, bt, cl, 0.35, "f32", bs)
    assert np.all(np.isfinite(out))
    # non-contiguous blocks read back in logical order
    seq_b = oracle.gather(kc, bt[1], int(cl[1]), bs)
    assert np.array_equal(seq_b[bs:2 * bs], kc[b[1]])


def test_page_defaults_in_configs():
    g = json.load(open(os.path.join(GOLDEN, "page_defaults.json")))
    assert g["block_size"]["value"] == 256
    assert g["chunked_prefill_budget"]["value"] == 512
    w4 = W.make_config(4)
    assert w4.block_size == g["block_size"]["value"]


# ---------------------------------------------------------------- planted mistakes must fail a pin


def _mutant_decode(kind):
    def impl(q, k_cache, v_cache, block_tables, context_lens, scale, dtype, block_size):
        qd = oracle.widen(q, dtype)
        B, Hq, D = qd.shape
        Hkv = k_cache.shape[2]
        G = Hq // Hkv
        out = np.zeros_like(qd)
        for b in range(B):
            L = int(context_lens[b])
            if kind == "drop_newest":
                L = max(L - 1, 1)
            rows_k, rows_v = [], []
            for t in range(L):
                j = t // block_size
                if kind == "off_by_one_block" and t % block_size == block_size - 1:
                    j = (t + 1) // block_size
                if kind == "transposed_table":
                    blk = int(block_tables.T.reshape(-1)[(b * block_tables.shape[1] + j) % block_tables.size])
                else:
                    blk = int(block_tables[b, j])
                rows_k.append(k_cache[blk, t % block_size])
                rows_v.append(v_cache[blk, t % block_size])
            K = oracle.widen(np.stack(rows_k), dtype)
            V = oracle.widen(np.stack(rows_v), dtype)
            s_ = 1.0 / scale if kind == "inverse_scale" else scale
            for h in range(Hq):
                g = h % Hkv if kind == "interleaved_heads" else h // G
                out[b, h] = oracle.attend(qd[b, h][None], K[:, g], V[:, g], s_)[0]
        return out

    return impl


def _mutant_prefill_top_left(q, k, v, cu_q, cu_k, bt, scale, dtype, bs):
    qd = oracle.widen(q, dtype)
    out = np.zeros_like(qd)
    Hq, Hkv = qd.shape[1], k.shape[-2]
    G = Hq // Hkv
    for b in range(len(cu_q) - 1):
        Lq, Lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        K = oracle.widen(oracle.gather(k, bt[b], Lk, bs), dtype)
        V = oracle.widen(oracle.gather(v, bt[b], Lk, bs), dtype)
        for i in range(Lq):
            p = i  # aligned to the top-left instead of the newest token
            for g in range(Hkv):
                hs = slice(g * G, (g + 1) * G)
                out[cu_q[b] + i, hs] = oracle.attend(qd[cu_q[b] + i, hs], K[:p + 1, g], V[:p + 1, g], scale)
    return out


@pytest.mark.parametrize("kind", ["interleaved_heads", "drop_newest", "off_by_one_block", "inverse_scale",
                                  "transposed_table"])
def test_planted_decode_mistakes_fail_a_pin(kind):
    impl = _mutant_decode(kind)
    caught = (not pin_decode_vs_sdpa(impl, G=2, Hkv=2, lens=(3, 6, 9, 5)) or not pin_permutation_invariance(impl))
    assert caught, kind


def test_planted_top_left_causal_fails_a_pin():
    assert not pin_prefill_vs_sdpa(_mutant_prefill_top_left)
    assert not pin_prefill_equals_tokenwise_decode(_mutant_prefill_top_left, oracle.decode)
