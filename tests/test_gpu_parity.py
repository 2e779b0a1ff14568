"""HIP path vs the fp64 oracle, element by element (GPU).

kv_store and the block gather are compared bitwise over the whole pool;
attention outputs within 2e-2 (bf16 inputs) or 1e-5 (fp32 inputs) max-abs.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_gqa_mapping_amd as pkv
import workloads as W
from gpu_harness import DeviceStep, bits, log, max_abs, oracle_caches, oracle_decode, tol, to_dev, to_host

pytestmark = pytest.mark.gpu


def _decode_case(dtype, hq, hkv, d, bs, lens, seed=0):
    seqs = [W.SeqSpec("decode", int(L), 1) for L in lens]
    return W.build(f"dec-{dtype}-{hq}-{hkv}-{d}-{bs}", seed, dtype, hq, hkv, d, bs, seqs)


def _prefill_case(dtype, hq, hkv, d, bs, pairs, seed=0):
    # pairs: (Lq new queries, Lk total keys)
    seqs = [W.SeqSpec("prefill", int(lk), int(lq)) for lq, lk in pairs]
    return W.build(f"pre-{dtype}-{hq}-{hkv}-{d}-{bs}", seed, dtype, hq, hkv, d, bs, seqs)


def _check_store(step, w):
    kc, vc = oracle_caches(w)
    assert np.array_equal(bits(to_host(step.k_cache, w.dtype)), bits(kc)), "k_cache differs from the oracle"
    assert np.array_equal(bits(to_host(step.v_cache, w.dtype)), bits(vc)), "v_cache differs from the oracle"
    return kc, vc


DECODE_SHAPES = [
    # dtype, Hq, Hkv, D, bs
    ("f32", 4, 2, 64, 16),
    ("f32", 8, 8, 128, 16),
    ("f32", 32, 8, 128, 256),
    ("bf16", 16, 8, 128, 256),
    ("bf16", 32, 8, 128, 16),
    ("bf16", 8, 1, 128, 32),
    ("bf16", 16, 2, 64, 8),
    ("bf16", 64, 8, 128, 64),
    ("bf16", 4, 4, 64, 16),
    ("bf16", 16, 4, 64, 32),    # four query heads per KV head at D = 64 (3-deep load ring, 4 KV heads per wave)
    ("bf16", 32, 8, 64, 256),   # the same with 8 KV heads per wave
    ("bf16", 8, 2, 128, 1024),  # the largest block size the ABI takes
    ("f32", 8, 2, 64, 8),       # the smallest
]


@pytest.mark.parametrize("split", [0, 64, pkv.SPLIT_BALANCED])
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_decode_tiny_sweep(shape, split):
    dtype, hq, hkv, d, bs = shape
    lens = [1, 2, bs - 1, bs, bs + 1, 3 * bs + 1, 63, 64, 65, 200, 517]
    w = _decode_case(dtype, hq, hkv, d, bs, lens, seed=hq + d + bs)
    log(f"decode sweep {shape} split={split}")
    step = DeviceStep(w)
    step.step(split_tokens=split)
    kc, vc = _check_store(step, w)
    ref = oracle_decode(w, kc, vc)
    err = max_abs(to_host(step.dec_out, dtype), ref, dtype)
    assert err <= tol(dtype), f"max abs error {err}"


# (query tokens, keys) per sequence; the last two walk 9-12 key tiles of 128 with few query
# tiles, so the three V tile buffers of the bf16 kernel are each reused several times
PREFILL_PAIRS = [(1, 1), (1, 40), (5, 5), (31, 31), (32, 32), (33, 100), (64, 64), (65, 200), (130, 130),
                 (97, 300), (200, 700), (3, 1500), (64, 1100)]
PREFILL_SHAPES = [
    ("bf16", 32, 8, 128, 256),
    ("bf16", 64, 8, 128, 16),   # 8 query heads per KV head: 8 heads x 32 positions per workgroup
    ("bf16", 4, 4, 64, 8),      # no grouping at D = 64: one head x 256 positions per workgroup
    ("bf16", 32, 8, 128, 16),
    ("bf16", 16, 8, 128, 64),
    ("bf16", 8, 8, 128, 32),
    ("bf16", 64, 8, 64, 16),
    ("bf16", 8, 4, 64, 256),
    ("f32", 8, 2, 64, 16),
    ("f32", 32, 8, 128, 256),
    ("bf16", 32, 8, 128, 1024),  # the largest block size the ABI takes
    ("bf16", 16, 4, 128, 8),     # the smallest
]


@pytest.mark.parametrize("planned", [True, False], ids=["planned", "one-launch"])
@pytest.mark.parametrize("shape", PREFILL_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_prefill_tiny_sweep(shape, planned):
    """With the planned work lists the pairs (3, 1500) and (64, 1100) are cut into
    pieces of 4 key tiles (the smallest cap), so the piece merge is covered."""
    dtype, hq, hkv, d, bs = shape
    w = _prefill_case(dtype, hq, hkv, d, bs, PREFILL_PAIRS, seed=hq * 3 + bs)
    log(f"prefill sweep {shape} planned={planned}")
    step = DeviceStep(w)
    step.step(planned=planned)
    kc, vc = _check_store(step, w)
    ref = oracle.prefill(w.pre_q, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, w.pre_block_tables, w.scale, dtype,
                         w.block_size)
    err = max_abs(to_host(step.pre_out, dtype), ref, dtype)
    assert err <= tol(dtype), f"max abs error {err}"


def test_prefill_planned_repeats_bitwise_and_rejects_small_workspace():
    """The last piece to arrive merges all pieces in piece order, so repeated
    calls give the same bits whichever piece finishes last."""
    w = _prefill_case("bf16", 32, 8, 128, 16, [(3, 1500), (64, 1100), (200, 700), (700, 3000)], seed=21)
    step = DeviceStep(w)
    step.step()
    first = step.pre_out.clone()
    for _ in range(3):
        step.prefill()
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.int16), step.pre_out.view(torch.int16))
    need = pkv.prefill_workspace_bytes(4, w.max_seqlen_q, 32, 8, 128, 1)
    small = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(pkv.PkvError, match="workspace"):
        pkv.paged_prefill_attn(step.pre_q, step.k_cache, step.v_cache, step.cu_q, step.cu_k, step.pre_bt,
                               step.pre_out, max_seqlen_q=w.max_seqlen_q, max_seqlen_k=w.max_seqlen_k,
                               scale=w.scale, workspace=small)


@pytest.mark.parametrize("planned", [True, False], ids=["planned", "one-launch"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_sequences_without_new_queries(dtype, planned):
    """Sequences of a batch may bring no new queries (an empty chunk, Lq = 0,
    between others): they launch no work, and their neighbours' rows, keys
    and stored tokens are unaffected."""
    pairs = [(0, 40), (5, 5), (0, 300), (40, 300), (0, 1), (129, 1000)]
    w = _prefill_case(dtype, 32, 8, 128, 16, pairs, seed=23)
    log(f"prefill with empty chunks {dtype} planned={planned}")
    step = DeviceStep(w)
    step.step(planned=planned)
    kc, vc = _check_store(step, w)
    ref = oracle.prefill(w.pre_q, kc, vc, w.cu_seqlens_q, w.cu_seqlens_k, w.pre_block_tables, w.scale, dtype,
                         w.block_size)
    err = max_abs(to_host(step.pre_out, dtype), ref, dtype)
    assert err <= tol(dtype), f"max abs error {err}"


# packed k/v (no block table): group sizes 1-8, both head dims; the last pair walks 12 key tiles
PACKED_SHAPES = [("bf16", 16, 4, 128), ("f32", 16, 4, 128), ("bf16", 64, 8, 128), ("bf16", 8, 8, 64),
                 ("bf16", 16, 8, 64), ("f32", 8, 2, 64)]


@pytest.mark.parametrize("shape", PACKED_SHAPES, ids=lambda s: "-".join(map(str, s)))
def test_prefill_packed_kv(shape):
    dtype, hq, hkv, d = shape
    pairs = [(3, 3), (40, 90), (64, 64), (129, 300), (1, 17), (70, 1500)]
    lq = [a for a, _ in pairs]
    lk = [b for _, b in pairs]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = W.fill_normal((int(cu_q[-1]), hq, d), dtype, 9, 1)
    k = W.fill_normal((int(cu_k[-1]), hkv, d), dtype, 9, 2)
    v = W.fill_normal((int(cu_k[-1]), hkv, d), dtype, 9, 3)
    log(f"prefill packed {shape}")
    out = torch.empty((int(cu_q[-1]), hq, d), dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device="cuda")
    pkv.paged_prefill_attn(to_dev(q, dtype), to_dev(k, dtype), to_dev(v, dtype), to_dev(cu_q), to_dev(cu_k), None,
                           out, scale=0.09)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, cu_q, cu_k, None, 0.09, dtype)
    err = max_abs(to_host(out, dtype), ref, dtype)
    assert err <= tol(dtype), f"max abs error {err}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_gather_bitwise(dtype):
    w = _decode_case(dtype, 8, 4, 64, 16, [1, 15, 16, 17, 100, 333], seed=5)
    cu = np.concatenate([[0], np.cumsum(w.dec_context_lens)]).astype(np.int32)
    log(f"gather {dtype}")
    step = DeviceStep(w)
    ko, vo = pkv.paged_gather(step.k_cache, step.v_cache, step.dec_bt, to_dev(cu))
    torch.cuda.synchronize()
    ko, vo = to_host(ko, dtype), to_host(vo, dtype)
    for b, L in enumerate(w.dec_context_lens.tolist()):
        rk = oracle.gather(w.k_cache, w.dec_block_tables[b], L, w.block_size)
        rv = oracle.gather(w.v_cache, w.dec_block_tables[b], L, w.block_size)
        assert np.array_equal(bits(ko[cu[b]:cu[b + 1]]), bits(rk))
        assert np.array_equal(bits(vo[cu[b]:cu[b + 1]]), bits(rv))


def test_kv_store_negative_slots_skipped():
    w = _decode_case("bf16", 8, 8, 128, 16, [5, 9, 30], seed=6)
    w.slot_mapping = w.slot_mapping.copy()
    w.slot_mapping[1] = -1
    log("kv_store negative slot")
    step = DeviceStep(w)
    step.store()
    torch.cuda.synchronize()
    _check_store(step, w)


# ------------------------------------------------------------------ the five workloads


def test_config1_tiny_decode_f32():
    w = W.make_config(1)
    log("config 1")
    step = DeviceStep(w)
    step.step()
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, w.dtype), oracle_decode(w, kc, vc), w.dtype)
    assert err <= 1e-5, err


@pytest.mark.parametrize("dtype", [None, "f32"])
def test_config2_qwen3_decode(dtype):
    w = W.make_config(2, dtype=dtype)
    log(f"config 2 dtype={w.dtype}")
    step = DeviceStep(w)
    step.step()
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, w.dtype), oracle_decode(w, kc, vc), w.dtype)
    log(f"config 2 max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


@pytest.mark.parametrize("dtype", [None, "f32"])
def test_config3_long_decode_splitk(dtype):
    w = W.make_config(3, dtype=dtype)
    log(f"config 3 dtype={w.dtype}")
    step = DeviceStep(w)
    step.step()
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, w.dtype), oracle_decode(w, kc, vc), w.dtype)
    log(f"config 3 max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


@pytest.mark.parametrize("config", [2, 3])
@pytest.mark.parametrize("dtype", [None, "f32"])
def test_balanced_pieces_full_configs(config, dtype):
    """Token-balanced ranges (1024 waves of equal step counts, cut across the
    batch) on the Qwen3-shaped and long-context decode workloads, every row."""
    w = W.make_config(config, dtype=dtype)
    log(f"config {config} dtype={w.dtype} balanced pieces")
    step = DeviceStep(w)
    step.step(split_tokens=pkv.SPLIT_BALANCED)
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, w.dtype), oracle_decode(w, kc, vc), w.dtype)
    log(f"config {config} balanced max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_balanced_pieces_more_sequences_than_pieces():
    """1100 short sequences and one long one over at most 1024 waves: most
    waves' ranges cover several whole sequences (written in the first pass),
    the long one is cut into many parts."""
    rng = np.random.default_rng(16)
    lens = [int(x) for x in rng.integers(1, 300, size=1100)] + [5000]
    w = _decode_case("f32", 8, 2, 64, 16, lens, seed=16)
    log("balanced pieces, 1101 sequences")
    step = DeviceStep(w)
    step.step(split_tokens=pkv.SPLIT_BALANCED)
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, "f32"), oracle_decode(w, kc, vc), "f32")
    assert err <= 1e-5, err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_balanced_single_long_sequence(dtype):
    """One 24000-token sequence cut into hundreds of parts (375 in bf16, 512 =
    the most per sequence in f32), so the merge runs its eight-wave slice
    path; f32 makes 1e-5 see a single lost part."""
    w = _decode_case(dtype, 32, 8, 128, 16, [24000], seed=21)
    log(f"balanced single long sequence {dtype}")
    step = DeviceStep(w)
    step.step(split_tokens=pkv.SPLIT_BALANCED)
    kc, vc = _check_store(step, w)
    err = max_abs(to_host(step.dec_out, w.dtype), oracle_decode(w, kc, vc), w.dtype)
    log(f"balanced single long sequence max abs error {err:.3g}")
    assert err <= tol(w.dtype), err


def test_balanced_ranges_cross_sequences_with_empty_contexts():
    """Ranges that end inside one sequence and start the next, with empty
    contexts (zero rows) and a one-token context among them, and a step count
    below 16 * 1024 (fewer waves than the cap)."""
    rng = np.random.default_rng(22)
    lens = [int(x) for x in rng.integers(1, 700, size=90)]
    lens[7] = 1
    w = _decode_case("f32", 16, 4, 64, 32, lens, seed=22)
    log("balanced ranges across sequences, empty contexts")
    step = DeviceStep(w)
    step.store()
    kc, vc = _check_store(step, w)
    empty = (3, 40, 89)
    cl_host = np.asarray(w.dec_context_lens, dtype=np.int32).copy()
    cl_host[list(empty)] = 0
    cl = torch.from_numpy(cl_host).cuda()
    step.dec_out.fill_(1.0)
    pkv.paged_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, cl, w.scale, step.dec_out,
                          max_context_len=int(cl_host.max()), split_tokens=pkv.SPLIT_BALANCED)
    torch.cuda.synchronize()
    got = to_host(step.dec_out, "f32")
    rows = [b for b in range(len(lens)) if b not in empty]
    err = max_abs(got[rows], oracle_decode(w, kc, vc, rows=rows), "f32")
    assert err <= 1e-5, err
    for b in empty:
        assert not np.any(got[b]), f"row {b} of an empty context is not zero"


# The prefix-cached prefill and mixed-step workloads are compared row by row in
# test_gpu_full_size.py.


# ------------------------------------------------------------------ properties


def test_decode_deterministic_and_permutation_invariant():
    w = _decode_case("bf16", 32, 8, 128, 16, [700, 1, 33, 2049], seed=11)
    log("decode determinism / permutation")
    step = DeviceStep(w)
    step.step(split_tokens=128)
    a = to_host(step.dec_out, "bf16").copy()
    step.decode(split_tokens=128)
    torch.cuda.synchronize()
    assert np.array_equal(a, to_host(step.dec_out, "bf16"))
    # move every block to another physical id, data with it
    perm = np.random.default_rng(3).permutation(w.num_blocks)
    inv = torch.from_numpy(np.argsort(perm)).cuda()
    k2 = step.k_cache[inv].contiguous()  # new block j holds old block inv[j]  (perm[old] = new)
    v2 = step.v_cache[inv].contiguous()
    bt2 = to_dev(perm[w.dec_block_tables].astype(np.int32))
    out2 = torch.empty_like(step.dec_out)
    pkv.paged_decode_attn(step.dec_q, k2, v2, bt2, step.dec_cl, w.scale, out2, max_context_len=w.max_context_len,
                          split_tokens=128)
    torch.cuda.synchronize()
    assert np.array_equal(a, to_host(out2, "bf16"))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_context_one_returns_v_bitwise(dtype):
    w = _decode_case(dtype, 16, 8, 128, 16, [1, 1, 1], seed=12)
    log(f"context one {dtype}")
    step = DeviceStep(w)
    step.step()
    got = to_host(step.dec_out, dtype)
    for b in range(3):
        v0 = w.new_v[b]  # the only token is the one just stored
        assert np.array_equal(bits(got[b]), bits(np.repeat(v0, 2, axis=0)))


def test_prefill_first_row_returns_v_bitwise():
    w = _prefill_case("bf16", 32, 8, 128, 16, [(40, 40), (7, 7)], seed=13)
    log("prefill first row")
    step = DeviceStep(w)
    step.step()
    got = to_host(step.pre_out, "bf16")
    for s in range(2):
        q0 = int(w.cu_seqlens_q[s])
        tok = int(w.cu_seqlens_q[s])  # first new token of the sequence (no cached prefix)
        assert np.array_equal(bits(got[q0]), bits(np.repeat(w.new_v[tok], 4, axis=0)))


def test_split_paths_agree():
    w = _decode_case("f32", 32, 8, 128, 16, [3000, 64, 65, 640], seed=14)
    log("split paths")
    step = DeviceStep(w)
    step.store()
    outs = []
    for split in (64, 192, 1024, 4096):
        step.decode(split_tokens=split)
        torch.cuda.synchronize()
        outs.append(to_host(step.dec_out, "f32").copy())
    kc, vc = oracle_caches(w)
    ref = oracle_decode(w, kc, vc)
    for o in outs:
        assert max_abs(o, ref, "f32") <= 1e-5


@pytest.mark.parametrize("split", [0, pkv.SPLIT_BALANCED])
def test_zero_length_context_gives_zeros(split):
    w = _decode_case("bf16", 16, 8, 128, 16, [5, 7], seed=15)
    step = DeviceStep(w)
    step.store()
    cl = torch.tensor([0, 7], dtype=torch.int32, device="cuda")
    step.dec_out.fill_(1.0)
    pkv.paged_decode_attn(step.dec_q, step.k_cache, step.v_cache, step.dec_bt, cl, w.scale, step.dec_out,
                          max_context_len=7, split_tokens=split)
    torch.cuda.synchronize()
    got = to_host(step.dec_out, "bf16")
    assert (got[0] == 0).all()
