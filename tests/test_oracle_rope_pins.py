"""Pins of the oracle's rotary embedding and fused rope + cache write (CPU only).

The pages name the rotary embedding layer and the per-token positions but
print no formula (reading: the RoFormer rotation, see ``oracle.rope``).  So
the pins are the properties that define a rotary embedding, not a retyped
formula: position 0 is the identity; one pair is the complex product with
e^{i t} (numpy complex arithmetic); the turn rates of the pairs form the
geometric sequence from 1 rad per position down towards 1/theta; norms are
kept; the score of a rotated query and key depends only on the distance of
their positions; rotations compose; the interleaved and rotate-half layouts
are the same map up to a permutation of dimensions.  Planted mistakes at the
bottom each fail at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
import workloads as W

TOL = 1e-12


def _x(seed, N, H, D):
    return np.random.default_rng(seed).standard_normal((N, H, D))


# ---------------------------------------------------------------- pins (functions of impl)


def pin_position_zero_is_identity(rope, interleaved):
    x = _x(1, 5, 3, 16)
    assert np.array_equal(rope(x, np.zeros(5, dtype=np.int64), 1e4, interleaved), x)


def pin_one_pair_is_complex_product(rope, interleaved):
    """D = 2: the only pair turns at 1 rad per position, as x0 + i x1 times e^{i p}."""
    pos = np.array([0, 1, 2, 3, 7, 100, 4095, 32767])
    x = _x(2, len(pos), 4, 2)
    z = (x[..., 0] + 1j * x[..., 1]) * np.exp(1j * pos.astype(np.float64))[:, None]
    out = rope(x, pos, 1e6, interleaved)
    np.testing.assert_allclose(out[..., 0], z.real, rtol=0, atol=TOL)
    np.testing.assert_allclose(out[..., 1], z.imag, rtol=0, atol=TOL)


def _turn_rates(rope, D, theta, interleaved):
    """Angle per position of each pair, read back with atan2 from a rotation at position 1."""
    first, second = oracle.rope_pairs(D, interleaved)  # only used to place the probe vectors
    rates = []
    for j in range(D // 2):
        x = np.zeros((1, 1, D))
        x[0, 0, first[j]] = 1.0
        out = rope(x, np.array([1]), theta, interleaved)[0, 0]
        others = np.delete(out, [first[j], second[j]])
        assert np.all(others == 0), "a pair leaked into other dimensions"
        rates.append(math.atan2(out[second[j]], out[first[j]]))
    return np.array(rates)


def pin_turn_rates_geometric_to_one_over_theta(rope, interleaved):
    """Pair 0 turns 1 rad per position; each next pair turns by a constant factor
    less, and D/2 such factors take 1 rad down to 1/theta."""
    for D, theta in ((8, 1e4), (16, 1e4), (64, 1e6), (128, 1e6)):
        r = _turn_rates(rope, D, theta, interleaved)
        assert abs(r[0] - 1.0) < TOL
        ratio = r[1:] / r[:-1]
        np.testing.assert_allclose(ratio, ratio[0], rtol=1e-9)
        assert abs(ratio[0] ** (D // 2) * theta - 1.0) < 1e-9


def pin_norms_kept(rope, interleaved):
    x = _x(3, 9, 4, 32)
    pos = np.array([0, 1, 5, 17, 255, 256, 1000, 8191, 30000])
    out = rope(x, pos, 1e4, interleaved)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(x, axis=-1), rtol=TOL)


def pin_scores_depend_on_distance_only(rope, interleaved):
    rng = np.random.default_rng(4)
    D = 64
    q = rng.standard_normal((1, 1, D))
    k = rng.standard_normal((1, 1, D))
    for p, r, shift in ((10, 3, 1), (100, 100, 517), (4000, 17, 12345), (0, 9, 3)):
        a = np.dot(rope(q, [p], 1e4, interleaved)[0, 0], rope(k, [r], 1e4, interleaved)[0, 0])
        b = np.dot(rope(q, [p + shift], 1e4, interleaved)[0, 0], rope(k, [r + shift], 1e4, interleaved)[0, 0])
        assert abs(a - b) < 1e-9 * (1 + abs(a))


def pin_rotations_compose(rope, interleaved):
    x = _x(5, 4, 2, 16)
    a = np.array([1, 30, 400, 5000])
    b = np.array([2, 7, 0, 2000])
    np.testing.assert_allclose(rope(rope(x, a, 1e4, interleaved), b, 1e4, interleaved),
                               rope(x, a + b, 1e4, interleaved), rtol=0, atol=1e-10)


def pin_layouts_are_one_map_up_to_permutation(rope):
    """Interleaved rotation = de-interleave, rotate-half rotation, re-interleave."""
    D = 16
    x = _x(6, 3, 2, D)
    pos = np.array([3, 77, 9000])
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])  # interleaved dim of half-layout slot
    half = rope(x[..., perm], pos, 1e4, False)
    back = np.empty_like(half)
    back[..., perm] = half
    np.testing.assert_allclose(rope(x, pos, 1e4, True), back, rtol=0, atol=TOL)


PINS = [pin_position_zero_is_identity, pin_one_pair_is_complex_product,
        pin_turn_rates_geometric_to_one_over_theta, pin_norms_kept,
        pin_scores_depend_on_distance_only, pin_rotations_compose]


@pytest.mark.parametrize("interleaved", [False, True])
@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_rope_pin(pin, interleaved):
    pin(oracle.rope, interleaved)


def test_rope_layouts_one_map():
    pin_layouts_are_one_map_up_to_permutation(oracle.rope)


def test_rope_pairs_are_a_partition():
    for D in (2, 8, 64, 128):
        for inter in (False, True):
            a, b = oracle.rope_pairs(D, inter)
            assert sorted(np.concatenate([a, b]).tolist()) == list(range(D))


# ---------------------------------------------------------------- fused rope + cache write


def _store_case(dtype, seed=7, N=6, Hq=4, Hkv=2, D=16, bs=4, nb=5):
    q = W.fill_normal((N, Hq, D), dtype, seed, 21)
    k = W.fill_normal((N, Hkv, D), dtype, seed, 22)
    v = W.fill_normal((N, Hkv, D), dtype, seed, 23)
    kc = W.fill_normal((nb, bs, Hkv, D), dtype, seed, 24)
    vc = W.fill_normal((nb, bs, Hkv, D), dtype, seed, 25)
    slots = np.array([3, 17, -1, 0, 9, 12], dtype=np.int32)
    pos = np.array([0, 5, 6, 100, 2047, 30000], dtype=np.int32)
    return q, k, v, kc, vc, slots, pos, bs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rope_kv_store_at_position_zero_is_plain_store(dtype):
    q, k, v, kc, vc, slots, _, bs = _store_case(dtype)
    pos = np.zeros(len(slots), dtype=np.int32)
    q_rot, kc_out, vc_out = oracle.rope_kv_store(q, k, v, pos, kc, vc, slots, bs, 1e4, False, dtype)
    kc_plain, vc_plain = oracle.kv_store(kc, vc, k, v, slots, bs)
    assert np.array_equal(q_rot, oracle.widen(q, dtype))
    assert np.array_equal(kc_out, oracle.widen(kc_plain, dtype))
    assert np.array_equal(vc_out, vc_plain)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_kv_store_writes_rotated_rows_only_at_slots(interleaved):
    dtype = "f32"
    q, k, v, kc, vc, slots, pos, bs = _store_case(dtype)
    q_rot, kc_out, vc_out = oracle.rope_kv_store(q, k, v, pos, kc, vc, slots, bs, 1e6, interleaved, dtype)
    kc0 = oracle.widen(kc, dtype)
    flat_out = kc_out.reshape(-1, *kc_out.shape[2:])
    flat_in = kc0.reshape(-1, *kc0.shape[2:])
    written = set(int(s) for s in slots if s >= 0)
    for s in range(flat_in.shape[0]):
        if s not in written:
            assert np.array_equal(flat_out[s], flat_in[s])
    for i, s in enumerate(slots):
        if s < 0:
            continue
        # norms of the stored rows are those of k (a rotation), and position 0 stores k itself
        np.testing.assert_allclose(np.linalg.norm(flat_out[s], axis=-1),
                                   np.linalg.norm(oracle.widen(k, dtype)[i], axis=-1), rtol=TOL)
    assert np.array_equal(flat_out[slots[0]], oracle.widen(k, dtype)[0])  # slot 3 holds position 0
    # a negative slot still rotates its query
    np.testing.assert_allclose(np.linalg.norm(q_rot[2], axis=-1),
                               np.linalg.norm(oracle.widen(q, dtype)[2], axis=-1), rtol=TOL)
    assert not np.allclose(q_rot[2], oracle.widen(q, dtype)[2])
    # v is a plain copy
    _, vc_plain = oracle.kv_store(kc, vc, k, v, slots, bs)
    assert np.array_equal(vc_out, vc_plain)


def test_rotated_attention_is_shift_invariant():
    """Decode over rotated queries and keys gives the same output when every
    position moves by the same amount (the property rotary embeddings exist for)."""
    dtype = "f32"
    rng = np.random.default_rng(8)
    L, Hq, Hkv, D, bs = 11, 4, 2, 32, 4
    k = rng.standard_normal((L, Hkv, D))
    v = rng.standard_normal((L, Hkv, D))
    q = rng.standard_normal((1, Hq, D))
    bt = np.array([[2, 0, 1]], dtype=np.int32)
    outs = []
    for shift in (0, 1000):
        kr = oracle.rope(k, np.arange(L) + shift, 1e4)
        qr = oracle.rope(q, [L - 1 + shift], 1e4)
        kc = np.zeros((3, bs, Hkv, D))
        vc = np.zeros((3, bs, Hkv, D))
        slots = [int(bt[0, t // bs]) * bs + t % bs for t in range(L)]
        kc, vc = oracle.kv_store(kc, vc, kr, v, slots, bs)
        outs.append(oracle.decode(qr.astype(np.float32), kc.astype(np.float32), vc.astype(np.float32),
                                  bt, [L], 1 / math.sqrt(D), dtype, bs))
    np.testing.assert_allclose(outs[0], outs[1], rtol=0, atol=1e-6)


# ---------------------------------------------------------------- planted mistakes


def _mutant(kind):
    def rope(x, positions, theta, interleaved=False):
        x = np.asarray(x, dtype=np.float64)
        N, H, D = x.shape
        first, second = oracle.rope_pairs(D, (not interleaved) if kind == "pairs" else interleaved)
        expo = -1.0 if kind == "exponent" else -2.0
        inv = float(theta) ** (expo * np.arange(D // 2) / D)
        p = np.asarray(positions, dtype=np.float64) + (1.0 if kind == "position" else 0.0)
        ang = p[:, None] * inv[None, :]
        c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
        if kind == "cos_sin":
            c, s = s, c
        sg = -1.0 if kind == "sign" else 1.0
        out = np.empty_like(x)
        out[:, :, first] = x[:, :, first] * c - sg * x[:, :, second] * s
        out[:, :, second] = sg * x[:, :, first] * s + x[:, :, second] * c
        return out
    return rope


@pytest.mark.parametrize("kind", ["sign", "exponent", "pairs", "position", "cos_sin"])
def test_planted_rope_mistakes_fail_a_pin(kind):
    bad = _mutant(kind)
    failed = 0
    for pin in PINS:
        for inter in (False, True):
            try:
                pin(bad, inter)
            except AssertionError:
                failed += 1
    try:
        pin_layouts_are_one_map_up_to_permutation(bad)
    except AssertionError:
        failed += 1
    assert failed > 0, f"mutant {kind} passed every pin"
