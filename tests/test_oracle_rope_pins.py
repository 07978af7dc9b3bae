"""Pins of the rotary-embedding oracle (CPU only).

Each pin checks the oracle against something other than its own formula:
  * R1 identity: position 0 rotates by angle 0 and returns the row.
  * R2 closed form: with head_dim 128 and base 10000, pair i = 32 has
    frequency 10000^(-1/2) = 1/100, so at position 100 the unit vector e_32
    turns by exactly 1 radian into cos(1) e_32 + sin(1) e_96; pair 0 has
    frequency 1 (angle = position).
  * R3 rotation: every (i, i + d/2) pair keeps its length.
  * R4 composition: rotating by positions m then n equals rotating by m + n
    (a sign or pairing slip breaks the group law).
  * R5 relative position: the dot product of a rotated query and key
    depends only on the distance between their positions -- the property
    the embedding exists for.
  * R6 store: the pool after the fused call equals store_kv of the rotated
    k (bit patterns), with v stored unchanged and padding rows skipped.
  * R7 rounding: the bf16 result is the exact rotation rounded once.
"""

import math

import numpy as np
import pytest

import oracle


def _unit(d, i):
    x = np.zeros((1, 1, d))
    x[0, 0, i] = 1.0
    return x


def test_r1_position_zero_is_identity():
    rng = np.random.default_rng(1)
    tab = oracle.rope_table(4, 64, 10000.0)
    x = rng.standard_normal((3, 2, 64))
    y = oracle.rope_f64(x, np.zeros(3, np.int64), tab)
    assert np.array_equal(x, y)


def test_r2_closed_form_angles():
    d = 128
    tab = oracle.rope_table(101, d, 10000.0)
    y = oracle.rope_f64(_unit(d, 32), np.array([100]), tab)[0, 0]
    assert abs(y[32] - math.cos(1.0)) < 1e-12 and abs(y[96] - math.sin(1.0)) < 1e-12
    assert np.count_nonzero(np.abs(y) > 1e-12) == 2
    for p in (1, 7, 100):
        y0 = oracle.rope_f64(_unit(d, 0), np.array([p]), tab)[0, 0]
        assert abs(y0[0] - math.cos(p)) < 1e-12 and abs(y0[64] - math.sin(p)) < 1e-12


@pytest.mark.parametrize("d,base", [(64, 10000.0), (128, 500000.0)])
def test_r3_pairs_keep_their_length(d, base):
    rng = np.random.default_rng(3)
    tab = oracle.rope_table(4096, d, base)
    x = rng.standard_normal((16, 4, d))
    pos = rng.integers(0, 4096, 16)
    y = oracle.rope_f64(x, pos, tab)
    h = d // 2
    assert np.allclose(x[..., :h] ** 2 + x[..., h:] ** 2, y[..., :h] ** 2 + y[..., h:] ** 2,
                       rtol=0, atol=1e-9)


def test_r4_composition():
    d = 64
    rng = np.random.default_rng(4)
    tab = oracle.rope_table(3000, d, 10000.0)
    x = rng.standard_normal((8, 2, d))
    m = rng.integers(0, 1500, 8)
    n = rng.integers(0, 1500, 8)
    twice = oracle.rope_f64(oracle.rope_f64(x, m, tab), n, tab)
    once = oracle.rope_f64(x, m + n, tab)
    assert np.allclose(twice, once, rtol=0, atol=1e-9)


def test_r5_scores_depend_on_distance_only():
    d = 128
    rng = np.random.default_rng(5)
    tab = oracle.rope_table(5000, d, 10000.0)
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    for m, n in ((10, 3), (400, 17), (2000, 1999)):
        base = float(np.sum(oracle.rope_f64(q, [m], tab) * oracle.rope_f64(k, [n], tab)))
        for s in (1, 250, 2900):
            shifted = float(np.sum(oracle.rope_f64(q, [m + s], tab) * oracle.rope_f64(k, [n + s], tab)))
            assert abs(base - shifted) < 1e-9
    # and it does depend on the distance
    a = float(np.sum(oracle.rope_f64(q, [10], tab) * oracle.rope_f64(k, [3], tab)))
    b = float(np.sum(oracle.rope_f64(q, [10], tab) * oracle.rope_f64(k, [4], tab)))
    assert abs(a - b) > 1e-6


def test_r6_fused_store_rotates_k_and_copies_v():
    rng = np.random.default_rng(6)
    hq, hkv, d, S = 4, 2, 64, 40
    pool = rng.integers(0, 1 << 16, (2, 1, 10, 4, hkv, d)).astype(np.uint16)
    tab = oracle.rope_table(64, d, 10000.0)
    q = oracle.float_to_bf16_bits(rng.standard_normal((5, hq, d)))
    k = oracle.float_to_bf16_bits(rng.standard_normal((5, hkv, d)))
    v = oracle.float_to_bf16_bits(rng.standard_normal((5, hkv, d)))
    loc = np.array([3, -1, 17, 39, 0])
    pos = np.array([0, 5, 63, 9, 30])
    q_rot, out = oracle.rope_store_kv(pool, 0, q, k, v, loc, pos, tab)
    kview = out[0, 0].reshape(S, hkv, d)
    vview = out[1, 0].reshape(S, hkv, d)
    k_rot = oracle.rope(k, pos, tab)
    for t, s in enumerate(loc):
        if s < 0:
            continue
        assert np.array_equal(kview[s], k_rot[t]) and np.array_equal(vview[s], v[t])
    untouched = np.setdiff1d(np.arange(S), loc[loc >= 0])
    assert np.array_equal(kview[untouched], pool[0, 0].reshape(S, hkv, d)[untouched])
    assert np.array_equal(q_rot[0], q[0])  # position 0
    assert np.array_equal(k_rot[0], k[0])


def test_r7_single_rounding():
    rng = np.random.default_rng(7)
    tab = oracle.rope_table(100, 64, 10000.0)
    x = oracle.float_to_bf16_bits(rng.standard_normal((6, 3, 64)))
    pos = rng.integers(0, 100, 6)
    exact = oracle.rope_f64(oracle.bf16_bits_to_float(x, np.float64), pos, tab)
    got = oracle.bf16_bits_to_float(oracle.rope(x, pos, tab), np.float64)
    # within half a bf16 ulp of the exact value (one rounding), for normal values
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(exact), 1e-30))) - 7)
    assert np.all(np.abs(got - exact) <= 0.5 * ulp)


def test_r7_direct_rounding_against_brute_force():
    # f64_to_bf16_bits picks, among the bf16 values around x, the nearest
    # (ties to the even pattern): compare with an exhaustive search over the
    # two neighbouring bf16 patterns, on values that sit exactly on or just
    # beside bf16 midpoints (where rounding through binary32 goes wrong)
    rng = np.random.default_rng(8)
    lo = rng.integers(0x3000, 0x5000, 2000).astype(np.uint16)
    a = oracle.bf16_bits_to_float(lo, np.float64)
    b = oracle.bf16_bits_to_float(lo + np.uint16(1), np.float64)
    mid = (a + b) / 2
    xs = np.concatenate([mid, mid + (b - a) * 2.0 ** -30, mid - (b - a) * 2.0 ** -30])
    got = oracle.f64_to_bf16_bits(xs)
    for x, g in zip(xs, got):
        base = oracle.float_to_bf16_bits(np.float32(x))  # a neighbour to start from
        cands = [int(base) - 1, int(base), int(base) + 1]
        vals = [float(oracle.bf16_bits_to_float(np.array([c], np.uint16), np.float64)[0]) for c in cands]
        dist = [abs(v - x) for v in vals]
        best = min(dist)
        winners = [c for c, dd in zip(cands, dist) if dd == best]
        want = winners[0] if len(winners) == 1 else [c for c in winners if c % 2 == 0][0]
        assert int(g) == want, (x, int(g), want)
