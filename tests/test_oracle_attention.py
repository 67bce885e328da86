"""Pins for the oracle's fp64 decode attention, split partials and combine
(CPU only): a stdlib brute force on tiny contexts, closed forms, invariances,
and the exactness of the split/merge identity."""
import itertools
import math

import numpy as np
import pytest

from oracle import brute
from oracle import oracle as O

TYPES = ["f16", "q8_0", "q4_0"]


def make_cache(t, x_f16):
    """x_f16: (B, Hkv, C, D) float16 -> (type, data, scales) in the oracle layout."""
    d, s = O.quantize(t, x_f16)
    return (t, d, s)


def rand_f16(rng, shape, scale=1.0):
    return (rng.standard_normal(shape) * scale).astype(np.float16)


@pytest.mark.parametrize("tK,tV", list(itertools.product(TYPES, TYPES)))
def test_brute_force_tiny(tK, tV):
    rng = np.random.default_rng(3 * TYPES.index(tK) + TYPES.index(tV))
    for D, G, L in [(32, 1, 1), (32, 2, 3), (64, 5, 8), (32, 5, 5), (64, 1, 7)]:
        Hkv, B, C = 2, 2, 8
        Hq = G * Hkv
        q = rand_f16(rng, (B, Hq, D))
        k = rand_f16(rng, (B, Hkv, C, D))
        v = rand_f16(rng, (B, Hkv, C, D))
        kc, vc = make_cache(tK, k), make_cache(tV, v)
        lens = np.array([L, max(1, L - 1)], np.int32)
        scale = 1 / math.sqrt(D)
        out, lse = O.attend(q, kc, vc, lens, Hkv, scale)
        for b in range(B):
            for h in range(Hq):
                g = h // G
                krows = [brute.dequant_row(tK, kc[1][b, g, t].tobytes(), kc[2][b, g, t] if tK != "f16" else None, D)
                         for t in range(lens[b])]
                vrows = [brute.dequant_row(tV, vc[1][b, g, t].tobytes(), vc[2][b, g, t] if tV != "f16" else None, D)
                         for t in range(lens[b])]
                qv = [float(x) for x in q[b, h].astype(np.float64)]
                o_ref, lse_ref = brute.attend_rows(qv, krows, vrows, scale)
                assert np.allclose(out[b, h], o_ref, rtol=0, atol=1e-12)
                assert abs(lse[b, h] - lse_ref) < 1e-12


def test_single_token_is_that_value_row():
    rng = np.random.default_rng(1)
    D, Hkv, G = 64, 2, 3
    q = rand_f16(rng, (1, Hkv * G, D))
    k = rand_f16(rng, (1, Hkv, 4, D))
    v = rand_f16(rng, (1, Hkv, 4, D))
    for t in TYPES:
        kc, vc = make_cache(t, k), make_cache(t, v)
        out, lse = O.attend(q, kc, vc, [1], Hkv, 0.125)
        vhat = O.dequantize(t, vc[1], vc[2], D)
        khat = O.dequantize(t, kc[1], kc[2], D)
        for h in range(Hkv * G):
            assert np.array_equal(out[0, h], vhat[0, h // G, 0])
            s0 = 0.125 * np.dot(q[0, h].astype(np.float64), khat[0, h // G, 0])
            assert abs(lse[0, h] - s0) < 1e-12


def test_zero_query_gives_mean_and_log_length():
    rng = np.random.default_rng(2)
    D, Hkv, L = 32, 1, 37
    q = np.zeros((1, 4, D), np.float16)
    v = rand_f16(rng, (1, Hkv, 40, D))
    k = rand_f16(rng, (1, Hkv, 40, D))
    for t in TYPES:
        kc, vc = make_cache(t, k), make_cache(t, v)
        out, lse = O.attend(q, kc, vc, [L], Hkv, 1.0)
        vhat = O.dequantize(t, vc[1], vc[2], D)[0, 0, :L]
        assert np.allclose(out[0, 0], vhat.mean(axis=0), atol=1e-14)
        assert abs(lse[0, 0] - math.log(L)) < 1e-13


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    D, L = 128, 300
    q = rand_f16(rng, (1, 1, D))
    k = rand_f16(rng, (1, 1, L, D), 0.1)
    k[0, 0, 123] = (q[0, 0].astype(np.float32) * 4).astype(np.float16)
    v = rand_f16(rng, (1, 1, L, D))
    out, _ = O.attend(q, make_cache("f16", k), make_cache("f16", v), [L], 1, 1.0)
    assert np.allclose(out[0, 0], v[0, 0, 123].astype(np.float64), atol=1e-6)


def test_gqa_equals_mha_with_repeated_heads():
    rng = np.random.default_rng(4)
    D, Hkv, G, L = 64, 3, 4, 50
    q = rand_f16(rng, (2, Hkv * G, D))
    k = rand_f16(rng, (2, Hkv, L, D))
    v = rand_f16(rng, (2, Hkv, L, D))
    for tK, tV in [("q8_0", "q4_0"), ("f16", "f16")]:
        kc, vc = make_cache(tK, k), make_cache(tV, v)
        out_g, lse_g = O.attend(q, kc, vc, [L, L - 7], Hkv, 0.1)
        rep = lambda c: (c[0], np.repeat(c[1], G, axis=1), np.repeat(c[2], G, axis=1))
        out_m, lse_m = O.attend(q, rep(kc), rep(vc), [L, L - 7], Hkv * G, 0.1)
        assert np.array_equal(out_g, out_m) and np.array_equal(lse_g, lse_m)


def test_joint_row_permutation_invariance():
    rng = np.random.default_rng(5)
    D, L = 64, 80
    q = rand_f16(rng, (1, 2, D))
    k = rand_f16(rng, (1, 1, L, D))
    v = rand_f16(rng, (1, 1, L, D))
    perm = rng.permutation(L)
    for t in TYPES:
        a = O.attend(q, make_cache(t, k), make_cache(t, v), [L], 1, 0.125)
        b = O.attend(q, make_cache(t, k[:, :, perm]), make_cache(t, v[:, :, perm]), [L], 1, 0.125)
        assert np.allclose(a[0], b[0], atol=1e-13) and np.allclose(a[1], b[1], atol=1e-13)


def test_context_beyond_length_is_ignored():
    rng = np.random.default_rng(6)
    D, L, C = 32, 20, 64
    q = rand_f16(rng, (1, 1, D))
    k = rand_f16(rng, (1, 1, C, D))
    v = rand_f16(rng, (1, 1, C, D))
    a = O.attend(q, make_cache("q4_0", k), make_cache("q4_0", v), [L], 1, 0.2)
    k2, v2 = k.copy(), v.copy()
    k2[:, :, L:] = 100
    v2[:, :, L:] = -100
    b = O.attend(q, make_cache("q4_0", k2), make_cache("q4_0", v2), [L], 1, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("split_tokens", [1, 7, 16, 64, 1000])
def test_split_then_combine_equals_whole(split_tokens):
    rng = np.random.default_rng(split_tokens)
    D, Hkv, G = 64, 2, 5
    lens = np.array([300, 1, 129], np.int32)
    C = 300
    q = rand_f16(rng, (3, Hkv * G, D))
    k = rand_f16(rng, (3, Hkv, C, D))
    v = rand_f16(rng, (3, Hkv, C, D))
    kc, vc = make_cache("q8_0", k), make_cache("q4_0", v)
    S = -(-C // split_tokens)
    po, pl = O.attend_split(q, kc, vc, lens, Hkv, 0.125, split_tokens, S)
    out, lse = O.combine(po, pl)
    ref, ref_lse = O.attend(q, kc, vc, lens, Hkv, 0.125)
    assert np.allclose(out, ref, atol=1e-12) and np.allclose(lse, ref_lse, atol=1e-12)
    # splits past the end of a sequence are empty: lse = -inf, o = 0
    for b in range(3):
        nb = -(-lens[b] // split_tokens)
        assert np.all(np.isneginf(pl[b, :, nb:])) and np.all(po[b, :, nb:] == 0)
        assert np.all(np.isfinite(pl[b, :, :nb]))


def test_combine_of_one_split_is_identity_and_all_empty_is_zero():
    rng = np.random.default_rng(8)
    po = rng.standard_normal((5, 1, 16))
    pl = rng.standard_normal((5, 1))
    out, lse = O.combine(po, pl)
    assert np.array_equal(out, po[:, 0]) and np.array_equal(lse, pl[:, 0])
    out, lse = O.combine(np.zeros((2, 4, 8)), np.full((2, 4), -np.inf))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


def test_combine_closed_form_two_regions():
    """Two regions with lse a, b: weights e^a/(e^a+e^b) and e^b/(e^a+e^b)."""
    po = np.array([[[1.0, 0.0], [0.0, 1.0]]])
    pl = np.array([[math.log(3.0), math.log(1.0)]])
    out, lse = O.combine(po, pl)
    assert np.allclose(out[0], [0.75, 0.25], atol=1e-15)
    assert abs(lse[0] - math.log(4.0)) < 1e-15


def identity_values(rng, t, shape, e):
    """Values 2^e * k that format t stores exactly (one per-block extreme forces
    the scale to be 2^e)."""
    if t == "q8_0":
        k = rng.integers(-127, 128, shape)
        k[..., ::32] = 127
    else:
        k = rng.integers(-7, 8, shape)
        k[..., ::32] = -8
    x = np.ldexp(k.astype(np.float64), e).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), np.ldexp(k.astype(np.float64), e))
    return x


def test_identity_quantisation_matches_f16_cache_exactly():
    """K and V built from values the format holds exactly: the attention over
    the quantised caches equals the attention over f16 caches of the same
    values, bit for bit."""
    rng = np.random.default_rng(12)
    D, Hkv, G, L = 64, 2, 5, 33
    q = rand_f16(rng, (1, Hkv * G, D))
    for tK, tV in [("q4_0", "q4_0"), ("q8_0", "q4_0"), ("q8_0", "q8_0")]:
        k = identity_values(rng, tK, (1, Hkv, L, D), -7 if tK == "q8_0" else -3)
        v = identity_values(rng, tV, (1, Hkv, L, D), -6 if tV == "q8_0" else -2)
        ref = O.attend(q, make_cache("f16", k), make_cache("f16", v), [L], Hkv, 0.125)
        got = O.attend(q, make_cache(tK, k), make_cache(tV, v), [L], Hkv, 0.125)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])


def test_thread_count_does_not_change_results():
    rng = np.random.default_rng(13)
    D, Hkv, G, L = 128, 2, 5, 500
    q = rand_f16(rng, (1, Hkv * G, D))
    k = rand_f16(rng, (1, Hkv, L, D))
    v = rand_f16(rng, (1, Hkv, L, D))
    kc, vc = make_cache("q8_0", k), make_cache("q4_0", v)
    a = O.attend(q, kc, vc, [L], Hkv, 0.1, nthreads=1)
    b = O.attend(q, kc, vc, [L], Hkv, 0.1, nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ------------------------------------------------ regions of a mixed cache

def test_regions_one_region_equals_attend():
    rng = np.random.default_rng(21)
    B, Hkv, G, D, C = 2, 2, 3, 64, 50
    lens = [50, 17]
    q = rand_f16(rng, (B, Hkv * G, D))
    kc = make_cache("q8_0", rand_f16(rng, (B, Hkv, C, D)))
    vc = make_cache("q4_0", rand_f16(rng, (B, Hkv, C, D)))
    ref, ref_lse = O.attend(q, kc, vc, lens, Hkv, 0.125)
    got, got_lse = O.attend_regions(q, [(kc, vc, lens)], Hkv, 0.125)
    assert np.allclose(got, ref, atol=1e-12, rtol=0) and np.allclose(got_lse, ref_lse, atol=1e-12)


def test_regions_cutting_one_cache_in_two_changes_nothing():
    """Rows [0, a) as one region and [a, L) as another give the attention over
    [0, L) (the regions are a partition of the rows)."""
    rng = np.random.default_rng(22)
    B, Hkv, G, D, C = 1, 2, 4, 64, 90
    L, a = 90, 37
    q = rand_f16(rng, (B, Hkv * G, D))
    for tK, tV in [("q8_0", "q4_0"), ("f16", "q8_0")]:
        kt, vt = rand_f16(rng, (B, Hkv, C, D)), rand_f16(rng, (B, Hkv, C, D))
        kc, vc = make_cache(tK, kt), make_cache(tV, vt)
        ref, ref_lse = O.attend(q, kc, vc, [L], Hkv, 0.125)
        head = lambda c: (c[0], c[1][:, :, :a], c[2][:, :, :a])
        tail = lambda c: (c[0], np.ascontiguousarray(c[1][:, :, a:]), np.ascontiguousarray(c[2][:, :, a:]))
        got, got_lse = O.attend_regions(q, [(head(kc), head(vc), [a]), (tail(kc), tail(vc), [L - a])],
                                        Hkv, 0.125)
        assert np.allclose(got, ref, atol=1e-12, rtol=0)
        assert np.allclose(got_lse, ref_lse, atol=1e-12)


def test_regions_fp16_window_and_exact_quantised_tail_equal_one_f16_cache():
    """A q8_0/q4_0 tail holding values the format stores exactly, plus an fp16
    window: the same attention as one fp16 cache of all the rows."""
    rng = np.random.default_rng(23)
    B, Hkv, G, D = 2, 2, 5, 64
    Lt, Lw = [40, 0], [9, 13]
    q = rand_f16(rng, (B, Hkv * G, D))
    kt = identity_values(rng, "q8_0", (B, Hkv, 40, D), -7)
    vt = identity_values(rng, "q4_0", (B, Hkv, 40, D), -2)
    kw, vw = rand_f16(rng, (B, Hkv, 13, D)), rand_f16(rng, (B, Hkv, 13, D))
    got, got_lse = O.attend_regions(q, [(make_cache("q8_0", kt), make_cache("q4_0", vt), Lt),
                                        (make_cache("f16", kw), make_cache("f16", vw), Lw)], Hkv, 0.125)
    for b in range(B):
        k_all = np.concatenate([kt[b:b + 1, :, :Lt[b]], kw[b:b + 1, :, :Lw[b]]], axis=2)
        v_all = np.concatenate([vt[b:b + 1, :, :Lt[b]], vw[b:b + 1, :, :Lw[b]]], axis=2)
        ref, ref_lse = O.attend(q[b:b + 1], make_cache("f16", k_all), make_cache("f16", v_all),
                                [Lt[b] + Lw[b]], Hkv, 0.125)
        assert np.allclose(got[b:b + 1], ref, atol=1e-12, rtol=0)
        assert np.allclose(got_lse[b:b + 1], ref_lse, atol=1e-12)


def test_regions_all_empty_gives_zero_and_minus_infinity():
    rng = np.random.default_rng(24)
    q = rand_f16(rng, (1, 2, 32))
    kc = make_cache("q4_0", rand_f16(rng, (1, 1, 4, 32)))
    got, got_lse = O.attend_regions(q, [(kc, kc, [0]), (kc, kc, [0])], 1, 0.2)
    assert np.all(got == 0) and np.all(np.isneginf(got_lse))
