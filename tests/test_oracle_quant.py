"""Pins for the oracle's quantiser and fp16 primitives (CPU only).

What pins what:
  * hand-worked blocks (tests/golden/worked_blocks.txt) fix every reading of
    the quantiser: stored-scale division, half-away ties, the q4_0 tie-break,
    clamp, -0.0 scale and nibble order;
  * binary16 decode/encode against numpy's IEEE implementation (a special case
    that reduces to a library routine);
  * round-trip error bounds and code ranges (invariants of any correct
    block quantiser with these formulas);
  * identity inputs, where quantisation must reproduce the input exactly;
  * a stdlib brute force (oracle/brute.py) written independently.
"""
import os

import numpy as np
import pytest

from oracle import brute
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.txt")


def load_worked_blocks():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        wid, t, inputs, scale, data = line.split()
        x = np.zeros(32, np.uint16)
        if inputs != "-":
            for item in inputs.split(","):
                i, h = item.split("=")
                x[int(i)] = int(h, 16)
        rows.append((wid, t, x, int(scale, 16), bytes.fromhex(data)))
    return rows


WORKED = load_worked_blocks()


@pytest.mark.parametrize("wid,t,x,scale,data", WORKED, ids=[w[0] for w in WORKED])
def test_worked_block_oracle(wid, t, x, scale, data):
    d, s = O.quantize(t, x[None, :])
    assert int(s[0, 0]) == scale, f"{wid}: scale {int(s[0,0]):#06x} != {scale:#06x}"
    assert d[0].tobytes() == data, f"{wid}: {d[0].tobytes().hex()} != {data.hex()}"


@pytest.mark.parametrize("wid,t,x,scale,data", WORKED, ids=[w[0] for w in WORKED])
def test_worked_block_brute(wid, t, x, scale, data):
    if t == "q8_0":
        s, q = brute.quant_q8_0([int(v) for v in x])
        got = bytes((v & 0xFF) for v in q)
    else:
        s, got = brute.quant_q4_0([int(v) for v in x])
        got = bytes(got)
    assert s == scale and got == data


def test_f16_decode_all_patterns():
    """Every finite binary16 pattern decodes to numpy's value (bitwise)."""
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = np.isfinite(h.view(np.float16))
    rows = h[finite].reshape(-1)
    pad = (-rows.size) % 32
    rows = np.concatenate([rows, np.zeros(pad, np.uint16)]).reshape(-1, 32)
    data, sc = O.quantize("f16", rows)
    got = O.dequantize("f16", data, sc, 32).reshape(-1)[: finite.sum()]
    want = h[finite].view(np.float16).astype(np.float64)
    assert np.array_equal(got, want)
    # sign of zero survives
    assert np.signbit(got[want == 0]).sum() == 1


def _f16_grid_f32():
    """binary32 values around every binary16 value: the value itself, the
    midpoints to its neighbours, and one binary32 ulp either side of them."""
    h = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float64)
    nxt = np.append(v[1:], 65536.0)
    mids = (v + nxt) / 2
    base = np.concatenate([v, mids]).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    allv = np.concatenate([base, up, dn])
    allv = allv[(allv >= 0) & (allv < 65520)]
    return np.concatenate([allv, -allv])


def test_f32_to_f16_matches_numpy_rne():
    x = _f16_grid_f32()
    rng = np.random.default_rng(7)
    x = np.concatenate([x, rng.standard_normal(200000).astype(np.float32) * 10,
                        (rng.standard_normal(50000) * 1e-6).astype(np.float32)])
    got = O.f32_to_f16_bits(x)
    want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def _blocks_with_amax(amax_bits: np.ndarray) -> np.ndarray:
    x = np.zeros((amax_bits.size, 32), np.uint16)
    x[:, 0] = amax_bits
    return x


def test_q8_scale_every_positive_f16_amax():
    """Scale bits for every finite positive binary16 maximum: numpy binary32
    division by 127 then numpy RNE to binary16 (IEEE library arithmetic)."""
    amax = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16)
    _, s = O.quantize("q8_0", _blocks_with_amax(amax))
    want = (amax.view(np.float16).astype(np.float32) / np.float32(127)).astype(np.float16)
    assert np.array_equal(s[:, 0], want.view(np.uint16))


def test_q4_scale_every_nonzero_f16_smax():
    pos = np.arange(1, 0x7C00, dtype=np.uint32).astype(np.uint16)
    smax = np.concatenate([pos, pos | 0x8000]).astype(np.uint16)
    _, s = O.quantize("q4_0", _blocks_with_amax(smax))
    want = (smax.view(np.float16).astype(np.float32) / np.float32(-8)).astype(np.float16)
    assert np.array_equal(s[:, 0], want.view(np.uint16))
    # the scale has the opposite sign to the signed maximum
    assert np.all((s[:, 0] >> 15) != (smax >> 15))


def _codes(t, data):
    if t == "q8_0":
        return data.view(np.int8).astype(np.int64)
    lo = (data & 15).astype(np.int64)
    hi = (data >> 4).astype(np.int64)
    out = np.empty(data.shape[:-1] + (data.shape[-1] * 2,), np.int64)
    nb = data.shape[-1] // 16
    for b in range(nb):
        out[..., 32 * b:32 * b + 16] = lo[..., 16 * b:16 * b + 16] - 8
        out[..., 32 * b + 16:32 * b + 32] = hi[..., 16 * b:16 * b + 16] - 8
    return out


def _check_nearest(t, x, data, scales):
    """Invariant: each code is the integer nearest x/d (d = stored scale) within
    the binary32 quotient's rounding, ties go away from zero, and codes outside
    the type's range are clamped."""
    q = _codes(t, data)
    d = scales.view(np.float16).astype(np.float64).repeat(32, axis=-1)
    xv = x.view(np.float16).astype(np.float64)
    lo, hi = (-127, 127) if t == "q8_0" else (-8, 7)
    assert q.min() >= lo and q.max() <= hi
    nz = d != 0
    assert np.all(q[~nz] == 0)
    r = np.zeros_like(xv)
    r[nz] = xv[nz] / d[nz]
    inrange = nz & (r >= lo - 0.5) & (r <= hi + 0.5)
    # binary32 quotient rounding can move r by at most |r| * 2^-24
    slack = np.abs(r) * 2.0 ** -23
    assert np.all(np.abs(r[inrange] - q[inrange]) <= 0.5 + slack[inrange])
    # exact ties (2x == (2k+1) d, both sides exact in fp64) round away from zero
    k2 = np.floor(2 * r)
    tie = inrange & (np.abs(2 * xv - np.where(k2 % 2 == 1, k2, 0) * d) == 0) & (k2 % 2 == 1)
    away = np.sign(r) * np.floor(np.abs(r) + 0.5)
    tie &= (away >= lo) & (away <= hi)
    assert np.all(q[tie] == away[tie])
    # outside the representable range the code is the clamp
    assert np.all(q[nz & (r > hi + 0.5)] == hi)
    assert np.all(q[nz & (r < lo - 0.5)] == lo)
    return q, d, xv, int(tie.sum())


def _random_blocks(rng, n):
    kinds = [
        rng.standard_normal((n, 32)),
        rng.standard_normal((n, 32)) * np.where(rng.random((n, 32)) < 0.05, 8.0, 1.0),
        rng.standard_normal((n, 32)) * 1e-5,          # subnormal-scale territory
        rng.integers(-20, 20, (n, 32)) / 8.0,         # many exact ties
        rng.standard_normal((n, 32)) * 3000.0,
    ]
    return np.concatenate(kinds).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("t", ["q8_0", "q4_0"])
def test_round_trip_bounds(t):
    rng = np.random.default_rng(11)
    x = _random_blocks(rng, 20000)
    data, scales = O.quantize(t, x)
    q, d, xv, nties = _check_nearest(t, x, data, scales)
    assert nties > 1000
    xhat = O.dequantize(t, data, scales, 32)
    assert np.array_equal(xhat, d * q)
    err = np.abs(xv - xhat)
    ad = np.abs(d)
    normal = ad >= 2.0 ** -14
    if t == "q8_0":
        assert np.all(err[normal] <= ad[normal] / 2 * (1 + 2.0 ** -20))
    else:
        clamped = (q == 7) & (np.abs(xv / np.where(ad > 0, d, 1)) > 7.5)
        ok = ~clamped & normal
        assert np.all(err[ok] <= ad[ok] / 2 * (1 + 2.0 ** -20))
        assert np.all(err[clamped & normal] <= ad[clamped & normal] * (1 + 2.0 ** -10))
        assert clamped.any()
    # zero input elements reconstruct to zero whenever the scale is zero
    assert np.all(xhat[(d == 0)] == 0)


def test_every_f16_value_at_many_scales():
    """Every finite binary16 x with |x| <= amax, quantised in blocks whose
    maximum is amax, for 64 values of amax spread over the normal range."""
    allh = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    allv = allh.view(np.float16).astype(np.float64)
    for t in ("q8_0", "q4_0"):
        ntie = 0
        amaxes = np.unique(np.geomspace(2.0 ** -13, 60000.0, 64).astype(np.float16))
        for a in amaxes:
            xs = allh[allv <= float(a)]
            xs = np.concatenate([xs, xs | 0x8000])
            pad = (-xs.size) % 31
            xs = np.concatenate([xs, np.zeros(pad, np.uint16)]).reshape(-1, 31)
            # put the maximum first with a negative sign for q4_0 so every
            # block shares the same positive scale
            first = np.full((xs.shape[0], 1), a.view(np.uint16) | (0x8000 if t == "q4_0" else 0),
                            np.uint16)
            blocks = np.concatenate([first, xs], axis=1)
            data, scales = O.quantize(t, blocks)
            assert np.all(scales == scales[0, 0])
            ntie += _check_nearest(t, blocks, data, scales)[3]
        assert ntie > 100


@pytest.mark.parametrize("t", ["q8_0", "q4_0"])
def test_identity_inputs_are_exact(t):
    """x = 2^e * k with integer k that the format holds exactly: dequantise
    (quantise (x)) == x for every element."""
    rng = np.random.default_rng(5)
    blocks = []
    for e in range(-14, 6):
        for _ in range(50):
            if t == "q8_0":
                k = rng.integers(-127, 128, 32)
                k[rng.integers(32)] = rng.choice([-127, 127])
            else:
                if rng.random() < 0.5:
                    k = rng.integers(-7, 8, 32)
                    k[rng.integers(32)] = -8
                else:
                    k = rng.integers(-7, 9, 32)
                    k[k == -8] = 0
                    k[rng.integers(32)] = 8
            blocks.append(np.ldexp(k.astype(np.float64), e))
    x = np.array(blocks).astype(np.float16)
    assert np.array_equal(x.astype(np.float64), np.array(blocks))
    data, scales = O.quantize(t, x.view(np.uint16))
    xhat = O.dequantize(t, data, scales, 32)
    assert np.array_equal(xhat, x.astype(np.float64))


@pytest.mark.parametrize("t", ["q8_0", "q4_0"])
def test_brute_force_agrees_bitwise(t):
    rng = np.random.default_rng(3)
    x = _random_blocks(rng, 300)
    data, scales = O.quantize(t, x)
    for i in range(x.shape[0]):
        if t == "q8_0":
            s, q = brute.quant_q8_0([int(v) for v in x[i]])
            got = bytes((v & 0xFF) for v in q)
        else:
            s, got = brute.quant_q4_0([int(v) for v in x[i]])
            got = bytes(got)
        assert s == int(scales[i, 0]) and got == data[i].tobytes(), i


def test_rows_of_several_blocks_are_blockwise():
    """A row of D values is D/32 independent blocks laid out in order."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((7, 256)).astype(np.float16).view(np.uint16)
    for t, rb in (("q8_0", 32), ("q4_0", 16)):
        data, scales = O.quantize(t, x)
        assert data.shape == (7, 256 // 32 * rb) and scales.shape == (7, 8)
        for b in range(8):
            d1, s1 = O.quantize(t, np.ascontiguousarray(x[:, 32 * b:32 * b + 32]))
            assert np.array_equal(data[:, rb * b:rb * b + rb], d1)
            assert np.array_equal(scales[:, b:b + 1], s1)
