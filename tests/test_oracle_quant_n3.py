"""Pins for the oracle's further scalar types q4_1, q5_0, q5_1 and q6_0 (CPU
only).  The pages give their block sizes (HAL #582 "per-layer KV compression
study", section 1 size table and section 5 P1 ladder) but no layout or
quantiser; the readings are documented in oracle/kvq_oracle.c.

What pins what:
  * hand-worked blocks (tests/golden/worked_blocks_n3.txt) fix the scale and
    minimum formulas, half-away ties, the clamp, the -0 scale of a zero block,
    the nibble order and the placement of the high bits;
  * the stdlib brute force (oracle/brute.py), written independently, agrees
    bit for bit on random blocks and on dequantised values;
  * round-trip error bounds and exact reproduction of on-grid inputs
    (invariants of any quantiser with these formulas);
  * block sizes: data plus scale bytes per block equal the pages' 20, 22, 24
    and 26 bytes.
"""
import os
import struct

import numpy as np
import pytest

from oracle import brute
from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks_n3.txt")
TYPES = ["q4_1", "q5_0", "q5_1", "q6_0"]
LEVELS = {"q4_1": 15, "q5_1": 31}
BITS = {"q5_0": 5, "q6_0": 6}


def f16_bits(v: float) -> int:
    return struct.unpack("<H", struct.pack("<e", v))[0]


def parse_inputs(spec: str) -> np.ndarray:
    x = np.zeros(32, np.uint16)
    if spec == "-":
        return x
    if spec.startswith("ramp="):
        a, s = (float(t) for t in spec[5:].split(","))
        return np.array([f16_bits(a + s * i) for i in range(32)], np.uint16)
    if spec.startswith("rampc="):
        a, s, c = (float(t) for t in spec[6:].split(","))
        return np.array([f16_bits(min(a + s * i, c)) for i in range(32)], np.uint16)
    if spec.startswith("all="):
        return np.full(32, int(spec[4:], 16), np.uint16)
    for item in spec.split(","):
        i, h = item.split("=")
        x[int(i)] = int(h, 16)
    return x


def load():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        wid, t, inputs, scales, data = line.split()
        rows.append((wid, t, parse_inputs(inputs), [int(h, 16) for h in scales.split(",")],
                     bytes.fromhex(data)))
    return rows


WORKED = load()


@pytest.mark.parametrize("wid,t,x,scales,data", WORKED, ids=[w[0] for w in WORKED])
def test_worked_block_oracle(wid, t, x, scales, data):
    d, s = O.quantize(t, x.reshape(1, 32))
    assert bytes(d[0]) == data, f"{wid} data {bytes(d[0]).hex()}"
    assert [int(v) for v in s[0]] == scales, f"{wid} scales {[hex(v) for v in s[0]]}"


@pytest.mark.parametrize("wid,t,x,scales,data", WORKED, ids=[w[0] for w in WORKED])
def test_worked_block_brute(wid, t, x, scales, data):
    bits = [int(h) for h in x]
    if t in BITS:
        d16, n = brute.quant_sym(bits, BITS[t])
        sc = [d16]
    else:
        d16, m16, n = brute.quant_minmax(bits, LEVELS[t])
        sc = [d16, m16]
    assert sc == scales
    assert brute.pack_row(t, [n]) == data


def test_block_sizes_match_the_pages():
    # bytes per 32 values, data plus scales: q4_1 20, q5_0 22, q5_1 24, q6_0 26
    want = {"q4_1": 20, "q5_0": 22, "q5_1": 24, "q6_0": 26}
    for t, n in want.items():
        for D in (32, 128, 512):
            assert (O.data_row_bytes(t, D) + O.scale_row_bytes(t, D)) * 32 == n * D


def random_blocks(rng, n):
    """Blocks of several shapes: normal, wide dynamic range, few distinct
    values (ties), all-positive (the min/max types' offset), constant."""
    out = []
    for k in range(n):
        kind = k % 5
        if kind == 0:
            v = rng.standard_normal(32)
        elif kind == 1:
            v = rng.standard_normal(32) * np.exp(rng.uniform(-8, 8, 32))
        elif kind == 2:
            v = rng.integers(-6, 7, 32) * 0.25
        elif kind == 3:
            v = 3.0 + rng.random(32) * 5
        else:
            v = np.full(32, rng.standard_normal())
        out.append(v.astype(np.float16).view(np.uint16))
    return np.stack(out)


@pytest.mark.parametrize("t", TYPES)
def test_brute_force_agrees_bitwise(t):
    rng = np.random.default_rng(7)
    x = random_blocks(rng, 400)
    d, s = O.quantize(t, x)
    for i in range(x.shape[0]):
        bits = [int(h) for h in x[i]]
        if t in BITS:
            d16, n = brute.quant_sym(bits, BITS[t])
            sc = [d16]
        else:
            d16, m16, n = brute.quant_minmax(bits, LEVELS[t])
            sc = [d16, m16]
        assert [int(v) for v in s[i]] == sc, f"block {i}"
        assert bytes(d[i]) == brute.pack_row(t, [n]), f"block {i}"
        # the dequantised values of both agree exactly
        assert O.dequantize(t, d[i:i + 1], s[i:i + 1], 32)[0].tolist() == \
            brute.dequant_row(t, bytes(d[i]), [int(v) for v in s[i]], 32)


@pytest.mark.parametrize("t", TYPES)
def test_round_trip_error_bounds(t):
    """|x - value| <= d/2 for every element the clamp does not reach; the
    clamp reaches only the top code of the symmetric types (|x - value| <= d)
    and, for the min/max types, the top code when d rounded down (bounded by
    levels * |d - d_exact| + d/2)."""
    rng = np.random.default_rng(11)
    x = random_blocks(rng, 600)
    d, s = O.quantize(t, x)
    xv = x.view(np.float16).astype(np.float64)
    deq = O.dequantize(t, d, s, 32)
    for i in range(x.shape[0]):
        dd = O.load().kvo_f16_value(int(s[i][0]))
        err = np.abs(deq[i] - xv[i])
        if t in BITS:
            assert np.all(err <= abs(dd) * (1 + 1e-6)), f"block {i}"
            inner = err[np.abs(xv[i]) < abs(dd) * ((1 << (BITS[t] - 1)) - 1)]
            assert np.all(inner <= abs(dd) / 2 * (1 + 1e-6)), f"block {i}"
        else:
            lv = LEVELS[t]
            d_exact = float(np.float32(np.float32(xv[i].max()) - np.float32(xv[i].min()))) / lv
            bound = abs(dd) / 2 + lv * abs(dd - d_exact) + 1e-12
            assert np.all(err <= bound * (1 + 1e-6)), f"block {i}"


@pytest.mark.parametrize("t", TYPES)
def test_on_grid_inputs_are_exact(t):
    """Inputs that lie on the block's own grid come back exactly."""
    rng = np.random.default_rng(13)
    for trial in range(50):
        if t in BITS:
            half = 1 << (BITS[t] - 1)
            step = 2.0 ** int(rng.integers(-6, 3))
            codes = rng.integers(-half, half, 32)
            codes[int(rng.integers(0, 32))] = -half          # the first absmax sets d = step
            codes[:int(np.argmax(codes == -half))] = np.clip(codes[:int(np.argmax(codes == -half))],
                                                              -half + 1, half - 1)
            v = codes * step
        else:
            lv = LEVELS[t]
            step = 2.0 ** int(rng.integers(-6, 3))
            base = float(rng.integers(-20, 20)) * step
            codes = rng.integers(0, lv + 1, 32)
            codes[0], codes[1] = 0, lv                       # min and max on the grid ends
            v = base + codes * step
        x = v.astype(np.float16)
        assert np.array_equal(x.astype(np.float64), v)
        d, s = O.quantize(t, x.view(np.uint16).reshape(1, 32))
        assert np.array_equal(O.dequantize(t, d, s, 32)[0], v), f"trial {trial}"


@pytest.mark.parametrize("t", TYPES)
def test_rows_are_blockwise_with_high_bits_after_the_nibbles(t):
    """A row of four blocks: its low nibbles are the four blocks' nibbles in
    order, then the four blocks' high-bit words; each block quantises alone."""
    rng = np.random.default_rng(17)
    x = random_blocks(rng, 4)
    d1, s1 = O.quantize(t, x)                           # four rows of one block
    d4, s4 = O.quantize(t, x.reshape(1, 128))           # one row of four blocks
    lo = b"".join(bytes(d1[i][:16]) for i in range(4))
    hi = b"".join(bytes(d1[i][16:]) for i in range(4))
    assert bytes(d4[0]) == lo + hi
    assert np.array_equal(s4[0], s1.reshape(-1))
