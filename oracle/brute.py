"""Stdlib-only brute force for tiny cases (test infrastructure only).

A second, independent transcription of the same definitions as the C oracle,
written with Python's own binary16/binary32 packing (``struct`` 'e' and 'f',
both round-to-nearest-even) and ``math.fsum``.  It exists to pin the C oracle:
the two share no code.  Only the tests import it.

Double rounding note: binary32 results are formed here as a binary64 operation
followed by a rounding to binary32.  For division of two binary32 operands this
equals the correctly rounded binary32 quotient, because binary64 carries more
than 2*24 + 2 significand bits.
"""
from __future__ import annotations

import math
import struct


def f16_bits_to_float(h: int) -> float:
    return struct.unpack("<e", struct.pack("<H", h))[0]


def float_to_f16_bits(x: float) -> int:
    return struct.unpack("<H", struct.pack("<e", x))[0]


def to_f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def div_f32(a: float, b: float) -> float:
    return to_f32(a / b)


def round_half_away(v: float) -> int:
    r = math.floor(abs(v) + 0.5)
    return -r if v < 0 else r


def quant_q8_0(block_bits):
    """32 fp16 bit patterns -> (scale bits, list of 32 ints in [-127, 127])."""
    xs = [f16_bits_to_float(h) for h in block_bits]
    amax = max(abs(x) for x in xs)
    d16 = float_to_f16_bits(div_f32(amax, 127.0))
    d = f16_bits_to_float(d16)
    if d == 0.0:
        return d16, [0] * 32
    q = [max(-127, min(127, round_half_away(div_f32(x, d)))) for x in xs]
    return d16, q


def quant_q4_0(block_bits):
    """32 fp16 bit patterns -> (scale bits, 16 packed bytes)."""
    xs = [f16_bits_to_float(h) for h in block_bits]
    best = 0
    for i, x in enumerate(xs):
        if abs(x) > abs(xs[best]):
            best = i
    smax = xs[best] if abs(xs[best]) > 0 else 0.0
    d16 = float_to_f16_bits(div_f32(smax, -8.0))
    d = f16_bits_to_float(d16)
    if d == 0.0:
        n = [8] * 32
    else:
        n = [max(-8, min(7, round_half_away(div_f32(x, d)))) + 8 for x in xs]
    return d16, [n[j] | (n[j + 16] << 4) for j in range(16)]


def _first_absmax(xs):
    best = 0
    for i, x in enumerate(xs):
        if abs(x) > abs(xs[best]):
            best = i
    return xs[best] if abs(xs[best]) > 0 else 0.0


def quant_sym(block_bits, bits: int):
    """q5_0 (bits 5) / q6_0 (bits 6): 32 fp16 bit patterns -> (scale bits,
    32 codes in [0, 2^bits))."""
    half = 1 << (bits - 1)
    xs = [f16_bits_to_float(h) for h in block_bits]
    d16 = float_to_f16_bits(div_f32(_first_absmax(xs), -float(half)))
    d = f16_bits_to_float(d16)
    if d == 0.0:
        return d16, [half] * 32
    return d16, [max(-half, min(half - 1, round_half_away(div_f32(x, d)))) + half for x in xs]


def quant_minmax(block_bits, levels: int):
    """q4_1 (levels 15) / q5_1 (levels 31): 32 fp16 bit patterns -> (scale
    bits, minimum bits, 32 codes in [0, levels])."""
    xs = [f16_bits_to_float(h) for h in block_bits]
    mn, mx = min(xs), max(xs)
    d16 = float_to_f16_bits(div_f32(to_f32(mx - mn), float(levels)))
    m16 = float_to_f16_bits(mn)
    d, m = f16_bits_to_float(d16), f16_bits_to_float(m16)
    if d == 0.0:
        return d16, m16, [0] * 32
    return d16, m16, [max(0, min(levels, round_half_away(div_f32(to_f32(x - m), d)))) for x in xs]


def pack_row(t: str, codes_per_block):
    """Data-plane bytes of one row from its blocks' codes: every block's low
    nibbles (byte j = element j | element j+16 << 4), then every block's high
    bits (q5: 32-bit word, bit j = bit 4 of element j; q6: 64-bit word, bits
    2j and 2j+1 = bits 4 and 5 of element j), little endian."""
    lo = bytearray()
    hi = bytearray()
    hb = {"q4_1": 0, "q5_0": 1, "q5_1": 1, "q6_0": 2}[t]
    for n in codes_per_block:
        lo += bytes((n[j] & 15) | ((n[j + 16] & 15) << 4) for j in range(16))
        if hb:
            w = sum((n[j] >> 4) << (hb * j) for j in range(32))
            hi += w.to_bytes(4 * hb, "little")
    return bytes(lo + hi)


def dequant_row(t: str, data: bytes, scales, D: int):
    """One stored row -> list of D floats (exact products)."""
    if t == "f16":
        return [f16_bits_to_float(int.from_bytes(data[2 * i:2 * i + 2], "little")) for i in range(D)]
    if t in ("q4_1", "q5_0", "q5_1", "q6_0"):
        hb = {"q4_1": 0, "q5_0": 1, "q5_1": 1, "q6_0": 2}[t]
        out = []
        for b in range(D // 32):
            w = int.from_bytes(data[D // 2 + 4 * hb * b:D // 2 + 4 * hb * (b + 1)], "little") if hb else 0
            for e in range(32):
                byte = data[16 * b + (e % 16)]
                n = (byte & 15 if e < 16 else byte >> 4) | (((w >> (hb * e)) & ((1 << hb) - 1)) << 4)
                if t == "q5_0":
                    out.append(f16_bits_to_float(scales[b]) * (n - 16))
                elif t == "q6_0":
                    out.append(f16_bits_to_float(scales[b]) * (n - 32))
                else:
                    out.append(f16_bits_to_float(scales[2 * b]) * n + f16_bits_to_float(scales[2 * b + 1]))
        return out
    out = []
    for b in range(D // 32):
        d = f16_bits_to_float(scales[b])
        for e in range(32):
            if t == "q8_0":
                q = data[32 * b + e]
                q = q - 256 if q > 127 else q
            else:
                byte = data[16 * b + (e % 16)]
                q = (byte & 15 if e < 16 else byte >> 4) - 8
            out.append(d * q)
    return out


def attend_rows(q, krows, vrows, scale: float):
    """Softmax attention of one query (list of floats) over lists of rows.
    Returns (out list, lse)."""
    s = [scale * math.fsum(a * b for a, b in zip(q, k)) for k in krows]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    lsum = math.fsum(p)
    D = len(vrows[0])
    out = [math.fsum(p[t] * vrows[t][i] for t in range(len(p))) / lsum for i in range(D)]
    return out, m + math.log(lsum)
