"""The pins can see a plausible mistake: each planted mistake, compiled into a
separate copy of the oracle on the CPU, must fail at least one pin.  (Only the
oracle is ever mutated; nothing here runs on a GPU.)"""
import os

import numpy as np
import pytest

from oracle import brute
from oracle import oracle as O

from .test_oracle_quant import WORKED
from .test_oracle_quant_n3 import BITS, LEVELS, WORKED as WORKED_N3

MUTANTS = {
    1: "round half to even",
    2: "divide by the unrounded binary32 scale",
    3: "q4_0 signed maximum taken at the last index on ties",
    4: "q4_0 nibbles packed as adjacent pairs",
    5: "combine drops the last split",
    6: "q4_1 / q5_1 divide by the unrounded binary32 scale",
    7: "q5 / q6 high bits of adjacent elements swapped",
    8: "q5_0 / q6_0 clamp one level too high",
    9: "query head h reads KV head h mod Hkv",
    10: "softmax scale dropped from the scores",
    11: "V rows decoded from the K planes",
    12: "q4_0 decoded with offset 7",
}


def worked_blocks_pass(lib) -> bool:
    for _, t, x, scale, data in WORKED:
        d, s = O.quantize(t, x[None, :], lib=lib)
        if int(s[0, 0]) != scale or d[0].tobytes() != data:
            return False
    return True


def brute_agrees(lib) -> bool:
    rng = np.random.default_rng(21)
    x = np.concatenate([rng.standard_normal((200, 32)),
                        rng.integers(-20, 20, (200, 32)) / 8.0]).astype(np.float16).view(np.uint16)
    for t in ("q8_0", "q4_0"):
        data, scales = O.quantize(t, x, lib=lib)
        for i in range(x.shape[0]):
            if t == "q8_0":
                s, q = brute.quant_q8_0([int(v) for v in x[i]])
                got = bytes((v & 0xFF) for v in q)
            else:
                s, got = brute.quant_q4_0([int(v) for v in x[i]])
                got = bytes(got)
            if s != int(scales[i, 0]) or got != data[i].tobytes():
                return False
    return True


def split_combine_matches(lib) -> bool:
    rng = np.random.default_rng(22)
    D, Hkv, C = 32, 1, 100
    q = rng.standard_normal((1, 2, D)).astype(np.float16)
    k = rng.standard_normal((1, Hkv, C, D)).astype(np.float16)
    v = rng.standard_normal((1, Hkv, C, D)).astype(np.float16)
    kc = ("f16",) + O.quantize("f16", k, lib=lib)
    vc = ("f16",) + O.quantize("f16", v, lib=lib)
    po, pl = O.attend_split(q, kc, vc, [C], Hkv, 0.2, 16, 7, lib=lib)
    out, lse = O.combine(po, pl, lib=lib)
    ref, ref_lse = O.attend(q, kc, vc, [C], Hkv, 0.2, lib=lib)
    return bool(np.allclose(out, ref, atol=1e-12) and np.allclose(lse, ref_lse, atol=1e-12))


def n3_worked_blocks_pass(lib) -> bool:
    for _, t, x, scales, data in WORKED_N3:
        d, s = O.quantize(t, x[None, :], lib=lib)
        if [int(v) for v in s[0]] != scales or d[0].tobytes() != data:
            return False
    return True


def n3_brute_agrees(lib) -> bool:
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.standard_normal((100, 32)), 2 + rng.random((100, 32)),
                        rng.integers(-20, 20, (100, 32)) / 8.0]).astype(np.float16).view(np.uint16)
    for t in ("q4_1", "q5_0", "q5_1", "q6_0"):
        data, scales = O.quantize(t, x, lib=lib)
        for i in range(x.shape[0]):
            bits = [int(v) for v in x[i]]
            if t in BITS:
                d16, n = brute.quant_sym(bits, BITS[t])
                sc = [d16]
            else:
                d16, m16, n = brute.quant_minmax(bits, LEVELS[t])
                sc = [d16, m16]
            if [int(v) for v in scales[i]] != sc or brute.pack_row(t, [n]) != data[i].tobytes():
                return False
    return True


def attention_brute_agrees(lib) -> bool:
    """fp64 attention of the oracle against the stdlib brute force (its own
    row decoding, math.fsum sums) on tiny contexts: 2 sequences, 2 distinct KV
    heads, 3 query heads each, q8_0 K and q4_0 V."""
    rng = np.random.default_rng(24)
    B, Hkv, G, D, C = 2, 2, 3, 32, 6
    lens = [6, 3]
    q = rng.standard_normal((B, Hkv * G, D)).astype(np.float16)
    k = rng.standard_normal((B, Hkv, C, D)).astype(np.float16)
    v = rng.standard_normal((B, Hkv, C, D)).astype(np.float16)
    kc = ("q8_0",) + O.quantize("q8_0", k, lib=lib)
    vc = ("q4_0",) + O.quantize("q4_0", v, lib=lib)
    out, lse = O.attend(q, kc, vc, lens, Hkv, 0.3, lib=lib)
    for b in range(B):
        for h in range(Hkv * G):
            g = h // G
            krows = [brute.dequant_row("q8_0", kc[1][b, g, t].tobytes(), [int(x) for x in kc[2][b, g, t]], D)
                     for t in range(lens[b])]
            vrows = [brute.dequant_row("q4_0", vc[1][b, g, t].tobytes(), [int(x) for x in vc[2][b, g, t]], D)
                     for t in range(lens[b])]
            qf = [float(x) for x in q[b, h].astype(np.float64)]
            ref, ref_lse = brute.attend_rows(qf, krows, vrows, 0.3)
            if not (np.allclose(out[b, h], ref, atol=1e-12) and abs(lse[b, h] - ref_lse) <= 1e-12):
                return False
    return True


BATTERY = [worked_blocks_pass, brute_agrees, split_combine_matches, n3_worked_blocks_pass, n3_brute_agrees,
           attention_brute_agrees]


def test_unmutated_oracle_passes_battery():
    lib = O.load()
    assert all(f(lib) for f in BATTERY)


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_planted_mistake_is_caught(mutant, tmp_path):
    path = O.build(str(tmp_path / f"liboracle_m{mutant}.so"), mutant=mutant)
    lib = O.load(path)
    results = {f.__name__: f(lib) for f in BATTERY}
    assert not all(results.values()), f"mutant '{MUTANTS[mutant]}' passed every pin: {results}"
