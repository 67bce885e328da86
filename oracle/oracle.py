"""Python face of the CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this module.  It loads ``liboracle.so`` built from ``kvq_oracle.c``
(plain C, fp64 attention) and wraps it for numpy arrays.  Nothing here touches a
GPU, and nothing here shares code with the HIP library.

Storage formats and the quantiser readings are documented in ``kvq_oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "kvq_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

F16, Q8_0, Q4_0 = 0, 1, 2
Q4_1, Q5_0, Q5_1, Q6_0 = 4, 5, 6, 7
TYPE_NAMES = {"f16": F16, "q8_0": Q8_0, "q4_0": Q4_0, "q4_1": Q4_1, "q5_0": Q5_0, "q5_1": Q5_1,
              "q6_0": Q6_0}

CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
          "-std=c11", "-Wall", "-Wextra", "-Wno-missing-field-initializers"]


def build(out: str = LIB, mutant: int = 0) -> str:
    """Compile the oracle with gcc (``mutant`` > 0 plants a known mistake; used
    only by the test that shows the pins catch such mistakes)."""
    cmd = ["gcc", *CFLAGS, f"-DKVO_MUTANT={int(mutant)}", SRC, "-o", out, "-lm"]
    subprocess.run(cmd, check=True)
    return out


_libs: dict[str, ctypes.CDLL] = {}


def load(path: str = LIB) -> ctypes.CDLL:
    if path in _libs:
        return _libs[path]
    if path == LIB and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build(LIB)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, dbl = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.kvo_f16_value.argtypes = [ctypes.c_uint16]
    lib.kvo_f16_value.restype = dbl
    lib.kvo_f32_to_f16.argtypes = [ctypes.c_float]
    lib.kvo_f32_to_f16.restype = ctypes.c_uint16
    lib.kvo_f32_to_f16_array.argtypes = [P, i64, P]
    lib.kvo_f32_to_f16_array.restype = None
    lib.kvo_round_half_away.argtypes = [dbl]
    lib.kvo_round_half_away.restype = dbl
    lib.kvo_data_row_bytes.argtypes = [i32, i32]
    lib.kvo_data_row_bytes.restype = i64
    lib.kvo_scale_row_bytes.argtypes = [i32, i32]
    lib.kvo_scale_row_bytes.restype = i64
    lib.kvo_quantize_rows.argtypes = [i32, P, i64, i32, P, P]
    lib.kvo_quantize_rows.restype = i32
    lib.kvo_dequant_rows.argtypes = [i32, P, P, i64, i32, P]
    lib.kvo_dequant_rows.restype = i32
    lib.kvo_attend.argtypes = [i32, i32, i32, i32, i32, P, P, i32, P, P, i32, P, P, dbl, P, P, i32]
    lib.kvo_attend.restype = i32
    lib.kvo_attend_split.argtypes = [i32, i32, i32, i32, i32, P, P, i32, P, P, i32, P, P, dbl,
                                     i32, i32, P, P, i32]
    lib.kvo_attend_split.restype = i32
    lib.kvo_combine.argtypes = [i32, i32, i32, P, P, P, P]
    lib.kvo_combine.restype = i32
    _libs[path] = lib
    return lib


def _ptr(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _tcode(t) -> int:
    return TYPE_NAMES[t] if isinstance(t, str) else int(t)


def f32_to_f16_bits(x: np.ndarray, lib=None) -> np.ndarray:
    """The oracle's own binary32 -> binary16 rounding, element-wise."""
    lib = lib or load()
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(x.shape, np.uint16)
    lib.kvo_f32_to_f16_array(_ptr(x), x.size, _ptr(out))
    return out


def data_row_bytes(t, D: int, lib=None) -> int:
    return int((lib or load()).kvo_data_row_bytes(_tcode(t), D))


def scale_row_bytes(t, D: int, lib=None) -> int:
    return int((lib or load()).kvo_scale_row_bytes(_tcode(t), D))


def quantize(t, x_f16: np.ndarray, lib=None):
    """Quantise rows of fp16 values.  ``x_f16``: (..., D) float16 or uint16 bits.
    Returns (data uint8 (..., data_row_bytes), scales uint16 (..., scale_row_bytes
    / 2): D/32 scales, or D/32 (scale, minimum) pairs for q4_1 / q5_1); the
    scale plane is an empty last axis for the f16 type."""
    lib = lib or load()
    t = _tcode(t)
    x = np.ascontiguousarray(x_f16).view(np.uint16)
    D = x.shape[-1]
    lead = x.shape[:-1]
    n = int(np.prod(lead, dtype=np.int64)) if lead else 1
    data = np.zeros(lead + (data_row_bytes(t, D, lib),), np.uint8)
    scales = np.zeros(lead + (scale_row_bytes(t, D, lib) // 2,), np.uint16)
    sc = scales if t != F16 else np.zeros(1, np.uint16)
    rc = lib.kvo_quantize_rows(t, _ptr(x), n, D, _ptr(data), _ptr(sc))
    if rc != 0:
        raise ValueError("kvo_quantize_rows failed")
    return data, scales


def dequantize(t, data: np.ndarray, scales: np.ndarray, D: int, lib=None) -> np.ndarray:
    lib = lib or load()
    t = _tcode(t)
    data = np.ascontiguousarray(data)
    lead = data.shape[:-1]
    n = int(np.prod(lead, dtype=np.int64)) if lead else 1
    out = np.zeros(lead + (D,), np.float64)
    sc = np.ascontiguousarray(scales) if t != F16 else np.zeros(1, np.uint16)
    rc = lib.kvo_dequant_rows(t, _ptr(data), _ptr(sc), n, D, _ptr(out))
    if rc != 0:
        raise ValueError("kvo_dequant_rows failed")
    return out


def _cache_args(kc, vc):
    tK, kd, ks = kc
    tV, vd, vs = vc
    tK, tV = _tcode(tK), _tcode(tV)
    kd = np.ascontiguousarray(kd)
    vd = np.ascontiguousarray(vd)
    ks = np.ascontiguousarray(ks) if tK != F16 else np.zeros(1, np.uint16)
    vs = np.ascontiguousarray(vs) if tV != F16 else np.zeros(1, np.uint16)
    return tK, kd, ks, tV, vd, vs


def attend(q_f16, kc, vc, seq_lens, Hkv: int, scale: float, nthreads: int | None = None, lib=None):
    """fp64 decode attention.  ``q_f16``: (B, Hq, D) fp16.  ``kc``/``vc``:
    (type, data (B, Hkv, C, data_row_bytes), scales (B, Hkv, C, D/32)).
    Returns (out (B, Hq, D) float64, lse (B, Hq) float64)."""
    lib = lib or load()
    q = np.ascontiguousarray(q_f16).view(np.uint16)
    B, Hq, D = q.shape
    tK, kd, ks, tV, vd, vs = _cache_args(kc, vc)
    C = kd.shape[2]
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.zeros((B, Hq), np.float64)
    nt = nthreads or len(os.sched_getaffinity(0))
    rc = lib.kvo_attend(B, Hq, Hkv, D, C, _ptr(L), _ptr(q), tK, _ptr(kd), _ptr(ks), tV, _ptr(vd),
                        _ptr(vs), float(scale), _ptr(out), _ptr(lse), nt)
    if rc != 0:
        raise ValueError("kvo_attend failed")
    return out, lse


def attend_split(q_f16, kc, vc, seq_lens, Hkv: int, scale: float, split_tokens: int,
                 max_splits: int, nthreads: int | None = None, lib=None):
    """Per-split fp64 partials: (o (B, Hq, S, D), lse (B, Hq, S))."""
    lib = lib or load()
    q = np.ascontiguousarray(q_f16).view(np.uint16)
    B, Hq, D = q.shape
    tK, kd, ks, tV, vd, vs = _cache_args(kc, vc)
    C = kd.shape[2]
    L = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((B, Hq, max_splits, D), np.float64)
    lse = np.zeros((B, Hq, max_splits), np.float64)
    nt = nthreads or len(os.sched_getaffinity(0))
    rc = lib.kvo_attend_split(B, Hq, Hkv, D, C, _ptr(L), _ptr(q), tK, _ptr(kd), _ptr(ks), tV,
                              _ptr(vd), _ptr(vs), float(scale), int(split_tokens), int(max_splits),
                              _ptr(out), _ptr(lse), nt)
    if rc != 0:
        raise ValueError("kvo_attend_split failed")
    return out, lse


def combine(part_o: np.ndarray, part_lse: np.ndarray, lib=None):
    """Exact fp64 merge of partials (..., S, D), (..., S) -> (..., D), (...)."""
    lib = lib or load()
    po = np.ascontiguousarray(part_o, dtype=np.float64)
    pl = np.ascontiguousarray(part_lse, dtype=np.float64)
    lead = pl.shape[:-1]
    S, D = po.shape[-2], po.shape[-1]
    BH = int(np.prod(lead, dtype=np.int64)) if lead else 1
    out = np.zeros(lead + (D,), np.float64)
    lse = np.zeros(lead, np.float64)
    rc = lib.kvo_combine(BH, S, D, _ptr(po), _ptr(pl), _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("kvo_combine failed")
    return out, lse


def attend_regions(q_f16, regions, Hkv: int, scale: float, lib=None):
    """fp64 decode attention over the union of the rows of several caches (the
    regions of a mixed cache, HAL #582 section 5 P2: an fp16 window of recent
    tokens and a quantised tail).  ``regions``: list of (kc, vc, seq_lens) with
    kc / vc as for ``attend``; region i contributes its rows [0, seq_lens[b]).
    Every row is dequantised exactly (``dequantize``) and the scores of all
    regions' rows share one softmax, by the plain definition:
        s_t = scale * q . k_t,  p_t = exp(s_t - max s),  o = sum p_t v_t / sum p_t,
        lse = max s + ln sum p_t  (no rows: o = 0, lse = -inf).
    Returns (out (B, Hq, D) float64, lse (B, Hq) float64)."""
    lib = lib or load()
    q = np.ascontiguousarray(q_f16).view(np.uint16)
    B, Hq, D = q.shape
    G = Hq // Hkv
    qv = q.view(np.float16).astype(np.float64)
    deq = []
    for kc, vc, lens in regions:
        lens = [int(x) for x in lens]
        n = max(lens) if lens else 0
        k = dequantize(kc[0], kc[1][:, :, :n], kc[2][:, :, :n], D, lib)
        v = dequantize(vc[0], vc[1][:, :, :n], vc[2][:, :, :n], D, lib)
        deq.append((k, v, lens))
    out = np.zeros((B, Hq, D), np.float64)
    lse = np.full((B, Hq), -np.inf, np.float64)
    for b in range(B):
        for g in range(Hkv):
            K = np.concatenate([k[b, g, :lens[b]] for k, _, lens in deq], axis=0)
            V = np.concatenate([v[b, g, :lens[b]] for _, v, lens in deq], axis=0)
            if K.shape[0] == 0:
                continue
            for h in range(g * G, (g + 1) * G):
                s = scale * (K @ qv[b, h])
                m = s.max()
                p = np.exp(s - m)
                l = p.sum()
                out[b, h] = (p @ V) / l
                lse[b, h] = m + np.log(l)
    return out, lse
