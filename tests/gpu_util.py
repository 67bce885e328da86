"""Helpers for the GPU parity tests: caches quantised by the CPU oracle and
uploaded (so every oracle input is the oracle's own), the decode path run
through the C ABI, and the comparison with the oracle."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from oracle import oracle as O  # noqa: E402
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

# Tolerances for attention outputs (fp32 kernels against the fp64 oracle on
# unit-variance inputs): element-wise |d| <= ATOL + RTOL * |ref|, plus per-head
# relative L2 and log-sum-exp checks that see a dropped or misweighted split
# even when the outputs themselves are small.
ATOL, RTOL = 2e-3, 1e-2
REL_L2 = 1e-3
LSE_ATOL = 1e-4


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    C._lib.load()  # raises if the HIP library is not built


def note(msg: str):
    """Name the case on stdout before any GPU step (flushed)."""
    print(f"[gpu-case] {msg}", flush=True)


def to_host_u16(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_quantize(t, x_u16: np.ndarray, nthreads: int | None = None):
    """The oracle's quantiser over (..., D) fp16 bits, with the leading axis cut
    into chunks run on threads (ctypes releases the GIL; the arithmetic is the
    oracle's, row by row)."""
    from concurrent.futures import ThreadPoolExecutor
    x = np.ascontiguousarray(x_u16)
    n = x.shape[0]
    nt = max(1, min(nthreads or oracle_threads(), n))
    cuts = np.linspace(0, n, nt + 1).astype(int)
    with ThreadPoolExecutor(nt) as ex:
        parts = list(ex.map(lambda i: O.quantize(t, x[cuts[i]:cuts[i + 1]]), range(nt)))
    return np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts])


def oracle_planes(t, x_u16: np.ndarray, capacity: int | None = None):
    """Planes of rows x (B, Hkv, L, D) fp16 bits quantised by the oracle, padded
    with zero rows to `capacity`: (type name, data, scales) on the host."""
    B, Hkv, L, D = x_u16.shape
    cap = capacity or L
    name = t if isinstance(t, str) else {v: k for k, v in O.TYPE_NAMES.items()}[t]
    data, sc = oracle_quantize(name, x_u16.reshape(B * Hkv, L, D))
    rb = data.shape[-1]
    d = np.zeros((B, Hkv, cap, rb), np.uint8)
    s = np.zeros((B, Hkv, cap, O.scale_row_bytes(name, D) // 2), np.uint16)
    d[:, :, :L] = data.reshape(B, Hkv, L, rb)
    s[:, :, :L] = sc.reshape(B, Hkv, L, -1)
    return (name, d, s)


def fill_pair(tk, tv, k_f16, v_f16, capacity=None):
    """Device cache planes holding the oracle's quantisation of k, v (B, Hkv, L,
    D) fp16; each carries its host copy as `.oracle` for the oracle side."""
    kh, vh = to_host_u16(k_f16), to_host_u16(v_f16)
    kc = upload_oracle_planes(*oracle_planes(tk, kh, capacity))
    vc = upload_oracle_planes(*oracle_planes(tv, vh, capacity))
    return kc, vc


def planes_to_oracle(p: C.CachePlanes):
    """The oracle-side (type name, data, scales) of planes built by fill_pair:
    the oracle's own bytes, never bytes written by the library."""
    return p.oracle


def upload_oracle_planes(name: str, data: np.ndarray, scales: np.ndarray) -> C.CachePlanes:
    B, Hkv, cap, _ = data.shape
    D = scales.shape[-1] * 32 // (O.scale_row_bytes(name, 32) // 2) if name != "f16" else data.shape[-1] // 2
    p = C.CachePlanes.alloc(name, B, Hkv, cap, D)
    p.data.copy_(torch.from_numpy(np.ascontiguousarray(data)))
    if p.scales is not None:
        p.scales.copy_(torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)))
    p.oracle = (name, data, scales)
    return p


def download_planes(p: C.CachePlanes):
    """What the library holds in a cache on the device (for byte comparisons)."""
    data = p.data.cpu().numpy()
    sc = p.scales.cpu().numpy().view(np.uint16) if p.scales is not None else np.zeros(
        p.data.shape[:3] + (0,), np.uint16)
    return data, sc


def run_decode(kc, vc, q, lens, split_tokens, variant="auto", scale=None, out_f16=False):
    """K2 + K3 through the C ABI.  Returns (out fp32 host (B,Hq,D), lse host (B,Hq),
    partials (o, lse) host); the partials of splits that hold no row are NaN
    (their sentinel, left untouched)."""
    B, Hq, D = q.shape
    lens_t = torch.tensor(lens, dtype=torch.int32, device=q.device)
    max_len = max(lens)
    part = C.Partials(B, Hq, D, max_len, split_tokens)
    # sentinel: splits that hold no row must be left untouched
    part.o.fill_(float("nan"))
    part.lse.fill_(float("nan"))
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    C.decode(kc, vc, q, lens_t, max_len, part, scale, variant)
    out = torch.empty((B, Hq, D), dtype=torch.float16 if out_f16 else torch.float32, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    C.combine(part, lens_t, out, lse)
    torch.cuda.synchronize()
    return (out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
            (part.o.cpu().numpy(), part.lse.cpu().numpy()))


def assert_close(out, lse, ref, ref_lse, what=""):
    """The parity bar for attention outputs; returns (max abs err, max rel err)."""
    err = np.abs(out - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    assert not bad.any(), f"{what}: {bad.sum()} elements beyond tolerance, max err {err.max():.3g}"
    num = np.sqrt(((out - ref) ** 2).sum(-1))
    den = np.sqrt((ref ** 2).sum(-1))
    rel = num / np.maximum(den, 1e-30)
    assert rel.max() <= REL_L2, f"{what}: per-head relative L2 {rel.max():.3g} > {REL_L2}"
    dl = np.abs(lse - ref_lse)
    assert np.all(dl <= LSE_ATOL), f"{what}: lse error {dl.max():.3g} > {LSE_ATOL}"
    big = np.abs(ref) >= 1e-3
    max_rel = float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0
    return float(err.max()), max_rel


def oracle_threads() -> int:
    return min(16, len(os.sched_getaffinity(0)))


def live_splits(lens, split_tokens, Hq, S):
    """(B, Hq, S) mask of the splits that hold a row: s < ceil(L_b / split_tokens)."""
    m = np.zeros((len(lens), Hq, S), dtype=bool)
    for b, L in enumerate(lens):
        m[b, :, :-(-L // split_tokens)] = True
    return m


def assert_partials(po, pl, ro, rl, lens, split_tokens):
    """Split partials against the oracle's: splits that hold a row match it
    (lse within 1e-4, o within the element bound), the others are untouched."""
    live = live_splits(lens, split_tokens, pl.shape[1], pl.shape[2])
    assert np.array_equal(np.isfinite(rl), live)
    assert np.all(np.isnan(pl[~live])) and np.all(np.isnan(po[~live])), "a split with no row was written"
    assert np.all(np.abs(pl[live] - rl[live]) <= 1e-4)
    assert np.all(np.abs(po[live] - ro[live]) <= 2e-3 + 1e-2 * np.abs(ro[live]))
