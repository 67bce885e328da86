"""Helpers for the GPU parity tests: build caches through the HIP library, run
the decode path through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")

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


def fill_pair(tk, tv, k_f16, v_f16, capacity=None, stream=None):
    B, Hkv, L, D = k_f16.shape
    cap = capacity or L
    kc = C.CachePlanes.alloc(tk, B, Hkv, cap, D)
    vc = C.CachePlanes.alloc(tv, B, Hkv, cap, D)
    pos = torch.zeros(B, dtype=torch.int32, device=k_f16.device)
    C.append(kc, vc, k_f16.permute(0, 2, 1, 3).contiguous(), v_f16.permute(0, 2, 1, 3).contiguous(),
             pos, L, stream)
    return kc, vc


def planes_to_oracle(p: C.CachePlanes):
    """(type name, data uint8 (B,Hkv,C,rb), scales uint16 (B,Hkv,C,nb)) on the host."""
    name = {0: "f16", 1: "q8_0", 2: "q4_0"}[p.type]
    data = p.data.cpu().numpy()
    sc = p.scales.cpu().numpy().view(np.uint16) if p.scales is not None else np.zeros(
        p.data.shape[:3] + (0,), np.uint16)
    return (name, data, sc)


def upload_oracle_planes(name: str, data: np.ndarray, scales: np.ndarray) -> C.CachePlanes:
    B, Hkv, cap, _ = data.shape
    D = scales.shape[-1] * 32 if name != "f16" else data.shape[-1] // 2
    p = C.CachePlanes.alloc(name, B, Hkv, cap, D)
    p.data.copy_(torch.from_numpy(np.ascontiguousarray(data)))
    if p.scales is not None:
        p.scales.copy_(torch.from_numpy(np.ascontiguousarray(scales).view(np.int16)))
    return p


def run_decode(kc, vc, q, lens, split_tokens, variant="auto", scale=None, out_f16=False):
    """K2 + K3 through the C ABI.  Returns (out fp32 host (B,Hq,D), lse host (B,Hq),
    partials (o, lse) host)."""
    B, Hq, D = q.shape
    lens_t = torch.tensor(lens, dtype=torch.int32, device=q.device)
    max_len = max(lens)
    part = C.Partials(B, Hq, D, max_len, split_tokens)
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
