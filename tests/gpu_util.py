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


def gpu_row_scores(kc, vc, q_rows, g, n_rows, scale, chunk=32768):
    """The attention kernel's own score of every row t < n_rows of KV head g
    (sequence 0) for the query rows q_rows ((G, D) fp16 on the device).  Each
    row is presented as a sequence of length 1 through a plane view whose
    sequence stride is one row, so the log-sum-exp of that one-row split is
    the kernel's score of the row.  Returns (G, n_rows) float64."""
    from quantised_kv_long_amd import _lib
    G, D = q_rows.shape
    dev = q_rows.device
    out = np.empty((G, n_rows))

    def view(p, t0):
        rb = _lib.kvq_data_row_bytes(p.type, D)
        sb = _lib.kvq_scale_row_bytes(p.type, D)
        row0 = g * p.capacity + t0
        return _lib.kvq_plane_desc(p.type, 1, p.data.data_ptr() + row0 * rb,
                                   p.scales.data_ptr() + row0 * sb if p.scales is not None else None, 1, 0)

    for t0 in range(0, n_rows, chunk):
        nb = min(chunk, n_rows - t0)
        q = q_rows.unsqueeze(0).expand(nb, G, D).contiguous()
        lens = torch.ones(nb, dtype=torch.int32, device=dev)
        po = torch.empty((nb, G, 1, D), dtype=torch.float32, device=dev)
        pl = torch.empty((nb, G, 1), dtype=torch.float32, device=dev)
        _lib.kvq_decode_attn(view(kc, t0), view(vc, t0), q, lens, nb, G, 1, D, scale, 1, 64, 1, po, pl)
        torch.cuda.synchronize()
        out[:, t0:t0 + nb] = pl[:, :, 0].T.cpu().numpy()
    return out


def oracle_row_scores(kc, q_rows_u16, g, n_rows, scale):
    """The oracle's fp64 scores scale * q . k_t of rows t < n_rows of KV head g
    (sequence 0) for the query rows q_rows ((G, D) fp16 bits): the plain
    definition over the oracle's dequantised rows."""
    name, data, scales = planes_to_oracle(kc)
    D = q_rows_u16.shape[-1]
    k = O.dequantize(name, data[0, g, :n_rows], scales[0, g, :n_rows], D)     # (n, D) fp64
    qf = q_rows_u16.view(np.float16).astype(np.float64)                          # (G, D)
    return scale * (qf @ k.T)


def assert_step_matches_three_calls(out_step, lse_step, out_three, lse_three, v_new_max, what=""):
    """A decode step against the same step as three calls.  The step merges the
    new row as one term: its score is the fp32 sum of q times the decoded
    row, its weight w an fp32 value.  The attention launch reads the row back
    inside a tile: the weight enters the matrix-core product rounded to fp16
    (relative error up to 2^-11), and a quantised K row's score is summed on
    the matrix cores as (code + offset) * q, the offset removed afterwards,
    whose fp32 cancellation costs up to about 2^-24 * 32 * (15 + 8) * |q| *
    |scale| per block (a few 1e-6 to 1e-5 here).  So the outputs of head h
    differ by at most 2^-11 * w * max|v_new| (w <= 1) plus a relative 1e-4
    from the weights' score errors; the LSEs by 5e-5.  v_new_max: (B, Hq) the
    largest |value| of the new V row each head reads."""
    a = np.asarray(out_step, np.float64)
    c = np.asarray(out_three, np.float64)
    assert np.array_equal(np.isfinite(a), np.isfinite(c)), what
    bound = 2e-6 + 1e-4 * np.abs(c) + 2.0 ** -11 * np.asarray(v_new_max, np.float64)[..., None]
    err = np.abs(a - c)
    f = np.isfinite(c)
    assert np.all(err[f] <= bound[f]), f"{what}: step and three calls differ by {err[f].max():.3g}"
    la, lc = np.asarray(lse_step, np.float64), np.asarray(lse_three, np.float64)
    assert np.array_equal(np.isneginf(la), np.isneginf(lc)), what
    g = np.isfinite(lc)
    d = np.abs(la[g] - lc[g])
    assert np.all(d <= 5e-5 + 2e-6 * np.abs(lc[g])), f"{what}: LSE differs by {d.max():.3g}"


def new_row_vmax(v_new, G):
    """(B, Hq) the largest |value| of the new V row (B, Hkv, D) fp16 read by
    each query head (head h reads KV head h // G), with room for the
    quantised row's rounding (|v_hat| <= |v| * (1 + 1/14) for q4_0's
    clamped codes)."""
    m = v_new.float().abs().amax(dim=-1).cpu().numpy().astype(np.float64)   # (B, Hkv)
    return np.repeat(m, G, axis=1) * 1.1


def replay_and_compare(call, outputs, planes, scratch, what, replays=3):
    """Runs call() eagerly, captures it in a graph and replays the graph
    `replays` times; every replay's outputs and cache planes must equal the eager
    call's bit for bit."""
    call()
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs]
    want_planes = [t.clone() for t in planes]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for r in range(replays):
        for t in list(outputs) + list(scratch):
            t.fill_(float("nan"))
        (torch.randn(1 << 20, device="cuda") * 2.0).sum().item()   # other eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, w) in enumerate(zip(outputs, want)):
            assert torch.equal(t, w), f"{what}: replay {r}, output {i} differs from the eager call"
        for i, (t, w) in enumerate(zip(planes, want_planes)):
            assert torch.equal(t, w), f"{what}: replay {r}, cache plane {i} differs from the eager call"
    return want


def plane_tensors(*caches):
    """The device tensors holding the given caches' planes (data, and scales
    where the type has them)."""
    out = []
    for p in caches:
        out.append(p.data)
        if p.scales is not None:
            out.append(p.scales)
    return out
