"""Device memory for the KV cache planes and the split partials, allocated with
torch, and the plane descriptors the C ABI takes.  No computation happens
here: every step of the decode path runs in the library's HIP kernels.

Layout (matches kvq_plane_desc): for cache tensor X of one layer,
    data   : uint8  [B, Hkv, capacity, data_row_bytes(type, D)]
    scales : int16  [B, Hkv, capacity, scale_row_bytes(type, D) / 2]   (absent for f16)
so row t of KV head g of sequence b is row (b * Hkv + g) * capacity + t.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

from . import _lib


@dataclass
class CachePlanes:
    type: int
    B: int
    Hkv: int
    capacity: int
    D: int
    data: torch.Tensor
    scales: torch.Tensor | None

    @classmethod
    def alloc(cls, t, B: int, Hkv: int, capacity: int, D: int, device="cuda") -> "CachePlanes":
        t = _lib._tcode(t)
        rb = _lib.kvq_data_row_bytes(t, D)
        if rb == 0:
            raise ValueError(f"unsupported type/head_dim {t}/{D}")
        data = torch.empty((B, Hkv, capacity, rb), dtype=torch.uint8, device=device)
        scales = None
        if t != _lib.F16:
            ns = _lib.kvq_scale_row_bytes(t, D) // 2
            scales = torch.empty((B, Hkv, capacity, ns), dtype=torch.int16, device=device)
        return cls(t, B, Hkv, capacity, D, data, scales)

    def desc(self) -> _lib.kvq_plane_desc:
        return _lib.kvq_plane_desc(
            self.type, self.capacity, self.data.data_ptr(),
            self.scales.data_ptr() if self.scales is not None else None,
            self.Hkv * self.capacity, self.capacity)

    def stored_bytes(self, lengths) -> int:
        """Bytes of the rows [0, L_b) of every (b, head): the algorithmic bytes a
        decode pass over this tensor reads."""
        per_row = _lib.kvq_data_row_bytes(self.type, self.D) + _lib.kvq_scale_row_bytes(self.type, self.D)
        return int(sum(lengths)) * self.Hkv * per_row


class Partials:
    """Split partial buffers for kvq_decode_attn / kvq_combine."""

    def __init__(self, B: int, Hq: int, D: int, max_seq_len: int, split_tokens: int, device="cuda"):
        self.split_tokens = split_tokens
        self.max_splits = max(1, math.ceil(max_seq_len / split_tokens))
        self.o = torch.empty((B, Hq, self.max_splits, D), dtype=torch.float32, device=device)
        self.lse = torch.empty((B, Hq, self.max_splits), dtype=torch.float32, device=device)


def append(kc: CachePlanes, vc: CachePlanes, k_new: torch.Tensor, v_new: torch.Tensor,
           positions: torch.Tensor, max_end: int, stream=None):
    """kvq_quantize_append on torch tensors: k_new, v_new (B, n_new, Hkv, D) fp16."""
    B, n_new, Hkv, D = k_new.shape
    return _lib.kvq_quantize_append(kc.desc(), vc.desc(), k_new, v_new, positions, B, n_new, Hkv,
                                    D, max_end, stream)


def quantize_rows(kc: CachePlanes, vc: CachePlanes, k_src: CachePlanes, v_src: CachePlanes,
                  counts: torch.Tensor, positions: torch.Tensor, max_rows: int, max_end: int,
                  stream=None):
    """kvq_quantize_rows: rows [0, counts[b]) of the fp16 planes k_src / v_src
    into rows positions[b] + r of kc / vc."""
    return _lib.kvq_quantize_rows(kc.desc(), vc.desc(), k_src.desc(), v_src.desc(), counts, positions,
                                  kc.B, max_rows, kc.Hkv, kc.D, max_end, stream)


def decode_mixed(tail, win, q: torch.Tensor, tail_lens: torch.Tensor, win_lens: torch.Tensor,
                 tail_part: "Partials", win_part: "Partials", softmax_scale: float, stream=None,
                 tail_max_len=None, win_max_len=None):
    """kvq_decode_attn_mixed: ``tail`` and ``win`` are (K, V) CachePlanes pairs
    (the window fp16); max lengths default to the caches' capacities."""
    B, Hq, D = q.shape
    kt, vt = tail
    kw, vw = win
    return _lib.kvq_decode_attn_mixed(kt.desc(), vt.desc(), kw.desc(), vw.desc(), q, tail_lens, win_lens,
                                      B, Hq, kt.Hkv, D, softmax_scale, tail_max_len or kt.capacity,
                                      tail_part.split_tokens, tail_part.max_splits, tail_part.o,
                                      tail_part.lse, win_max_len or kw.capacity,
                                      win_part.split_tokens, win_part.max_splits, win_part.o, win_part.lse,
                                      stream)


def decode_step_mixed(tail, win, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      tail_lens: torch.Tensor, win_lens: torch.Tensor, tail_part: "Partials",
                      win_part: "Partials", softmax_scale: float, out: torch.Tensor, lse_out=None,
                      stream=None, tail_max_len=None, win_max_len=None):
    """kvq_decode_step_mixed: the new row (B, Hkv, D) fp16 into the fp16 window
    at row win_lens[b] - 1, attention over both regions, the region merge into
    ``out`` (B, Hq, D)."""
    B, Hq, D = q.shape
    kt, vt = tail
    kw, vw = win
    ot = "f16" if out.dtype == torch.float16 else "f32"
    return _lib.kvq_decode_step_mixed(kt.desc(), vt.desc(), kw.desc(), vw.desc(), k_new, v_new, q,
                                      tail_lens, win_lens, B, Hq, kt.Hkv, D, softmax_scale,
                                      tail_max_len or kt.capacity, tail_part.split_tokens,
                                      tail_part.max_splits, tail_part.o, tail_part.lse,
                                      win_max_len or kw.capacity, win_part.split_tokens,
                                      win_part.max_splits, win_part.o, win_part.lse, ot, out, lse_out,
                                      stream)


# Workgroups of the matrix-core decode kernel resident at once on the 256
# compute units: every instance runs two waves per SIMD (eight per CU), in
# workgroups of two waves at head_dim 256 and of four otherwise.
def resident_workgroups(D: int, cus: int = 256) -> int:
    return cus * (4 if D == 256 else 2)


def mixed_splits(tail_len: int, win_len: int, tail_row_bytes: int, win_row_bytes: int, B: int,
                 Hkv: int, D: int, granule: int = _lib.SPLIT_GRANULE) -> tuple[int, int]:
    """Split sizes (tail, window) for kvq_decode_attn_mixed: the resident
    workgroups are shared between the two regions so that one round of
    workgroups covers both, and the split whose workgroup reads the most bytes
    is as small as it can be.  Row bytes are the K plus V bytes of one row of
    one KV head (codes and scales)."""
    def cdiv(a, b):
        return -(-a // b)

    units = max(2, resident_workgroups(D) // max(1, B * Hkv))
    best = None
    for n_w in range(1, units):
        n_t = units - n_w
        st = cdiv(cdiv(max(1, tail_len), n_t), granule) * granule
        sw = cdiv(cdiv(max(1, win_len), n_w), granule) * granule
        cost = (max(st * tail_row_bytes, sw * win_row_bytes), cdiv(tail_len, st) + cdiv(win_len, sw))
        if best is None or cost < best[0]:
            best = (cost, st, sw)
    return best[1], best[2]


def combine_regions(parts, seq_lens, out: torch.Tensor, lse_out=None, stream=None):
    """kvq_combine_regions over the Partials of several regions (one seq_lens
    tensor per region) into ``out`` (B, Hq, D) fp16 or fp32."""
    B, Hq, D = out.shape
    ot = "f16" if out.dtype == torch.float16 else "f32"
    return _lib.kvq_combine_regions([p.o for p in parts], [p.lse for p in parts], list(seq_lens),
                                    [p.split_tokens for p in parts], [p.max_splits for p in parts],
                                    B, Hq, D, ot, out, lse_out, stream)


def decode_multi(kc: CachePlanes, vc: CachePlanes, q: torch.Tensor, seq_lens: torch.Tensor,
                 max_seq_len: int, part: "Partials", softmax_scale: float, stream=None):
    """kvq_decode_attn_multi: q (B, n_q, Hq, D) fp16; ``part`` built for n_q * Hq
    heads."""
    B, n_q, Hq, D = q.shape
    return _lib.kvq_decode_attn_multi(kc.desc(), vc.desc(), q, seq_lens, B, n_q, Hq, kc.Hkv, D,
                                      softmax_scale, max_seq_len, part.split_tokens,
                                      part.max_splits, part.o, part.lse, stream)


def decode_step_multi(kc: CachePlanes, vc: CachePlanes, k_new: torch.Tensor, v_new: torch.Tensor,
                      q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, part: "Partials",
                      softmax_scale: float, out: torch.Tensor, lse_out=None, stream=None):
    """kvq_decode_step_multi: k_new, v_new (B, n_q, Hkv, D) fp16 written at rows
    seq_lens[b] - n_q .., then kvq_decode_attn_multi and the merge into ``out``
    (B, n_q * Hq, D); ``part`` built for n_q * Hq heads."""
    B, n_q, Hq, D = q.shape
    ot = "f16" if out.dtype == torch.float16 else "f32"
    return _lib.kvq_decode_step_multi(kc.desc(), vc.desc(), k_new, v_new, q, seq_lens, B, n_q, Hq, kc.Hkv, D,
                                      softmax_scale, max_seq_len, part.split_tokens, part.max_splits,
                                      part.o, part.lse, ot, out, lse_out, stream)


def decode(kc: CachePlanes, vc: CachePlanes, q: torch.Tensor, seq_lens: torch.Tensor,
           max_seq_len: int, part: Partials, softmax_scale: float, variant="auto", stream=None):
    """kvq_decode_attn_variant on torch tensors: q (B, Hq, D) fp16."""
    B, Hq, D = q.shape
    return _lib.kvq_decode_attn_variant(kc.desc(), vc.desc(), q, seq_lens, B, Hq, kc.Hkv, D,
                                        softmax_scale, max_seq_len, part.split_tokens,
                                        part.max_splits, part.o, part.lse, variant, stream)


def combine(part: Partials, seq_lens: torch.Tensor, out: torch.Tensor, lse_out=None, stream=None):
    """kvq_combine into ``out`` (B, Hq, D) fp16 or fp32."""
    B, Hq, D = out.shape
    ot = "f16" if out.dtype == torch.float16 else "f32"
    return _lib.kvq_combine(part.o, part.lse, seq_lens, B, Hq, D, part.split_tokens,
                            part.max_splits, ot, out, lse_out, stream)


def decode_step(kc: CachePlanes, vc: CachePlanes, k_new: torch.Tensor, v_new: torch.Tensor,
                q: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, part: Partials,
                softmax_scale: float, out: torch.Tensor, lse_out=None, stream=None):
    """kvq_decode_step: k_new, v_new (B, Hkv, D) fp16 written at row seq_lens[b] - 1,
    then attention over rows [0, seq_lens[b]) into ``out`` (B, Hq, D)."""
    B, Hq, D = q.shape
    ot = "f16" if out.dtype == torch.float16 else "f32"
    return _lib.kvq_decode_step(kc.desc(), vc.desc(), k_new, v_new, q, seq_lens, B, Hq, kc.Hkv, D,
                                softmax_scale, max_seq_len, part.split_tokens, part.max_splits,
                                part.o, part.lse, ot, out, lse_out, stream)
