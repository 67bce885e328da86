"""ctypes binding of the C ABI in include/kvq.h (argument marshalling only).

Every function here has the name of the C entry point it calls and does
nothing but check and convert arguments: torch tensors become device pointers,
``stream=None`` becomes torch's current HIP stream.  All computation happens in
the HIP kernels of ``libkvq.so``.  If the library is missing, every call raises
``KVQLibraryMissing``; there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkvq.so")

F16, Q8_0, Q4_0 = 0, 1, 2
OUT_F32 = 3
Q4_1, Q5_0, Q5_1, Q6_0 = 4, 5, 6, 7
TYPES = {"f16": F16, "q8_0": Q8_0, "q4_0": Q4_0, "q4_1": Q4_1, "q5_0": Q5_0, "q5_1": Q5_1, "q6_0": Q6_0}
VARIANT_AUTO, VARIANT_VALU, VARIANT_MFMA = 0, 1, 2
VARIANTS = {"auto": VARIANT_AUTO, "valu": VARIANT_VALU, "mfma": VARIANT_MFMA}
SPLIT_GRANULE = 64
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_NULL", -2: "KVQ_ERR_SHAPE", -3: "KVQ_ERR_TYPE",
          -4: "KVQ_ERR_ALIGN", -5: "KVQ_ERR_CAPACITY", -6: "KVQ_ERR_SPLITS", -7: "KVQ_ERR_LAUNCH"}


class KVQLibraryMissing(RuntimeError):
    pass


class KVQError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {message}")
        self.status = status


class kvq_plane_desc(ctypes.Structure):
    _fields_ = [
        ("type", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("data", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
        ("seq_stride_rows", ctypes.c_int64),
        ("head_stride_rows", ctypes.c_int64),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libkvq.so (built by ``quantised_kv_long_amd.build``)."""
    global _lib
    if _lib is not None:
        return _lib
    # Bind to the HIP runtime torch has loaded (one runtime per process: the
    # library's libamdhip64.so.7 dependency resolves to the copy already loaded),
    # so torch's streams and events are valid handles for the library.
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise KVQLibraryMissing(
            f"{path} is not built; run `python -m quantised_kv_long_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, i32, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    DP = ctypes.POINTER(kvq_plane_desc)
    lib.kvq_data_row_bytes.argtypes = [i32, i32]
    lib.kvq_data_row_bytes.restype = ctypes.c_size_t
    lib.kvq_scale_row_bytes.argtypes = [i32, i32]
    lib.kvq_scale_row_bytes.restype = ctypes.c_size_t
    i64 = ctypes.c_int64
    lib.kvq_tier_cache_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.kvq_tier_cache_bytes.restype = i64
    lib.kvq_select_kv_tier.argtypes = [i64, i32, i32, i32, i64, i64, i64, ctypes.POINTER(i64),
                                       ctypes.POINTER(i64)]
    lib.kvq_select_kv_tier.restype = i32
    lib.kvq_tier_types.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.kvq_tier_types.restype = i32
    lib.kvq_status_string.argtypes = [i32]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_quantize_append.argtypes = [DP, DP, P, P, P, i32, i32, i32, i32, i32, P]
    lib.kvq_quantize_append.restype = i32
    lib.kvq_quantize_rows.argtypes = [DP, DP, DP, DP, P, P, i32, i32, i32, i32, i32, P]
    lib.kvq_quantize_rows.restype = i32
    lib.kvq_combine_regions.argtypes = [i32, ctypes.POINTER(P), ctypes.POINTER(P), ctypes.POINTER(P),
                                        ctypes.POINTER(i32), ctypes.POINTER(i32), i32, i32, i32, i32,
                                        P, P, P]
    lib.kvq_combine_regions.restype = i32
    lib.kvq_decode_attn_mixed.argtypes = [DP, DP, DP, DP, P, P, P, i32, i32, i32, i32, f32, i32, i32,
                                          i32, P, P, i32, i32, i32, P, P, P]
    lib.kvq_decode_attn_mixed.restype = i32
    lib.kvq_decode_step_mixed.argtypes = [DP, DP, DP, DP, P, P, P, P, P, i32, i32, i32, i32, f32, i32,
                                          i32, i32, P, P, i32, i32, i32, P, P, i32, P, P, P]
    lib.kvq_decode_step_mixed.restype = i32
    lib.kvq_decode_step_multi.argtypes = [DP, DP, P, P, P, P, i32, i32, i32, i32, i32, f32, i32, i32, i32,
                                          P, P, i32, P, P, P]
    lib.kvq_decode_step_multi.restype = i32
    lib.kvq_decode_attn_multi.argtypes = [DP, DP, P, P, i32, i32, i32, i32, i32, f32, i32, i32, i32,
                                          P, P, P]
    lib.kvq_decode_attn_multi.restype = i32
    lib.kvq_decode_attn.argtypes = [DP, DP, P, P, i32, i32, i32, i32, f32, i32, i32, i32, P, P, P]
    lib.kvq_decode_attn.restype = i32
    lib.kvq_decode_attn_variant.argtypes = [DP, DP, P, P, i32, i32, i32, i32, f32, i32, i32, i32,
                                            P, P, i32, P]
    lib.kvq_decode_attn_variant.restype = i32
    lib.kvq_combine.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, P, P, P]
    lib.kvq_combine.restype = i32
    lib.kvq_decode_step.argtypes = [DP, DP, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, i32, P, P,
                                    i32, P, P, P]
    lib.kvq_decode_step.restype = i32
    lib.kvq_decode_step_noalloc_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.kvq_decode_step_noalloc_bytes.restype = ctypes.c_size_t
    lib.kvq_decode_step_noalloc.argtypes = [DP, DP, P, P, P, P, i32, i32, i32, i32, f32, i32, i32, i32, P, P,
                                            P]
    lib.kvq_decode_step_noalloc.restype = i32
    _lib = lib
    return lib


def _check(fn: str, rc: int) -> int:
    if rc != 0:
        raise KVQError(fn, rc, load().kvq_status_string(rc).decode())
    return rc


def _ptr(x) -> int | None:
    """A torch tensor (must be on a GPU and contiguous), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("expected a device tensor")
    if not x.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return x.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _tcode(t) -> int:
    return TYPES[t] if isinstance(t, str) else int(t)


def kvq_data_row_bytes(t, head_dim: int) -> int:
    return int(load().kvq_data_row_bytes(_tcode(t), head_dim))


def kvq_scale_row_bytes(t, head_dim: int) -> int:
    return int(load().kvq_scale_row_bytes(_tcode(t), head_dim))


TIERS = {0: ("f16", "f16"), 1: ("q8_0", "q8_0"), 2: ("q8_0", "q4_0"), 3: ("q5_1", "q4_0")}


def kvq_tier_cache_bytes(tier: int, n_ctx: int, n_layers: int, Hkv: int, D: int) -> int:
    return int(load().kvq_tier_cache_bytes(tier, n_ctx, n_layers, Hkv, D))


def kvq_select_kv_tier(n_ctx: int, n_layers: int, Hkv: int, D: int, free_bytes: int,
                       resident_bytes: int, vram_target_bytes: int = 0):
    """Returns (tier, budget bytes, cache bytes of the tier)."""
    budget, cache = ctypes.c_int64(), ctypes.c_int64()
    rc = load().kvq_select_kv_tier(n_ctx, n_layers, Hkv, D, free_bytes, resident_bytes,
                                   vram_target_bytes, ctypes.byref(budget), ctypes.byref(cache))
    if rc < 0:
        _check("kvq_select_kv_tier", rc)
    return rc, budget.value, cache.value


def kvq_tier_types(tier: int):
    tk, tv = ctypes.c_int(), ctypes.c_int()
    _check("kvq_tier_types", load().kvq_tier_types(tier, ctypes.byref(tk), ctypes.byref(tv)))
    return tk.value, tv.value


def kvq_status_string(status: int) -> str:
    return load().kvq_status_string(status).decode()


def kvq_quantize_append(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, k_new, v_new, positions,
                        B: int, n_new: int, Hkv: int, D: int, max_end: int, stream=None) -> int:
    rc = load().kvq_quantize_append(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(k_new),
                                    _ptr(v_new), _ptr(positions), B, n_new, Hkv, D, max_end,
                                    _stream(stream))
    return _check("kvq_quantize_append", rc)


def kvq_quantize_rows(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, k_src: kvq_plane_desc,
                      v_src: kvq_plane_desc, counts, positions, B: int, max_rows: int, Hkv: int, D: int,
                      max_end: int, stream=None) -> int:
    rc = load().kvq_quantize_rows(ctypes.byref(k_cache), ctypes.byref(v_cache), ctypes.byref(k_src),
                                  ctypes.byref(v_src), _ptr(counts), _ptr(positions), B, max_rows, Hkv,
                                  D, max_end, _stream(stream))
    return _check("kvq_quantize_rows", rc)


def kvq_decode_attn(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, q, seq_lens, B: int, Hq: int,
                    Hkv: int, D: int, softmax_scale: float, max_seq_len: int, split_tokens: int,
                    max_splits: int, part_o, part_lse, stream=None) -> int:
    rc = load().kvq_decode_attn(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(q),
                                _ptr(seq_lens), B, Hq, Hkv, D, float(softmax_scale), max_seq_len,
                                split_tokens, max_splits, _ptr(part_o), _ptr(part_lse),
                                _stream(stream))
    return _check("kvq_decode_attn", rc)


def kvq_decode_attn_mixed(k_tail: kvq_plane_desc, v_tail: kvq_plane_desc, k_win: kvq_plane_desc,
                          v_win: kvq_plane_desc, q, tail_lens, win_lens, B: int, Hq: int, Hkv: int,
                          D: int, softmax_scale: float, tail_max_len: int, tail_split_tokens: int,
                          tail_max_splits: int, tail_part_o, tail_part_lse, win_max_len: int,
                          win_split_tokens: int, win_max_splits: int, win_part_o, win_part_lse,
                          stream=None) -> int:
    rc = load().kvq_decode_attn_mixed(ctypes.byref(k_tail), ctypes.byref(v_tail), ctypes.byref(k_win),
                                      ctypes.byref(v_win), _ptr(q), _ptr(tail_lens), _ptr(win_lens), B,
                                      Hq, Hkv, D, float(softmax_scale), tail_max_len, tail_split_tokens,
                                      tail_max_splits, _ptr(tail_part_o), _ptr(tail_part_lse),
                                      win_max_len, win_split_tokens, win_max_splits, _ptr(win_part_o),
                                      _ptr(win_part_lse), _stream(stream))
    return _check("kvq_decode_attn_mixed", rc)


def kvq_decode_step_mixed(k_tail: kvq_plane_desc, v_tail: kvq_plane_desc, k_win: kvq_plane_desc,
                          v_win: kvq_plane_desc, k_new, v_new, q, tail_lens, win_lens, B: int, Hq: int,
                          Hkv: int, D: int, softmax_scale: float, tail_max_len: int,
                          tail_split_tokens: int, tail_max_splits: int, tail_part_o, tail_part_lse,
                          win_max_len: int, win_split_tokens: int, win_max_splits: int, win_part_o,
                          win_part_lse, out_type, out, lse_out=None, stream=None) -> int:
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_decode_step_mixed(ctypes.byref(k_tail), ctypes.byref(v_tail), ctypes.byref(k_win),
                                      ctypes.byref(v_win), _ptr(k_new), _ptr(v_new), _ptr(q),
                                      _ptr(tail_lens), _ptr(win_lens), B, Hq, Hkv, D,
                                      float(softmax_scale), tail_max_len, tail_split_tokens,
                                      tail_max_splits, _ptr(tail_part_o), _ptr(tail_part_lse),
                                      win_max_len, win_split_tokens, win_max_splits, _ptr(win_part_o),
                                      _ptr(win_part_lse), ot, _ptr(out), _ptr(lse_out),
                                      _stream(stream))
    return _check("kvq_decode_step_mixed", rc)


def kvq_decode_step_multi(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, k_new, v_new, q, seq_lens,
                          B: int, n_q: int, Hq: int, Hkv: int, D: int, softmax_scale: float,
                          max_seq_len: int, split_tokens: int, max_splits: int, part_o, part_lse, out_type,
                          out, lse_out=None, stream=None) -> int:
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_decode_step_multi(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(k_new), _ptr(v_new),
                                      _ptr(q), _ptr(seq_lens), B, n_q, Hq, Hkv, D, float(softmax_scale),
                                      max_seq_len, split_tokens, max_splits, _ptr(part_o), _ptr(part_lse),
                                      ot, _ptr(out), _ptr(lse_out), _stream(stream))
    return _check("kvq_decode_step_multi", rc)


def kvq_decode_attn_multi(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, q, seq_lens, B: int,
                          n_q: int, Hq: int, Hkv: int, D: int, softmax_scale: float,
                          max_seq_len: int, split_tokens: int, max_splits: int, part_o, part_lse,
                          stream=None) -> int:
    rc = load().kvq_decode_attn_multi(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(q),
                                      _ptr(seq_lens), B, n_q, Hq, Hkv, D, float(softmax_scale),
                                      max_seq_len, split_tokens, max_splits, _ptr(part_o),
                                      _ptr(part_lse), _stream(stream))
    return _check("kvq_decode_attn_multi", rc)


def kvq_decode_attn_variant(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, q, seq_lens, B: int,
                            Hq: int, Hkv: int, D: int, softmax_scale: float, max_seq_len: int,
                            split_tokens: int, max_splits: int, part_o, part_lse, variant,
                            stream=None) -> int:
    v = VARIANTS[variant] if isinstance(variant, str) else int(variant)
    rc = load().kvq_decode_attn_variant(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(q),
                                        _ptr(seq_lens), B, Hq, Hkv, D, float(softmax_scale),
                                        max_seq_len, split_tokens, max_splits, _ptr(part_o),
                                        _ptr(part_lse), v, _stream(stream))
    return _check("kvq_decode_attn_variant", rc)


def kvq_combine(part_o, part_lse, seq_lens, B: int, Hq: int, D: int, split_tokens: int,
                max_splits: int, out_type, out, lse_out=None, stream=None) -> int:
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_combine(_ptr(part_o), _ptr(part_lse), _ptr(seq_lens), B, Hq, D, split_tokens,
                            max_splits, ot, _ptr(out), _ptr(lse_out), _stream(stream))
    return _check("kvq_combine", rc)


def kvq_combine_regions(part_o, part_lse, seq_lens, split_tokens, max_splits, B: int, Hq: int,
                        D: int, out_type, out, lse_out=None, stream=None) -> int:
    """Each of part_o, part_lse, seq_lens, split_tokens, max_splits is a list with
    one entry per region."""
    n = len(part_o)
    if not (len(part_lse) == len(seq_lens) == len(split_tokens) == len(max_splits) == n):
        raise ValueError("one entry per region in every list")
    P = ctypes.c_void_p
    arr = lambda xs: (P * max(n, 1))(*[_ptr(x) for x in xs])
    ints = lambda xs: (ctypes.c_int * max(n, 1))(*[int(x) for x in xs])
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_combine_regions(n, arr(part_o), arr(part_lse), arr(seq_lens), ints(split_tokens),
                                    ints(max_splits), B, Hq, D, ot, _ptr(out), _ptr(lse_out),
                                    _stream(stream))
    return _check("kvq_combine_regions", rc)


def kvq_decode_step(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, k_new, v_new, q, seq_lens,
                    B: int, Hq: int, Hkv: int, D: int, softmax_scale: float, max_seq_len: int,
                    split_tokens: int, max_splits: int, part_o, part_lse, out_type, out,
                    lse_out=None, stream=None) -> int:
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_decode_step(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(k_new),
                                _ptr(v_new), _ptr(q), _ptr(seq_lens), B, Hq, Hkv, D,
                                float(softmax_scale), max_seq_len, split_tokens, max_splits,
                                _ptr(part_o), _ptr(part_lse), ot, _ptr(out),
                                _ptr(lse_out), _stream(stream))
    return _check("kvq_decode_step", rc)


def kvq_decode_step_noalloc_bytes(B: int, Hq: int, D: int, max_seq_len: int, split_tokens: int) -> int:
    return int(load().kvq_decode_step_noalloc_bytes(B, Hq, D, max_seq_len, split_tokens))


def kvq_decode_step_noalloc(k_cache: kvq_plane_desc, v_cache: kvq_plane_desc, k_new, v_new, q, seq_lens,
                            B: int, Hq: int, Hkv: int, D: int, softmax_scale: float, max_seq_len: int,
                            split_tokens: int, out_type, out, lse_out=None, stream=None) -> int:
    ot = OUT_F32 if out_type in ("f32", OUT_F32) else _tcode(out_type)
    rc = load().kvq_decode_step_noalloc(ctypes.byref(k_cache), ctypes.byref(v_cache), _ptr(k_new),
                                        _ptr(v_new), _ptr(q), _ptr(seq_lens), B, Hq, Hkv, D,
                                        float(softmax_scale), max_seq_len, split_tokens, ot, _ptr(out),
                                        _ptr(lse_out), _stream(stream))
    return _check("kvq_decode_step_noalloc", rc)
