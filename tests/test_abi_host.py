"""The C-ABI library on the host, no GPU: it builds, loads, exports every entry
point include/kvq.h declares, reproduces the pages' byte counts, and rejects
every invalid argument with the documented status before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

from quantised_kv_long_amd import _lib  # noqa: E402
from quantised_kv_long_amd import build as B  # noqa: E402

from .test_page_sizes import ROWS, UNIT  # noqa: E402


@pytest.fixture(scope="module")
def lib():
    srcs = B.sources()
    if not os.path.exists(B.LIB) or os.path.getmtime(B.LIB) < max(os.path.getmtime(s) for s in srcs):
        B.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("kvq_quantize_append", "kvq_decode_attn", "kvq_combine", "kvq_decode_attn_variant",
              "kvq_decode_step", "kvq_quantize_rows", "kvq_combine_regions", "kvq_decode_attn_multi",
              "kvq_decode_attn_mixed", "kvq_decode_step_mixed", "kvq_decode_step_multi",
              "kvq_select_kv_tier", "kvq_tier_cache_bytes", "kvq_tier_types", "kvq_data_row_bytes",
              "kvq_scale_row_bytes", "kvq_status_string", "kvq_decode_step_noalloc",
              "kvq_decode_step_noalloc_bytes"):
        assert n in names


def test_every_declared_function_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in kvq.h but not exported"


def test_status_strings(lib):
    for code in range(-7, 1):
        assert _lib.kvq_status_string(code) != "unknown status"
    assert _lib.kvq_status_string(5) == "unknown status"


def test_row_bytes(lib):
    for D in (32, 64, 128, 256, 512):
        assert _lib.kvq_data_row_bytes("f16", D) == 2 * D
        assert _lib.kvq_data_row_bytes("q8_0", D) == D
        assert _lib.kvq_data_row_bytes("q4_0", D) == D // 2
        assert _lib.kvq_scale_row_bytes("f16", D) == 0
        assert _lib.kvq_scale_row_bytes("q8_0", D) == D // 16
        assert _lib.kvq_scale_row_bytes("q4_0", D) == D // 16
        assert _lib.kvq_data_row_bytes("q4_1", D) == D // 2
        assert _lib.kvq_data_row_bytes("q5_0", D) == _lib.kvq_data_row_bytes("q5_1", D) == 5 * D // 8
        assert _lib.kvq_data_row_bytes("q6_0", D) == 3 * D // 4
        assert _lib.kvq_scale_row_bytes("q5_0", D) == _lib.kvq_scale_row_bytes("q6_0", D) == D // 16
        assert _lib.kvq_scale_row_bytes("q4_1", D) == _lib.kvq_scale_row_bytes("q5_1", D) == D // 8
    assert _lib.kvq_data_row_bytes("q8_0", 48) == 0
    assert _lib.kvq_data_row_bytes(3, 128) == 0
    assert _lib.kvq_data_row_bytes(8, 128) == 0


def test_row_bytes_agree_with_the_oracle():
    from oracle import oracle as O
    for t in ("f16", "q8_0", "q4_0", "q4_1", "q5_0", "q5_1", "q6_0"):
        for D in (32, 128, 512):
            assert _lib.kvq_data_row_bytes(t, D) == O.data_row_bytes(t, D)
            assert _lib.kvq_scale_row_bytes(t, D) == O.scale_row_bytes(t, D)


@pytest.mark.parametrize("layers,heads,D,tK,tV,tokens,value,unit,cite", ROWS,
                         ids=[f"{r[3]}-{r[4]}-{r[5]}-{r[2]}" for r in ROWS])
def test_library_sizes_reproduce_page_figures(lib, layers, heads, D, tK, tV, tokens, value, unit,
                                              cite):
    per_row = lambda t: _lib.kvq_data_row_bytes(t, D) + _lib.kvq_scale_row_bytes(t, D)
    total = layers * heads * tokens * (per_row(tK) + per_row(tV))
    assert total / UNIT[unit] == pytest.approx(value, rel=1e-12), cite


# ------------------------------------------------------------- validation
# Fake, well-aligned device addresses: every call below must fail validation,
# which happens before any HIP call.  The fake addresses are never dereferenced;
# to stay safe even if validation had a bug, these tests run only where no GPU
# is visible.

def _no_gpu():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


nogpu = pytest.mark.skipif(not _no_gpu(), reason="fake-pointer validation tests run only without a GPU")
A = 0x10000  # aligned fake address


def plane(t=2, cap=100, data=A, scales=A + 0x100000, seq=800, head=100):
    return _lib.kvq_plane_desc(t, cap, data, scales, seq, head)


def append(lib, k=None, v=None, kn=A, vn=A, pos=A, B=2, n=1, H=8, D=128, max_end=100):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    kp = ctypes.byref(k) if k is not False else None
    vp = ctypes.byref(v) if v is not False else None
    return lib.kvq_quantize_append(kp, vp, kn, vn, pos, B, n, H, D, max_end, None)


@nogpu
def test_append_validation(lib):
    assert append(lib, kn=None) == -1
    assert append(lib, pos=None) == -1
    assert append(lib, k=False) == -1
    assert append(lib, k=plane(t=2, scales=None)) == -1        # quant type needs a scale plane
    assert append(lib, k=plane(data=None)) == -1
    assert append(lib, B=-1) == -2
    assert append(lib, n=-1) == -2
    assert append(lib, H=0) == -2
    assert append(lib, D=48) == -2
    assert append(lib, D=544) == -2
    assert append(lib, D=0) == -2
    assert append(lib, k=plane(t=3)) == -3
    assert append(lib, v=plane(t=-1)) == -3
    assert append(lib, k=plane(data=A + 8)) == -4
    assert append(lib, v=plane(scales=A + 2)) == -4
    # 4-byte aligned scales pass the alignment check (which comes before the
    # capacity check): the call fails on the capacity instead
    assert append(lib, v=plane(scales=A + 4), max_end=101) == -5
    assert append(lib, kn=A + 2) == -4
    assert append(lib, pos=A + 2) == -4
    assert append(lib, max_end=101) == -5
    assert append(lib, v=plane(cap=50), max_end=60) == -5
    assert append(lib, k=plane(seq=0)) == -2                   # B > 1 with a zero sequence stride
    assert append(lib, k=plane(head=0)) == -2
    assert append(lib, max_end=0, n=1) == -2                    # max_end < n_new
    # nothing to do: returns OK without touching the device
    assert append(lib, B=0) == 0
    assert append(lib, n=0, max_end=0) == 0
    assert append(lib, B=0, kn=None, vn=None, pos=None, k=False, v=False) == 0


def decode(lib, k=None, v=None, q=A, lens=A, B=1, Hq=40, Hkv=8, D=128, scale=0.088, max_len=100,
           split=64, max_splits=2, po=A, pl=A, variant=None):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    args = (ctypes.byref(k), ctypes.byref(v), q, lens, B, Hq, Hkv, D, scale, max_len, split,
            max_splits, po, pl)
    if variant is None:
        return lib.kvq_decode_attn(*args, None)
    return lib.kvq_decode_attn_variant(*args, variant, None)


@nogpu
def test_decode_validation(lib):
    assert decode(lib, q=None) == -1
    assert decode(lib, lens=None) == -1
    assert decode(lib, po=None) == -1
    assert decode(lib, pl=None) == -1
    assert decode(lib, k=plane(scales=None)) == -1
    assert decode(lib, Hq=41) == -2                             # Hq % Hkv != 0
    assert decode(lib, Hq=8 * 17) == -2                         # group of 17 > 16
    assert decode(lib, B=0) == -2
    assert decode(lib, D=96 + 8) == -2
    assert decode(lib, D=1024) == -2
    assert decode(lib, scale=float("nan")) == -2
    assert decode(lib, max_len=0) == -2
    assert decode(lib, k=plane(t=8)) == -3
    assert decode(lib, k=plane(t=3)) == -3                      # 3 names fp32 output, not a storage type
    assert decode(lib, variant=3) == -3
    assert decode(lib, q=A + 4) == -4
    assert decode(lib, po=A + 4) == -4
    assert decode(lib, max_len=101) == -5
    assert decode(lib, v=plane(cap=99)) == -5
    assert decode(lib, split=100) == -6                         # not a multiple of 64
    assert decode(lib, split=0) == -6
    assert decode(lib, max_splits=1) == -6                      # 1 * 64 < 100
    assert decode(lib, max_splits=0) == -6


def combine(lib, po=A, pl=A, lens=A, B=1, Hq=40, D=128, split=64, max_splits=4, ot=3, out=A,
            lse=None):
    return lib.kvq_combine(po, pl, lens, B, Hq, D, split, max_splits, ot, out, lse, None)


@nogpu
def test_combine_validation(lib):
    assert combine(lib, po=None) == -1
    assert combine(lib, out=None) == -1
    assert combine(lib, lens=None) == -1
    assert combine(lib, ot=1) == -3
    assert combine(lib, ot=2) == -3
    assert combine(lib, B=0) == -2
    assert combine(lib, D=40) == -2
    assert combine(lib, split=32) == -6
    assert combine(lib, max_splits=0) == -6
    assert combine(lib, po=A + 8) == -4
    assert combine(lib, out=A + 1, ot=0) == -4
    assert combine(lib, out=A + 8, ot=3) == -4
    assert combine(lib, lse=A + 2) == -4


def step(lib, k=None, v=None, kn=A, vn=A, q=A, lens=A, B=1, Hq=40, Hkv=8, D=128, scale=0.088,
         max_len=100, split=64, max_splits=2, po=A, pl=A, ot=0, out=A, lse=None):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    return lib.kvq_decode_step(ctypes.byref(k), ctypes.byref(v), kn, vn, q, lens, B, Hq, Hkv, D,
                               scale, max_len, split, max_splits, po, pl, ot, out, lse, None)


@nogpu
def test_decode_step_validation(lib):
    # the decode arguments are checked exactly as kvq_decode_attn checks them
    assert step(lib, q=None) == -1
    assert step(lib, po=None) == -1
    assert step(lib, Hq=41) == -2
    assert step(lib, D=1024) == -2
    assert step(lib, k=plane(t=8)) == -3
    assert step(lib, max_len=101) == -5
    assert step(lib, split=100) == -6
    # and the step's own arguments
    assert step(lib, kn=None) == -1
    assert step(lib, vn=None) == -1
    assert step(lib, out=None) == -1
    assert step(lib, ot=1) == -3
    assert step(lib, ot=2) == -3
    assert step(lib, kn=A + 2) == -4
    assert step(lib, vn=A + 8) == -4
    assert step(lib, out=A + 8) == -4
    assert step(lib, lse=A + 2) == -4


def step_noalloc(lib, k=None, v=None, kn=A, vn=A, q=A, lens=A, B=1, Hq=40, Hkv=8, D=128, scale=0.088,
                 max_len=100, split=64, ot=0, out=A, lse=None):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    return lib.kvq_decode_step_noalloc(ctypes.byref(k), ctypes.byref(v), kn, vn, q, lens, B, Hq, Hkv, D,
                                       scale, max_len, split, ot, out, lse, None)


def test_noalloc_scratch_bytes(lib):
    """The partials a no-allocation step needs: B*Hq*S*D fp32 rows (rounded up
    to 256 bytes) then B*Hq*S fp32 LSEs, S = ceil(max_seq_len / split_tokens)."""
    assert _lib.kvq_decode_step_noalloc_bytes(1, 40, 128, 65536, 1024) == 40 * 64 * 128 * 4 + 40 * 64 * 4
    assert _lib.kvq_decode_step_noalloc_bytes(2, 5, 32, 65, 64) == 2 * 5 * 2 * 32 * 4 + 2 * 5 * 2 * 4
    assert _lib.kvq_decode_step_noalloc_bytes(1, 3, 32, 1, 64) == 512 + 12
    assert _lib.kvq_decode_step_noalloc_bytes(0, 3, 32, 1, 64) == 0


@nogpu
def test_decode_step_noalloc_validation(lib):
    """Every status of kvq_decode_step, and KVQ_ERR_CAPACITY for partials beyond
    the library's array, all before any HIP call."""
    assert step_noalloc(lib, q=None) == -1
    assert step_noalloc(lib, kn=None) == -1
    assert step_noalloc(lib, out=None) == -1
    assert step_noalloc(lib, Hq=41) == -2
    assert step_noalloc(lib, D=1024) == -2
    assert step_noalloc(lib, B=0) == -2
    assert step_noalloc(lib, k=plane(t=8)) == -3
    assert step_noalloc(lib, ot=1) == -3
    assert step_noalloc(lib, kn=A + 2) == -4
    assert step_noalloc(lib, max_len=101) == -5
    assert step_noalloc(lib, split=100) == -6
    assert step_noalloc(lib, split=32) == -6
    # 40 heads x 4097 splits x 129 floats is beyond 64 MiB
    big = plane(cap=1 << 25, seq=8 << 25, head=1 << 25)
    assert _lib.kvq_decode_step_noalloc_bytes(1, 40, 128, 4096 * 4097, 4096) > 64 << 20
    assert step_noalloc(lib, k=big, v=big, max_len=4096 * 4097, split=4096) == -5
    # more splits than the partials' index allows
    assert step_noalloc(lib, k=big, v=big, max_len=64 * 65536, split=64) == -6


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    """The product path has no fallback: a missing library raises."""
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.KVQLibraryMissing):
        _lib.load(str(tmp_path / "libkvq.so"))


def qrows(lib, k=None, v=None, ks=None, vs=None, counts=A, pos=A, B=2, max_rows=16, H=8, D=128,
          max_end=100):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    ks = ks if ks is not None else plane(t=0, cap=16)
    vs = vs if vs is not None else plane(t=0, cap=16)
    return lib.kvq_quantize_rows(ctypes.byref(k), ctypes.byref(v), ctypes.byref(ks), ctypes.byref(vs),
                                 counts, pos, B, max_rows, H, D, max_end, None)


@nogpu
def test_quantize_rows_validation(lib):
    assert qrows(lib, B=0) == 0 and qrows(lib, max_rows=0) == 0      # nothing to do
    assert qrows(lib, B=-1) == -2
    assert qrows(lib, D=48) == -2
    assert qrows(lib, counts=None) == -1
    assert qrows(lib, pos=None) == -1
    assert qrows(lib, ks=plane(t=1, cap=16)) == -3                  # sources are fp16
    assert qrows(lib, vs=plane(t=2, cap=16)) == -3
    assert qrows(lib, ks=plane(t=0, cap=8)) == -5                   # max_rows beyond the source
    assert qrows(lib, max_end=101) == -5
    assert qrows(lib, counts=A + 2) == -4
    assert qrows(lib, ks=plane(t=0, cap=16, data=A + 8)) == -4


def cregions(lib, n=2, po=(A, A), pl=(A, A), lens=(A, A), split=(64, 64), ms=(4, 4), B=1, Hq=40,
             D=128, ot=3, out=A, lse=None):
    P = ctypes.c_void_p
    k = max(n, 1)
    arr = lambda xs: (P * k)(*(list(xs) + [None] * k)[:k])
    ints = lambda xs: (ctypes.c_int * k)(*(list(xs) + [0] * k)[:k])
    return lib.kvq_combine_regions(n, arr(po), arr(pl), arr(lens), ints(split), ints(ms), B, Hq, D, ot,
                                   out, lse, None)


@nogpu
def test_combine_regions_validation(lib):
    assert cregions(lib, n=0) == -2
    assert cregions(lib, n=5, po=[A] * 5, pl=[A] * 5, lens=[A] * 5, split=[64] * 5, ms=[4] * 5) == -2
    assert cregions(lib, po=(A, None)) == -1
    assert cregions(lib, lens=(None, A)) == -1
    assert cregions(lib, out=None) == -1
    assert cregions(lib, ot=1) == -3
    assert cregions(lib, D=40) == -2
    assert cregions(lib, split=(64, 32)) == -6
    assert cregions(lib, ms=(0, 4)) == -6
    assert cregions(lib, po=(A, A + 8)) == -4
    assert cregions(lib, out=A + 8, ot=3) == -4


def multi(lib, k=None, v=None, q=A, lens=A, B=1, nq=3, Hq=40, Hkv=8, D=128, scale=0.088, max_len=100,
          split=64, max_splits=2, po=A, pl=A):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    return lib.kvq_decode_attn_multi(ctypes.byref(k), ctypes.byref(v), q, lens, B, nq, Hq, Hkv, D, scale,
                                     max_len, split, max_splits, po, pl, None)


@nogpu
def test_decode_multi_validation(lib):
    assert multi(lib, q=None) == -1                 # the decode checks come first
    assert multi(lib, Hq=41) == -2
    assert multi(lib, split=100) == -6
    assert multi(lib, nq=0) == -2
    assert multi(lib, nq=4) == -2                   # 4 tokens x 5 heads = 20 columns
    assert multi(lib, nq=3, max_len=2, max_splits=1) == -2   # fewer rows than query tokens
    assert multi(lib, D=64, nq=1) == -2             # the matrix-core kernel covers D 128/256/512


def mixed(lib, kt=None, vt=None, kw=None, vw=None, q=A, tl=A, wl=A, B=1, Hq=40, Hkv=8, D=128,
          scale=0.088, tmax=100, tsplit=64, tms=2, tpo=A, tpl=A, wmax=100, wsplit=64, wms=2, wpo=A,
          wpl=A):
    kt = kt if kt is not None else plane()
    vt = vt if vt is not None else plane()
    kw = kw if kw is not None else plane(t=0)
    vw = vw if vw is not None else plane(t=0)
    return lib.kvq_decode_attn_mixed(ctypes.byref(kt), ctypes.byref(vt), ctypes.byref(kw), ctypes.byref(vw),
                                     q, tl, wl, B, Hq, Hkv, D, scale, tmax, tsplit, tms, tpo, tpl, wmax,
                                     wsplit, wms, wpo, wpl, None)


@nogpu
def test_decode_mixed_validation(lib):
    # each region takes the decode checks; the window must be fp16 in K and V
    assert mixed(lib, q=None) == -1
    assert mixed(lib, tl=None) == -1
    assert mixed(lib, wl=None) == -1
    assert mixed(lib, wpo=None) == -1
    assert mixed(lib, Hq=41) == -2
    assert mixed(lib, kw=plane(t=1)) == -3
    assert mixed(lib, vw=plane(t=2)) == -3
    assert mixed(lib, kw=plane(t=7)) == -3
    assert mixed(lib, tpl=A + 2) == -4
    assert mixed(lib, wmax=101) == -5
    assert mixed(lib, tsplit=100) == -6
    assert mixed(lib, wms=1) == -6


def step_mixed(lib, kt=None, vt=None, kw=None, vw=None, kn=A, vn=A, q=A, tl=A, wl=A, B=1, Hq=40, Hkv=8,
               D=128, scale=0.088, tmax=100, tsplit=64, tms=2, tpo=A, tpl=A, wmax=100, wsplit=64, wms=2,
               wpo=A, wpl=A, ot=0, out=A, lse=None):
    kt = kt if kt is not None else plane()
    vt = vt if vt is not None else plane()
    kw = kw if kw is not None else plane(t=0)
    vw = vw if vw is not None else plane(t=0)
    return lib.kvq_decode_step_mixed(ctypes.byref(kt), ctypes.byref(vt), ctypes.byref(kw), ctypes.byref(vw),
                                     kn, vn, q, tl, wl, B, Hq, Hkv, D, scale, tmax, tsplit, tms, tpo, tpl,
                                     wmax, wsplit, wms, wpo, wpl, ot, out, lse, None)


@nogpu
def test_decode_step_mixed_validation(lib):
    assert step_mixed(lib, q=None) == -1
    assert step_mixed(lib, kn=None) == -1
    assert step_mixed(lib, out=None) == -1
    assert step_mixed(lib, Hq=41) == -2
    assert step_mixed(lib, kw=plane(t=2)) == -3
    assert step_mixed(lib, ot=1) == -3
    assert step_mixed(lib, vn=A + 2) == -4
    assert step_mixed(lib, out=A + 4) == -4
    assert step_mixed(lib, lse=A + 2) == -4
    assert step_mixed(lib, wmax=101) == -5
    assert step_mixed(lib, tms=1) == -6


def step_multi(lib, k=None, v=None, kn=A, vn=A, q=A, lens=A, B=1, nq=3, Hq=40, Hkv=8, D=128, scale=0.088,
               max_len=100, split=64, max_splits=2, po=A, pl=A, ot=0, out=A, lse=None):
    k = k if k is not None else plane()
    v = v if v is not None else plane()
    return lib.kvq_decode_step_multi(ctypes.byref(k), ctypes.byref(v), kn, vn, q, lens, B, nq, Hq, Hkv, D,
                                     scale, max_len, split, max_splits, po, pl, ot, out, lse, None)


@nogpu
def test_decode_step_multi_validation(lib):
    assert step_multi(lib, q=None) == -1            # the decode checks come first
    assert step_multi(lib, Hq=41) == -2
    assert step_multi(lib, split=100) == -6
    assert step_multi(lib, nq=0) == -2
    assert step_multi(lib, nq=4) == -2              # 4 tokens x 5 heads = 20 columns
    assert step_multi(lib, nq=3, max_len=2, max_splits=1) == -2
    assert step_multi(lib, kn=None) == -1
    assert step_multi(lib, out=None) == -1
    assert step_multi(lib, ot=2) == -3
    assert step_multi(lib, vn=A + 2) == -4
    assert step_multi(lib, lse=A + 1) == -4
    assert step_multi(lib, D=64, nq=1) == -2        # the matrix-core kernel covers D 128/256/512
