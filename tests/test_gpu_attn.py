"""K2 (kvq_decode_attn) + K3 (kvq_combine) on the GPU against the CPU oracle.

Small cases span several 64-row tiles, ragged tails and every K/V type pair;
the workloads at their full sizes run in the launch configuration the
benchmark times (same split_tokens), compared on every output (or on sampled
heads where the oracle would be slow)."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, assert_partials, fill_pair, gpu_row_scores, note, oracle_row_scores,
                       oracle_threads, planes_to_oracle, require_gpu, run_decode, to_host_u16)
from .test_oracle_attention import identity_values

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu
TYPES = ["f16", "q8_0", "q4_0"]
VARIANTS = ["valu", "mfma"]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def variant_ok(variant, D, G, tk, tv):
    """Whether the library runs `variant` for this shape (the MFMA kernel covers a
    subset of shapes; the dispatcher reports KVQ_ERR_SHAPE otherwise)."""
    from quantised_kv_long_amd import _lib
    if variant == "valu":
        return True
    try:
        B, Hkv = 1, 1
        kc = C.CachePlanes.alloc(tk, B, Hkv, 64, D)
        vc = C.CachePlanes.alloc(tv, B, Hkv, 64, D)
        q = torch.zeros((B, Hkv * G, D), dtype=torch.float16, device="cuda")
        lens = torch.ones(B, dtype=torch.int32, device="cuda")
        part = C.Partials(B, Hkv * G, D, 64, 64)
        C.decode(kc, vc, q, lens, 64, part, 1.0, variant)
        torch.cuda.synchronize()
        return True
    except _lib.KVQError as e:
        if e.status == -2:
            return False
        raise


def oracle_ref(kc, vc, q, lens, Hkv, scale=None):
    D = q.shape[-1]
    scale = scale if scale is not None else 1.0 / math.sqrt(D)
    return O.attend(to_host_u16(q), planes_to_oracle(kc), planes_to_oracle(vc), lens, Hkv, scale,
                    nthreads=oracle_threads())


SMALL = [
    # (B, Hkv, G, D, lens, split_tokens)
    (2, 2, 5, 128, [1000, 65], 256),
    (1, 2, 8, 256, [777], 128),
    (2, 1, 16, 64, [64, 63], 64),
    (1, 2, 1, 512, [300], 64),
    (3, 2, 4, 32, [1, 129, 200], 64),
    # head_dim 192: the vector-ALU kernel, and a merge in two 96-column chunks
    (1, 1, 3, 192, [500], 128),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("tk,tv", list(itertools.product(TYPES, TYPES)))
@pytest.mark.parametrize("case", range(len(SMALL)))
def test_small_cases_all_type_pairs(variant, tk, tv, case):
    B, Hkv, G, D, lens, st = SMALL[case]
    if not variant_ok(variant, D, G, tk, tv):
        pytest.skip(f"{variant} does not cover D={D} G={G}")
    note(f"decode {variant} {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} lens={lens} split={st}")
    dev = "cuda"
    cap = max(lens) + 17
    seed = 1000 + case
    k = synth.normal_f16((B, Hkv, cap, D), seed, dev)
    v = synth.normal_f16((B, Hkv, cap, D), seed + 1, dev)
    q = synth.normal_f16((B, Hkv * G, D), seed + 2, dev)
    kc, vc = fill_pair(tk, tv, k, v)
    out, lse, (po, pl) = run_decode(kc, vc, q, lens, st, variant)
    ref, ref_lse = oracle_ref(kc, vc, q, lens, Hkv)
    assert_close(out, lse, ref, ref_lse, f"{variant} {tk}/{tv} case {case}")
    # partials of every split against the oracle's split partials
    S = po.shape[2]
    ro, rl = O.attend_split(to_host_u16(q), planes_to_oracle(kc), planes_to_oracle(vc), lens, Hkv,
                            1 / math.sqrt(D), st, S)
    assert_partials(po, pl, ro, rl, lens, st)


@pytest.mark.parametrize("variant", VARIANTS)
def test_partials_past_max_seq_len_untouched(variant):
    """Partials sized for a capacity beyond max_seq_len: only the splits that
    hold a row of their sequence (s < ceil(L_b / split_tokens)) are written,
    and the merge, which reads only those, matches the oracle."""
    dev = "cuda"
    B, Hkv, G, D, st = 2, 2, 5, 128, 64
    lens, max_len, cap = [700, 123], 700, 2000
    if not variant_ok(variant, D, G, "q8_0", "q4_0"):
        pytest.skip(f"{variant} does not cover D={D} G={G}")
    note(f"partials past max_seq_len {variant}")
    k = synth.normal_f16((B, Hkv, cap, D), 1301, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 1302, dev)
    q = synth.normal_f16((B, Hkv * G, D), 1303, dev)
    kc, vc = fill_pair("q8_0", "q4_0", k, v)
    part = C.Partials(B, Hkv * G, D, cap, st)
    part.o.fill_(5.0)
    part.lse.fill_(5.0)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    C.decode(kc, vc, q, lt, max_len, part, 1 / math.sqrt(D), variant)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
    C.combine(part, lt, out, lse)
    torch.cuda.synchronize()
    assert part.max_splits > -(-max_len // st)
    for b, L in enumerate(lens):
        nb = -(-L // st)
        assert torch.all(part.o[b, :, nb:] == 5.0) and torch.all(part.lse[b, :, nb:] == 5.0)
        assert torch.all(part.lse[b, :, :nb] != 5.0)
    ref, ref_lse = oracle_ref(kc, vc, q, lens, Hkv)
    assert_close(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64), ref, ref_lse,
                 variant)


@pytest.mark.parametrize("D", [32, 128, 160, 192, 256, 512])
@pytest.mark.parametrize("S", [40, 300])
def test_combine_alone_on_oracle_partials(D, S):
    """K3 fed the oracle's split partials (rounded to fp32) reproduces the
    oracle's exact merge: rows of up to 128 columns in one workgroup, wider
    rows in column chunks (160: five of 32, 192: two of 96, 256 / 512: two /
    four of 128); 300 splits take several batches of loads."""
    note(f"combine on oracle partials D={D} S={S}")
    rng = np.random.default_rng(3 + D + S)
    B, Hq, st = 3, 6, 64
    lens = [1, 1000, 64 * S]
    po = rng.standard_normal((B, Hq, S, D))
    pl = rng.standard_normal((B, Hq, S)) * 5
    for b in range(B):
        nb = -(-lens[b] // st)
        pl[b, :, nb:] = -np.inf
        po[b, :, nb:] = 0
    ref, ref_lse = O.combine(po, pl)
    part = C.Partials(B, Hq, D, max(lens), st)
    part.o.copy_(torch.from_numpy(po.astype(np.float32)))
    part.lse.copy_(torch.from_numpy(pl.astype(np.float32)))
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    for out_dtype in (torch.float32, torch.float16):
        out = torch.empty((B, Hq, D), dtype=out_dtype, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        C.combine(part, lt, out, lse)
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        tol = 1e-5 if out_dtype == torch.float32 else 2e-3
        assert np.allclose(got, ref, atol=tol, rtol=tol)
        assert np.allclose(lse.cpu().numpy(), ref_lse, atol=1e-5)


@pytest.mark.parametrize("B", [1, 3])
def test_combine_ignores_dead_splits(B):
    """Splits at or past a sequence's ceil(L / split_tokens) carry no weight
    whatever their memory holds: they are filled with NaN rows and an lse
    that would dominate every live one (one sequence: the merge loads them
    and masks them; several: it reads the lengths first and does not load
    them)."""
    note(f"combine dead splits B={B}")
    rng = np.random.default_rng(11 + B)
    Hq, D, S, st = 5, 128, 40, 64
    lens = [1000] if B == 1 else [1, 1000, 64 * 17 + 5]
    po = rng.standard_normal((B, Hq, S, D))
    pl = rng.standard_normal((B, Hq, S)) * 5
    live = po.copy(), pl.copy()
    for b in range(B):
        nb = -(-lens[b] // st)
        live[1][b, :, nb:] = -np.inf
        live[0][b, :, nb:] = 0
        po[b, :, nb:] = np.nan
        pl[b, :, nb:] = 50.0
    ref, ref_lse = O.combine(*live)
    # max_seq_len of the partials: every split of the buffer may be loaded
    part = C.Partials(B, Hq, D, S * st, st)
    part.o.copy_(torch.from_numpy(po.astype(np.float32)))
    part.lse.copy_(torch.from_numpy(pl.astype(np.float32)))
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    C.combine(part, lt, out, lse)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert np.allclose(got, ref, atol=1e-5, rtol=1e-5)
    assert np.allclose(lse.cpu().numpy(), ref_lse, atol=1e-5)


@pytest.mark.parametrize("variant", VARIANTS)
def test_split_count_invariance_and_determinism(variant):
    dev = "cuda"
    B, Hkv, G, D, L = 1, 2, 5, 128, 5000
    if not variant_ok(variant, D, G, "q8_0", "q4_0"):
        pytest.skip("variant does not cover the shape")
    note(f"split invariance {variant}")
    k = synth.normal_f16((B, Hkv, L, D), 71, dev)
    v = synth.normal_f16((B, Hkv, L, D), 72, dev)
    q = synth.normal_f16((B, Hkv * G, D), 73, dev)
    kc, vc = fill_pair("q8_0", "q4_0", k, v)
    ref, ref_lse = oracle_ref(kc, vc, q, [L], Hkv)
    outs = {}
    for st in (64, 256, 1024, 5056):
        outs[st] = run_decode(kc, vc, q, [L], st, variant)
        assert_close(outs[st][0], outs[st][1], ref, ref_lse, f"split {st}")
    again = run_decode(kc, vc, q, [L], 256, variant)
    assert np.array_equal(again[0], outs[256][0]) and np.array_equal(again[1], outs[256][1])


@pytest.mark.parametrize("variant", VARIANTS)
def test_identity_quantisation_equals_f16_cache(variant):
    """Values every format stores exactly: the quantised caches and the f16
    caches give the same outputs (within the kernel's rounding)."""
    dev = "cuda"
    rng = np.random.default_rng(17)
    B, Hkv, G, D, L = 1, 2, 5, 128, 700
    q = synth.normal_f16((B, Hkv * G, D), 5, dev)
    for tk, tv in (("q8_0", "q4_0"), ("q4_0", "q4_0"), ("q8_0", "q8_0")):
        if not variant_ok(variant, D, G, tk, tv):
            pytest.skip("variant does not cover the shape")
        note(f"identity {variant} {tk}/{tv}")
        k = identity_values(rng, tk, (B, Hkv, L, D), -7 if tk == "q8_0" else -3)
        v = identity_values(rng, tv, (B, Hkv, L, D), -6 if tv == "q8_0" else -2)
        kt = torch.from_numpy(k.view(np.int16)).to(dev).view(torch.float16)
        vt = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.float16)
        kq, vq = fill_pair(tk, tv, kt, vt)
        kf, vf = fill_pair("f16", "f16", kt, vt)
        a = run_decode(kq, vq, q, [L], 256, variant)
        b = run_decode(kf, vf, q, [L], 256, variant)
        # same real values, different fp32 summation: the quantised route
        # accumulates (code + offset) * q and removes the offset after, the f16
        # route sums the products directly; both are fp32-rounding apart
        d = np.abs(a[0] - b[0])
        assert np.all(d <= 1e-5 + 1e-4 * np.abs(b[0])), f"{tk}/{tv}: max diff {d.max():.3g}"
        assert np.allclose(a[1], b[1], atol=1e-5), f"{tk}/{tv}: lse diff {np.abs(a[1] - b[1]).max():.3g}"


def test_valu_and_mfma_agree():
    """Two kernel families on the same cache agree within fp32 rounding."""
    dev = "cuda"
    B, Hkv, G, D, L = 2, 2, 5, 128, 3000
    if not variant_ok("mfma", D, G, "q4_0", "q4_0"):
        pytest.skip("MFMA kernel not available for this shape")
    note("valu vs mfma")
    k = synth.normal_f16((B, Hkv, L, D), 81, dev)
    v = synth.normal_f16((B, Hkv, L, D), 82, dev)
    q = synth.normal_f16((B, Hkv * G, D), 83, dev)
    for tk, tv in (("q4_0", "q4_0"), ("q8_0", "q4_0"), ("f16", "f16")):
        kc, vc = fill_pair(tk, tv, k, v)
        a = run_decode(kc, vc, q, [L, L - 100], 512, "valu")
        b = run_decode(kc, vc, q, [L, L - 100], 512, "mfma")
        assert np.allclose(a[0], b[0], atol=2e-4, rtol=2e-3)
        assert np.allclose(a[1], b[1], atol=1e-4)


# ----------------------------------------------------------------- workloads

def build_workload(wl, tk, tv, layer=0, needle_pos=None):
    """Cache, query and lengths of one layer of a workload; the cache rows are
    the oracle's quantisation of the seeded values."""
    dev = "cuda"
    lens = wl.lengths()
    cap = max(lens)
    B, Hkv, D = wl.B, wl.Hkv, wl.D
    k = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "k"), dev)
    v = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "v"), dev)
    q = synth.normal_f16((B, wl.Hq, D), synth.seed_for(wl.seed, layer, "q"), dev)
    if wl.k_outlier_frac:
        ch = synth.outlier_channels(D, synth.seed_for(wl.seed, layer, "aux"), wl.k_outlier_frac)
        k[..., ch] = (k[..., ch].float() * 8).half()
    if wl.needle:
        p = needle_pos if needle_pos is not None else lens[0] // 3
        for g in range(Hkv):
            k[0, p, g] = synth.needle_row(q[0, g * wl.G], synth.seed_for(wl.seed, g, "aux"))
    # (B, rows, Hkv, D) -> planes (B, Hkv, rows, .) quantised by the oracle
    kc, vc = fill_pair(tk, tv, k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3))
    return kc, vc, q, lens


def workload_case(name, tk, tv, variant, heads=None, layer=0, needle_pos=None, split_tokens=None):
    wl = synth.WORKLOADS[name]
    if not variant_ok(variant, wl.D, wl.G, tk, tv):
        pytest.skip("variant does not cover the shape")
    st = split_tokens or wl.split_tokens
    note(f"workload {name} {tk}/{tv} {variant} layer={layer} split={st}")
    kc, vc, q, lens = build_workload(wl, tk, tv, layer, needle_pos)
    out, lse, _ = run_decode(kc, vc, q, lens, st, variant)
    if heads is None:
        ref, ref_lse = oracle_ref(kc, vc, q, lens, wl.Hkv)
        assert_close(out, lse, ref, ref_lse, name)
    else:
        # sampled query heads: the oracle restricted to the KV heads they read
        for h in heads:
            g = h // wl.G
            sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]), np.ascontiguousarray(p[2][:, g:g + 1]))
            qh = to_host_u16(q[:, h:h + 1])
            ref, ref_lse = O.attend(qh, sub(planes_to_oracle(kc)), sub(planes_to_oracle(vc)), lens, 1,
                                    1 / math.sqrt(wl.D), nthreads=oracle_threads())
            assert_close(out[:, h:h + 1], lse[:, h:h + 1], ref, ref_lse, f"{name} head {h}")
    return kc, vc, q, lens, out, lse


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("tk,tv", list(itertools.product(TYPES, repeat=2)))
def test_workload_gqa5_d128_ctx4k(variant, tk, tv):
    """The one-layer 4096-row workload (128-row splits), every pair of the
    base types, every output against the oracle."""
    workload_case("gqa5_d128_ctx4k", tk, tv, variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("tk,tv", [("f16", "f16"), ("q8_0", "q8_0"), ("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_workload_hybrid_d256_ctx32k(variant, tk, tv):
    workload_case("hybrid_d256_ctx32k", tk, tv, variant)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("tk,tv", [("f16", "f16"), ("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_workload_stack48_layers_sampled(variant, tk, tv):
    """Layers 0, 23 and 47 of the 48-layer stack (each layer is an independent
    65536-row cache; every output of those layers is checked)."""
    for layer in (0, 23, 47):
        workload_case("stack48_d128_ctx64k", tk, tv, variant, layer=layer)


def assert_needle_argmax(kc, vc, q, g, h, p, n_rows, D):
    """The needle pin: row p has the largest score of query head h (the head
    its needle was built from) among all n_rows rows of KV head g, in the
    oracle's fp64 scores and in the attention kernel's own scores, which also
    agree row by row within fp32 rounding."""
    scale = 1 / math.sqrt(D)
    so = oracle_row_scores(kc, to_host_u16(q[0, h:h + 1]), g, n_rows, scale)[0]
    sg = gpu_row_scores(kc, vc, q[0, h:h + 1], g, n_rows, scale)[0]
    assert int(np.argmax(so)) == p, f"oracle: argmax {int(np.argmax(so))} != needle row {p} (KV head {g})"
    assert int(np.argmax(sg)) == p, f"GPU: argmax {int(np.argmax(sg))} != needle row {p} (KV head {g})"
    err = np.abs(sg - so)
    assert np.all(err <= 1e-4 + 1e-5 * np.abs(so)), f"scores differ by {err.max():.3g}"


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_workload_long_ctx256k_with_needle(variant, tk, tv):
    """All 40 heads at 262144 rows against the oracle.  The planted needle: for
    every KV head, row p is the argmax of the constructing head's scores in
    both the oracle and the kernel, and carries a visible share of that head's
    attention."""
    kc, vc, q, lens, out, lse = workload_case("long_d128_ctx256k", tk, tv, variant)
    wl = synth.WORKLOADS["long_d128_ctx256k"]
    p = lens[0] // 3
    vneedle = O.dequantize(tv, planes_to_oracle(vc)[1][0, :, p], planes_to_oracle(vc)[2][0, :, p], wl.D)
    for g in range(wl.Hkv):
        if variant == "mfma":
            assert_needle_argmax(kc, vc, q, g, g * wl.G, p, lens[0], wl.D)
        o = out[0, g * wl.G]
        cos = float(o @ vneedle[g] / (np.linalg.norm(o) * np.linalg.norm(vneedle[g])))
        assert cos > 0.5, f"needle of KV head {g} not visible (cos {cos:.3f})"


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
@pytest.mark.parametrize("split_tokens", [2048, 1024])
def test_workload_long_ctx256k_128_and_256_splits(tk, tv, split_tokens):
    """The 262144-row layer cut into 128 and 256 splits (the benchmark's 64 are
    covered above), all 40 heads against the oracle."""
    workload_case("long_d128_ctx256k", tk, tv, "mfma", split_tokens=split_tokens)


@pytest.mark.parametrize("variant", VARIANTS)
def test_needle_at_split_boundaries(variant):
    """Needle at row 0, at split boundaries +-1 and at the last row, on a
    shortened (32768-row) copy of the long-context workload."""
    wl0 = synth.WORKLOADS["long_d128_ctx256k"]
    import dataclasses
    wl = dataclasses.replace(wl0, ctx=32768, name="long_needle_32k")
    synth.WORKLOADS[wl.name] = wl
    try:
        st = wl.split_tokens
        for p in (0, st - 1, st, st + 1, 5 * st, wl.ctx - 1):
            kc, vc, q, lens, out, lse = workload_case(wl.name, "q8_0", "q4_0", variant,
                                                      heads=[0, wl.G * 3], needle_pos=p)
            if variant == "mfma":
                for g in (0, 3):
                    assert_needle_argmax(kc, vc, q, g, g * wl.G, p, lens[0], wl.D)
    finally:
        del synth.WORKLOADS[wl.name]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("name", ["batch16_ragged", "batch16_ragged_d512"])
@pytest.mark.parametrize("tk,tv", [("q4_0", "q4_0"), ("q8_0", "q4_0")])
def test_workload_batch16_ragged(variant, name, tk, tv):
    wl = synth.WORKLOADS[name]
    # one query head of every KV head, at a different place in each group
    heads = [g * wl.G + g % wl.G for g in range(wl.Hkv)]
    workload_case(name, tk, tv, variant, heads=heads)
