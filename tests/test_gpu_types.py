"""The further scalar types q4_1, q5_0, q5_1 and q6_0 on the GPU against the
CPU oracle: quantise-on-write bit-exact, decode attention (the vector-ALU
kernel, which covers every type pair) within the parity tolerance, the decode
step and the window eviction into these types.  The layouts and quantisers
are the oracle's readings (oracle/kvq_oracle.c); the block sizes are the
pages' (HAL #582 section 1 size table, section 5 P1 ladder)."""
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, assert_partials, fill_pair, note, oracle_threads, planes_to_oracle,
                       require_gpu, run_decode, to_host_u16)
from .test_oracle_quant_n3 import WORKED as WORKED_N3

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import _lib  # noqa: E402
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu
NEW = ["q4_1", "q5_0", "q5_1", "q6_0"]
# the pages' served pairs that use these types, the ladder's last rung, and
# each new type against the existing ones
PAIRS = [("q8_0", "q6_0"), ("q8_0", "q5_0"), ("q6_0", "q6_0"), ("q6_0", "q4_0"), ("q5_0", "q5_0"),
         ("q5_1", "q5_1"), ("q4_1", "q4_1"), ("q5_1", "q4_0"), ("f16", "q5_1"), ("q4_1", "q8_0")]


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def sentinel_planes(t, B, Hkv, cap, D):
    p = C.CachePlanes.alloc(t, B, Hkv, cap, D)
    p.data.fill_(0xA5)
    if p.scales is not None:
        p.scales.fill_(0x5A5A)
    return p


def structured_rows(shape, seed, dev):
    """N(0,1) rows, with some rows tiny, some huge, some all-zero, some
    all-positive with an offset (the min/max types' case), some holding exact
    ties."""
    x = synth.normal_f16(shape, seed, dev).float()
    x[:, ::7] *= 1e-5
    x[:, 1::7] *= 2000.0
    x[:, 2::7] = 0.0
    x[:, 3::7] = torch.randint(-20, 20, x[:, 3::7].shape, device=dev).float() / 8.0
    x[:, 4::7] = 5.0 + x[:, 4::7].abs()
    return x.half()


@pytest.mark.parametrize("t", NEW)
@pytest.mark.parametrize("D", [32, 128, 512])
def test_append_bit_exact(t, D):
    dev = "cuda"
    B, n_new, Hkv, cap = 3, 29, 2, 80
    positions = [0, 7, 51]
    note(f"append {t} D={D}")
    x = structured_rows((B, n_new, Hkv, D), 31 + D, dev)
    kc = sentinel_planes(t, B, Hkv, cap, D)
    vc = sentinel_planes(t, B, Hkv, cap, D)
    pos = torch.tensor(positions, dtype=torch.int32, device=dev)
    C.append(kc, vc, x, x, pos, max(positions) + n_new)
    torch.cuda.synchronize()
    qd, qs = O.quantize(t, to_host_u16(x))          # (B, n_new, Hkv, ...)
    got_d = kc.data.cpu().numpy()
    got_s = kc.scales.cpu().numpy().view(np.uint16)
    for b in range(B):
        p0 = positions[b]
        assert np.array_equal(got_d[b, :, p0:p0 + n_new], qd[b].transpose(1, 0, 2)), f"data b={b}"
        assert np.array_equal(got_s[b, :, p0:p0 + n_new], qs[b].transpose(1, 0, 2)), f"scales b={b}"
        # rows outside [p0, p0 + n_new) untouched
        assert np.all(got_d[b, :, :p0] == 0xA5) and np.all(got_d[b, :, p0 + n_new:] == 0xA5)
    assert torch.equal(kc.data, vc.data) and torch.equal(kc.scales, vc.scales)


@pytest.mark.parametrize("t", NEW)
def test_append_every_finite_f16_value(t):
    """All 63488 finite binary16 values, in 4 seeded shuffles, through K1."""
    dev = "cuda"
    note(f"append every f16 value {t}")
    pos = np.arange(0, 0x7C00, dtype=np.uint32).astype(np.uint16)
    vals = np.concatenate([pos, pos | 0x8000])
    rng = np.random.default_rng(98)
    allv = np.concatenate([rng.permutation(vals) for _ in range(4)])
    D = 128
    rows = allv.reshape(1, -1, 1, D)
    x = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.float16)
    n_new = rows.shape[1]
    kc = sentinel_planes(t, 1, 1, n_new, D)
    C.append(kc, kc, x, x, torch.zeros(1, dtype=torch.int32, device=dev), n_new)
    torch.cuda.synchronize()
    want_d, want_s = O.quantize(t, rows[0, :, 0])
    assert np.array_equal(kc.data[0, 0].cpu().numpy(), want_d)
    assert np.array_equal(kc.scales[0, 0].cpu().numpy().view(np.uint16), want_s)


def test_append_worked_blocks():
    dev = "cuda"
    note("append worked blocks of the further types")
    for wid, t, x, scales, data in WORKED_N3:
        xt = torch.from_numpy(x.reshape(1, 1, 1, 32).view(np.int16)).to(dev).view(torch.float16)
        kc = sentinel_planes(t, 1, 1, 1, 32)
        C.append(kc, kc, xt, xt, torch.zeros(1, dtype=torch.int32, device=dev), 1)
        torch.cuda.synchronize()
        assert kc.data[0, 0, 0].cpu().numpy().tobytes() == data, wid
        assert [int(v) for v in kc.scales[0, 0, 0].cpu().numpy().view(np.uint16)] == scales, wid


CASES = [
    # (B, Hkv, G, D, lens, split_tokens)
    (2, 2, 5, 128, [1000, 65], 256),
    (1, 2, 8, 256, [777], 128),
    (3, 2, 4, 32, [1, 129, 200], 64),
    (1, 2, 1, 512, [300], 64),
    (2, 1, 16, 64, [64, 0], 64),
]


# pairs with the further types that the matrix-core kernel is built for
# (head_dim 128, 256 and 512; one or several query tokens)
MFMA_PAIRS = {("q8_0", "q6_0"), ("q8_0", "q5_0"), ("q6_0", "q6_0"), ("q6_0", "q4_0"), ("q5_0", "q5_0"),
              ("q5_1", "q5_1"), ("q4_1", "q4_1"), ("q5_1", "q4_0")}


@pytest.mark.parametrize("variant", ["valu", "mfma"])
@pytest.mark.parametrize("tk,tv", PAIRS)
@pytest.mark.parametrize("case", range(len(CASES)))
def test_decode_matches_oracle(tk, tv, case, variant):
    B, Hkv, G, D, lens, st = CASES[case]
    covered = (tk, tv) in MFMA_PAIRS and D in (128, 256, 512)
    note(f"decode {variant} {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} lens={lens} split={st}")
    dev = "cuda"
    seed = 3300 + case
    cap = max(lens) + 9
    kc, vc = fill_pair(tk, tv, synth.normal_f16((B, Hkv, cap, D), seed, dev),
                       synth.normal_f16((B, Hkv, cap, D), seed + 1, dev))
    q = synth.normal_f16((B, Hkv * G, D), seed + 2, dev)
    if variant == "mfma" and not covered:
        with pytest.raises(_lib.KVQError) as e:
            run_decode(kc, vc, q, lens, st, variant="mfma")
        assert e.value.status == -2
        return
    out, lse, (po, pl) = run_decode(kc, vc, q, lens, st, variant=variant)
    ref, ref_lse = O.attend(to_host_u16(q), planes_to_oracle(kc), planes_to_oracle(vc), lens, Hkv,
                            1 / math.sqrt(D), nthreads=oracle_threads())
    live = [b for b, L in enumerate(lens) if L > 0]
    assert_close(out[live], lse[live], ref[live], ref_lse[live], f"{tk}/{tv} case {case}")
    for b, L in enumerate(lens):
        if L == 0:   # no rows: output 0, LSE -inf
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
    # the split partials too
    ro, rl = O.attend_split(to_host_u16(q), planes_to_oracle(kc), planes_to_oracle(vc), lens, Hkv,
                            1 / math.sqrt(D), st, po.shape[2])
    assert_partials(po, pl, ro, rl, lens, st)


def test_matrix_core_kernel_reports_what_it_does_not_cover():
    """The further types on the matrix cores: the listed pairs at head_dim 128,
    256 and 512 only (KVQ_ERR_SHAPE otherwise, also for multi-query decode;
    kvq_decode_attn falls back to the vector ALUs for single-token decode)."""
    dev = "cuda"
    for (tk, tv), D, nq in ((("q5_1", "q4_0"), 64, 1), (("q5_1", "q4_0"), 64, 2),
                            (("q4_1", "q8_0"), 256, 1), (("q4_1", "q8_0"), 256, 2)):
        kc, vc = fill_pair(tk, tv, synth.normal_f16((1, 1, 64, D), 1, dev),
                           synth.normal_f16((1, 1, 64, D), 2, dev))
        with pytest.raises(_lib.KVQError) as e:
            if nq == 1:
                run_decode(kc, vc, synth.normal_f16((1, 5, D), 3, dev), [64], 64, variant="mfma")
            else:
                part = C.Partials(1, nq * 5, D, 64, 64)
                C.decode_multi(kc, vc, synth.normal_f16((1, nq, 5, D), 3, dev),
                               torch.tensor([64], dtype=torch.int32, device=dev), 64, part, 0.1)
        assert e.value.status == -2


@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("tk,tv", [("q5_1", "q4_0"), ("q6_0", "q6_0"), ("q4_1", "q4_1")])
def test_decode_step_is_append_attention_merge(tk, tv, D):
    """kvq_decode_step on these types (the attention kernel writes the new row,
    then the merge) equals the three calls bit for bit, and the oracle over
    the oracle-quantised rows within the tolerance."""
    dev = "cuda"
    B, Hkv, G, st = 2, 2, 5, 128
    lens = [300, 77]
    cap = max(lens)
    note(f"decode step {tk}/{tv} D={D}")
    k = synth.normal_f16((B, Hkv, cap, D), 71, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 72, dev)
    q = synth.normal_f16((B, Hkv * G, D), 73, dev)
    kn = synth.normal_f16((B, Hkv, D), 74, dev)
    vn = synth.normal_f16((B, Hkv, D), 75, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    res = []
    for fused in (True, False):
        kc, vc = fill_pair(tk, tv, k, v)
        part = C.Partials(B, Hkv * G, D, cap, st)
        out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
        lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
        if fused:
            C.decode_step(kc, vc, kn, vn, q, lt, cap, part, 1 / math.sqrt(D), out, lse)
        else:
            C.append(kc, vc, kn.unsqueeze(1), vn.unsqueeze(1), lt - 1, cap)
            C.decode(kc, vc, q, lt, cap, part, 1 / math.sqrt(D))
            C.combine(part, lt, out, lse)
        torch.cuda.synchronize()
        res.append((kc, vc, out, lse))
    (k1, v1, o1, l1), (k2, v2, o2, l2) = res
    assert torch.equal(k1.data, k2.data) and torch.equal(k1.scales, k2.scales)
    assert torch.equal(v1.data, v2.data) and torch.equal(o1, o2) and torch.equal(l1, l2)
    # the oracle: rows quantised by the oracle, the new row at L - 1
    kh, vh = to_host_u16(k).copy(), to_host_u16(v).copy()
    for b, L in enumerate(lens):
        kh[b, :, L - 1] = to_host_u16(kn)[b]
        vh[b, :, L - 1] = to_host_u16(vn)[b]
    from .gpu_util import oracle_planes
    ref, ref_lse = O.attend(to_host_u16(q), oracle_planes(tk, kh), oracle_planes(tv, vh), lens, Hkv,
                            1 / math.sqrt(D), nthreads=oracle_threads())
    assert_close(o1.cpu().numpy().astype(np.float64), l1.cpu().numpy().astype(np.float64), ref, ref_lse,
                 f"step {tk}/{tv}")


@pytest.mark.parametrize("tk,tv", [("q5_1", "q4_0"), ("q4_1", "q6_0")])
def test_window_eviction_into_the_types(tk, tv):
    """kvq_quantize_rows from fp16 window planes into a tail of these types:
    bit-exact with the oracle's quantiser of the same rows."""
    dev = "cuda"
    B, Hkv, D, W, cap = 2, 2, 128, 48, 200
    note(f"eviction into {tk}/{tv}")
    win_k = synth.normal_f16((B, Hkv, W, D), 81, dev)
    win_v = synth.normal_f16((B, Hkv, W, D), 82, dev)
    wk, wv = fill_pair("f16", "f16", win_k, win_v)
    kc, vc = sentinel_planes(tk, B, Hkv, cap, D), sentinel_planes(tv, B, Hkv, cap, D)
    counts = torch.tensor([W, 17], dtype=torch.int32, device=dev)
    posq = torch.tensor([100, 3], dtype=torch.int32, device=dev)
    C.quantize_rows(kc, vc, wk, wv, counts, posq, W, 100 + W)
    torch.cuda.synchronize()
    for planes, t, src in ((kc, tk, win_k), (vc, tv, win_v)):
        qd, qs = O.quantize(t, to_host_u16(src))
        d = planes.data.cpu().numpy()
        s = planes.scales.cpu().numpy().view(np.uint16)
        for b, (n, p0) in enumerate(((W, 100), (17, 3))):
            assert np.array_equal(d[b, :, p0:p0 + n], qd[b, :, :n]), f"{t} data b={b}"
            assert np.array_equal(s[b, :, p0:p0 + n], qs[b, :, :n]), f"{t} scales b={b}"
            assert np.all(d[b, :, p0 + n:] == 0xA5)


def test_ladder_last_rung_full_size_64k():
    """The tier ladder's last rung (q5_1 K, q4_0 V) on a 64k-row layer of the
    48-layer workload: sampled query heads against the oracle restricted to the
    KV heads they read."""
    wl = synth.WORKLOADS["stack48_d128_ctx64k"]
    B, Hkv, D, G, L = wl.B, wl.Hkv, wl.D, wl.G, wl.ctx
    dev = "cuda"
    note("q5_1/q4_0 full size 64k")
    assert _lib.kvq_tier_types(3) == (_lib.Q5_1, _lib.Q4_0)
    kc, vc = fill_pair("q5_1", "q4_0", synth.normal_f16((B, Hkv, L, D), 3401, dev),
                       synth.normal_f16((B, Hkv, L, D), 3402, dev))
    q = synth.normal_f16((B, wl.Hq, D), 3403, dev)
    out, lse, _ = run_decode(kc, vc, q, [L], wl.split_tokens)
    for h in (0, 21, 39):
        g = h // G
        sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]), np.ascontiguousarray(p[2][:, g:g + 1]))
        ref, ref_lse = O.attend(to_host_u16(q[:, h:h + 1]), sub(planes_to_oracle(kc)),
                                sub(planes_to_oracle(vc)), [L], 1, 1 / math.sqrt(D),
                                nthreads=oracle_threads())
        assert_close(out[:, h:h + 1], lse[:, h:h + 1], ref, ref_lse, f"head {h}")


@pytest.mark.parametrize("t", NEW)
def test_fused_step_rows_bit_exact(t):
    """The decode step writes the new row from the attention kernel (32 lanes
    per block, cross-lane extremes and ballots for the high bits): the stored
    bytes equal the oracle's quantiser on rows of every kind -- zeros, a mix
    of +0 and -0, exact ties, tiny and huge values, an offset range."""
    dev = "cuda"
    B, Hkv, G, D = 7, 2, 5, 128
    cap, L = 96, 90
    note(f"fused step rows {t}")
    x = synth.normal_f16((B, Hkv, D), 91, dev).float()
    x[0] = 0.0
    x[1] = torch.where(torch.arange(D, device=dev) % 3 == 0, torch.tensor(-0.0, device=dev),
                       torch.tensor(0.0, device=dev)).expand(Hkv, D)
    x[1, :, 5::32] = 1.0                                   # one nonzero per block among signed zeros
    x[2] = torch.randint(-20, 20, (Hkv, D), device=dev).float() / 8.0
    x[3] *= 1e-5
    x[4] *= 3000.0
    x[5] = 7.0 + x[5].abs()
    kn = x.half()
    vn = synth.normal_f16((B, Hkv, D), 92, dev)
    lens = [L] * B
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    kc = sentinel_planes(t, B, Hkv, cap, D)
    vc = sentinel_planes(t, B, Hkv, cap, D)
    # the rows the attention reads before the new one: any valid codes
    base = synth.normal_f16((B, L - 1, Hkv, D), 93, dev)
    C.append(kc, vc, base, base, torch.zeros(B, dtype=torch.int32, device=dev), L - 1)
    part = C.Partials(B, Hkv * G, D, cap, 64)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    C.decode_step(kc, vc, kn, vn, synth.normal_f16((B, Hkv * G, D), 94, dev), lt, cap, part,
                  1 / math.sqrt(D), out)
    torch.cuda.synchronize()
    for planes, src in ((kc, kn), (vc, vn)):
        qd, qs = O.quantize(t, to_host_u16(src))            # (B, Hkv, ...)
        d = planes.data.cpu().numpy()[:, :, L - 1]
        s = planes.scales.cpu().numpy().view(np.uint16)[:, :, L - 1]
        assert np.array_equal(d, qd), "data"
        assert np.array_equal(s, qs), "scales"
    assert np.all(np.isfinite(out.cpu().numpy()))


@pytest.mark.parametrize("D", [128, 256, 512])
@pytest.mark.parametrize("tk,tv", sorted(MFMA_PAIRS))
def test_multi_query_decode_matches_oracle(tk, tv, D):
    """Multi-query decode (n_q tokens, causal among them) of the further types on
    the matrix cores against the oracle, token by token; and the fused
    multi-query step equals append + attention + merge bit for bit."""
    from .test_gpu_multi import oracle_multi, run_multi
    dev = "cuda"
    B, Hkv, G, nq, st = 2, 2, 5, 3, 64
    lens = [300, 130]                      # the second: query tokens across a split boundary
    note(f"multi {tk}/{tv} D={D}")
    cap = max(lens)
    kc, vc = fill_pair(tk, tv, synth.normal_f16((B, Hkv, cap, D), 61, dev),
                       synth.normal_f16((B, Hkv, cap, D), 62, dev))
    q = synth.normal_f16((B, nq, Hkv * G, D), 63, dev)
    out, lse = run_multi(kc, vc, q, lens, st)
    ref, ref_lse = oracle_multi(kc, vc, q, lens)
    assert_close(out.reshape(B, -1, D), lse.reshape(B, -1), ref.reshape(B, -1, D), ref_lse.reshape(B, -1),
                 f"multi {tk}/{tv}")
    k_new = synth.normal_f16((B, nq, Hkv, D), 64, dev)
    v_new = synth.normal_f16((B, nq, Hkv, D), 65, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    res = []
    for fused in (True, False):
        k2, v2 = fill_pair(tk, tv, synth.normal_f16((B, Hkv, cap, D), 61, dev),
                           synth.normal_f16((B, Hkv, cap, D), 62, dev))
        part = C.Partials(B, nq * Hkv * G, D, cap, st)
        o = torch.empty((B, nq * Hkv * G, D), dtype=torch.float32, device=dev)
        ls = torch.empty((B, nq * Hkv * G), dtype=torch.float32, device=dev)
        if fused:
            C.decode_step_multi(k2, v2, k_new, v_new, q, lt, cap, part, 1 / math.sqrt(D), o, ls)
        else:
            C.append(k2, v2, k_new, v_new, lt - nq, cap)
            C.decode_multi(k2, v2, q, lt, cap, part, 1 / math.sqrt(D))
            C.combine(part, lt, o, ls)
        torch.cuda.synchronize()
        res.append((k2, v2, o, ls))
    (a1, b1, o1, l1), (a2, b2, o2, l2) = res
    assert torch.equal(a1.data, a2.data) and torch.equal(a1.scales, a2.scales)
    assert torch.equal(b1.data, b2.data) and torch.equal(b1.scales, b2.scales)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
