"""The position-axis mixed cache (HAL #582 "per-layer KV compression study",
section 5 P2): recent tokens in an fp16 window, older ones in a quantised tail.
Each region gets its own kvq_decode_attn launch, kvq_combine_regions merges
the two sets of partials, and kvq_quantize_rows quantises the window's rows
into the tail when the window is evicted.

Checked against the oracle: the merged output against its fp64 attention over
the union of the regions' rows (attend_regions), the evicted rows byte for
byte against its quantiser, and a run of decode steps with evictions in
between against the oracle at every step."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, download_planes, fill_pair, new_row_vmax, note, oracle_planes,
                       oracle_threads, planes_to_oracle, require_gpu, to_host_u16,
                       upload_oracle_planes)

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import _lib  # noqa: E402
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu
SENT_D, SENT_S = 0xA5, 0x5A5A


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def attend_mixed(tail, win, q, tail_lens, win_lens, st_tail, st_win, out_dtype=torch.float32,
                 one_call=True):
    """Attention over both regions (kvq_decode_attn_mixed, or one
    kvq_decode_attn per region) and the region merge; returns host fp64
    (out, lse)."""
    B, Hq, D = q.shape
    scale = 1.0 / math.sqrt(D)
    parts, lens_t = [], []
    for (kc, vc), lens, st in ((tail, tail_lens, st_tail), (win, win_lens, st_win)):
        lens_t.append(torch.tensor(lens, dtype=torch.int32, device=q.device))
        parts.append(C.Partials(B, Hq, D, kc.capacity, st))
    if one_call:
        C.decode_mixed(tail, win, q, lens_t[0], lens_t[1], parts[0], parts[1], scale)
    else:
        for (kc, vc), lt, part in zip((tail, win), lens_t, parts):
            C.decode(kc, vc, q, lt, kc.capacity, part, scale)
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    C.combine_regions(parts, lens_t, out, lse)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def oracle_mixed(tail, win, q, tail_lens, win_lens):
    D = q.shape[-1]
    return O.attend_regions(to_host_u16(q), [(planes_to_oracle(tail[0]), planes_to_oracle(tail[1]), tail_lens),
                                             (planes_to_oracle(win[0]), planes_to_oracle(win[1]), win_lens)],
                            tail[0].Hkv, 1.0 / math.sqrt(D), lib=None)


CASES = [
    # (B, Hkv, G, D, tail_lens, tail capacity, win_lens, window capacity, tail split, window split)
    (2, 2, 5, 128, [1000, 300], 1000, [37, 64], 64, 256, 64),
    (3, 2, 4, 128, [0, 129, 2000], 2000, [5, 0, 64], 64, 256, 64),
    (1, 2, 8, 256, [777], 800, [100], 128, 128, 64),
    (2, 1, 4, 512, [300, 65], 300, [1, 33], 64, 64, 64),
    (2, 2, 5, 64, [200, 1], 200, [17, 64], 64, 64, 64),
]


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("q8_0", "q8_0"), ("f16", "q4_0"),
                                   ("q5_1", "q4_0"), ("q6_0", "q6_0")])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_regions_match_oracle(tk, tv, case):
    B, Hkv, G, D, tl, tcap, wl, wcap, st_t, st_w = CASES[case]
    note(f"mixed {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} tail={tl} window={wl}")
    dev = "cuda"
    seed = 2100 + case
    tail = fill_pair(tk, tv, synth.normal_f16((B, Hkv, tcap, D), seed, dev),
                     synth.normal_f16((B, Hkv, tcap, D), seed + 1, dev))
    win = fill_pair("f16", "f16", synth.normal_f16((B, Hkv, wcap, D), seed + 2, dev),
                    synth.normal_f16((B, Hkv, wcap, D), seed + 3, dev))
    q = synth.normal_f16((B, Hkv * G, D), seed + 4, dev)
    out, lse = attend_mixed(tail, win, q, tl, wl, st_t, st_w)
    ref, ref_lse = oracle_mixed(tail, win, q, tl, wl)
    empty = np.isneginf(ref_lse)
    assert np.array_equal(np.isneginf(lse), empty)
    assert np.all(out[empty] == 0)
    live = ~empty
    if live.any():
        assert_close(out[live], lse[live], ref[live], ref_lse[live], f"mixed {tk}/{tv} case {case}")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "q4_0"), ("q5_1", "q4_0"),
                                   ("q4_1", "q4_1")])
@pytest.mark.parametrize("case", [0, 2, 3, 4])
def test_mixed_call_is_the_two_calls_bit_for_bit(tk, tv, case):
    """kvq_decode_attn_mixed (one launch where the matrix-core kernel covers the
    shape, two launches otherwise) writes the same partials as kvq_decode_attn
    over each region."""
    B, Hkv, G, D, tl, tcap, wl, wcap, st_t, st_w = CASES[case]
    note(f"mixed call vs two calls {tk}/{tv} case {case}")
    dev = "cuda"
    seed = 2900 + case
    tail = fill_pair(tk, tv, synth.normal_f16((B, Hkv, tcap, D), seed, dev),
                     synth.normal_f16((B, Hkv, tcap, D), seed + 1, dev))
    win = fill_pair("f16", "f16", synth.normal_f16((B, Hkv, wcap, D), seed + 2, dev),
                    synth.normal_f16((B, Hkv, wcap, D), seed + 3, dev))
    q = synth.normal_f16((B, Hkv * G, D), seed + 4, dev)
    scale = 1.0 / math.sqrt(D)
    ltt = torch.tensor(tl, dtype=torch.int32, device=dev)
    ltw = torch.tensor(wl, dtype=torch.int32, device=dev)
    p1 = (C.Partials(B, Hkv * G, D, tcap, st_t), C.Partials(B, Hkv * G, D, wcap, st_w))
    p2 = (C.Partials(B, Hkv * G, D, tcap, st_t), C.Partials(B, Hkv * G, D, wcap, st_w))
    for p in p1 + p2:
        p.o.fill_(7.0)
        p.lse.fill_(7.0)
    C.decode_mixed(tail, win, q, ltt, ltw, p1[0], p1[1], scale)
    C.decode(tail[0], tail[1], q, ltt, tcap, p2[0], scale)
    C.decode(win[0], win[1], q, ltw, wcap, p2[1], scale)
    torch.cuda.synchronize()
    for a, b in zip(p1, p2):
        assert torch.equal(a.o, b.o) and torch.equal(a.lse, b.lse)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "q4_0")])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_mixed_is_append_attention_merge(tk, tv, case):
    """kvq_decode_step_mixed equals kvq_quantize_append of the new row into the
    window at row win_lens[b] - 1, kvq_decode_attn_mixed and
    kvq_combine_regions: window rows and tail partials bit for bit, window
    partials, output and LSE up to fp32 rounding (a sequence whose window
    length is 0 gets no row)."""
    note(f"step_mixed vs three calls {tk}/{tv} case {case}")
    step_mixed_vs_three_calls(tk, tv, CASES[case], 3100 + case)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_step_mixed_full_size_64k_tail_and_window(tk, tv):
    """The same comparison on a layer of the 64k workload as the benchmark
    runs it: 63488 quantised tail rows, a 2048-row fp16 window whose last row
    the step writes, the split sizes of mixed_splits."""
    wl = synth.WORKLOADS["stack48_d128_ctx64k"]
    Lw, Lt = 2048, wl.ctx - 2048
    row_t = sum(_lib.kvq_data_row_bytes(t, wl.D) + _lib.kvq_scale_row_bytes(t, wl.D) for t in (tk, tv))
    st, sw = C.mixed_splits(Lt, Lw, row_t, 4 * wl.D, wl.B, wl.Hkv, wl.D)
    note(f"step_mixed vs three calls full size {tk}/{tv} splits {st}/{sw}")
    step_mixed_vs_three_calls(tk, tv, (wl.B, wl.Hkv, wl.G, wl.D, [Lt], Lt, [Lw], Lw, st, sw), 3190)


def step_mixed_vs_three_calls(tk, tv, shape, seed):
    B, Hkv, G, D, tl, tcap, wl, wcap, st_t, st_w = shape
    dev = "cuda"
    kt = synth.normal_f16((B, Hkv, tcap, D), seed, dev)
    vt = synth.normal_f16((B, Hkv, tcap, D), seed + 1, dev)
    kw = synth.normal_f16((B, Hkv, wcap, D), seed + 2, dev)
    vw = synth.normal_f16((B, Hkv, wcap, D), seed + 3, dev)
    q = synth.normal_f16((B, Hkv * G, D), seed + 4, dev)
    k_new = synth.normal_f16((B, Hkv, D), seed + 5, dev)
    v_new = synth.normal_f16((B, Hkv, D), seed + 6, dev)
    scale = 1.0 / math.sqrt(D)
    ltt = torch.tensor(tl, dtype=torch.int32, device=dev)
    ltw = torch.tensor(wl, dtype=torch.int32, device=dev)
    res = []
    for fused in (True, False):
        tail = fill_pair(tk, tv, kt, vt)
        win = fill_pair("f16", "f16", kw, vw)   # rows [0, wcap) written; the step overwrites one
        parts = (C.Partials(B, Hkv * G, D, tcap, st_t), C.Partials(B, Hkv * G, D, wcap, st_w))
        out = torch.full((B, Hkv * G, D), 7.0, dtype=torch.float32, device=dev)
        lse = torch.full((B, Hkv * G), 7.0, dtype=torch.float32, device=dev)
        if fused:
            C.decode_step_mixed(tail, win, k_new, v_new, q, ltt, ltw, parts[0], parts[1], scale, out, lse)
        else:
            C.append(win[0], win[1], k_new.unsqueeze(1), v_new.unsqueeze(1), ltw - 1, wcap)
            C.decode_mixed(tail, win, q, ltt, ltw, parts[0], parts[1], scale)
            C.combine_regions(parts, [ltt, ltw], out, lse)
        torch.cuda.synchronize()
        res.append((win[0].data.clone(), win[1].data.clone(), parts[0].o.clone(), parts[0].lse.clone(),
                    parts[1].o.clone(), parts[1].lse.clone(), out, lse))
    names = ("window K", "window V", "tail part_o", "tail part_lse", "window part_o", "window part_lse",
             "out", "lse")
    vmax = new_row_vmax(v_new, G)

    def close(a, c, what):
        # outputs (B, Hq, D) and LSEs (B, Hq): the step's new-row term (an
        # fp32 weight) against the tile's fp16-rounded one
        a, c = a.cpu().numpy().astype(np.float64), c.cpu().numpy().astype(np.float64)
        assert np.array_equal(np.isneginf(a), np.isneginf(c)), what
        f = np.isfinite(c)
        if a.ndim == 2:
            assert np.all(np.abs(a[f] - c[f]) <= 2e-6 * np.maximum(1.0, np.abs(c[f]))), what
        else:
            bound = 2e-6 + 2e-5 * np.abs(c) + 2.0 ** -11 * vmax[..., None]
            assert np.all(np.abs(a[f] - c[f]) <= bound[f]), f"{what}: {np.abs(a[f] - c[f]).max():.3g}"

    # the window bytes are identical; the tail partials too (the tail is not
    # written); the step merges the new row's decoded values as a term of its
    # window split with an fp32 weight, where the three calls read the row
    # back inside a tile and round its weight to fp16 for the matrix cores:
    # the window partials and the outputs agree within 2^-11 of that weight
    # times the row's largest value, plus fp32 rounding
    for n, a, b in zip(names, *res):
        if n.endswith("part_o") or n.endswith("part_lse"):
            # splits past a sequence's last one are not written by either path
            continue
        if n in ("out", "lse"):
            close(a, b, n)
        else:
            assert torch.equal(a, b), n
    for b in range(B):
        for (n, a, c), L, st in zip(((2, res[0][2], res[1][2]), (4, res[0][4], res[1][4])), (tl, wl),
                                    (st_t, st_w)):
            S = -(-L[b] // st)
            if n == 2:
                assert torch.equal(a[b, :, :S], c[b, :, :S]), f"{names[n]} b {b}"
                assert torch.equal(res[0][n + 1][b, :, :S], res[1][n + 1][b, :, :S]), f"{names[n + 1]} b {b}"
            else:
                # window partials (Hq, S, D), and their LSEs (Hq, S)
                pa, pc = a[b, :, :S], c[b, :, :S]
                fa = pa.cpu().numpy().astype(np.float64)
                fc = pc.cpu().numpy().astype(np.float64)
                bound = 2e-6 + 2e-5 * np.abs(fc) + 2.0 ** -11 * vmax[b][:, None, None]
                assert np.all(np.abs(fa - fc) <= bound), f"{names[n]} b {b}"
                la = res[0][n + 1][b, :, :S].cpu().numpy().astype(np.float64)
                lc = res[1][n + 1][b, :, :S].cpu().numpy().astype(np.float64)
                assert np.all(np.abs(la - lc) <= 2e-6 * np.maximum(1.0, np.abs(lc))), f"{names[n + 1]} b {b}"
    # the new row is in the window where the lengths say
    kh = to_host_u16(k_new)
    wk = res[0][0].cpu().numpy().view(np.uint16)
    for b in range(B):
        if wl[b] > 0:
            assert np.array_equal(wk[b, :, wl[b] - 1], kh[b])


def test_one_region_merge_equals_combine():
    """kvq_combine_regions over one region gives kvq_combine's output (the same
    merge; the loads are batched differently, so within fp32 rounding)."""
    B, Hkv, G, D, L, st = 2, 2, 5, 128, [5000, 700], 64
    note("combine_regions with one region")
    dev = "cuda"
    kc, vc = fill_pair("q8_0", "q4_0", synth.normal_f16((B, Hkv, max(L), D), 2201, dev),
                       synth.normal_f16((B, Hkv, max(L), D), 2202, dev))
    q = synth.normal_f16((B, Hkv * G, D), 2203, dev)
    lt = torch.tensor(L, dtype=torch.int32, device=dev)
    part = C.Partials(B, Hkv * G, D, max(L), st)
    C.decode(kc, vc, q, lt, max(L), part, 1 / math.sqrt(D))
    o1 = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    l1 = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
    o2, l2 = torch.empty_like(o1), torch.empty_like(l1)
    C.combine(part, lt, o1, l1)
    C.combine_regions([part], [lt], o2, l2)
    torch.cuda.synchronize()
    assert torch.allclose(o1, o2, atol=1e-6, rtol=1e-5)
    assert torch.allclose(l1, l2, atol=1e-6)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q8_0"), ("f16", "q4_0")])
def test_quantize_rows_bit_exact(tk, tv):
    """Rows [0, counts[b]) of fp16 window planes land at rows positions[b] + r
    of the tail, byte for byte the oracle's quantisation; no other row of the
    tail changes."""
    B, Hkv, D, W, cap = 3, 2, 128, 40, 200
    counts, positions = [40, 0, 17], [0, 100, 183]
    note(f"quantize_rows {tk}/{tv}")
    dev = "cuda"
    kw = synth.normal_f16((B, Hkv, W, D), 2301, dev)
    vw = synth.normal_f16((B, Hkv, W, D), 2302, dev)
    win = fill_pair("f16", "f16", kw, vw)
    k_exp, v_exp = oracle_planes(tk, np.zeros((B, Hkv, cap, D), np.uint16)), \
        oracle_planes(tv, np.zeros((B, Hkv, cap, D), np.uint16))
    for p in (k_exp, v_exp):
        p[1][:] = SENT_D
        p[2][:] = SENT_S
    k_dev = upload_oracle_planes(k_exp[0], k_exp[1].copy(), k_exp[2].copy())
    v_dev = upload_oracle_planes(v_exp[0], v_exp[1].copy(), v_exp[2].copy())
    kq = oracle_planes(tk, to_host_u16(kw))
    vq = oracle_planes(tv, to_host_u16(vw))
    for b in range(B):
        n, p0 = counts[b], positions[b]
        k_exp[1][b, :, p0:p0 + n] = kq[1][b, :, :n]
        k_exp[2][b, :, p0:p0 + n] = kq[2][b, :, :n]
        v_exp[1][b, :, p0:p0 + n] = vq[1][b, :, :n]
        v_exp[2][b, :, p0:p0 + n] = vq[2][b, :, :n]
    ct = torch.tensor(counts, dtype=torch.int32, device=dev)
    pt = torch.tensor(positions, dtype=torch.int32, device=dev)
    C.quantize_rows(k_dev, v_dev, win[0], win[1], ct, pt, W, max(c + p for c, p in zip(counts, positions)))
    torch.cuda.synchronize()
    for dev_p, want, what in ((k_dev, k_exp, "K"), (v_dev, v_exp, "V")):
        d, s = download_planes(dev_p)
        assert np.array_equal(d, want[1]), f"{what} data"
        if want[0] != "f16":
            assert np.array_equal(s, want[2]), f"{what} scales"


@pytest.mark.parametrize("fused", [True, False])
@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_rolling_window_decode_steps(tk, tv, fused):
    """Decode steps on a mixed cache: each new token goes into the fp16 window;
    when the window is full its rows are quantised into the tail
    (kvq_quantize_rows) and it starts empty.  Fused: kvq_decode_step_mixed
    writes the token and attends; otherwise kvq_quantize_append on the fp16
    planes (a copy), kvq_decode_attn_mixed and the region merge.  Every step's
    output against the oracle over tail + window, and the tail's bytes
    against the oracle's quantiser of the same tokens."""
    B, Hkv, G, D, W = 2, 2, 5, 128, 16
    L0 = [300, 45]                      # tokens in the tail at the start
    steps = 40
    cap = max(L0) + steps + W
    dev = "cuda"
    note(f"rolling window {tk}/{tv}")
    # every token's K and V (the tail holds tokens [0, Lq), the window the next Lw)
    k_all = synth.normal_f16((B, Hkv, cap, D), 2401, dev)
    v_all = synth.normal_f16((B, Hkv, cap, D), 2402, dev)
    kh, vh = to_host_u16(k_all), to_host_u16(v_all)
    k_q, v_q = oracle_planes(tk, kh), oracle_planes(tv, vh)        # expected tail bytes
    tail_k = upload_oracle_planes(k_q[0], k_q[1].copy(), k_q[2].copy())
    tail_v = upload_oracle_planes(v_q[0], v_q[1].copy(), v_q[2].copy())
    # the tail on the device holds only tokens [0, L0) written by the oracle;
    # later rows must come from evictions: blank them
    for p in (tail_k, tail_v):
        for b in range(B):
            p.data[b, :, L0[b]:] = SENT_D
            if p.scales is not None:
                p.scales[b, :, L0[b]:] = SENT_S
    win_k = C.CachePlanes.alloc("f16", B, Hkv, W, D)
    win_v = C.CachePlanes.alloc("f16", B, Hkv, W, D)
    Lq, Lw = list(L0), [0] * B
    q_all = synth.normal_f16((steps, B, Hkv * G, D), 2403, dev)
    for i in range(steps):
        # the new token of sequence b is token Lq[b] + Lw[b]
        tok = [Lq[b] + Lw[b] for b in range(B)]
        k_new = torch.stack([k_all[b, :, tok[b]] for b in range(B)]).unsqueeze(1).contiguous()
        v_new = torch.stack([v_all[b, :, tok[b]] for b in range(B)]).unsqueeze(1).contiguous()
        q = q_all[i].contiguous()
        if fused:
            Lw = [x + 1 for x in Lw]
            ltt = torch.tensor(Lq, dtype=torch.int32, device=dev)
            ltw = torch.tensor(Lw, dtype=torch.int32, device=dev)
            parts = (C.Partials(B, Hkv * G, D, cap, 64), C.Partials(B, Hkv * G, D, W, 64))
            o = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
            ls = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
            C.decode_step_mixed((tail_k, tail_v), (win_k, win_v), k_new[:, 0].contiguous(),
                                v_new[:, 0].contiguous(), q, ltt, ltw, parts[0], parts[1],
                                1 / math.sqrt(D), o, ls)
            torch.cuda.synchronize()
            out = o.cpu().numpy().astype(np.float64)
            lse = ls.cpu().numpy().astype(np.float64)
        else:
            pos = torch.tensor(Lw, dtype=torch.int32, device=dev)
            C.append(win_k, win_v, k_new, v_new, pos, max(Lw) + 1)
            Lw = [x + 1 for x in Lw]
            out, lse = attend_mixed((tail_k, tail_v), (win_k, win_v), q, Lq, Lw, 64, 64)
        # the oracle: tail rows from its own quantiser, window rows the tokens' fp16 values
        ref, ref_lse = O.attend_regions(
            to_host_u16(q), [(k_q, v_q, Lq), (k_win_ref(kh, Lq, Lw, W), k_win_ref(vh, Lq, Lw, W), Lw)],
            Hkv, 1 / math.sqrt(D))
        assert_close(out, lse, ref, ref_lse, f"step {i} tail {Lq} window {Lw}")
        full = [b for b in range(B) if Lw[b] == W]
        if full:
            counts = torch.tensor([Lw[b] if b in full else 0 for b in range(B)], dtype=torch.int32, device=dev)
            posq = torch.tensor(Lq, dtype=torch.int32, device=dev)
            C.quantize_rows(tail_k, tail_v, win_k, win_v, counts, posq, W, max(Lq) + W)
            for b in full:
                Lq[b] += W
                Lw[b] = 0
            torch.cuda.synchronize()
            d, s = download_planes(tail_k)
            for b in range(B):
                assert np.array_equal(d[b, :, :Lq[b]], k_q[1][b, :, :Lq[b]]), f"tail K bytes after step {i}"
                assert np.array_equal(s[b, :, :Lq[b]], k_q[2][b, :, :Lq[b]])
            d, s = download_planes(tail_v)
            for b in range(B):
                assert np.array_equal(d[b, :, :Lq[b]], v_q[1][b, :, :Lq[b]]), f"tail V bytes after step {i}"
                assert np.array_equal(s[b, :, :Lq[b]], v_q[2][b, :, :Lq[b]])
    assert sum(Lq) > sum(L0), "no eviction happened"


def k_win_ref(xh, Lq, Lw, W):
    """The window as the oracle sees it: fp16 planes of tokens [Lq_b, Lq_b + Lw_b)."""
    B, Hkv, _, D = xh.shape
    w = np.zeros((B, Hkv, W, D), np.uint16)
    for b in range(B):
        w[b, :, :Lw[b]] = xh[b, :, Lq[b]:Lq[b] + Lw[b]]
    return oracle_planes("f16", w)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_mixed_full_size_64k_tail_and_window(tk, tv):
    """A layer of the 64k workload split as 63488 quantised tail rows and a
    2048-row fp16 window, in the launch configuration of the benchmark (the
    splits of mixed_splits, one round of resident workgroups); sampled query
    heads against the oracle restricted to the KV heads they read."""
    wl = synth.WORKLOADS["stack48_d128_ctx64k"]
    B, Hkv, D, G = wl.B, wl.Hkv, wl.D, wl.G
    Lw, Lt = 2048, wl.ctx - 2048
    dev = "cuda"
    note(f"mixed full size {tk}/{tv}")
    tail = fill_pair(tk, tv, synth.normal_f16((B, Hkv, Lt, D), 2501, dev),
                     synth.normal_f16((B, Hkv, Lt, D), 2502, dev))
    win = fill_pair("f16", "f16", synth.normal_f16((B, Hkv, Lw, D), 2503, dev),
                    synth.normal_f16((B, Hkv, Lw, D), 2504, dev))
    q = synth.normal_f16((B, wl.Hq, D), 2505, dev)
    row_t = sum(_lib.kvq_data_row_bytes(t, D) + _lib.kvq_scale_row_bytes(t, D) for t in (tk, tv))
    st, sw = C.mixed_splits(Lt, Lw, row_t, 4 * D, B, Hkv, D)
    out, lse = attend_mixed(tail, win, q, [Lt], [Lw], st, sw)
    for h in (0, 17, 39):
        g = h // G
        sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]), np.ascontiguousarray(p[2][:, g:g + 1]))
        ref, ref_lse = O.attend_regions(
            to_host_u16(q[:, h:h + 1]),
            [(sub(planes_to_oracle(tail[0])), sub(planes_to_oracle(tail[1])), [Lt]),
             (sub(planes_to_oracle(win[0])), sub(planes_to_oracle(win[1])), [Lw])], 1, 1 / math.sqrt(D))
        assert_close(out[:, h:h + 1], lse[:, h:h + 1], ref, ref_lse, f"head {h}")
