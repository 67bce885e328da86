"""The decode calls captured in a HIP graph and replayed, the way the benchmark
times them.  The eager call runs first, then the graph is replayed several
times with eager work of the program's own (the outputs and partials filled
with NaN, other kernels) and host synchronisations in between: every replay
must give the eager call's outputs, LSEs and cache bytes bit for bit (a step
writes its new rows with the same bytes each time, so replays repeat the same
work).  The eager single-token step is also checked against the oracle."""
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, fill_pair, note, oracle_threads, plane_tensors, replay_and_compare,
                       require_gpu, to_host_u16)

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


STEP_CASES = [
    # (B, Hkv, G, D, lens, split_tokens, tk, tv)
    (2, 2, 5, 128, [3000, 1700], 256, "q8_0", "q4_0"),
    (2, 2, 5, 128, [3000, 1700], 256, "q4_0", "q4_0"),
    (1, 2, 5, 128, [2049], 1024, "f16", "f16"),
    (1, 2, 8, 256, [2000], 128, "q8_0", "q8_0"),
    (3, 1, 4, 512, [900, 64, 513], 64, "q4_0", "q4_0"),
    (2, 2, 5, 128, [1200, 700], 128, "q5_1", "q4_0"),
]


@pytest.mark.parametrize("case", range(len(STEP_CASES)))
def test_step_graph_replays_equal_eager(case):
    B, Hkv, G, D, lens, st, tk, tv = STEP_CASES[case]
    note(f"graph decode_step {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} lens={lens} split={st}")
    cap = max(lens) + 5
    dev = "cuda"
    k = synth.normal_f16((B, Hkv, cap, D), 900 + case, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 950 + case, dev)
    q = synth.normal_f16((B, Hkv * G, D), 990 + case, dev)
    # the cache holds the oracle's quantisation of every row, the new row's
    # included: the step rewrites row L_b - 1 with the same bytes
    kc, vc = fill_pair(tk, tv, k, v, cap)
    idx = torch.tensor([L - 1 for L in lens], device=dev, dtype=torch.long)
    bi = torch.arange(B, device=dev)
    k_new, v_new = k[bi, :, idx].contiguous(), v[bi, :, idx].contiguous()
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    part = C.Partials(B, Hkv * G, D, max(lens), st)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
    scale = 1.0 / math.sqrt(D)

    def call():
        C.decode_step(kc, vc, k_new, v_new, q, lt, max(lens), part, scale, out, lse)

    got, got_lse = replay_and_compare(call, [out, lse], plane_tensors(kc, vc), [part.o, part.lse],
                                      f"step {tk}/{tv} case {case}")
    # the replays' cache bytes are the oracle's quantisation, the new rows'
    # included
    for p, what in ((kc, "K"), (vc, "V")):
        assert np.array_equal(p.data.cpu().numpy(), p.oracle[1]), f"{what} data plane differs from the oracle"
        if p.scales is not None:
            assert np.array_equal(p.scales.cpu().numpy().view(np.uint16), p.oracle[2]), \
                f"{what} scale plane differs from the oracle"
    ref, ref_lse = O.attend(to_host_u16(q), kc.oracle, vc.oracle, lens, Hkv, scale, nthreads=oracle_threads())
    assert_close(got.cpu().numpy().astype(np.float64), got_lse.cpu().numpy().astype(np.float64), ref,
                 ref_lse, f"graph step {tk}/{tv} case {case}")


def test_three_calls_graph_replays_equal_eager():
    B, Hkv, G, D, lens, st = 2, 2, 5, 128, [2500, 900], 256
    note(f"graph append+decode+combine q8_0/q4_0 lens={lens} split={st}")
    dev = "cuda"
    cap = max(lens)
    k = synth.normal_f16((B, Hkv, cap, D), 1200, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 1201, dev)
    q = synth.normal_f16((B, Hkv * G, D), 1202, dev)
    kc, vc = fill_pair("q8_0", "q4_0", k, v, cap)
    idx = torch.tensor([L - 1 for L in lens], device=dev, dtype=torch.long)
    bi = torch.arange(B, device=dev)
    k_new = k[bi, :, idx].unsqueeze(1).contiguous()          # (B, 1, Hkv, D)
    v_new = v[bi, :, idx].unsqueeze(1).contiguous()
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    pos = lt - 1
    part = C.Partials(B, Hkv * G, D, max(lens), st)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float16, device=dev)
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)

    def call():
        C.append(kc, vc, k_new, v_new, pos, max(lens))
        C.decode(kc, vc, q, lt, max(lens), part, 1.0 / math.sqrt(D))
        C.combine(part, lt, out, lse)

    replay_and_compare(call, [out, lse], plane_tensors(kc, vc), [part.o, part.lse], "three calls")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_step_multi_graph_replays_equal_eager(tk, tv):
    B, Hkv, G, D, lens, st, nq = 2, 2, 5, 128, [2000, 300], 256, 3
    note(f"graph decode_step_multi {tk}/{tv} nq={nq} lens={lens} split={st}")
    dev = "cuda"
    cap = max(lens)
    k = synth.normal_f16((B, Hkv, cap, D), 1300, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 1301, dev)
    q = synth.normal_f16((B, nq, Hkv * G, D), 1302, dev)
    kc, vc = fill_pair(tk, tv, k, v, cap)
    rows = torch.stack([torch.arange(L - nq, L, device=dev) for L in lens])        # (B, nq)
    bi = torch.arange(B, device=dev)[:, None]
    k_new = k[bi, :, rows].contiguous()                     # (B, nq, Hkv, D)
    v_new = v[bi, :, rows].contiguous()
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    part = C.Partials(B, nq * Hkv * G, D, max(lens), st)
    out = torch.empty((B, nq * Hkv * G, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, nq * Hkv * G), dtype=torch.float32, device=dev)

    def call():
        C.decode_step_multi(kc, vc, k_new, v_new, q, lt, max(lens), part, 1.0 / math.sqrt(D), out, lse)

    replay_and_compare(call, [out, lse], plane_tensors(kc, vc), [part.o, part.lse], f"step multi {tk}/{tv}")


def test_step_mixed_graph_replays_equal_eager():
    B, Hkv, G, D = 2, 2, 5, 128
    tl, tcap, wl, wcap = [1900, 640], 1920, [130, 7], 256
    dev = "cuda"
    st_t, st_w = C.mixed_splits(max(tl), max(wl), 136 + 72, 512, B, Hkv, D)
    note(f"graph decode_step_mixed q8_0/q4_0 tail={tl} window={wl} splits {st_t}/{st_w}")
    kt = synth.normal_f16((B, Hkv, tcap, D), 1400, dev)
    vt = synth.normal_f16((B, Hkv, tcap, D), 1401, dev)
    kw = synth.normal_f16((B, Hkv, wcap, D), 1402, dev)
    vw = synth.normal_f16((B, Hkv, wcap, D), 1403, dev)
    q = synth.normal_f16((B, Hkv * G, D), 1404, dev)
    k_new = synth.normal_f16((B, Hkv, D), 1405, dev)
    v_new = synth.normal_f16((B, Hkv, D), 1406, dev)
    tail = fill_pair("q8_0", "q4_0", kt, vt)
    win = fill_pair("f16", "f16", kw, vw)
    ltt = torch.tensor(tl, dtype=torch.int32, device=dev)
    ltw = torch.tensor(wl, dtype=torch.int32, device=dev)
    parts = (C.Partials(B, Hkv * G, D, tcap, st_t), C.Partials(B, Hkv * G, D, wcap, st_w))
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)

    def call():
        C.decode_step_mixed(tail, win, k_new, v_new, q, ltt, ltw, parts[0], parts[1], 1.0 / math.sqrt(D),
                            out, lse)

    replay_and_compare(call, [out, lse], plane_tensors(*tail, *win),
                       [parts[0].o, parts[0].lse, parts[1].o, parts[1].lse], "step mixed")
