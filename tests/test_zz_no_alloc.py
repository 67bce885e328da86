"""kvq_decode_step_noalloc (partials in the library's own device array)
against kvq_decode_step (partials in caller memory): the same cache rows and
the same outputs, bit for bit, on two calls in a row, the second smaller; and
the call captured in a HIP graph, as its callers use it, replaying the eager
call's results."""
import math

import numpy as np
import pytest

from .gpu_util import (note, oracle_planes, plane_tensors, replay_and_compare, require_gpu, to_host_u16,
                       upload_oracle_planes)

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import _lib  # noqa: E402
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def one_step(tk, tv, B, Hkv, G, D, lens, st, seed, noalloc):
    dev = "cuda"
    cap = max(lens)
    k = synth.normal_f16((B, Hkv, cap, D), seed, dev)
    v = synth.normal_f16((B, Hkv, cap, D), seed + 1, dev)
    kc = upload_oracle_planes(*oracle_planes(tk, to_host_u16(k)))
    vc = upload_oracle_planes(*oracle_planes(tv, to_host_u16(v)))
    q = synth.normal_f16((B, Hkv * G, D), seed + 2, dev)
    k_new = synth.normal_f16((B, Hkv, D), seed + 3, dev)
    v_new = synth.normal_f16((B, Hkv, D), seed + 4, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.full((B, Hkv * G, D), 7.0, dtype=torch.float32, device=dev)
    lse = torch.full((B, Hkv * G), 7.0, dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(D)
    if noalloc:
        _lib.kvq_decode_step_noalloc(kc.desc(), vc.desc(), k_new, v_new, q, lt, B, Hkv * G, Hkv, D, scale,
                                     cap, st, "f32", out, lse)
    else:
        part = C.Partials(B, Hkv * G, D, cap, st)
        C.decode_step(kc, vc, k_new, v_new, q, lt, cap, part, scale, out, lse)
    torch.cuda.synchronize()
    return kc, vc, out, lse


@pytest.mark.parametrize("tk,tv,D,G", [("q8_0", "q4_0", 128, 5), ("q4_0", "q4_0", 128, 5),
                                       ("q8_0", "q8_0", 256, 8), ("f16", "f16", 128, 5)])
def test_noalloc_step_equals_step_twice(tk, tv, D, G):
    # first a larger call, then a smaller one that reuses the array left with
    # the first call's partials
    for B, Hkv, lens, st, seed in ((3, 2, [5000, 1, 2049], 256, 101), (1, 1, [300], 64, 202)):
        note(f"noalloc step {tk}/{tv} D={D} B={B} lens={lens} split={st}")
        need = _lib.kvq_decode_step_noalloc_bytes(B, Hkv * G, D, max(lens), st)
        assert 0 < need <= 64 << 20
        a = one_step(tk, tv, B, Hkv, G, D, lens, st, seed, noalloc=True)
        b = one_step(tk, tv, B, Hkv, G, D, lens, st, seed, noalloc=False)
        for p, r in ((a[0], b[0]), (a[1], b[1])):
            assert torch.equal(p.data, r.data)
            if p.scales is not None:
                assert torch.equal(p.scales, r.scales)
        assert torch.equal(a[2], b[2]), f"out differs by {(a[2] - b[2]).abs().max().item():.3g}"
        assert torch.equal(a[3], b[3])
        assert np.all(np.isfinite(a[2].cpu().numpy()))


def test_noalloc_rejects_oversize_partials():
    dev = "cuda"
    B, Hkv, G, D, L, st = 1, 8, 5, 128, 4096 * 4097, 4096
    assert _lib.kvq_decode_step_noalloc_bytes(B, Hkv * G, D, L, st) > 64 << 20
    kc = C.CachePlanes.alloc("q4_0", B, Hkv, 64, D)
    desc = kc.desc()
    desc.capacity = L      # the call is rejected before anything reads the planes
    x = torch.zeros((B, Hkv, D), dtype=torch.float16, device=dev)
    q = torch.zeros((B, Hkv * G, D), dtype=torch.float16, device=dev)
    lt = torch.ones(B, dtype=torch.int32, device=dev)
    out = torch.zeros((B, Hkv * G, D), dtype=torch.float32, device=dev)
    with pytest.raises(_lib.KVQError) as e:
        _lib.kvq_decode_step_noalloc(desc, desc, x, x, q, lt, B, Hkv * G, Hkv, D, 0.1, L, st, "f32", out)
    assert e.value.status == -5


def test_noalloc_step_graph_replays_equal_eager():
    # the array keeps the last call's partials: each replay must rewrite
    # every partial the merge reads
    B, Hkv, G, D, lens, st = 2, 2, 5, 128, [3000, 700], 256
    note(f"noalloc step in a graph q8_0/q4_0 B={B} lens={lens} split={st}")
    dev = "cuda"
    cap = max(lens)
    k = synth.normal_f16((B, Hkv, cap, D), 303, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 304, dev)
    kc = upload_oracle_planes(*oracle_planes("q8_0", to_host_u16(k)))
    vc = upload_oracle_planes(*oracle_planes("q4_0", to_host_u16(v)))
    q = synth.normal_f16((B, Hkv * G, D), 305, dev)
    k_new = synth.normal_f16((B, Hkv, D), 306, dev)
    v_new = synth.normal_f16((B, Hkv, D), 307, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
    scale = 1 / math.sqrt(D)

    def call():
        _lib.kvq_decode_step_noalloc(kc.desc(), vc.desc(), k_new, v_new, q, lt, B, Hkv * G, Hkv, D, scale,
                                     cap, st, "f32", out, lse)

    got = replay_and_compare(call, [out, lse], plane_tensors(kc, vc), [], "noalloc step")
    # and the eager call is kvq_decode_step's result
    ref = one_step("q8_0", "q4_0", B, Hkv, G, D, lens, st, 303, noalloc=False)
    assert torch.equal(got[0], ref[2]) and torch.equal(got[1], ref[3])
