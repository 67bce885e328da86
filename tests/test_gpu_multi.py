"""Decode attention for n_q query tokens at once (kvq_decode_attn_multi, the
verify step of speculative decoding) against the oracle: token i of a
sequence of L rows attends over rows [0, L - n_q + 1 + i), which the oracle
computes as plain attention with that length."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, fill_pair, note, oracle_threads, planes_to_oracle, require_gpu,
                       to_host_u16)

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import _lib  # noqa: E402
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def run_multi(kc, vc, q, lens, st):
    """q (B, n_q, Hq, D): kvq_decode_attn_multi + kvq_combine over n_q * Hq heads.
    Returns host (out (B, n_q, Hq, D), lse (B, n_q, Hq)) fp64."""
    B, nq, Hq, D = q.shape
    lt = torch.tensor(lens, dtype=torch.int32, device=q.device)
    part = C.Partials(B, nq * Hq, D, max(lens), st)
    C.decode_multi(kc, vc, q, lt, max(lens), part, 1.0 / math.sqrt(D))
    out = torch.empty((B, nq * Hq, D), dtype=torch.float32, device=q.device)
    lse = torch.empty((B, nq * Hq), dtype=torch.float32, device=q.device)
    C.combine(part, lt, out, lse)
    torch.cuda.synchronize()
    return (out.view(B, nq, Hq, D).cpu().numpy().astype(np.float64),
            lse.view(B, nq, Hq).cpu().numpy().astype(np.float64))


def oracle_multi(kc, vc, q, lens, heads=None):
    B, nq, Hq, D = q.shape
    Hkv = kc.Hkv
    out = np.zeros((B, nq, Hq, D))
    lse = np.zeros((B, nq, Hq))
    for i in range(nq):
        li = [L - nq + 1 + i for L in lens]
        o, l = O.attend(to_host_u16(q[:, i]), planes_to_oracle(kc), planes_to_oracle(vc), li, Hkv,
                        1 / math.sqrt(D), nthreads=oracle_threads())
        out[:, i], lse[:, i] = o, l
    return out, lse


CASES = [
    # (B, Hkv, G, D, lens, split_tokens, n_q): n_q * G <= 16 score columns
    (2, 2, 5, 128, [1000, 70], 256, 3),
    (1, 2, 8, 256, [777], 128, 2),
    (2, 1, 4, 512, [300, 64], 64, 4),
    (3, 2, 1, 128, [16, 40, 1025], 64, 16),   # every row of the first sequence is a query token
    (2, 2, 2, 128, [65, 129], 64, 7),         # query tokens across a split boundary
]


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "f16"), ("q8_0", "q8_0"),
                                   ("q4_0", "f16")])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_multi_matches_oracle(tk, tv, case):
    B, Hkv, G, D, lens, st, nq = CASES[case]
    note(f"multi {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} lens={lens} split={st} n_q={nq}")
    dev = "cuda"
    seed = 2600 + case
    kc, vc = fill_pair(tk, tv, synth.normal_f16((B, Hkv, max(lens), D), seed, dev),
                       synth.normal_f16((B, Hkv, max(lens), D), seed + 1, dev))
    q = synth.normal_f16((B, nq, Hkv * G, D), seed + 2, dev)
    out, lse = run_multi(kc, vc, q, lens, st)
    ref, ref_lse = oracle_multi(kc, vc, q, lens)
    assert_close(out.reshape(B, -1, D), lse.reshape(B, -1), ref.reshape(B, -1, D), ref_lse.reshape(B, -1),
                 f"multi {tk}/{tv} case {case}")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "f16"), ("q8_0", "q8_0")])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_step_multi_is_append_attention_merge_bit_for_bit(tk, tv, case):
    """kvq_decode_step_multi equals kvq_quantize_append of the n_q new rows at
    rows L - n_q .. L - 1, kvq_decode_attn_multi and kvq_combine over n_q * Hq
    heads, bit for bit: cache rows, partials of every split that holds rows,
    output and LSE.  Cases include new rows that straddle a split boundary."""
    B, Hkv, G, D, lens, st, nq = CASES[case]
    note(f"step_multi vs three calls {tk}/{tv} case {case}")
    dev = "cuda"
    seed = 4100 + case
    cap = max(lens) + 5
    k = synth.normal_f16((B, Hkv, cap, D), seed, dev)
    v = synth.normal_f16((B, Hkv, cap, D), seed + 1, dev)
    q = synth.normal_f16((B, nq, Hkv * G, D), seed + 2, dev)
    k_new = synth.normal_f16((B, nq, Hkv, D), seed + 3, dev)
    v_new = synth.normal_f16((B, nq, Hkv, D), seed + 4, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    res = []
    for fused in (True, False):
        kc, vc = fill_pair(tk, tv, k, v)          # the rows the step writes hold other values first
        part = C.Partials(B, nq * Hkv * G, D, max(lens), st)
        out = torch.full((B, nq * Hkv * G, D), 7.0, dtype=torch.float32, device=dev)
        lse = torch.full((B, nq * Hkv * G), 7.0, dtype=torch.float32, device=dev)
        if fused:
            C.decode_step_multi(kc, vc, k_new, v_new, q, lt, max(lens), part, scale, out, lse)
        else:
            C.append(kc, vc, k_new, v_new, lt - nq, max(lens))
            C.decode_multi(kc, vc, q, lt, max(lens), part, scale)
            C.combine(part, lt, out, lse)
        torch.cuda.synchronize()
        res.append((kc, vc, part, out, lse))
    (k1, v1, p1, o1, l1), (k2, v2, p2, o2, l2) = res
    for a, c, what in ((k1, k2, "K"), (v1, v2, "V")):
        assert torch.equal(a.data, c.data), f"{what} data"
        if a.scales is not None:
            assert torch.equal(a.scales, c.scales), f"{what} scales"
    for bi, L in enumerate(lens):
        S = -(-L // st)
        assert torch.equal(p1.o[bi, :, :S], p2.o[bi, :, :S]) and torch.equal(p1.lse[bi, :, :S], p2.lse[bi, :, :S])
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_one_query_token_is_the_decode_call_bit_for_bit():
    B, Hkv, G, D, lens, st = 2, 2, 5, 128, [3000, 700], 256
    note("multi n_q=1 vs decode")
    dev = "cuda"
    kc, vc = fill_pair("q8_0", "q4_0", synth.normal_f16((B, Hkv, max(lens), D), 2701, dev),
                       synth.normal_f16((B, Hkv, max(lens), D), 2702, dev))
    q = synth.normal_f16((B, 1, Hkv * G, D), 2703, dev)
    lt = torch.tensor(lens, dtype=torch.int32, device=dev)
    p1 = C.Partials(B, Hkv * G, D, max(lens), st)
    p2 = C.Partials(B, Hkv * G, D, max(lens), st)
    C.decode_multi(kc, vc, q, lt, max(lens), p1, 1 / math.sqrt(D))
    C.decode(kc, vc, q[:, 0].contiguous(), lt, max(lens), p2, 1 / math.sqrt(D))
    torch.cuda.synchronize()
    # every split that holds a row (the others are written by neither call)
    for b, L in enumerate(lens):
        S = -(-L // st)
        assert torch.equal(p1.o[b, :, :S], p2.o[b, :, :S]) and torch.equal(p1.lse[b, :, :S], p2.lse[b, :, :S])


def test_multi_rejects_what_it_does_not_cover():
    dev = "cuda"
    kc, vc = fill_pair("q8_0", "q4_0", synth.normal_f16((1, 1, 64, 64), 1, dev),
                       synth.normal_f16((1, 1, 64, 64), 2, dev))
    q = synth.normal_f16((1, 2, 4, 64), 3, dev)
    part = C.Partials(1, 8, 64, 64, 64)
    lt = torch.tensor([64], dtype=torch.int32, device=dev)
    with pytest.raises(_lib.KVQError):           # head_dim 64: vector-ALU kernel only
        C.decode_multi(kc, vc, q, lt, 64, part, 0.125)
    kc, vc = fill_pair("q8_0", "q4_0", synth.normal_f16((1, 1, 64, 128), 1, dev),
                       synth.normal_f16((1, 1, 64, 128), 2, dev))
    q = synth.normal_f16((1, 5, 4, 128), 3, dev)  # 5 tokens x 4 heads = 20 columns > 16
    part = C.Partials(1, 20, 128, 64, 64)
    with pytest.raises(_lib.KVQError):
        C.decode_multi(kc, vc, q, lt, 64, part, 0.125)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_multi_full_size_64k_three_tokens(tk, tv):
    """A 64k layer of the stack workload verifying 3 draft tokens (15 of the 16
    columns); sampled heads of every token against the oracle restricted to the
    KV head they read."""
    wl = synth.WORKLOADS["stack48_d128_ctx64k"]
    B, Hkv, D, G, L, nq = wl.B, wl.Hkv, wl.D, wl.G, wl.ctx, 3
    dev = "cuda"
    note(f"multi full size {tk}/{tv}")
    kc, vc = fill_pair(tk, tv, synth.normal_f16((B, Hkv, L, D), 2801, dev),
                       synth.normal_f16((B, Hkv, L, D), 2802, dev))
    q = synth.normal_f16((B, nq, wl.Hq, D), 2803, dev)
    out, lse = run_multi(kc, vc, q, [L], wl.split_tokens)
    for h in (0, 21, 39):
        g = h // G
        sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]), np.ascontiguousarray(p[2][:, g:g + 1]))
        for i in range(nq):
            ref, ref_lse = O.attend(to_host_u16(q[:, i, h:h + 1]), sub(planes_to_oracle(kc)),
                                    sub(planes_to_oracle(vc)), [L - nq + 1 + i], 1, 1 / math.sqrt(D),
                                    nthreads=oracle_threads())
            assert_close(out[:, i, h:h + 1], lse[:, i, h:h + 1], ref, ref_lse, f"token {i} head {h}")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_step_multi_full_size_64k_three_tokens(tk, tv):
    """A layer of the 64k workload with three query tokens, in the launch
    configuration of the benchmark (kvq_decode_step_multi, 1024-row splits):
    the step writes the three new rows and attends; sampled query heads of
    every token against the oracle over the same rows (its own bytes)."""
    wl = synth.WORKLOADS["stack48_d128_ctx64k"]
    B, Hkv, D, G, L, st, nq = wl.B, wl.Hkv, wl.D, wl.G, wl.ctx, wl.split_tokens, 3
    dev = "cuda"
    note(f"step_multi full size {tk}/{tv}")
    # rows L - 3 .. L - 1 are the new tokens: the oracle's planes hold its own
    # quantisation of them, the step writes them from k_new / v_new
    k = synth.normal_f16((B, Hkv, L, D), 4201, dev)
    v = synth.normal_f16((B, Hkv, L, D), 4202, dev)
    kc, vc = fill_pair(tk, tv, k, v)
    q = synth.normal_f16((B, nq, wl.Hq, D), 4203, dev)
    k_new = k[:, :, L - nq:].transpose(1, 2).contiguous()
    v_new = v[:, :, L - nq:].transpose(1, 2).contiguous()
    del k, v
    lt = torch.tensor([L] * B, dtype=torch.int32, device=dev)
    part = C.Partials(B, nq * wl.Hq, D, L, st)
    out = torch.empty((B, nq * wl.Hq, D), dtype=torch.float32, device=dev)
    lse = torch.empty((B, nq * wl.Hq), dtype=torch.float32, device=dev)
    C.decode_step_multi(kc, vc, k_new, v_new, q, lt, L, part, 1.0 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    out = out.view(B, nq, wl.Hq, D).cpu().numpy().astype(np.float64)
    lse = lse.view(B, nq, wl.Hq).cpu().numpy().astype(np.float64)
    kp, vp = planes_to_oracle(kc), planes_to_oracle(vc)
    for h in (0, 17, 39):
        g = h // G
        sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]), np.ascontiguousarray(p[2][:, g:g + 1]))
        for i in range(nq):
            ref, ref_lse = O.attend(to_host_u16(q[:, i, h:h + 1]), sub(kp), sub(vp), [L - nq + 1 + i], 1,
                                    1 / math.sqrt(D), nthreads=oracle_threads())
            assert_close(out[:, i, h:h + 1], lse[:, i, h:h + 1], ref, ref_lse, f"token {i} head {h}")
