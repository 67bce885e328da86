"""kvq_decode_step (quantise-on-write of the new token + split-KV attention +
log-sum-exp merge in one call) on the GPU against the CPU oracle.

The cache holds the oracle's quantisation of rows [0, L_b - 1) and a sentinel
at row L_b - 1, which the step must overwrite with the new token, bit-exact.
Outputs are compared with the oracle's attention over the oracle's planes, and
with the three-call path (kvq_quantize_append, kvq_decode_attn, kvq_combine),
which runs the same kernel code and must agree bit for bit."""
import itertools
import math

import numpy as np
import pytest

from oracle import oracle as O

from .gpu_util import (assert_close, assert_step_matches_three_calls, download_planes, new_row_vmax, note,
                       oracle_planes, oracle_threads, require_gpu, to_host_u16, upload_oracle_planes)

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu
TYPES = ["f16", "q8_0", "q4_0"]
SENT_D, SENT_S = 0xA5, 0x5A5A


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


def step_setup(tk, tv, B, Hkv, G, D, lens, cap, seed):
    """Seeded rows, the oracle's planes of all of them (the expected cache after
    the step), and device planes where row L_b - 1 is a sentinel."""
    dev = "cuda"
    k = synth.normal_f16((B, Hkv, cap, D), seed, dev)
    v = synth.normal_f16((B, Hkv, cap, D), seed + 1, dev)
    q = synth.normal_f16((B, Hkv * G, D), seed + 2, dev)
    kh, vh = to_host_u16(k), to_host_u16(v)
    k_exp, v_exp = oracle_planes(tk, kh), oracle_planes(tv, vh)
    # rows at and beyond L_b hold the sentinel on the device
    k_dev = (k_exp[0], k_exp[1].copy(), k_exp[2].copy())
    v_dev = (v_exp[0], v_exp[1].copy(), v_exp[2].copy())
    for b, L in enumerate(lens):
        for p in (k_dev, v_dev):
            p[1][b, :, L - 1:] = SENT_D
            p[2][b, :, L - 1:] = SENT_S
    # rows beyond L_b are not touched by the step: expect the sentinel there
    for b, L in enumerate(lens):
        for p in (k_exp, v_exp):
            p[1][b, :, L:] = SENT_D
            p[2][b, :, L:] = SENT_S
    kc, vc = upload_oracle_planes(*k_dev), upload_oracle_planes(*v_dev)
    idx = torch.tensor([L - 1 for L in lens], device=dev, dtype=torch.long)
    bi = torch.arange(B, device=dev)
    k_new = k[bi, :, idx].contiguous()   # (B, Hkv, D)
    v_new = v[bi, :, idx].contiguous()
    return kc, vc, q, k_new, v_new, k_exp, v_exp


def run_step(kc, vc, k_new, v_new, q, lens, st, out_dtype=torch.float32, part=None):
    B, Hq, D = q.shape
    lt = torch.tensor(lens, dtype=torch.int32, device=q.device)
    part = part or C.Partials(B, Hq, D, max(lens), st)
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    C.decode_step(kc, vc, k_new, v_new, q, lt, max(lens), part, 1.0 / math.sqrt(D), out, lse)
    torch.cuda.synchronize()
    return out, lse, part


def run_three_calls(kc, vc, k_new, v_new, q, lens, st, out_dtype=torch.float32):
    B, Hq, D = q.shape
    lt = torch.tensor(lens, dtype=torch.int32, device=q.device)
    pos = torch.tensor([L - 1 for L in lens], dtype=torch.int32, device=q.device)
    C.append(kc, vc, k_new.unsqueeze(1).contiguous(), v_new.unsqueeze(1).contiguous(), pos,
             max(lens))
    part = C.Partials(B, Hq, D, max(lens), st)
    C.decode(kc, vc, q, lt, max(lens), part, 1.0 / math.sqrt(D))
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    C.combine(part, lt, out, lse)
    torch.cuda.synchronize()
    return out, lse


def check_planes(p, want, what):
    d, s = download_planes(p)
    assert np.array_equal(d, want[1]), f"{what}: data plane differs from the oracle"
    if want[0] != "f16":
        assert np.array_equal(s, want[2]), f"{what}: scale plane differs from the oracle"


STEP_CASES = [
    # (B, Hkv, G, D, lens, split_tokens): D 128 / 256 take the one-launch
    # matrix-core step where it covers the types, the others the three kernels
    (2, 2, 5, 128, [1000, 65], 256),
    # the new row alone in its split (L - 1 at a split boundary; L = 1)
    (3, 2, 5, 128, [257, 1, 64], 256),
    (1, 2, 8, 256, [777], 128),
    (2, 1, 4, 512, [300, 64], 64),
    (3, 2, 4, 64, [1, 129, 200], 64),
]


@pytest.mark.parametrize("tk,tv", list(itertools.product(TYPES, TYPES)))
@pytest.mark.parametrize("case", range(len(STEP_CASES)))
def test_step_matches_oracle_and_three_calls(tk, tv, case):
    B, Hkv, G, D, lens, st = STEP_CASES[case]
    cap = max(lens) + 9
    note(f"decode_step {tk}/{tv} B={B} Hkv={Hkv} G={G} D={D} lens={lens} split={st}")
    kc, vc, q, k_new, v_new, k_exp, v_exp = step_setup(tk, tv, B, Hkv, G, D, lens, cap, 500 + case)
    out, lse, part = run_step(kc, vc, k_new, v_new, q, lens, st)
    check_planes(kc, k_exp, "K")
    check_planes(vc, v_exp, "V")
    ref, ref_lse = O.attend(to_host_u16(q), k_exp, v_exp, lens, Hkv, 1 / math.sqrt(D),
                            nthreads=oracle_threads())
    got = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    assert_close(got, got_lse, ref, ref_lse, f"step {tk}/{tv} case {case}")

    # the same step again (the new row is rewritten with the same bytes):
    # identical results
    out2, lse2, _ = run_step(kc, vc, k_new, v_new, q, lens, st, part=part)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)

    # the three-call path on a fresh copy of the sentinel cache: the same
    # cache bytes, and the same results up to fp32 rounding (the step merges
    # the new row's decoded values as a term of its split's merge, the
    # attention launch reads the row back inside a tile)
    kc3, vc3, *_ = step_setup(tk, tv, B, Hkv, G, D, lens, cap, 500 + case)
    out3, lse3 = run_three_calls(kc3, vc3, k_new, v_new, q, lens, st)
    check_planes(kc3, k_exp, "K (three calls)")
    check_planes(vc3, v_exp, "V (three calls)")
    assert_step_matches_three_calls(out.cpu().numpy(), lse.cpu().numpy(), out3.cpu().numpy(),
                                    lse3.cpu().numpy(), new_row_vmax(v_new, G), f"step {tk}/{tv} case {case}")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_step_f16_output(tk, tv):
    B, Hkv, G, D, lens, st = 2, 2, 5, 128, [700, 64], 128
    note(f"decode_step f16 out {tk}/{tv}")
    kc, vc, q, k_new, v_new, k_exp, v_exp = step_setup(tk, tv, B, Hkv, G, D, lens, 704, 611)
    out, lse, _ = run_step(kc, vc, k_new, v_new, q, lens, st, torch.float16)
    ref, ref_lse = O.attend(to_host_u16(q), k_exp, v_exp, lens, Hkv, 1 / math.sqrt(D))
    assert_close(out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                 ref, ref_lse, "f16 out")


@pytest.mark.parametrize("D,G", [(128, 5), (512, 4)])
def test_consecutive_steps_cross_split_and_tile_boundaries(D, G):
    """Decode steps one token at a time, sequence 0 from L = 126 to 131 and
    sequence 1 from 62 to 67 (split_tokens 64: the number of splits changes
    between calls), each checked against the oracle, with one set of partials
    for all calls."""
    tk, tv, B, Hkv, st = "q8_0", "q4_0", 2, 2, 64
    L0, n_steps = [126, 62], 6
    cap = max(L0) + n_steps
    dev = "cuda"
    note(f"consecutive decode steps D={D} G={G}")
    k = synth.normal_f16((B, Hkv, cap, D), 700, dev)
    v = synth.normal_f16((B, Hkv, cap, D), 701, dev)
    k_exp, v_exp = oracle_planes(tk, to_host_u16(k)), oracle_planes(tv, to_host_u16(v))
    k_dev = (tk, k_exp[1].copy(), k_exp[2].copy())
    v_dev = (tv, v_exp[1].copy(), v_exp[2].copy())
    for b in range(B):
        for p in (k_dev, v_dev):
            p[1][b, :, L0[b] - 1:] = SENT_D
            p[2][b, :, L0[b] - 1:] = SENT_S
    kc, vc = upload_oracle_planes(*k_dev), upload_oracle_planes(*v_dev)
    part = C.Partials(B, Hkv * G, D, cap, st)
    for i in range(n_steps):
        lens = [L0[b] + i for b in range(B)]
        q = synth.normal_f16((B, Hkv * G, D), 800 + i, dev)
        k_new = torch.stack([k[b, :, lens[b] - 1] for b in range(B)]).contiguous()
        v_new = torch.stack([v[b, :, lens[b] - 1] for b in range(B)]).contiguous()
        out, lse, _ = run_step(kc, vc, k_new, v_new, q, lens, st, part=part)
        ref, ref_lse = O.attend(to_host_u16(q), k_exp, v_exp, lens, Hkv, 1 / math.sqrt(D))
        assert_close(out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                     ref, ref_lse, f"step {i} lens {lens}")
        d, s = download_planes(kc)
        for b in range(B):
            assert np.array_equal(d[b, :, :lens[b]], k_exp[1][b, :, :lens[b]])
            assert np.array_equal(s[b, :, :lens[b]], k_exp[2][b, :, :lens[b]])
            assert np.all(d[b, :, lens[b]:] == SENT_D)


# ------------------------------------------------- full-size workloads

def workload_step(name, tk, tv, heads, layer=0):
    """One decode step of one layer of a workload at its full size, in the launch
    configuration the benchmark times; sampled query heads against the oracle
    restricted to the KV heads they read, and the new rows bit-exact."""
    wl = synth.WORKLOADS[name]
    dev = "cuda"
    lens = wl.lengths()
    cap = max(lens)
    B, Hkv, D = wl.B, wl.Hkv, wl.D
    note(f"decode_step workload {name} {tk}/{tv} layer={layer}")
    k = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "k"), dev)
    v = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "v"), dev)
    q = synth.normal_f16((B, wl.Hq, D), synth.seed_for(wl.seed, layer, "q"), dev)
    if wl.k_outlier_frac:
        ch = synth.outlier_channels(D, synth.seed_for(wl.seed, layer, "aux"), wl.k_outlier_frac)
        k[..., ch] = (k[..., ch].float() * 8).half()
    kt, vt = k.permute(0, 2, 1, 3), v.permute(0, 2, 1, 3)      # (B, Hkv, rows, D)
    k_exp, v_exp = oracle_planes(tk, to_host_u16(kt)), oracle_planes(tv, to_host_u16(vt))
    k_dev = (tk, k_exp[1].copy(), k_exp[2].copy())
    v_dev = (tv, v_exp[1].copy(), v_exp[2].copy())
    for b, L in enumerate(lens):
        for p in (k_dev, v_dev):
            p[1][b, :, L - 1] = SENT_D
            p[2][b, :, L - 1] = SENT_S
    kc, vc = upload_oracle_planes(*k_dev), upload_oracle_planes(*v_dev)
    del k_dev, v_dev
    k_new = torch.stack([kt[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    v_new = torch.stack([vt[b, :, lens[b] - 1] for b in range(B)]).contiguous()
    out, lse, _ = run_step(kc, vc, k_new, v_new, q, lens, wl.split_tokens)
    d, s = download_planes(kc)
    for b, L in enumerate(lens):
        assert np.array_equal(d[b, :, L - 1], k_exp[1][b, :, L - 1])
        assert np.array_equal(s[b, :, L - 1], k_exp[2][b, :, L - 1])
    d, s = download_planes(vc)
    for b, L in enumerate(lens):
        assert np.array_equal(d[b, :, L - 1], v_exp[1][b, :, L - 1])
        assert np.array_equal(s[b, :, L - 1], v_exp[2][b, :, L - 1])
    got = out.cpu().numpy().astype(np.float64)
    got_lse = lse.cpu().numpy().astype(np.float64)
    if heads is None:
        # every head: the whole oracle
        ref, ref_lse = O.attend(to_host_u16(q), k_exp, v_exp, lens, Hkv, 1 / math.sqrt(D),
                                nthreads=oracle_threads())
        assert_close(got, got_lse, ref, ref_lse, f"{name} step")
        return
    for h in heads:
        g = h // wl.G
        sub = lambda p: (p[0], np.ascontiguousarray(p[1][:, g:g + 1]),
                         np.ascontiguousarray(p[2][:, g:g + 1]))
        ref, ref_lse = O.attend(to_host_u16(q[:, h:h + 1]), sub(k_exp), sub(v_exp), lens, 1,
                                1 / math.sqrt(D), nthreads=oracle_threads())
        assert_close(got[:, h:h + 1], got_lse[:, h:h + 1], ref, ref_lse, f"{name} head {h}")


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0"), ("f16", "f16")])
def test_step_stack48_layer_full_size(tk, tv):
    """A layer of the 64k stack, every head."""
    workload_step("stack48_d128_ctx64k", tk, tv, heads=None, layer=5)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
def test_step_long_ctx256k_full_size(tk, tv):
    """The 262144-row layer, every head."""
    workload_step("long_d128_ctx256k", tk, tv, heads=None)


@pytest.mark.parametrize("tk,tv", [("f16", "f16"), ("q8_0", "q8_0"), ("q4_0", "q4_0")])
def test_step_hybrid_d256_ctx32k_full_size(tk, tv):
    """The hybrid model's full-attention layer (16 query / 2 KV heads, head_dim
    256, 32768 rows, outlier K channels), every head."""
    workload_step("hybrid_d256_ctx32k", tk, tv, heads=None)


@pytest.mark.parametrize("tk,tv", [("q4_1", "q4_1"), ("q5_0", "q5_0"), ("q5_1", "q5_1"), ("q6_0", "q6_0"),
                                   ("q6_0", "q4_0"), ("q8_0", "q5_0"), ("q8_0", "q6_0"), ("q5_1", "q4_0")])
def test_step_types_stack48_layer_full_size(tk, tv):
    """The further scalar types' pairs of the 64k types workload, a layer at
    full size in the benchmark's launch configuration: the new row bit-exact
    and sampled heads of three KV heads against the oracle."""
    workload_step("stack48_d128_ctx64k_types", tk, tv, heads=[0, 17, 39], layer=2)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q5_1", "q4_0"), ("q6_0", "q6_0"), ("q4_1", "q4_1"),
                                   ("q5_0", "q5_0"), ("q8_0", "q6_0")])
def test_step_types_hybrid_d256_ctx32k_full_size(tk, tv):
    """The hybrid layer (head_dim 256, 2 KV heads, outlier K channels) with the
    pairs its types profile measures, every head."""
    workload_step("hybrid_d256_ctx32k", tk, tv, heads=None)


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q4_0")])
@pytest.mark.parametrize("name", ["batch16_ragged", "batch16_ragged_d512"])
def test_step_batch16_ragged_full_size(name, tk, tv):
    """16 ragged sequences (16k-128k rows), head_dim 128 and 512, every head."""
    workload_step(name, tk, tv, heads=None)


# ------------------------------------------- the new row's quantisation

def edge_blocks():
    """32-value fp16 blocks that exercise every branch of the block quantiser
    on finite inputs: the worked blocks, zero and negative-zero blocks,
    magnitude ties (the first index must win), the maximum in the last lane,
    halfway values, tiny and huge scales, the largest finite values."""
    from .test_oracle_quant import WORKED
    out = [x.copy() for _, _, x, _, _ in WORKED]
    f = lambda a: np.asarray(a, np.float16).view(np.uint16)
    rng = np.random.default_rng(5)
    out.append(np.zeros(32, np.uint16))
    out.append(np.full(32, 0x8000, np.uint16))
    b = np.zeros(32, np.float16); b[3], b[17] = 2.0, -2.0; out.append(b.view(np.uint16))
    b = np.zeros(32, np.float16); b[17], b[3] = 2.0, -2.0; out.append(b.view(np.uint16))
    b = rng.standard_normal(32).astype(np.float16); b[31] = 9.0; out.append(b.view(np.uint16))
    out.append(f((rng.integers(-40, 40, 32) / 8.0)))
    out.append(f(rng.standard_normal(32) * 1e-5))
    out.append(f(rng.standard_normal(32) * 2000.0))
    b = rng.standard_normal(32).astype(np.float16); b[12] = 65504.0; out.append(b.view(np.uint16))
    b = rng.standard_normal(32).astype(np.float16); b[0] = -65504.0; b[31] = 65504.0
    out.append(b.view(np.uint16))
    out.append(f(rng.standard_normal(32)))
    return out


@pytest.mark.parametrize("tk,tv", [("q8_0", "q4_0"), ("q4_0", "q8_0"), ("q8_0", "q8_0"),
                                   ("q4_0", "q4_0"), ("f16", "q4_0")])
def test_step_new_row_edge_blocks_bit_exact(tk, tv):
    """The decode step's own write of the new row (one lane per value in the
    matrix-core kernel) against the oracle's quantiser, block by block."""
    blocks = edge_blocks()
    D = 128
    nb = D // 32
    while len(blocks) % nb:
        blocks.append(np.zeros(32, np.uint16))
    Hkv = len(blocks) // nb
    B, G, L, st = 1, 1, 65, 64
    dev = "cuda"
    note(f"decode_step edge blocks {tk}/{tv} Hkv={Hkv}")
    rows = np.stack(blocks).reshape(1, Hkv, D)                   # the new rows
    vrows = np.roll(rows, 1, axis=1).copy()
    base_k = synth.normal_f16((B, Hkv, L, D), 901, dev)
    base_v = synth.normal_f16((B, Hkv, L, D), 902, dev)
    kh, vh = to_host_u16(base_k), to_host_u16(base_v)
    kh[:, :, L - 1], vh[:, :, L - 1] = rows, vrows
    k_exp, v_exp = oracle_planes(tk, kh), oracle_planes(tv, vh)
    k_dev = (tk, k_exp[1].copy(), k_exp[2].copy())
    v_dev = (tv, v_exp[1].copy(), v_exp[2].copy())
    for p in (k_dev, v_dev):
        p[1][:, :, L - 1] = SENT_D
        p[2][:, :, L - 1] = SENT_S
    kc, vc = upload_oracle_planes(*k_dev), upload_oracle_planes(*v_dev)
    k_new = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.float16)
    v_new = torch.from_numpy(vrows.view(np.int16)).to(dev).view(torch.float16)
    q = synth.normal_f16((B, Hkv * G, D), 903, dev)
    run_step(kc, vc, k_new, v_new, q, [L], st)        # the rows only; outputs are checked elsewhere
    check_planes(kc, k_exp, "K")
    check_planes(vc, v_exp, "V")
