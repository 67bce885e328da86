"""Calls on two streams at once: kvq_decode_step (and the three calls) keep
no state between calls beyond the caller's buffers, so two problems stepped
concurrently on two streams of default priority give the results each gives
alone, bit for bit."""
import math

import pytest

from .gpu_util import fill_pair, note, plane_tensors, require_gpu

torch = pytest.importorskip("torch")
from quantised_kv_long_amd import cache as C  # noqa: E402
from quantised_kv_long_amd import synth  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    require_gpu()


class Problem:
    def __init__(self, tk, tv, B, Hkv, G, D, lens, st, seed, three_calls=False):
        dev = "cuda"
        cap = max(lens)
        k = synth.normal_f16((B, Hkv, cap, D), seed, dev)
        v = synth.normal_f16((B, Hkv, cap, D), seed + 1, dev)
        self.q = synth.normal_f16((B, Hkv * G, D), seed + 2, dev)
        self.kc, self.vc = fill_pair(tk, tv, k, v, cap)
        self.k_new = synth.normal_f16((B, Hkv, D), seed + 3, dev)
        self.v_new = synth.normal_f16((B, Hkv, D), seed + 4, dev)
        self.lt = torch.tensor(lens, dtype=torch.int32, device=dev)
        self.pos = self.lt - 1
        self.max_len = cap
        self.part = C.Partials(B, Hkv * G, D, cap, st)
        self.out = torch.empty((B, Hkv * G, D), dtype=torch.float32, device=dev)
        self.lse = torch.empty((B, Hkv * G), dtype=torch.float32, device=dev)
        self.scale = 1.0 / math.sqrt(D)
        self.three = three_calls

    def run(self, stream):
        if self.three:
            C.append(self.kc, self.vc, self.k_new.unsqueeze(1), self.v_new.unsqueeze(1), self.pos, self.max_len,
                     stream)
            C.decode(self.kc, self.vc, self.q, self.lt, self.max_len, self.part, self.scale, stream=stream)
            C.combine(self.part, self.lt, self.out, self.lse, stream)
        else:
            C.decode_step(self.kc, self.vc, self.k_new, self.v_new, self.q, self.lt, self.max_len, self.part,
                          self.scale, self.out, self.lse, stream)

    def state(self):
        return [t.clone() for t in [self.out, self.lse] + plane_tensors(self.kc, self.vc)]


def test_two_streams_give_the_results_of_each_alone():
    probs = [Problem("q8_0", "q4_0", 2, 2, 5, 128, [6000, 3100], 512, 2100),
             Problem("q4_0", "q4_0", 1, 2, 8, 256, [4000], 256, 2200),
             Problem("q8_0", "q4_0", 3, 1, 5, 128, [2500, 64, 1025], 128, 2300, three_calls=True)]
    note("two streams: decode steps and three calls of three problems")
    # each alone, in order, on the current stream (each call rewrites its new
    # rows with the same bytes, so repeating a call repeats its results)
    want = []
    for p in probs:
        p.run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        want.append(p.state())
    for p in probs:
        p.out.fill_(float("nan"))
        p.lse.fill_(float("nan"))
    torch.cuda.synchronize()
    s = [torch.cuda.Stream(), torch.cuda.Stream()]     # default priority
    # problems 0 and 2 on one stream, problem 1 on the other; each problem's
    # repeats stay in order on its stream
    for rep in range(4):
        for i, p in enumerate(probs):
            p.run(s[i % 2])
    torch.cuda.synchronize()
    for i, p in enumerate(probs):
        for j, (a, b) in enumerate(zip(p.state(), want[i])):
            assert torch.equal(a, b), f"problem {i}: tensor {j} differs from the call alone"
