#!/usr/bin/env python3
"""Decode-attention benchmark over a block-quantised KV cache on one MI355X.

One step = the whole hot path for every layer of the workload: quantise-on-write
of one new token per sequence, split-KV decode attention over every row and
the exact log-sum-exp combine, on inputs already resident in HBM.  The timed
path is kvq_decode_step (two launches per layer where the matrix-core kernel
covers the shape: attention with the new row's write, then the merge); the same step as three calls (kvq_quantize_append,
kvq_decode_attn, kvq_combine) and the attention launch alone are timed beside
it and reported per arm.  The default workload is the 48-layer stack at 65536 rows
(40 query / 8 KV heads, head_dim 128) with the f16, q8_0K/q4_0V and q4_0/q4_0
arms; the headline value is the q8_0K/q4_0V arm.

value = stored KV bytes read per step / step time (GB/s, 1e9 bytes/s), where
stored bytes = sum_b L_b * Hkv * (row bytes of K + row bytes of V) summed over
layers (f16 2*D, q8_0 34*D/32, q4_0 18*D/32 bytes per row).

Prints ONE JSON line.  Steps are captured once in a HIP graph and replayed
(--no-graph replays eager launches instead).

Two further modes time the wider calls on the same workloads:
  --queries N  N query tokens per sequence and step (the verify step of
               speculative decoding): kvq_decode_step_multi (the attention
               kernel writes the N rows, then kvq_combine over N * Hq heads);
  --window W   a mixed cache: the last W rows of each sequence in an fp16 window,
               the rest in the arm's types; append the new token to the window,
               attention over both regions in one launch (kvq_decode_attn_mixed),
               kvq_combine_regions.  The eviction of a full window into the
               tail (kvq_quantize_rows) is timed on its own and reported per
               layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn KV GB/s (stored bytes) and % of MI355X HBM peak; µs/step at 64k–256k"
HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
# sources of the attention kernel: a traffic record taken from the counters is
# used only while these are unchanged
KERNEL_SOURCES = ["decode_mfma.hip", "kvq_device.hpp", "kvq_internal.hpp", "kvq_quant.hpp"]


def kernel_sources_sha256() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "quantised_kv_long_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def traffic_record(workload: str, tk: str, tv: str):
    """Measured HBM bytes per launch of the attention kernel for this workload
    and arm, from a committed rocprofv3 counter summary (FETCH_SIZE and
    WRITE_SIZE per dispatch, scaled by the calibration on a copy of known
    size), or None when there is none for the current kernel sources."""
    import glob
    import re
    sha = kernel_sources_sha256()
    for path in sorted(glob.glob(os.path.join(PROFILES, "*.md"))):
        for line in open(path, encoding="utf-8"):
            if not line.startswith("traffic-record:"):
                continue
            kv = dict(re.findall(r"(\w+)=(\S+)", line))
            if (kv.get("workload") == workload and kv.get("arm") == f"{tk}/{tv}"
                    and kv.get("sources_sha256") == sha):
                return int(kv["fetch_bytes"]), int(kv["write_bytes"]), os.path.basename(path)
    return None


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="stack48_d128_ctx64k")
    p.add_argument("--arms", default=None, help="comma list like q8_0/q4_0,f16/f16 (default: all)")
    p.add_argument("--variant", default="auto", choices=["auto", "valu", "mfma"])
    p.add_argument("--split-tokens", type=int, default=None)
    p.add_argument("--queries", type=int, default=1,
                   help="query tokens per sequence and step (> 1: multi-query decode, "
                        "kvq_decode_step_multi)")
    p.add_argument("--window", type=int, default=0,
                   help="> 0: mixed cache, the last WINDOW rows of each sequence in an fp16 window "
                        "and the rest in the arm's types (kvq_decode_attn_mixed and "
                        "kvq_combine_regions)")
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-long-ctx", dest="long_ctx", action="store_false",
                   help="skip the 262144-row layer that the default 64k run also times")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="approximate CPU time budget of the oracle baseline (0 disables it)")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only copy MIB MiB device to device once (a plain copy kernel of known "
                        "size, for scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    p.add_argument("--replicas", type=int, default=0,
                   help="cache copies rotated per step so the working set exceeds the 256 MB "
                        "last-level cache (0 = automatic)")
    return p.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


class Arm:
    """All device state of one (K type, V type) arm of a workload."""

    def __init__(self, wl, tk, tv, split_tokens, replicas, dev, queries=1, window=0, win_split_tokens=None):
        import torch

        from quantised_kv_long_amd import _lib
        from quantised_kv_long_amd import cache as C
        from quantised_kv_long_amd import synth

        self.tk, self.tv = tk, tv
        self.lens = wl.lengths()
        cap = max(self.lens)
        B, Hkv, Hq, D = wl.B, wl.Hkv, wl.Hq, wl.D
        self.wl = wl
        N, W = queries, window
        self.N, self.W = N, W
        if W and (N != 1 or min(self.lens) <= W):
            raise ValueError("a window needs one query token and sequences longer than the window")
        self.layers = []  # per layer: dict of planes and per-step tensors
        zero = torch.zeros(B, dtype=torch.int32, device=dev)
        n_copies = wl.layers * replicas
        for i in range(n_copies):
            layer = i % wl.layers
            k = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "k"), dev)
            v = synth.normal_f16((B, cap, Hkv, D), synth.seed_for(wl.seed, layer, "v"), dev)
            q = synth.normal_f16((B, N, Hq, D) if N > 1 else (B, Hq, D),
                                 synth.seed_for(wl.seed, layer, "q"), dev)
            if wl.k_outlier_frac:
                ch = synth.outlier_channels(D, synth.seed_for(wl.seed, layer, "aux"), wl.k_outlier_frac)
                k[..., ch] = (k[..., ch].float() * 8).half()
            if wl.needle:
                p = self.lens[0] // 3
                q0 = q[:, 0] if N > 1 else q
                for g in range(Hkv):
                    k[0, p, g] = synth.needle_row(q0[0, g * wl.G], synth.seed_for(wl.seed, g, "aux"))
            kc = C.CachePlanes.alloc(tk, B, Hkv, cap, D, dev)
            vc = C.CachePlanes.alloc(tv, B, Hkv, cap, D, dev)
            entry = dict(kc=kc, vc=vc, q=q)
            if W:
                # tail: rows [0, L - W) in the arm's types (capacity L, room for
                # an eviction); window: rows [0, W - 1) as fp16, the step
                # writes row W - 1
                C.append(kc, vc, k[:, :cap - W].contiguous(), v[:, :cap - W].contiguous(), zero, cap - W)
                kw = C.CachePlanes.alloc("f16", B, Hkv, W, D, dev)
                vw = C.CachePlanes.alloc("f16", B, Hkv, W, D, dev)
                C.append(kw, vw, k[:, cap - W:cap - 1].contiguous(), v[:, cap - W:cap - 1].contiguous(),
                         zero, W - 1)
                entry.update(kw=kw, vw=vw)
            else:
                C.append(kc, vc, k[:, :cap - N].contiguous(), v[:, :cap - N].contiguous(), zero, cap - N)
            del k, v
            entry["knew"] = synth.normal_f16((B, N, Hkv, D), synth.seed_for(wl.seed, layer, "k_new"), dev)
            entry["vnew"] = synth.normal_f16((B, N, Hkv, D), synth.seed_for(wl.seed, layer, "v_new"), dev)
            self.layers.append(entry)
        torch.cuda.synchronize()
        if W and len(set(self.lens)) != 1:
            raise ValueError("the window mode takes sequences of one length")
        self.pos = torch.tensor([(W if W else L) - N for L in self.lens], dtype=torch.int32, device=dev)
        self.lens_t = torch.tensor(self.lens, dtype=torch.int32, device=dev)
        self.max_len = cap
        if W and split_tokens is None:
            # one round of resident workgroups covers both regions
            row_t = sum(_lib.kvq_data_row_bytes(t, D) + _lib.kvq_scale_row_bytes(t, D) for t in (tk, tv))
            split_tokens, win_split_tokens = C.mixed_splits(cap - W, W, row_t, 4 * D, B, Hkv, D)
        elif W and win_split_tokens is None:
            win_split_tokens = split_tokens
        self.split_tokens, self.win_split_tokens = split_tokens, win_split_tokens
        self.part = C.Partials(B, N * Hq, D, cap, split_tokens, dev)
        self.out = torch.empty((B, N * Hq, D), dtype=torch.float16, device=dev)
        self.stored_bytes_layer = kc.stored_bytes(self.lens) + vc.stored_bytes(self.lens)
        if W:
            self.tail_lens = [L - W for L in self.lens]
            self.tail_lens_t = torch.tensor(self.tail_lens, dtype=torch.int32, device=dev)
            self.win_lens_t = torch.full((B,), W, dtype=torch.int32, device=dev)
            self.evict_pos = self.tail_lens_t
            self.part_w = C.Partials(B, Hq, D, W, win_split_tokens, dev)
            kw = self.layers[0]["kw"]
            self.stored_bytes_layer = (kc.stored_bytes(self.tail_lens) + vc.stored_bytes(self.tail_lens) +
                                       kw.stored_bytes([W] * B) * 2)
        self.stored_bytes_step = self.stored_bytes_layer * wl.layers
        self.replicas = replicas

    def prepare_calls(self, variant):
        """Pre-marshalled C calls (descriptors and pointers built once)."""
        import ctypes

        from quantised_kv_long_amd import _lib

        lib = _lib.load()
        wl = self.wl
        vcode = _lib.VARIANTS[variant]
        scale = 1.0 / math.sqrt(wl.D)
        part = self.part
        self.calls = []
        N, W, Hq = self.N, self.W, wl.Hq
        for L in self.layers:
            kd, vd = L["kc"].desc(), L["vc"].desc()
            L["descs"] = (kd, vd)  # keep alive
            if W:
                kwd, vwd = L["kw"].desc(), L["vw"].desc()
                L["wdescs"] = (kwd, vwd)
                pw = self.part_w
                P = ctypes.c_void_p
                regions = ((P * 2)(part.o.data_ptr(), pw.o.data_ptr()), (P * 2)(part.lse.data_ptr(), pw.lse.data_ptr()),
                           (P * 2)(self.tail_lens_t.data_ptr(), self.win_lens_t.data_ptr()),
                           (ctypes.c_int * 2)(part.split_tokens, pw.split_tokens),
                           (ctypes.c_int * 2)(part.max_splits, pw.max_splits))
                L["regions"] = regions
                self.calls.append(dict(
                    append=(ctypes.byref(kwd), ctypes.byref(vwd), L["knew"].data_ptr(), L["vnew"].data_ptr(),
                            self.pos.data_ptr(), wl.B, 1, wl.Hkv, wl.D, W),
                    decode=(ctypes.byref(kd), ctypes.byref(vd), L["q"].data_ptr(), self.tail_lens_t.data_ptr(),
                            wl.B, Hq, wl.Hkv, wl.D, scale, max(self.tail_lens), part.split_tokens,
                            part.max_splits, part.o.data_ptr(), part.lse.data_ptr(), vcode),
                    decode_w=(ctypes.byref(kwd), ctypes.byref(vwd), L["q"].data_ptr(), self.win_lens_t.data_ptr(),
                              wl.B, Hq, wl.Hkv, wl.D, scale, W, pw.split_tokens, pw.max_splits,
                              pw.o.data_ptr(), pw.lse.data_ptr(), vcode),
                    step_mixed=(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kwd), ctypes.byref(vwd),
                                L["knew"].data_ptr(), L["vnew"].data_ptr(), L["q"].data_ptr(),
                                self.tail_lens_t.data_ptr(), self.win_lens_t.data_ptr(), wl.B, Hq, wl.Hkv,
                                wl.D, scale, max(self.tail_lens), part.split_tokens, part.max_splits,
                                part.o.data_ptr(), part.lse.data_ptr(), W, pw.split_tokens, pw.max_splits,
                                pw.o.data_ptr(), pw.lse.data_ptr(), 0, self.out.data_ptr(), None),
                    mixed=(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kwd), ctypes.byref(vwd),
                           L["q"].data_ptr(), self.tail_lens_t.data_ptr(), self.win_lens_t.data_ptr(),
                           wl.B, Hq, wl.Hkv, wl.D, scale, max(self.tail_lens), part.split_tokens, part.max_splits,
                           part.o.data_ptr(), part.lse.data_ptr(), W, pw.split_tokens, pw.max_splits,
                           pw.o.data_ptr(), pw.lse.data_ptr()),
                    combine=(2, *regions, wl.B, Hq, wl.D, 0, self.out.data_ptr(), None),
                    evict=(ctypes.byref(kd), ctypes.byref(vd), ctypes.byref(kwd), ctypes.byref(vwd),
                           self.win_lens_t.data_ptr(), self.evict_pos.data_ptr(), wl.B, W, wl.Hkv, wl.D,
                           self.max_len),
                ))
                continue
            if N > 1:
                self.calls.append(dict(
                    append=(ctypes.byref(kd), ctypes.byref(vd), L["knew"].data_ptr(), L["vnew"].data_ptr(),
                            self.pos.data_ptr(), wl.B, N, wl.Hkv, wl.D, self.max_len),
                    step_multi=(ctypes.byref(kd), ctypes.byref(vd), L["knew"].data_ptr(), L["vnew"].data_ptr(),
                                L["q"].data_ptr(), self.lens_t.data_ptr(), wl.B, N, Hq, wl.Hkv, wl.D, scale,
                                self.max_len, part.split_tokens, part.max_splits, part.o.data_ptr(),
                                part.lse.data_ptr(), 0, self.out.data_ptr(), None),
                    multi=(ctypes.byref(kd), ctypes.byref(vd), L["q"].data_ptr(), self.lens_t.data_ptr(),
                           wl.B, N, Hq, wl.Hkv, wl.D, scale, self.max_len, part.split_tokens,
                           part.max_splits, part.o.data_ptr(), part.lse.data_ptr()),
                    combine=(part.o.data_ptr(), part.lse.data_ptr(), self.lens_t.data_ptr(), wl.B, N * Hq,
                             wl.D, part.split_tokens, part.max_splits, 0, self.out.data_ptr(), None),
                ))
                continue
            self.calls.append(dict(
                step=(ctypes.byref(kd), ctypes.byref(vd), L["knew"].data_ptr(), L["vnew"].data_ptr(),
                      L["q"].data_ptr(), self.lens_t.data_ptr(), wl.B, wl.Hq, wl.Hkv, wl.D, scale,
                      self.max_len, part.split_tokens, part.max_splits, part.o.data_ptr(),
                      part.lse.data_ptr(), 0, self.out.data_ptr(), None),
                append=(ctypes.byref(kd), ctypes.byref(vd), L["knew"].data_ptr(), L["vnew"].data_ptr(),
                        self.pos.data_ptr(), wl.B, 1, wl.Hkv, wl.D, self.max_len),
                decode=(ctypes.byref(kd), ctypes.byref(vd), L["q"].data_ptr(), self.lens_t.data_ptr(),
                        wl.B, wl.Hq, wl.Hkv, wl.D, scale, self.max_len, part.split_tokens,
                        part.max_splits, part.o.data_ptr(), part.lse.data_ptr(), vcode),
                combine=(part.o.data_ptr(), part.lse.data_ptr(), self.lens_t.data_ptr(), wl.B, wl.Hq,
                         wl.D, part.split_tokens, part.max_splits, 0, self.out.data_ptr(), None),
            ))
        self.lib = lib
        self.one_call = variant == "auto"

    def step(self, stream, rep=0, mode="step"):
        """One step over all layers of replica `rep`: mode "step" (kvq_decode_step),
        "three" (append + decode + combine) or "decode" (the attention launch alone).
        Multi-query: "step" is kvq_decode_step_multi (the attention kernel writes
        the N tokens); "three" appends them, runs kvq_decode_attn_multi and
        kvq_combine.  Window: "step" is kvq_decode_step_mixed (the attention
        kernel writes the token into the fp16 window); "three" appends the token,
        runs kvq_decode_attn_mixed and kvq_combine_regions.  With a forced
        variant both run one kvq_decode_attn_variant per region instead."""
        lib = self.lib
        n = self.wl.layers
        for c in self.calls[rep * n:(rep + 1) * n]:
            if self.W:
                if mode == "step" and self.one_call:
                    assert lib.kvq_decode_step_mixed(*c["step_mixed"], stream) == 0
                    continue
                if mode != "decode":
                    assert lib.kvq_quantize_append(*c["append"], stream) == 0
                if self.one_call:
                    assert lib.kvq_decode_attn_mixed(*c["mixed"], stream) == 0
                else:
                    assert lib.kvq_decode_attn_variant(*c["decode"], stream) == 0
                    assert lib.kvq_decode_attn_variant(*c["decode_w"], stream) == 0
                if mode != "decode":
                    assert lib.kvq_combine_regions(*c["combine"], stream) == 0
                continue
            if self.N > 1:
                if mode == "step":
                    assert lib.kvq_decode_step_multi(*c["step_multi"], stream) == 0
                    continue
                if mode != "decode":
                    assert lib.kvq_quantize_append(*c["append"], stream) == 0
                assert lib.kvq_decode_attn_multi(*c["multi"], stream) == 0
                if mode != "decode":
                    assert lib.kvq_combine(*c["combine"], stream) == 0
                continue
            if mode == "step":
                rc = lib.kvq_decode_step(*c["step"], stream)
                assert rc == 0, rc
                continue
            if mode == "three":
                rc = lib.kvq_quantize_append(*c["append"], stream)
                assert rc == 0, rc
            rc = lib.kvq_decode_attn_variant(*c["decode"], stream)
            assert rc == 0, rc
            if mode == "three":
                rc = lib.kvq_combine(*c["combine"], stream)
                assert rc == 0, rc


MODES = ("step", "three", "decode")


def time_arm(arm, steps, warmup, use_graph, variant):
    """ms per step for every mode, timed with HIP events on the stream the
    launches go to.  With graphs, the K timed steps of a mode are captured as
    one graph (step i uses cache replica i mod R) and replayed once, so launch
    gaps between graph replays do not enter the per-launch times."""
    import torch

    arm.prepare_calls(variant)
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    R = arm.replicas
    for mode in MODES:
        for i in range(warmup):
            arm.step(sh, i % R, mode)
    torch.cuda.synchronize()

    graphs = {}
    if use_graph:
        for m in MODES:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                for i in range(steps):
                    arm.step(cs, i % R, m)
            graphs[m] = g
            g.replay()                     # untimed: first replay of the new graph
        torch.cuda.synchronize()

    ms = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for mode in MODES:
        torch.cuda.synchronize()
        e0.record(stream)
        if use_graph:
            graphs[mode].replay()
        else:
            for i in range(steps):
                arm.step(sh, i % R, mode)
        e1.record(stream)
        torch.cuda.synchronize()
        ms[mode] = e0.elapsed_time(e1) / steps

    # distribution of the step time (mode "step"): graphs of n consecutive
    # steps (n steps cover about half a millisecond, so a graph launch's own
    # overhead is a small share of a sample), each replayed and timed on its
    # own; a sample is the replay's time divided by n
    samples = []
    per_sample = max(1, math.ceil(500.0 / max(ms["step"] * 1e3, 1e-3)))
    if use_graph:
        graphs_n = []
        for r in range(R):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                cs = torch.cuda.current_stream().cuda_stream
                for j in range(per_sample):
                    arm.step(cs, (r + j) % R, "step")
            graphs_n.append(g)
            g.replay()
        torch.cuda.synchronize()
        n_samples = max(steps, 20)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(n_samples)]
        for i in range(n_samples):
            ev[i][0].record(stream)
            graphs_n[i % R].replay()
            ev[i][1].record(stream)
        torch.cuda.synchronize()
        samples = [a.elapsed_time(b) * 1e3 / per_sample for a, b in ev]
    arm.steps_per_sample = per_sample
    return ms, samples


def step_path(args):
    """The entry points one step of one layer calls."""
    if args.window:
        return ("kvq_decode_step_mixed" if args.variant == "auto" else
                "kvq_quantize_append + kvq_decode_attn_variant x2 + kvq_combine_regions")
    if args.queries > 1:
        return "kvq_decode_step_multi"
    return "kvq_decode_step"


def workload_key(name, args):
    """The workload's name, with the multi-query / window mode appended."""
    return name + (f"+queries{args.queries}" if args.queries > 1 else "") + \
        (f"+window{args.window}" if args.window else "")


def time_evictions(arm, reps=10):
    """µs per layer of one eviction of the fp16 window into the tail
    (kvq_quantize_rows of WINDOW rows), from a graph of every layer's call."""
    import torch

    lib = arm.lib
    n = arm.wl.layers
    stream = torch.cuda.current_stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for c in arm.calls[:n]:
            assert lib.kvq_quantize_rows(*c["evict"], cs) == 0
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * n)


def percentile(xs, q):
    xs = sorted(xs)
    if not xs:
        return None
    k = (len(xs) - 1) * q
    lo, hi = int(k), min(int(k) + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def probe_read_bandwidth(nbytes=4 << 30, reps=4):
    """Achievable streaming-read rate of this GPU's HBM: the plain read kernel
    of libkvq_probe.so over a buffer far larger than the last-level cache, best
    over a few grid sizes.  None when the probe library is not built (it is not
    part of the decode path)."""
    import ctypes

    import torch

    from quantised_kv_long_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        return None
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.kvq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    lib.kvq_probe_stream_read.restype = ctypes.c_int
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda:0")
    grids = (4096, 8192, 16384)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda:0")
    stream = torch.cuda.current_stream()
    best = 0.0
    for blocks in grids:
        for i in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            rc = lib.kvq_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), blocks,
                                           stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize()
            assert rc == 0, rc
            if i:
                best = max(best, nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink
    torch.cuda.empty_cache()
    return best


def probe_same_bytes_us(nbytes, reps=5):
    """Per-launch time of the plain read kernel of libkvq_probe.so over
    exactly `nbytes` (the attention launch's stored bytes): launches over
    distinct buffers (>= 1 GiB in all, so the last-level cache cannot serve
    them), captured in one graph, best over a few grid sizes.  What a launch of
    that many bytes costs with no attention work: the start and the end of a
    launch included.  None when the probe library is not built."""
    import ctypes

    import torch

    from quantised_kv_long_amd import build as B

    if not os.path.exists(B.PROBE_LIB):
        return None
    lib = ctypes.CDLL(B.PROBE_LIB)
    lib.kvq_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                          ctypes.c_int, ctypes.c_void_p]
    lib.kvq_probe_stream_read.restype = ctypes.c_int
    nbytes = (nbytes + 15) // 16 * 16
    nbuf = max(2, math.ceil((1 << 30) / nbytes))
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda:0") for _ in range(nbuf)]
    grids = (512, 1024, 2048)
    sink = torch.empty(max(grids) * 256, dtype=torch.int32, device="cuda:0")
    s = torch.cuda.Stream()
    best = None
    for blocks in grids:
        def launch_all():
            for b in bufs:
                rc = lib.kvq_probe_stream_read(b.data_ptr(), nbytes, sink.data_ptr(), blocks, s.cuda_stream)
                assert rc == 0, rc
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            launch_all()                       # eager warm-up
            s.synchronize()
            with torch.cuda.graph(g, stream=s):
                launch_all()
        torch.cuda.synchronize()
        for i in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(s):
                e0.record(s)
                g.replay()
                e1.record(s)
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / nbuf
            if i and (best is None or us < best):
                best = us
        del g
    del bufs, sink
    torch.cuda.empty_cache()
    return best


def cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo (empty if unreadable)."""
    try:
        for line in open("/proc/cpuinfo", encoding="utf-8"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def cpu_baseline(arm, budget_s):
    """The oracle, as it stands, on a bounded sample of the same step: whole
    layers (quantise the new row, fp64 attention per split, exact combine) of
    the same cache bytes, timed on every core this process may run on, then
    one layer on a single thread."""
    import numpy as np
    import torch

    from oracle import oracle as O

    wl = arm.wl
    threads = len(os.sched_getaffinity(0))
    u16 = lambda t: t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    name = {0: "f16", 1: "q8_0", 2: "q4_0"}

    def host_layer(L):
        kc, vc = L["kc"], L["vc"]
        kp = (name[kc.type], kc.data.cpu().numpy(),
              kc.scales.cpu().numpy().view(np.uint16) if kc.scales is not None else None)
        vp = (name[vc.type], vc.data.cpu().numpy(),
              vc.scales.cpu().numpy().view(np.uint16) if vc.scales is not None else None)
        return kp, vp, u16(L["q"]), u16(L["knew"]), u16(L["vnew"])

    def one_layer(kp, vp, q, knew, vnew, nthreads):
        t0 = time.perf_counter()
        O.quantize(kp[0], knew)
        O.quantize(vp[0], vnew)
        po, pl = O.attend_split(q, kp, vp, arm.lens, wl.Hkv, 1 / math.sqrt(wl.D),
                                arm.part.split_tokens, arm.part.max_splits, nthreads=nthreads)
        O.combine(po, pl)
        return time.perf_counter() - t0

    done, elapsed = 0, 0.0
    for L in arm.layers[: wl.layers]:
        elapsed += one_layer(*host_layer(L), threads)
        done += 1
        if elapsed >= budget_s:
            break
    s_per_layer = elapsed / done
    gbs = arm.stored_bytes_layer / s_per_layer / 1e9
    s1 = one_layer(*host_layer(arm.layers[0]), 1)
    sample = (f"{done} of {wl.layers} layer(s) of {wl.name}, {arm.tk}/{arm.tv}: quantise the new "
              f"row, fp64 attention over {arm.part.max_splits} splits of {arm.part.split_tokens} "
              f"rows, exact combine; {s_per_layer * 1e3:.1f} ms per layer on {threads} threads, "
              f"{s1 * 1e3:.1f} ms for one layer on 1 thread; per-step figures scaled to "
              f"{wl.layers} layers")
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample, "cpu_model": cpu_model(),
            "us_per_step_scaled": round(s_per_layer * wl.layers * 1e6, 1),
            "one_thread": {"value": round(arm.stored_bytes_layer / s1 / 1e9, 4), "unit": "GB/s",
                           "us_per_step_scaled": round(s1 * wl.layers * 1e6, 1)}}


def run_arms(wl, arms, headline, split_tokens, args, dev):
    """Time every arm of a workload; returns (results per arm, the headline
    arm's device state)."""
    import torch

    import quantised_kv_long_amd as kvq

    results = {}
    head_arm = None
    for tk, tv in arms:
        per_layer = sum(wl.lengths()) * wl.Hkv * (
            kvq.kvq_data_row_bytes(tk, wl.D) + kvq.kvq_scale_row_bytes(tk, wl.D) +
            kvq.kvq_data_row_bytes(tv, wl.D) + kvq.kvq_scale_row_bytes(tv, wl.D))
        reps = args.replicas or max(1, math.ceil(1.0e9 / (per_layer * wl.layers)))
        log(f"arm {tk}/{tv}: building {wl.layers} layer(s) x {reps} replica(s)")
        arm = Arm(wl, tk, tv, split_tokens, reps, dev, args.queries, args.window)
        log(f"arm {tk}/{tv}: timing {args.steps} steps")
        ms, samples = time_arm(arm, args.steps, args.warmup, not args.no_graph, args.variant)
        per_launch = {m: ms[m] / wl.layers for m in MODES}
        evict_us = time_evictions(arm) if args.window else None
        r = {
            "us_per_step": round(ms["step"] * 1e3, 2),
            "stored_bytes_per_step": arm.stored_bytes_step,
            "GBps": round(arm.stored_bytes_step / (ms["step"] * 1e-3) / 1e9, 1),
            "frac_of_peak": round(arm.stored_bytes_step / (ms["step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "step_us_per_layer": round(per_launch["step"] * 1e3, 3),
            "three_call_us_per_step": round(ms["three"] * 1e3, 2),
            "decode_only_us_per_launch": round(per_launch["decode"] * 1e3, 3),
            "split_tokens": arm.split_tokens,
            **({"window_split_tokens": arm.win_split_tokens} if args.window else {}),
            "decode_only_GBps": round(arm.stored_bytes_layer / (per_launch["decode"] * 1e-3) / 1e9, 1),
            "replicas": reps,
        }
        if args.queries > 1:
            r["tokens_per_step"] = args.queries
            r["us_per_token_per_layer"] = round(per_launch["step"] * 1e3 / args.queries, 3)
        if evict_us is not None:
            # once every WINDOW steps per layer: quantise the window into the tail
            r["eviction_us_per_layer"] = round(evict_us, 3)
            r["eviction_us_per_step_layer_amortised"] = round(evict_us / args.window, 4)
        if samples:
            r["step_us_p10_p50_p90"] = [round(percentile(samples, q), 2) for q in (0.1, 0.5, 0.9)]
            r["steps_per_sample"] = arm.steps_per_sample
        results[f"{tk}/{tv}"] = r
        log(f"arm {tk}/{tv}: {r}")
        if (tk, tv) == headline:
            head_arm = arm
        else:
            del arm
            torch.cuda.empty_cache()
    return results, head_arm


def arm_ratios(results):
    """Speed-ups between the arms of one workload (median single steps and
    their p10-p90 separation where sampled)."""
    ratios = {}
    if "q4_0/q4_0" in results and "q8_0/q4_0" in results:
        ratios["q4q4_over_q8q4_speedup"] = round(results["q8_0/q4_0"]["us_per_step"] /
                                                 results["q4_0/q4_0"]["us_per_step"], 3)
        a, b = results["q8_0/q4_0"], results["q4_0/q4_0"]
        ratios["q4q4_over_q8q4_attention_speedup"] = round(a["decode_only_us_per_launch"] /
                                                           b["decode_only_us_per_launch"], 3)
        if "step_us_p10_p50_p90" in a and "step_us_p10_p50_p90" in b:
            pa, pb = a["step_us_p10_p50_p90"], b["step_us_p10_p50_p90"]
            ratios["q4q4_over_q8q4_median_step"] = round(pa[1] / pb[1], 3)
            ratios["q4q4_p90_below_q8q4_p10"] = pb[2] < pa[0]
    if "f16/f16" in results and "q8_0/q4_0" in results:
        ratios["q8q4_over_f16_speedup"] = round(results["f16/f16"]["us_per_step"] /
                                                results["q8_0/q4_0"]["us_per_step"], 3)
    if "f16/f16" in results and "q8_0/q8_0" in results:
        a, b = results["f16/f16"], results["q8_0/q8_0"]
        ratios["q8q8_over_f16_speedup"] = round(a["us_per_step"] / b["us_per_step"], 3)
        ratios["q8q8_over_f16_attention_speedup"] = round(a["decode_only_us_per_launch"] /
                                                          b["decode_only_us_per_launch"], 3)
        if "step_us_p10_p50_p90" in a and "step_us_p10_p50_p90" in b:
            ratios["q8q8_p90_below_f16_p10"] = b["step_us_p10_p50_p90"][2] < a["step_us_p10_p50_p90"][0]
    return ratios


def run_long_context(args, dev):
    """The 262144-row layer (40 query / 8 KV heads, head_dim 128, one planted
    needle per KV head) timed the same way, so one default run covers both ends
    of the 64k-256k range; its attention launch's fraction of peak is reported
    per arm."""
    import torch

    from quantised_kv_long_amd import synth

    wl = synth.WORKLOADS["long_d128_ctx256k"]
    arms = [("q8_0", "q4_0"), ("q4_0", "q4_0")]
    res, arm = run_arms(wl, arms, arms[0], wl.split_tokens, args, dev)
    del arm
    torch.cuda.empty_cache()
    for r in res.values():
        r["decode_only_frac_of_peak"] = round(r["decode_only_GBps"] / HBM_PEAK_GBS, 4)
    return {"workload": wl.name, "ctx": wl.ctx, "layers": wl.layers, "split_tokens": wl.split_tokens,
            "arms": res, "ratios": arm_ratios(res)}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
              "(the decode path would shard by sequence or KV head with no exchange, or by "
              "context with one all-gather of split partials).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}), flush=True)
        return

    import quantised_kv_long_amd as kvq
    from quantised_kv_long_amd import synth

    kvq.load()
    dev = "cuda:0"
    torch.cuda.set_device(0)
    wl = synth.WORKLOADS[args.workload]
    arms = wl.arms
    if args.arms:
        arms = [tuple(a.split("/")) for a in args.arms.split(",")]
    split_tokens = args.split_tokens or wl.split_tokens
    headline = ("q8_0", "q4_0") if ("q8_0", "q4_0") in arms else arms[0]

    results, head_arm = run_arms(wl, arms, headline, args.split_tokens if args.window else split_tokens,
                                 args, dev)
    h = results[f"{headline[0]}/{headline[1]}"]
    cpu = None
    if args.cpu_seconds > 0 and args.queries == 1 and not args.window:
        log("oracle CPU baseline")
        cpu = cpu_baseline(head_arm, args.cpu_seconds)
    ratios = arm_ratios(results)
    dec_us = h["decode_only_us_per_launch"]
    achieved = head_arm.stored_bytes_layer / (dec_us * 1e-6) / 1e9
    rec = traffic_record(workload_key(wl.name, args), headline[0], headline[1])
    traffic = None
    if rec is not None:
        traffic = round((rec[0] + rec[1]) / (dec_us * 1e-6) / 1e9, 1)
        log(f"traffic from {rec[2]}: {rec[0] + rec[1]} bytes per launch")
    probe = probe_read_bandwidth()
    probe = round(probe, 1) if probe else None
    log(f"probe read bandwidth {probe} GB/s")
    same = probe_same_bytes_us(head_arm.stored_bytes_layer)
    same = round(same, 3) if same else None
    log(f"plain read of the launch's {head_arm.stored_bytes_layer} bytes: {same} us per launch")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": ("decode_mfma_dual_kernel" if args.window and args.variant == "auto"
                           else "decode_mfma_kernel"), "avg_launch_us": dec_us,
                "algorithmic_bytes_per_launch": head_arm.stored_bytes_layer,
                "probe_read_GBps": probe,
                "frac_of_probe": round(achieved / probe, 4) if probe else None,
                # the same bytes read by the plain read kernel, one launch per
                # buffer: the time a launch of this size takes with no
                # attention work, and the attention launch's fraction of it
                "probe_same_bytes_us": same,
                "frac_of_same_bytes_probe": round(same / dec_us, 4) if same else None}
    line = {
        "metric": METRIC,
        "value": h["GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(h["us_per_step"] / 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the contractions take f16 operands (the codes as exact f16 values,
        # Q, and p times the V scale) on the matrix cores with fp32
        # accumulation; block scales, softmax and merge are fp32
        "dtype": "f16 MFMA operands, fp32 accumulate/softmax",
        "data": "synthetic",
        "config": {"workload": workload_key(wl.name, args), "arm": f"{headline[0]}K/{headline[1]}V",
                   "queries": args.queries, "window": args.window,
                   "layers": wl.layers, "batch": wl.B, "q_heads": wl.Hq, "kv_heads": wl.Hkv,
                   "head_dim": wl.D, "ctx": wl.ctx, "split_tokens": head_arm.split_tokens,
                   "path": step_path(args), "graph": not args.no_graph},
        # the dominant kernel is the split-KV attention kernel: its average
        # launch duration is measured with HIP events around graph replays of
        # that launch alone (one per layer, back to back)
        "roofline": roofline,
        "cpu_baseline": cpu,
        "arms": results,
        "ratios": ratios,
    }
    if args.long_ctx and args.workload == "stack48_d128_ctx64k" and args.queries == 1 and not args.window:
        del head_arm
        torch.cuda.empty_cache()
        log("long-context layer (262144 rows)")
        line["long_ctx"] = run_long_context(args, dev)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
