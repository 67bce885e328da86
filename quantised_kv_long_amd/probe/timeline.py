"""Per-workgroup timeline of the attention launch (not part of the decode path).

Runs a benchmark workload's layers through ``libkvq_timeline.so`` (the library
built with timeline points in the attention kernel, ``build_timeline()``),
replays them as one HIP graph so that every launch follows another one (the
steady state of a decode stack), and summarises the last layer's attention
launch: when its workgroups start, finish their tiles and end, per CU and per
XCC.  The clock is the GPU's 100 MHz constant clock, so times are multiples of
10 ns.

Usage:
    python3 quantised_kv_long_amd/probe/timeline.py --workload stack48_d128_ctx64k \\
        --arms q8_0/q4_0,q4_0/q4_0 --mode decode --replays 5
"""
from __future__ import annotations

import argparse
import ctypes
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TICKS_PER_US = 100.0


WORDS = 8   # per workgroup: clock at start, wave 0's loop end, end; ids; all loops done, merge written


def summarise(rec, nwg):
    """Summary of one launch from its records (nwg x WORDS uint64)."""
    start = [r[0] for r in rec[:nwg]]
    t0 = min(start)
    us = lambda t: (t - t0) / TICKS_PER_US
    s = [us(r[0]) for r in rec[:nwg]]
    le = [us(r[1]) if r[1] else None for r in rec[:nwg]]   # an empty split records no loop end
    e = [us(r[2]) for r in rec[:nwg]]
    xcc = [(r[3] >> 32) & 0xF for r in rec[:nwg]]
    cu = [(x, (r[3] >> 8) & 0xFF) for x, r in zip(xcc, rec[:nwg])]
    by_cu = {}
    for i, c in enumerate(cu):
        by_cu.setdefault(c, []).append(i)
    cu_end = [max(e[i] for i in v) for v in by_cu.values()]
    # two workgroups sharing a CU: loop time of the one whose loop ends first
    # over the other's, and whether that one has the lower workgroup number
    ratio, lower_first = [], 0
    for v in by_cu.values():
        if len(v) == 2 and all(le[i] is not None for i in v):
            a, b = sorted(v, key=lambda i: (le[i], i))
            if le[b] > s[b]:
                ratio.append((le[a] - s[a]) / (le[b] - s[b]))
                lower_first += a < b
    lev = [x for x in le if x is not None]
    q = lambda xs: (min(xs), statistics.median(xs), max(xs))
    # the four-wave merge: wave 0's loop end -> every loop done -> merge area
    # written -> end (medians over the workgroups that record them)
    ph = [(us(r[4]) - le[i], us(r[5]) - us(r[4]), e[i] - us(r[5]))
          for i, r in enumerate(rec[:nwg]) if r[1] and r[4] and r[5]]
    phases = tuple(statistics.median(x[k] for x in ph) for k in range(3)) if ph else None
    return dict(n=nwg, cus=len(by_cu), span=max(e), start=q(s), loop_end=q(lev), end=q(e), cu_end=q(cu_end),
                first_over_second=(statistics.median(ratio) if ratio else None), pairs=len(ratio),
                lower_first=lower_first, phases=phases,
                xcc_end=[max([e[i] for i in range(nwg) if xcc[i] == x], default=float("nan")) for x in range(8)])


def fmt3(t):
    return f"{t[0]:.2f} / {t[1]:.2f} / {t[2]:.2f}"


def main():
    import torch

    import bench
    from quantised_kv_long_amd import _lib
    from quantised_kv_long_amd import build as B
    from quantised_kv_long_amd import synth

    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--workload", default="stack48_d128_ctx64k", choices=sorted(synth.WORKLOADS))
    p.add_argument("--arms", default=None, help="K/V type pairs, comma-separated (default: the workload's)")
    p.add_argument("--mode", default="decode", choices=("decode", "step"),
                   help="decode: the attention launches alone; step: kvq_decode_step per layer")
    p.add_argument("--split-tokens", type=int, default=None)
    p.add_argument("--replays", type=int, default=5)
    args = p.parse_args()

    assert torch.cuda.is_available(), "the timeline needs a GPU"
    if not os.path.exists(B.TIMELINE_LIB):
        raise SystemExit(f"{B.TIMELINE_LIB} is not built (quantised_kv_long_amd.build.build_timeline)")
    lib = _lib.load(B.TIMELINE_LIB)   # every later _lib.load() returns this library
    lib.kvq_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.kvq_timeline_read.restype = ctypes.c_int
    cap = lib.kvq_timeline_capacity()

    wl = synth.WORKLOADS[args.workload]
    arms = [tuple(a.split("/")) for a in args.arms.split(",")] if args.arms else wl.arms
    st = args.split_tokens or wl.split_tokens
    dev = "cuda"
    print(f"# timeline: {wl.name}, mode {args.mode}, split_tokens {st}, {wl.layers} layers per graph")
    for tk, tv in arms:
        arm = bench.Arm(wl, tk, tv, st, 1, dev)
        arm.prepare_calls("auto")
        nwg = sum((L + st - 1) // st for L in arm.lens) * wl.Hkv
        if nwg > cap:
            raise SystemExit(f"{nwg} workgroups exceed the timeline's {cap}")
        g = torch.cuda.CUDAGraph()
        arm.step(torch.cuda.current_stream().cuda_stream, 0, args.mode)   # warm-up, eager
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            arm.step(torch.cuda.current_stream().cuda_stream, 0, args.mode)
        g.replay()
        torch.cuda.synchronize()
        print(f"\n## {tk}/{tv}: {nwg} workgroups (grid of the last layer's attention launch)\n")
        print("| replay | span µs | start spread µs | loop end min / median / max µs | end min / median / max µs "
              "| CUs | CU end min / median / max µs | two workgroups on a CU: loop time of the first to finish over "
              "the other's, median (CUs where the first to finish has the lower number) | "
              "last end per XCC 0-7 µs | merge phases, medians µs: wave 0's loop end to all loops done / "
              "merge area written / end |")
        print("|---|---|---|---|---|---|---|---|---|---|")
        for r in range(args.replays):
            g.replay()
            torch.cuda.synchronize()
            buf = (ctypes.c_uint64 * (WORDS * nwg))()
            assert lib.kvq_timeline_read(ctypes.addressof(buf), ctypes.sizeof(buf)) == 0
            rec = [tuple(buf[WORDS * i:WORDS * i + WORDS]) for i in range(nwg)]
            m = summarise(rec, nwg)
            fs = (f"{m['first_over_second']:.2f} ({m['lower_first']} of {m['pairs']} CUs)"
                  if m["first_over_second"] else "-")
            print(f"| {r} | {m['span']:.2f} | {m['start'][2] - m['start'][0]:.2f} | {fmt3(m['loop_end'])} | "
                  f"{fmt3(m['end'])} | {m['cus']} | {fmt3(m['cu_end'])} | {fs} | "
                  f"{' '.join(f'{x:.1f}' for x in m['xcc_end'])} | "
                  f"{' / '.join(f'{x:.2f}' for x in m['phases']) if m['phases'] else '-'} |", flush=True)
        del g, arm
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
