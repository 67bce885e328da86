"""The per-workgroup timeline probe's host side on the CPU: the summary of a
launch's records (start, wave 0's loop end, end, CU ids, merge phases), on
hand-made records whose figures are known."""
import importlib.util
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location(
    "kvq_timeline_probe", os.path.join(ROOT, "quantised_kv_long_amd", "probe", "timeline.py"))
T = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(T)


def rec(start, loop_end, end, xcc, cu, done=0, written=0):
    """One workgroup's record in clock ticks (100 per µs); hw id with the CU
    number in bits 8-15."""
    return (start, loop_end, end, (xcc << 32) | (cu << 8) | 5, done, written, 0, 0)


def test_summary_of_known_records():
    # CU (1, 3): workgroups 0 and 1; CU (2, 7): workgroups 2 and 3
    r = [rec(1000, 1600, 1700, 1, 3, 1620, 1660),
         rec(1010, 1900, 2000, 1, 3, 1920, 1950),
         rec(1005, 1650, 1760, 2, 7, 1670, 1700),
         rec(1000, 1300, 1400, 2, 7, 1310, 1350)]
    m = T.summarise(r, 4)
    assert m["n"] == 4 and m["cus"] == 2
    assert abs(m["span"] - 10.0) < 1e-9                   # last end 2000 - first start 1000 ticks
    assert m["start"] == (0.0, 0.025, 0.1)
    assert m["loop_end"] == (3.0, 6.25, 9.0)
    assert m["end"][0] == 4.0 and m["end"][2] == 10.0
    assert m["cu_end"] == (7.6, 8.8, 10.0)
    # loop times: CU 3: 6.0 (wg 0) vs 8.9 (wg 1); CU 7: 3.0 (wg 3) vs 6.45 (wg 2)
    assert m["pairs"] == 2
    assert abs(m["first_over_second"] - (6.0 / 8.9 + 3.0 / 6.45) / 2) < 1e-12
    assert m["lower_first"] == 1                           # on CU 7 the higher-numbered one ends first
    # merge phases (medians): loop end -> all loops done, -> merge written, -> end
    assert abs(m["phases"][0] - 0.2) < 1e-9
    assert abs(m["phases"][1] - 0.35) < 1e-9
    assert abs(m["phases"][2] - 0.5) < 1e-9
    assert m["xcc_end"][1] == 10.0 and m["xcc_end"][2] == 7.6


def test_split_without_rows_and_kernel_without_merge():
    # a split with no rows records no loop end (0), a wide-head kernel no
    # merge points: neither enters those figures
    r = [rec(1000, 0, 1100, 0, 1), rec(1000, 1500, 1600, 0, 2)]
    m = T.summarise(r, 2)
    assert m["loop_end"] == (5.0, 5.0, 5.0)
    assert m["phases"] is None
    assert m["pairs"] == 0 and m["first_over_second"] is None
