"""bench.py's host logic on the CPU: every name it loads is bound somewhere
(a call to a function that no longer exists would otherwise only show on a GPU),
its arguments parse, a request for more than one GPU exits with status 2, and
the committed counter summaries it reads its HBM traffic from parse."""
import ast
import builtins
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_every_loaded_name_is_bound():
    tree = ast.parse(open(BENCH).read())
    bound = set(dir(builtins)) | {"__file__"}
    for n in ast.walk(tree):
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            bound.add(n.name)
        elif isinstance(n, ast.Import):
            bound.update(a.asname or a.name.split(".")[0] for a in n.names)
        elif isinstance(n, ast.ImportFrom):
            bound.update(a.asname or a.name for a in n.names)
        elif isinstance(n, ast.Name) and isinstance(n.ctx, (ast.Store, ast.Del)):
            bound.add(n.id)
        elif isinstance(n, ast.arg):
            bound.add(n.arg)
    loads = {n.id for n in ast.walk(tree) if isinstance(n, ast.Name) and isinstance(n.ctx, ast.Load)}
    assert loads <= bound, f"unbound names in bench.py: {sorted(loads - bound)}"


def test_arguments_parse(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py", "--steps", "3", "--warmup", "1", "--no-long-ctx"])
    a = bench.parse()
    assert (a.steps, a.warmup, a.gpus, a.long_ctx) == (3, 1, 1, False)
    assert a.workload == "stack48_d128_ctx64k"


def test_more_than_one_gpu_exits_2():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_records_parse():
    """The counter summaries bench.py reads its measured HBM traffic from:
    every record line parses, its bytes are positive, its source hash is a
    sha256; the headline workload's record for the current kernel sources,
    where there is one, is within 10 % above the stored bytes of one launch
    (8 KV heads x 65536 rows x 208 bytes for q8_0 K + q4_0 V at head_dim 128)."""
    import glob
    import re

    import pytest

    sys.path.insert(0, ROOT)
    import bench
    n = 0
    for path in glob.glob(os.path.join(ROOT, "profiles", "*.md")):
        for line in open(path, encoding="utf-8"):
            if not line.startswith("traffic-record:"):
                continue
            kv = dict(re.findall(r"(\w+)=(\S+)", line))
            assert {"workload", "arm", "kernel", "fetch_bytes", "write_bytes", "sources_sha256"} <= set(kv), line
            assert int(kv["fetch_bytes"]) > 0 and int(kv["write_bytes"]) > 0, line
            assert re.fullmatch(r"[0-9a-f]{64}", kv["sources_sha256"]), line
            n += 1
    assert n > 0
    rec = bench.traffic_record("stack48_d128_ctx64k", "q8_0", "q4_0")
    if rec is None:
        pytest.skip("no counter summary taken on the current kernel sources")
    stored = 8 * 65536 * 208
    assert 1.0 <= (rec[0] + rec[1]) / stored <= 1.1, rec
