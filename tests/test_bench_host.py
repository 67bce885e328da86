"""bench.py's host logic on the CPU: every name it loads is bound somewhere
(a call to a function that no longer exists would otherwise only show on a GPU),
its arguments parse, and a request for more than one GPU exits with status 2."""
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
