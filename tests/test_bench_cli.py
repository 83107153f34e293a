"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message (before any GPU work), and the metric line's fixed fields are
the ones the headline is quoted with."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout.strip() == ""


def test_sweep_bytes_formula():
    sys.path.insert(0, ROOT)
    import bench
    # U 4*B*V + W2 2*r*V + W1 rows 2*B*r at the headline shape
    assert bench.sweep_bytes(128, 151936, 256, 2) == 155_648_000
    # GRU head: the fp32 states replace the W1 rows
    assert bench.sweep_bytes(256, 151936, 256, 2, 4) == 4 * 256 * 151936 + 2 * 256 * 151936 + 4 * 256 * 256


def test_measurement_modes_refuse_more_than_one_gpu():
    for mode in ("--verify-layout", "--sts-fit", "--schedule"):
        p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), mode, "--gpus", "2"],
                           capture_output=True, text=True, timeout=120)
        assert p.returncode == 2, mode
        assert "one GPU" in p.stderr


def test_every_called_name_is_defined():
    """Every plain name bench.py calls is a builtin, a module-level name, or
    bound inside the calling function (its imports, nested defs, assignments)."""
    import ast
    import builtins
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    top = set()
    for n in tree.body:
        if isinstance(n, (ast.FunctionDef, ast.ClassDef)):
            top.add(n.name)
        elif isinstance(n, (ast.Import, ast.ImportFrom)):
            top.update((a.asname or a.name).split(".")[0] for a in n.names)
        elif isinstance(n, ast.Assign):
            top.update(t.id for t in n.targets if isinstance(t, ast.Name))
    missing = []
    for fn in [n for n in tree.body if isinstance(n, ast.FunctionDef)]:
        bound = set()
        for n in ast.walk(fn):
            if isinstance(n, (ast.FunctionDef, ast.Lambda)) and n is not fn:
                if isinstance(n, ast.FunctionDef):
                    bound.add(n.name)
            elif isinstance(n, (ast.Import, ast.ImportFrom)):
                bound.update((a.asname or a.name).split(".")[0] for a in n.names)
            elif isinstance(n, ast.Name) and isinstance(n.ctx, ast.Store):
                bound.add(n.id)
            elif isinstance(n, ast.arg):
                bound.add(n.arg)
        for n in ast.walk(fn):
            if isinstance(n, ast.Call) and isinstance(n.func, ast.Name):
                name = n.func.id
                if name not in bound and name not in top and not hasattr(builtins, name):
                    missing.append(f"{fn.name} calls {name}")
    assert not missing, missing
