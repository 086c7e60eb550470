"""CPU: the benchmark's and the entry point's host-side contract.

- `bench.py --gpus N` with N > 1 exits with a message (one GPU is measured;
  sharding is described, not built), before touching a GPU;
- the entry module exposes build() and smoke();
- the product package does not import the oracle (the oracle is test
  infrastructure only).
"""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2", "--steps", "1"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_entry_points():
    src = open(os.path.join(ROOT, "__graft_entry__.py")).read()
    names = {n.name for n in ast.parse(src).body if isinstance(n, ast.FunctionDef)}
    assert {"build", "smoke"} <= names


def test_product_does_not_import_oracle():
    pkg = os.path.join(ROOT, "position_split_kv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert all(not a.name.startswith("oracle") for a in node.names), f
                elif isinstance(node, ast.ImportFrom):
                    assert not (node.module or "").startswith("oracle"), f
