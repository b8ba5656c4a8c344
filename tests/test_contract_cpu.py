"""Host-side contract checks that need no GPU: the benchmark refuses more
than one GPU before touching a device, and no module of the product path
(the package and its binding) imports the CPU oracle."""

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_kv_attention_append_amd")


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def _imports(path):
    tree = ast.parse(open(path).read(), path)
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            yield from (a.name for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_product_path_never_imports_the_oracle():
    files = [os.path.join(PKG, f) for f in os.listdir(PKG) if f.endswith(".py")]
    assert files
    for f in files:
        for name in _imports(f):
            assert not name.split(".")[0] == "oracle", f"{f} imports {name}"
    # and the compiled sources name no oracle file
    csrc = os.path.join(PKG, "csrc")
    for f in os.listdir(csrc):
        text = open(os.path.join(csrc, f), errors="replace").read()
        assert "oracle/" not in text and "#include \"oracle" not in text, f
