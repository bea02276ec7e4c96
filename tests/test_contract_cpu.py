"""Host-side contract checks that need no GPU: the binding fails loudly when
the HIP library is missing (there is no CPU fallback on the product path),
the product modules do not reach into the oracle, and the benchmark refuses
more than one GPU."""
import ast
import os
import subprocess
import sys

import pytest

from flow_matching_action_amd import pi_ae

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_missing_library_fails_loudly(tmp_path):
    saved = pi_ae._lib
    pi_ae._lib = None
    try:
        with pytest.raises(ImportError):
            pi_ae.load_library(str(tmp_path / "libpi_ae.so"))
    finally:
        pi_ae._lib = saved


def test_product_modules_do_not_import_the_oracle():
    pkg = os.path.join(ROOT, "flow_matching_action_amd")
    for name in sorted(os.listdir(pkg)):
        if not name.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(pkg, name)).read())
        for node in ast.walk(tree):
            mods = []
            if isinstance(node, ast.Import):
                mods = [a.name for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                mods = [node.module or ""]
            assert not any(m == "oracle" or m.startswith("oracle.") for m in mods), (name, mods)


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout.strip() == ""
