"""bench.py's measured path depends on the library and the input generator only: the oracle is
imported inside the CPU-baseline leg alone, and nothing under tests/ is put on the path or
imported. Checked on the source (no GPU needed)."""

import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _imports(node):
    for n in ast.walk(node):
        if isinstance(n, ast.Import):
            for a in n.names:
                yield a.name.split(".")[0], n
        elif isinstance(n, ast.ImportFrom) and n.module:
            yield n.module.split(".")[0], n


def test_bench_imports_the_oracle_only_in_the_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    owners = {}
    for fn in ast.walk(tree):
        if isinstance(fn, (ast.FunctionDef, ast.ClassDef)):
            for mod, node in _imports(fn):
                owners.setdefault(mod, set()).add(fn.name)
    assert owners.get("oracle", set()) <= {"cpu_baseline", "cpu_oracle_rate"}, owners["oracle"]
    assert "support" not in owners and "tests" not in owners
    top = {m for m, _ in _imports(ast.Module(body=[s for s in tree.body
                                                    if isinstance(s, (ast.Import, ast.ImportFrom))],
                                             type_ignores=[]))}
    assert "oracle" not in top and "support" not in top
    assert '"tests"' not in open(os.path.join(ROOT, "bench.py")).read()
