"""Host-only checks that the oracle stays test infrastructure: bench.py
runs it only in the cpu_baseline leg (its timed calls, whose result the GPU
output is then checked against), and the product package never imports it."""
import ast
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _functions_using(tree, pred):
    out = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if pred(node):
                    out.add(fn.name)
    return out


def test_bench_runs_the_oracle_only_in_the_cpu_baseline_leg():
    with open(os.path.join(ROOT, "bench.py")) as f:
        tree = ast.parse(f.read())

    def imports_oracle(node):
        if isinstance(node, ast.Import):
            return any(a.name.split(".")[0] == "oracle" for a in node.names)
        if isinstance(node, ast.ImportFrom):
            return (node.module or "").split(".")[0] == "oracle"
        return False

    def calls(name):
        return lambda node: isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id == name

    # no module-level import of the oracle
    assert not any(imports_oracle(node) for node in tree.body)
    assert _functions_using(tree, imports_oracle) == {"oracle_call"}
    assert _functions_using(tree, calls("oracle_call")) == {"cpu_baseline"}


def test_product_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "ring_all_reduce_allreduce_amd")
    for dirpath, _, files in os.walk(pkg):
        for name in files:
            if not name.endswith(".py"):
                continue
            with open(os.path.join(dirpath, name)) as f:
                tree = ast.parse(f.read())
            for node in ast.walk(tree):
                if isinstance(node, ast.Import):
                    assert all(a.name.split(".")[0] != "oracle" for a in node.names), name
                if isinstance(node, ast.ImportFrom):
                    assert (node.module or "").split(".")[0] != "oracle", name
