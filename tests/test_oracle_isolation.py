"""The oracle imports only the standard library and numpy: it shares no code with the HIP path."""
import ast
import os
import sys

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")
ALLOWED = {"numpy", "math"}


def test_oracle_imports_only_stdlib_and_numpy():
    stdlib = set(sys.stdlib_module_names)
    for fn in sorted(os.listdir(ORACLE)):
        if not fn.endswith(".py"):
            continue
        tree = ast.parse(open(os.path.join(ORACLE, fn)).read())
        for node in ast.walk(tree):
            if isinstance(node, ast.Import):
                names = [a.name.split(".")[0] for a in node.names]
            elif isinstance(node, ast.ImportFrom):
                if node.level > 0:
                    continue                       # relative import inside oracle/
                names = [node.module.split(".")[0]]
            else:
                continue
            for n in names:
                assert n in ALLOWED or n in stdlib, f"{fn} imports {n}"


ROOT = os.path.dirname(ORACLE)


def _imports(path):
    tree = ast.parse(open(path).read())
    out = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            out.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.level == 0:
            out.add(node.module.split(".")[0])
    return out


def test_product_and_shared_modules_never_import_the_oracle():
    """The package, the shared input generators and the device fill plumbing stay off the oracle."""
    dirs = [os.path.join(ROOT, "paged_kv_cache_283_amd"), os.path.join(ROOT, "workloads")]
    for d in dirs:
        for fn in sorted(os.listdir(d)):
            if fn.endswith(".py"):
                assert "oracle" not in _imports(os.path.join(d, fn)), f"{d}/{fn} imports the oracle"
    # the oracle does not import them either
    for fn in sorted(os.listdir(ORACLE)):
        if fn.endswith(".py"):
            imp = _imports(os.path.join(ORACLE, fn))
            assert not imp & {"paged_kv_cache_283_amd", "workloads", "torch"}, fn


def test_bench_imports_the_oracle_only_inside_its_cpu_baseline():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    for node in tree.body:                                   # module level: no oracle import
        if isinstance(node, (ast.Import, ast.ImportFrom)):
            names = [a.name for a in node.names] if isinstance(node, ast.Import) else [node.module]
            assert not any(n.split(".")[0] in ("oracle", "tests") for n in names)
    for node in ast.walk(tree):
        if isinstance(node, ast.FunctionDef) and node.name != "cpu_baseline":
            for sub in ast.walk(node):
                if isinstance(sub, ast.ImportFrom) and sub.module:
                    assert sub.module.split(".")[0] not in ("oracle", "tests"), (node.name, sub.module)
                if isinstance(sub, ast.Import):
                    assert not any(a.name.split(".")[0] in ("oracle", "tests") for a in sub.names), node.name
