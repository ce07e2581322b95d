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
