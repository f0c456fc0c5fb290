"""The product path never reaches the oracle: the package's modules do
not import it, bench.py imports it only inside its cpu_baseline functions
(the timed CPU baseline), and the built HIP library neither links the
oracle's library nor refers to any of its symbols."""
import ast
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "zero_sharded_optimizer_step_amd")


def _oracle_imports(tree):
    """(enclosing function name or None, line) of every import of `oracle`."""
    found = []

    def visit(node, func):
        for child in ast.iter_child_nodes(node):
            name = child.name if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else func
            if isinstance(child, ast.Import) and any(a.name.split(".")[0] == "oracle" for a in child.names):
                found.append((func, child.lineno))
            elif isinstance(child, ast.ImportFrom) and (child.module or "").split(".")[0] == "oracle":
                found.append((func, child.lineno))
            visit(child, name)
    visit(tree, None)
    return found


@pytest.mark.parametrize("path", sorted(glob.glob(os.path.join(PKG, "*.py"))),
                         ids=lambda p: os.path.basename(p))
def test_package_modules_do_not_import_the_oracle(path):
    assert _oracle_imports(ast.parse(open(path).read())) == []


def test_bench_imports_the_oracle_only_for_its_cpu_baseline():
    found = _oracle_imports(ast.parse(open(os.path.join(ROOT, "bench.py")).read()))
    assert found, "the bench's cpu_baseline times the oracle"
    for func, line in found:
        assert func is not None and func.startswith("cpu_baseline"), (func, line)


def test_hip_library_does_not_link_or_call_the_oracle():
    lib = os.path.join(PKG, "libzero_mi355x.so")
    needed = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in needed
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                               check=True).stdout
    assert "oracle" not in undefined


def test_oracle_does_not_use_the_library():
    """The other direction: the oracle's Python layer imports nothing of the
    package, and its C library refers to none of the HIP library's symbols."""
    tree = ast.parse(open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            assert all(not a.name.startswith("zero_sharded_optimizer_step_amd") for a in node.names)
        elif isinstance(node, ast.ImportFrom):
            assert not (node.module or "").startswith("zero_sharded_optimizer_step_amd")
    import oracle
    lib = oracle.build(force=False)
    undefined = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True, text=True,
                               check=True).stdout
    assert "zero_" not in undefined
    needed = subprocess.run(["readelf", "-d", lib], capture_output=True, text=True, check=True).stdout
    assert "zero_mi355x" not in needed
