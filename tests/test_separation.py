"""The oracle and the HIP path share no code (CPU only).

The oracle is test infrastructure: only the tests, the smoke check and the
bench's CPU-baseline leg may use it, and it uses nothing of the product. The
only module both sides' callers share is the seeded input generator, which
holds none of the method's arithmetic and imports neither side.
"""
import ast
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "quantized_gemm_quantize_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _files(top, exts):
    for dirpath, dirnames, filenames in os.walk(top):
        dirnames[:] = [d for d in dirnames if d != "__pycache__"]
        for f in filenames:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def _imports(path):
    """(module name, enclosing function names) of every import in a Python file."""
    tree = ast.parse(open(path).read(), path)
    out = []

    def walk(node, funcs):
        for child in ast.iter_child_nodes(node):
            inner = funcs + [child.name] if isinstance(child, (ast.FunctionDef, ast.AsyncFunctionDef)) else funcs
            if isinstance(child, ast.Import):
                out.extend((a.name, tuple(funcs)) for a in child.names)
            elif isinstance(child, ast.ImportFrom):
                out.append((child.module or "", tuple(funcs)))
            walk(child, inner)

    walk(tree, [])
    return out


def test_product_never_imports_the_oracle():
    for path in _files(PKG, (".py",)):
        for mod, _ in _imports(path):
            assert not mod.split(".")[0] == "oracle", f"{path} imports {mod}"


def test_product_sources_never_include_oracle_code():
    for path in _files(PKG, (".hip", ".hpp", ".h", ".cpp", ".c")):
        text = open(path).read()
        for inc in re.findall(r'#\s*include\s*[<"]([^>"]+)[>"]', text):
            assert "oracle" not in inc, f"{path} includes {inc}"


def test_oracle_never_uses_the_product():
    for path in _files(ORACLE, (".py",)):
        for mod, _ in _imports(path):
            assert not mod.startswith("quantized_gemm_quantize_amd"), f"{path} imports {mod}"
    for path in _files(ORACLE, (".c", ".h")):
        text = open(path).read()
        for inc in re.findall(r'#\s*include\s*[<"]([^>"]+)[>"]', text):
            assert "csrc" not in inc and "w8a8.h" not in inc, f"{path} includes {inc}"
            assert "hip" not in inc.lower(), f"{path} includes {inc}"


def test_input_generator_imports_neither_side():
    path = os.path.join(PKG, "inputs.py")
    for mod, _ in _imports(path):
        root = mod.split(".")[0]
        assert root != "oracle", mod
        assert not (root == "quantized_gemm_quantize_amd" and "binding" in mod), mod
        assert mod not in ("binding", ".binding"), mod


def test_bench_uses_the_oracle_only_for_its_cpu_baseline():
    for mod, funcs in _imports(os.path.join(ROOT, "bench.py")):
        if mod.split(".")[0] == "oracle":
            assert funcs and all("cpu_baseline" in f for f in funcs[:1]), (mod, funcs)
