"""The oracle and the HIP path stay apart, checked on the source text.

The oracle (oracle/) imports neither the product package nor the input
generators; the product package never imports the oracle; the input
generators (datagen.py) import neither.  Only tests/, __graft_entry__.smoke()
and bench.py's cpu_baseline may use the oracle, and the package's native
sources share no file with it.
"""
import ast
import glob
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "diffusion_transformer_attention_amd"


def _imports(path):
    tree = ast.parse(open(path).read(), filename=path)
    names = set()
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            names.update(a.name.split(".")[0] for a in node.names)
        elif isinstance(node, ast.ImportFrom) and node.module and node.level == 0:
            names.add(node.module.split(".")[0])
    return names


def test_oracle_imports_only_numpy_and_the_standard_library():
    for path in glob.glob(os.path.join(ROOT, "oracle", "*.py")):
        names = _imports(path)
        assert not names & {PKG, "datagen", "torch", "bench"}, (path, names)


def test_package_never_imports_the_oracle():
    for path in glob.glob(os.path.join(ROOT, PKG, "**", "*.py"), recursive=True):
        assert "oracle" not in _imports(path), path


def test_input_generators_import_neither_side():
    names = _imports(os.path.join(ROOT, "datagen.py"))
    assert not names & {PKG, "oracle"}, names


def test_oracle_use_in_bench_is_the_cpu_baseline_only():
    tree = ast.parse(open(os.path.join(ROOT, "bench.py")).read())
    users = set()
    for fn in ast.walk(tree):
        if isinstance(fn, ast.FunctionDef):
            for node in ast.walk(fn):
                if isinstance(node, ast.Import) and any(a.name == "oracle" for a in node.names):
                    users.add(fn.name)
    top = [n for n in tree.body if isinstance(n, (ast.Import, ast.ImportFrom))]
    assert not any(isinstance(n, ast.Import) and any(a.name == "oracle" for a in n.names) for n in top)
    assert users == {"cpu_baseline"}, users


def test_native_sources_do_not_reference_the_oracle():
    for path in glob.glob(os.path.join(ROOT, PKG, "csrc", "*")) + glob.glob(os.path.join(ROOT, "include", "*")):
        text = open(path, errors="replace").read()
        assert "oracle" not in text.lower(), path
