"""The product path and the oracle stay apart: the library binding and its build script
never import, read or name the oracle; the oracle and the HIP sources share no file;
the binding fails loudly, with no fallback, when the library is missing; and the
seeded input generators hold none of the method's arithmetic."""

import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "exact_attention_prefill_amd")


def _py_files(d):
    for base, _, files in os.walk(d):
        for f in files:
            if f.endswith(".py"):
                yield os.path.join(base, f)


def _imports(path):
    tree = ast.parse(open(path).read())
    for node in ast.walk(tree):
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield node.module or ""


def test_binding_never_touches_the_oracle():
    for f in _py_files(PKG):
        assert not any(m.split(".")[0] == "oracle" for m in _imports(f)), f
        assert "oracle" not in open(f).read().lower(), f
    for base, _, files in os.walk(os.path.join(PKG, "csrc")):
        for f in files:
            assert "oracle" not in open(os.path.join(base, f)).read().lower(), f


def test_oracle_imports_nothing_from_the_product():
    for f in _py_files(os.path.join(ROOT, "oracle")):
        mods = [m.split(".")[0] for m in _imports(f)]
        assert "exact_attention_prefill_amd" not in mods and "workloads" not in mods, f


def test_input_generators_hold_no_method_arithmetic():
    src = open(os.path.join(ROOT, "workloads", "__init__.py")).read()
    for word in ("softmax", "exp(", "matmul", "einsum", "logsumexp", "bmm("):
        assert word not in src, word
    tree = ast.parse(src)
    assert not any(isinstance(n, ast.BinOp) and isinstance(n.op, ast.MatMult) for n in ast.walk(tree))


def test_missing_library_fails_loudly(tmp_path):
    code = (
        "import exact_attention_prefill_amd as ea\n"
        f"ea.LIB_PATH = {str(tmp_path / 'absent.so')!r}\n"
        "try:\n"
        "    ea.lib()\n"
        "except ImportError as e:\n"
        "    print('raised', e)\n"
    )
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert "raised" in out.stdout, out.stdout + out.stderr


def test_bench_calls_the_oracle_only_in_its_host_leg():
    """bench.py imports the oracle only inside cpu_baseline() or under the
    `if not args.no_cpu_baseline` guard, so a run with --no-cpu-baseline (every
    profiled run) never loads it."""
    src = open(os.path.join(ROOT, "bench.py")).read()
    tree = ast.parse(src)
    parents = {}
    for node in ast.walk(tree):
        for child in ast.iter_child_nodes(node):
            parents[child] = node
    found = 0
    for node in ast.walk(tree):
        names = []
        if isinstance(node, ast.Import):
            names = [a.name.split(".")[0] for a in node.names]
        elif isinstance(node, ast.ImportFrom):
            names = [(node.module or "").split(".")[0]]
        if "oracle" not in names:
            continue
        found += 1
        p, ok = parents.get(node), False
        while p is not None and not ok:
            ok = (isinstance(p, ast.FunctionDef) and p.name == "cpu_baseline") or (
                isinstance(p, ast.If) and "no_cpu_baseline" in ast.get_source_segment(src, p.test))
            p = parents.get(p)
        assert ok, f"oracle imported outside the host leg at line {node.lineno}"
    assert found >= 1
