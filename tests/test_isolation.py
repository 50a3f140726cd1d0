"""The oracle and the GPU library stay apart, and the library fails loudly.

* Nothing under momentum_compression_amd/ (Python, HIP, headers) imports or
  includes anything from oracle/, and nothing under oracle/ imports the
  package or includes its sources or the C ABI header.
* bench.py and __graft_entry__.py import the oracle only inside the functions
  allowed to use it (the CPU baseline; smoke, and build, which compiles the
  checker).
* With the oracle made unimportable, the package and its binding still
  import; with libonebit.so absent, the binding raises instead of falling
  back to anything.
"""

import ast
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "momentum_compression_amd")
ORACLE = os.path.join(ROOT, "oracle")


def _files(top, exts):
    for dirpath, dirnames, filenames in os.walk(top):
        dirnames[:] = [d for d in dirnames if not d.startswith(("_build", "__pycache__"))]
        for f in filenames:
            if f.endswith(exts):
                yield os.path.join(dirpath, f)


def _strip_comments(text, path):
    if path.endswith(".py"):
        return "\n".join(line.split("#", 1)[0] for line in text.splitlines())
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.sub(r"//[^\n]*", "", text)


def test_library_sources_never_reach_the_oracle():
    bad = []
    for path in _files(PKG, (".py", ".hip", ".h", ".cpp")):
        code = _strip_comments(open(path).read(), path)
        if re.search(r"^\s*(from\s+oracle\b|import\s+oracle\b)", code, flags=re.M) or \
                re.search(r'#\s*include\s*[<"][^>"]*oracle', code):
            bad.append(os.path.relpath(path, ROOT))
    assert not bad, f"library files reaching the oracle: {bad}"


def test_oracle_sources_never_reach_the_library():
    bad = []
    for path in _files(ORACLE, (".py", ".cpp", ".h", ".c")):
        code = _strip_comments(open(path).read(), path)
        if re.search(r"^\s*(from|import)\s+momentum_compression_amd", code, flags=re.M) or \
                re.search(r'#\s*include\s*[<"][^>"]*(onebit\.h|common\.h|csrc)', code):
            bad.append(os.path.relpath(path, ROOT))
    assert not bad, f"oracle files reaching the library: {bad}"


def _oracle_imports_by_function(path):
    """Names of the top-level functions that import the oracle, and whether
    any import of it sits outside a function."""
    tree = ast.parse(open(path).read())
    inside, outside = set(), False
    for node in tree.body:
        nodes = list(ast.walk(node))
        hits = [n for n in nodes if isinstance(n, ast.ImportFrom) and (n.module or "").startswith("oracle")
                or isinstance(n, ast.Import) and any(a.name.startswith("oracle") for a in n.names)]
        if not hits:
            continue
        if isinstance(node, ast.FunctionDef):
            inside.add(node.name)
        else:
            outside = True
    return inside, outside


def test_bench_imports_the_oracle_only_for_the_cpu_baseline():
    inside, outside = _oracle_imports_by_function(os.path.join(ROOT, "bench.py"))
    assert not outside and inside == {"cpu_baseline"}


def test_entry_points_import_the_oracle_only_in_smoke_and_build():
    inside, outside = _oracle_imports_by_function(os.path.join(ROOT, "__graft_entry__.py"))
    assert not outside and inside <= {"smoke", "build"}


def _run(code):
    return subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                          timeout=300)


def test_package_imports_without_the_oracle():
    res = _run("import sys; sys.modules['oracle'] = None\n"
               "import momentum_compression_amd.onebit, momentum_compression_amd.state, "
               "momentum_compression_amd.checkpoint\n"
               "print('ok')")
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


def test_binding_raises_when_the_library_is_missing():
    res = _run("from momentum_compression_amd import onebit as ob\n"
               "ob.LIB_PATH = ob.LIB_PATH + '.absent'\n"
               "ob._lib = None\n"
               "try:\n"
               "    ob.load()\n"
               "except ImportError as e:\n"
               "    print('raised', 'missing' in str(e))\n")
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "raised True"
