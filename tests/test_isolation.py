"""The oracle and the product stay apart, and the product has no fallback.

- Nothing in the package (Python binding, build script, HIP sources) or in
  the C header imports, includes or names a path under oracle/.
- The oracle imports nothing from the package: the two share no code.
- bench.py and __graft_entry__.py import the oracle only inside the CPU
  baseline and smoke() functions, never at module level.
- Without libsfattn.so the binding raises on first use instead of computing
  anything another way.
"""
import ast
import os
import pathlib
import subprocess
import sys

ROOT = pathlib.Path(__file__).resolve().parents[1]
PKG = ROOT / "hidden_decoding_stream_amd"


def _imports(path: pathlib.Path, top_level_only: bool = False):
    tree = ast.parse(path.read_text(), filename=str(path))
    nodes = tree.body if top_level_only else ast.walk(tree)
    for node in nodes:
        if isinstance(node, ast.Import):
            for a in node.names:
                yield a.name
        elif isinstance(node, ast.ImportFrom):
            yield ("." * node.level) + (node.module or "")


def test_package_never_imports_the_oracle():
    for py in PKG.rglob("*.py"):
        for name in _imports(py):
            assert not name.split(".")[0] == "oracle", f"{py} imports {name}"
    for src in list((PKG / "csrc").rglob("*")) + list((ROOT / "include").rglob("*")):
        if src.is_file() and src.suffix in (".hip", ".h", ".cpp", ".hpp"):
            assert "oracle" not in src.read_text(), f"{src} names the oracle"


def test_oracle_imports_nothing_from_the_package():
    for py in (ROOT / "oracle").rglob("*.py"):
        for name in _imports(py):
            assert not name.startswith("hidden_decoding_stream_amd"), f"{py} imports {name}"


def test_entry_points_import_the_oracle_only_inside_functions():
    for f in ("bench.py", "__graft_entry__.py"):
        top = list(_imports(ROOT / f, top_level_only=True))
        assert not any(n.split(".")[0] == "oracle" for n in top), f"{f} imports the oracle at module level"


def test_missing_library_fails_loudly():
    code = ("import hidden_decoding_stream_amd as s\n"
            "try:\n"
            "    s.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "    raise SystemExit(3)\n"
            "raise SystemExit(0)\n")
    env = dict(os.environ, SFATTN_LIB=str(ROOT / "no_such_dir" / "libsfattn.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 3, (r.returncode, r.stdout, r.stderr)
    assert "is missing" in r.stdout
