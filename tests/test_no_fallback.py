"""The product path has no CPU fallback: without the HIP library every call
raises, and nothing in the package imports the oracle."""
import ast
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "int8_mixed_precision_outlier_amd")


def test_calls_raise_without_the_library():
    code = (
        "import int8_mixed_precision_outlier_amd as i8, torch\n"
        "i8.LIB_PATH = '/nonexistent/libint8mm.so'\n"
        "i8._lib = None\n"
        "try:\n"
        "    i8.workspace_size(16, 64, 64, 16)\n"
        "except RuntimeError as e:\n"
        "    print('raised', 'missing' in str(e))\n"
    )
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                         check=True).stdout.split()
    assert out == ["raised", "True"]


def test_package_never_imports_the_oracle():
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(dirpath, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                for n in names:
                    assert not n.split(".")[0] in ("oracle", "tests"), (f, n)
