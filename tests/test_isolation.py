"""Host-only checks of how the product is put together: the binding has no
fallback when the HIP library is missing, and no product file refers to the
oracle (which exists only to check the product)."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "dense_gemm_05_amd")


def test_binding_raises_without_library(tmp_path):
    """With the library path pointing at nothing, the first call raises
    ImportError instead of computing anything another way."""
    code = (
        "import dense_gemm_05_amd._lib as L\n"
        f"L.LIB_PATH = {str(tmp_path / 'missing.so')!r}\n"
        "L._lib = None\n"
        "try:\n"
        "    L.lib()\n"
        "except ImportError as e:\n"
        "    print('raised', e)\n"
        "else:\n"
        "    print('no error')\n")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    assert out.stdout.startswith("raised"), out.stdout


def _product_sources():
    for d, _, files in os.walk(PKG):
        if "_build" in d or "__pycache__" in d:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                yield os.path.join(d, f)
    yield os.path.join(ROOT, "include", "gemm05.h")


def test_product_never_refers_to_the_oracle():
    """Neither the package (binding, build script, kernels, C ABI) nor the
    public header imports, links or names the oracle."""
    pat = re.compile(r"\boracle\b|liboracle|oracle_gemm", re.IGNORECASE)
    hits = []
    for path in _product_sources():
        with open(path, encoding="utf-8") as fh:
            for n, line in enumerate(fh, 1):
                if pat.search(line):
                    hits.append(f"{os.path.relpath(path, ROOT)}:{n}: {line.strip()}")
    assert not hits, "\n".join(hits)


def test_oracle_never_refers_to_the_product():
    """The oracle shares no code with the HIP path: it neither imports the
    package nor includes its headers."""
    pat = re.compile(r"dense_gemm_05_amd|gemm05\.h|g5_|libgemm05")
    hits = []
    for d, _, files in os.walk(os.path.join(ROOT, "oracle")):
        if "__pycache__" in d:
            continue
        for f in files:
            if f.endswith((".py", ".c", ".h")):
                path = os.path.join(d, f)
                with open(path, encoding="utf-8") as fh:
                    for n, line in enumerate(fh, 1):
                        if pat.search(line):
                            hits.append(f"{os.path.relpath(path, ROOT)}:{n}: {line.strip()}")
    assert not hits, "\n".join(hits)
