"""The product path has no CPU fallback: the package refuses to import
without its HIP library, and no product source imports or includes the
oracle (CPU only)."""
import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "compressed_fp4_kv_amd")


def test_import_fails_loudly_without_the_library(tmp_path):
    dst = tmp_path / "compressed_fp4_kv_amd"
    dst.mkdir()
    shutil.copy(os.path.join(PKG, "__init__.py"), dst / "__init__.py")
    r = subprocess.run([sys.executable, "-c", "import compressed_fp4_kv_amd"], cwd=tmp_path,
                       capture_output=True, text=True, timeout=120,
                       env={**os.environ, "PYTHONPATH": str(tmp_path)})
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "no non-HIP implementation" in r.stderr


def test_product_sources_never_reach_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle|from\s+oracle|#\s*include\s*[<\"][^>\"]*oracle)",
                     re.M)
    for d, _, files in os.walk(PKG):
        if "__pycache__" in d or "_build" in os.path.relpath(d, PKG).split(os.sep)[0:1]:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                src = open(os.path.join(d, f), encoding="utf-8").read()
                assert not pat.search(src), f"{os.path.join(d, f)} reaches the oracle"
