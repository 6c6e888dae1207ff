"""Without the built HIP library the package refuses to load: there is no
CPU fallback for any step (CPU only; runs on a copy of the package's Python
files in a temporary directory, so the real library is untouched)."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = "mixture_experts_layer_gating_amd"


@pytest.mark.parametrize("module", [f"{PKG}._lib", f"{PKG}.layer"])
def test_import_without_library_fails_loudly(tmp_path, module):
    dst = tmp_path / PKG
    dst.mkdir()
    for name in os.listdir(os.path.join(ROOT, PKG)):
        if name.endswith(".py"):
            shutil.copy(os.path.join(ROOT, PKG, name), dst / name)
    assert not (dst / "libmoe.so").exists()
    code = (f"import sys; sys.path.insert(0, {str(tmp_path)!r})\n"
            f"try:\n    import {module}\n"
            f"except ImportError as e:\n    print('refused:', e); sys.exit(0)\n"
            f"sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "libmoe.so is missing" in r.stdout
