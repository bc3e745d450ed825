"""The product path has no CPU fallback: without the built library the
binding (and everything above it) refuses to import, loudly.  Checked on a
copy of the package that lacks libhpcattn.so, in a fresh interpreter."""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PKG = os.path.join(os.path.dirname(HERE), "load_balanced_split_amd")


def test_binding_refuses_to_import_without_the_library(tmp_path):
    dst = tmp_path / "load_balanced_split_amd"
    shutil.copytree(PKG, dst, ignore=shutil.ignore_patterns("*.so", "csrc", "__pycache__"))
    assert not any(p.suffix == ".so" for p in dst.iterdir())
    for mod in ("hpcattn", "runner"):
        r = subprocess.run([sys.executable, "-c",
                            "import load_balanced_split_amd.%s" % mod],
                           cwd=str(tmp_path), capture_output=True, text=True, timeout=120,
                           env=dict(os.environ, PYTHONPATH=str(tmp_path)))
        assert r.returncode != 0, mod
        assert "ImportError" in r.stderr and "libhpcattn.so is not built" in r.stderr, r.stderr
