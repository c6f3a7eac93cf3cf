"""__graft_entry__.build() works from a clean checkout: a copy of the source tree with no
built library compiles libgdn.so and the oracle, then imports the package."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SKIP_DIRS = {".git", "_work", "_build", "gpurun_out", "__pycache__", ".pytest_cache", "profiles"}


def _copy_sources(dst):
    for dirpath, dirnames, filenames in os.walk(ROOT):
        dirnames[:] = [d for d in dirnames if d not in SKIP_DIRS]
        rel = os.path.relpath(dirpath, ROOT)
        os.makedirs(os.path.join(dst, rel), exist_ok=True)
        for f in filenames:
            if f.endswith((".so", ".o", ".tmp", ".pyc")):
                continue
            shutil.copy2(os.path.join(dirpath, f), os.path.join(dst, rel, f))


@pytest.mark.skipif(shutil.which("hipcc") is None, reason="hipcc is not installed")
def test_build_from_clean_tree(tmp_path):
    dst = str(tmp_path / "repo")
    _copy_sources(dst)
    lib = os.path.join(dst, "gated_deltanet_state_amd", "libgdn.so")
    assert not os.path.exists(lib)
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build(); "
                        "import gated_deltanet_state_amd as m; print(m.library_path, m.gdn_version())"],
                       cwd=dst, capture_output=True, text=True, timeout=900)
    print(r.stdout[-2000:], r.stderr[-4000:])
    assert r.returncode == 0
    assert os.path.exists(lib) and os.path.exists(os.path.join(dst, "oracle", "liboracle.so"))
    assert lib in r.stdout
