"""__graft_entry__.build() works on a checkout where nothing is built yet: the
package refuses to import without libattn.so, so build() must compile before
it imports anything from the package.  The sources are copied into a fresh
directory and built there with hipcc (gfx950) and gcc; no GPU is needed."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _copy_sources(dst):
    shutil.copy(os.path.join(ROOT, "__graft_entry__.py"), dst)
    shutil.copy(os.path.join(ROOT, "workloads.py"), dst)
    shutil.copytree(os.path.join(ROOT, "include"), os.path.join(dst, "include"))
    keep = lambda d, names: [n for n in names if n.endswith((".so", ".o", ".pyc"))
                             or n in ("_build", "__pycache__")]
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"), ignore=keep)
    shutil.copytree(os.path.join(ROOT, "softmax_attention_attn_amd"),
                    os.path.join(dst, "softmax_attention_attn_amd"), ignore=keep)


@pytest.mark.skipif(not os.path.exists(os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")),
                    reason="hipcc is not installed")
def test_build_from_a_fresh_checkout(tmp_path):
    _copy_sources(str(tmp_path))
    lib = tmp_path / "softmax_attention_attn_amd" / "libattn.so"
    assert not lib.exists()
    r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"],
                       cwd=str(tmp_path), capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stderr[-3000:]
    assert lib.exists() and (tmp_path / "oracle" / "liboracle.so").exists()
