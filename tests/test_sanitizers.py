"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* libattn: every source is rebuilt with the sanitizers on its host code only
  (``-Xarch_host -fsanitize=...``; the gfx950 device code is built as usual),
  then ``tests/sanitize/abi_driver.py`` drives the argument validation (every
  rejected configuration, with degenerate and extreme sizes) and the size
  and layout queries through the C ABI, in a child process with clang's
  sanitizer runtime preloaded.  None of these calls reaches the GPU.
* The oracle: ``oracle.c`` is rebuilt with gcc's sanitizers and
  ``tests/sanitize/oracle_driver.py`` runs every routine on small inputs.

A sanitizer report makes the child exit with a non-zero status and the test
prints it.
"""
import glob
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "softmax_attention_attn_amd")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clang_asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def _gcc_runtime(name):
    r = subprocess.run(["gcc", "-print-file-name=" + name], capture_output=True, text=True)
    p = r.stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _run(cmd, env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    return subprocess.run(cmd, capture_output=True, text=True, env=env, timeout=300)


@pytest.fixture(scope="module")
def tmp():
    d = tempfile.mkdtemp(prefix="attn_san_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def test_libattn_host_code_sanitized(tmp):
    rt = _clang_asan_runtime()
    if rt is None or not os.path.exists(HIPCC):
        pytest.skip("clang sanitizer runtime or hipcc not available")
    sys.path.insert(0, PKG)
    import _build  # the library's own build flags
    sys.path.pop(0)
    srcs = _build.sources()

    def comp(src):
        obj = os.path.join(tmp, os.path.basename(src) + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [HIPCC] + _build.COMMON + ["-g"] + SAN + lang + ["-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(comp, srcs))
    lib = os.path.join(tmp, "libattn_san.so")
    r = subprocess.run([HIPCC, "--offload-arch=" + _build.ARCH, "-shared", "-fPIC"] + SAN +
                       objs + ["-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "abi_driver.py"), lib,
              os.path.join(PKG, "_abi.py")],
             {"LD_PRELOAD": rt, "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
              "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1"})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "all statuses as expected" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]


def test_oracle_sanitized(tmp):
    asan, ubsan = _gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not available")
    lib = os.path.join(tmp, "liboracle_san.so")
    r = subprocess.run(["gcc", "-O1", "-g", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                        "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                        "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "oracle.c"),
                        "-o", lib, "-lm"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = _run([sys.executable, os.path.join(ROOT, "tests", "sanitize", "oracle_driver.py"), lib],
             {"LD_PRELOAD": asan + ":" + ubsan,
              "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1",
              "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1", "OMP_NUM_THREADS": "4"})
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "every routine ran" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-6000:]
