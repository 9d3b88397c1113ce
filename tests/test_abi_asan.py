"""The C interface under AddressSanitizer, on the CPU: the library's host
code (argument checks, plan sizing, the host-side plan, the status strings)
is rebuilt with -fsanitize=address (host code only; the gfx950 device code
is compiled as usual and never runs here) and tests/test_abi.py runs against
that build in a child process with the ASan runtime preloaded. Any invalid
host memory access in those paths aborts the child with an ASan report."""
import hashlib
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OUT_DIR = os.path.join(ROOT, "_build", "asan")
LIB = os.path.join(OUT_DIR, "libmla_decode.so")
LLVM = "/opt/rocm/llvm/bin"


def _asan_runtime():
    clang = os.path.join(LLVM, "clang")
    if not os.path.exists(clang):
        return None
    path = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                          capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build():
    from mla_paged_kv_03_amd import build as B
    flags = [*B.HIP_FLAGS, "-Xarch_host", "-fsanitize=address",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
    srcs = B.sources()
    key = hashlib.sha256()
    for f in [*srcs, *sorted(os.path.join(ROOT, "include", n)
                             for n in os.listdir(os.path.join(ROOT, "include")))] + \
             sorted(os.path.join(B.PKG, "csrc", n) for n in os.listdir(os.path.join(B.PKG, "csrc"))
                    if n.endswith(".h")):
        key.update(open(f, "rb").read())
    key.update(" ".join(flags).encode())
    stamp = os.path.join(OUT_DIR, "stamp")
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == key.hexdigest():
        return
    os.makedirs(OUT_DIR, exist_ok=True)
    cmd = [B.hipcc(), *flags, "-I", os.path.join(ROOT, "include"), "-o", LIB, *srcs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    with open(stamp, "w") as f:
        f.write(key.hexdigest())


def test_abi_tests_pass_under_address_sanitizer():
    runtime = _asan_runtime()
    if runtime is None or shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("hipcc or the ASan runtime is not available")
    _build()
    # the build is instrumented: its host code calls the ASan report hooks
    readelf = os.path.join(LLVM, "llvm-readelf")
    if not os.path.exists(readelf):
        readelf = shutil.which("readelf")
    syms = subprocess.run([readelf, "--dyn-syms", "-W", LIB], capture_output=True,
                          text=True).stdout
    assert "__asan_report_load" in syms or "__asan_loadN" in syms, "no ASan instrumentation"
    env = dict(os.environ)
    env.update(MLA_DECODE_LIB=LIB, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                          "-m", "not gpu", os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = res.stdout + res.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert res.returncode == 0, out[-4000:]
    assert " passed" in out
