"""The C ABI's argument validation under AddressSanitizer and UndefinedBehaviorSanitizer,
on the CPU: int8mm_abi.hip is compiled with the sanitizers on its host code only
(`-Xarch_host`; the GPU code is untouched), linked with the library's other objects and a
driver (tests/abi_sanitize_main.cpp) that calls every entry point with arguments the
library must reject before touching the HIP runtime, plus the size helpers at the int64
limits. The driver must exit 0 with no sanitizer report."""

import os
import shutil
import subprocess
import tempfile

import pytest

from int8_mixed_precision_col_amd import build as pkg_build

HIPCC = pkg_build.HIPCC
HERE = os.path.dirname(os.path.abspath(__file__))
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(
    not (os.path.exists(HIPCC) and os.path.isdir(pkg_build.BUILD)),
    reason="hipcc or the library's build objects missing (run __graft_entry__.build())")


def test_abi_validation_under_host_sanitizers():
    others = [os.path.join(pkg_build.BUILD, os.path.splitext(s)[0] + ".o")
              for s in pkg_build.SOURCES if s != "int8mm_abi.hip"]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("library build objects missing (run __graft_entry__.build())")
    tmp = tempfile.mkdtemp(prefix="i8mm_san_")
    try:
        flags = [f for f in pkg_build.FLAGS if not f.startswith("-Rpass")]
        abi_o = os.path.join(tmp, "abi_san.o")
        drv_o = os.path.join(tmp, "driver.o")
        exe = os.path.join(tmp, "abi_san")
        steps = [
            [HIPCC, *flags, *SAN, "-c", os.path.join(pkg_build.CSRC, "int8mm_abi.hip"), "-o", abi_o],
            [HIPCC, *flags, *SAN, "-c", "-x", "hip", os.path.join(HERE, "abi_sanitize_main.cpp"), "-o", drv_o],
            [HIPCC, f"--offload-arch={pkg_build.ARCH}", *SAN, abi_o, drv_o, *others, "-o", exe],
        ]
        for cmd in steps:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
            assert r.returncode == 0, f"build step failed: {' '.join(cmd)}\n{r.stderr[-3000:]}"
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
        out = r.stdout + r.stderr
        assert "AddressSanitizer" not in out and "runtime error" not in out, out[-3000:]
        assert r.returncode == 0, out[-3000:]
        assert "all checks passed" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
