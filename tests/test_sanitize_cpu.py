"""Host AddressSanitizer and UndefinedBehaviorSanitizer on the CPU: the step library's host
code (validation, partition, chunk and tile tables, error paths; built with the
sanitizers on its host side only) and the oracle (built with gcc's sanitizers, under its
own pin tests).  Each run happens in a subprocess with the sanitizer runtime preloaded,
since the Python interpreter itself is not instrumented."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
HIPCC = "/opt/rocm/bin/hipcc"
CLANG = "/opt/rocm/llvm/bin/clang"
ENV = dict(ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:verify_asan_link_order=0",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")


def _runtime(cmd):
    path = subprocess.run(cmd, capture_output=True, text=True).stdout.strip()
    if not os.path.isabs(path) or not os.path.exists(path):
        pytest.skip(f"sanitizer runtime not found ({' '.join(cmd)})")
    return path


def test_library_host_code_under_asan_ubsan(tmp_path):
    if not os.path.exists(HIPCC):
        pytest.skip("hipcc not available")
    so = str(tmp_path / "libneox_zero1_san.so")
    sys.path.insert(0, ROOT)
    from mixed_precision_zero_amd.build import SOURCES as src
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "mixed_precision_zero_amd", "csrc"), *src, "-o", so],
                   check=True, capture_output=True)
    rt = _runtime([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"])
    r = subprocess.run([sys.executable, os.path.join(HERE, "host_sanitize_driver.py"), so],
                       env={**os.environ, **ENV, "LD_PRELOAD": rt},
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0 and "host code exercised" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]


def test_oracle_under_asan_ubsan(tmp_path):
    so = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                    "-fno-fast-math", "-fsanitize=address,undefined", "-fno-omit-frame-pointer",
                    "-o", so, os.path.join(ROOT, "oracle", "oracle.c"), "-lm"],
                   check=True, capture_output=True)
    rt = _runtime(["gcc", "-print-file-name=libasan.so"])
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(HERE, "test_oracle_step.py"),
                        os.path.join(HERE, "test_oracle_partition.py")],
                       env={**os.environ, **ENV, "LD_PRELOAD": rt, "NEOX_ORACLE_SO": so},
                       capture_output=True, text=True, timeout=900, cwd=ROOT)
    assert r.returncode == 0 and " passed" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
