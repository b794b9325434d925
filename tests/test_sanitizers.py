"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Two instrumented builds go into a temporary directory: the fp64 oracle
(oracle.c, clang -fsanitize=address,undefined, without OpenMP so each call
runs on one thread) and libsinkattn with its host code instrumented
(hipcc -Xarch_host -fsanitize=...; the gfx950 device code is built as usual).
The C-ABI tests (every argument check, the workspace arithmetic, the tile
choice, the no-alloc size check) and the oracle's pins then run in a child
process with clang's ASan runtime preloaded, the two libraries selected by
their path variables, and UBSan set to stop at the first report.  A planted
heap overflow in a third small library must be caught in the same
environment, which shows the runtime is live.  No GPU is used."""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LLVM = "/opt/rocm/llvm"
CLANG = os.path.join(LLVM, "bin", "clang")
RUNTIME = sorted(glob.glob(os.path.join(LLVM, "lib", "clang", "*", "lib", "linux",
                                        "libclang_rt.asan-x86_64.so")))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-shared-libsan"]

pytestmark = pytest.mark.skipif(not (os.path.exists(CLANG) and RUNTIME),
                                reason="ROCm clang or its ASan runtime is missing")

PLANTED = r"""
#include <stdlib.h>
int overflow(int n) {
  int* a = (int*)malloc(sizeof(int) * (size_t)n);
  for (int i = 0; i <= n; ++i) a[i] = i;   /* one past the end */
  int s = a[0];
  free(a);
  return s;
}
"""


def _env(lib, oracle):
    return dict(os.environ, LD_PRELOAD=RUNTIME[-1],
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
                UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1",
                SINKATTN_LIBRARY=lib, SINKATTN_ORACLE_LIB=oracle)


@pytest.fixture(scope="module")
def builds(tmp_path_factory):
    d = tmp_path_factory.mktemp("san")
    oracle = str(d / "liboracle_san.so")
    subprocess.run([CLANG, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    *SAN, os.path.join(ROOT, "oracle", "oracle.c"), "-o", oracle, "-lm"],
                   check=True)
    from attention_qk_rmsnorm_amd.build import CSRC, HIPCC_FLAGS, INCLUDE, sources
    flags = [f for f in HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"]
    for f in SAN:
        flags += ["-Xarch_host", f]
    lib = str(d / "libsinkattn_san.so")
    r = subprocess.run(["/opt/rocm/bin/hipcc", *flags, "-I", INCLUDE, "-I", CSRC, *sources(),
                        "-o", lib], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    planted = str(d / "libplanted.so")
    src = d / "planted.c"
    src.write_text(PLANTED)
    subprocess.run([CLANG, "-O0", "-g", "-fPIC", "-shared", *SAN, str(src), "-o", planted],
                   check=True)
    return lib, oracle, planted


def test_the_sanitizer_runtime_catches_a_planted_overflow(builds):
    lib, oracle, planted = builds
    code = f"import ctypes; ctypes.CDLL({planted!r}).overflow(8)"
    r = subprocess.run([sys.executable, "-c", code], env=_env(lib, oracle),
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-2000:]


def test_abi_and_oracle_pins_under_asan_and_ubsan(builds):
    lib, oracle, _ = builds
    tests = ["tests/test_abi.py", "tests/test_oracle_pins.py", "tests/test_oracle_bwd_pins.py",
             "tests/test_oracle_padded_pins.py"]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", *tests], cwd=ROOT, env=_env(lib, oracle),
                       capture_output=True, text=True, timeout=900)
    tail = (r.stdout + r.stderr)[-3000:]
    assert r.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error" not in tail, tail
    # the child really loaded the instrumented libraries
    code = ("import attention_qk_rmsnorm_amd as A, oracle.oracle as O; A.load_library(); "
            "O._load(); m = open('/proc/self/maps').read(); "
            f"assert {lib!r} in m and {oracle!r} in m and 'libclang_rt.asan' in m")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=_env(lib, oracle),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, (r.stdout + r.stderr)[-2000:]
