"""The host-side tests under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The HIP library is rebuilt with its host code instrumented (device code as
usual) and the oracle with clang and both sanitizers; the C-ABI checks, the
launch-planner tests and the oracle pins then run in a child process with
the sanitizer runtime preloaded, against those builds.  Any report (heap or
stack overflow, use after free, signed overflow, misaligned or out-of-range
access) fails the run.  The builds are cached next to the regular ones and
redone when a source changes.
"""
import glob
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "attention_prefill_amd")
SAN_LIB = os.path.join(PKG, "_build_san", "libattn_mi355x_san.so")
SAN_ORACLE = os.path.join(ROOT, "oracle", "liboracle_san.so")
HOST_TESTS = ["tests/test_abi.py", "tests/test_plan.py", "tests/test_oracle_pins.py",
              "tests/test_oracle_kv8_pins.py", "tests/test_oracle_fp8_pins.py", "tests/test_route_inputs.py"]


def asan_runtime():
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def stale(out, sources):
    return not os.path.exists(out) or any(os.path.getmtime(s) > os.path.getmtime(out) for s in sources)


@pytest.fixture(scope="module")
def sanitized_builds():
    rt = asan_runtime()
    if rt is None or not os.path.exists("/opt/rocm/bin/hipcc") or not os.path.exists("/opt/rocm/llvm/bin/clang"):
        pytest.skip("no ROCm clang sanitizer runtime")
    sys.path.insert(0, ROOT)
    from attention_prefill_amd.build import CSRC, SOURCES, build
    from oracle.build import build_oracle
    srcs = [os.path.join(CSRC, s) for s in SOURCES] + glob.glob(os.path.join(CSRC, "*.h")) + \
        [os.path.join(ROOT, "include", "attn.h")]
    os.makedirs(os.path.dirname(SAN_LIB), exist_ok=True)
    if stale(SAN_LIB, srcs):
        build(out=SAN_LIB, sanitize_host=True)
    if stale(SAN_ORACLE, [os.path.join(ROOT, "oracle", "oracle.c")]):
        build_oracle(out=SAN_ORACLE, sanitize=True)
    return rt


def test_host_tests_under_asan_and_ubsan(sanitized_builds):
    env = dict(os.environ)
    env.update({
        "LD_PRELOAD": sanitized_builds,
        # the interpreter itself is not instrumented and keeps objects alive
        # until exit: leak reports would be about it, not about this code
        "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=0",
        "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1",
        "ATTN_LIB_PATH": SAN_LIB,
        "ORACLE_LIB_PATH": SAN_ORACLE,
        "OMP_NUM_THREADS": "1",
    })
    # both instrumented builds are the ones the child process maps
    probe = ("import attention_prefill_amd as A, oracle, numpy as np; A.load(); oracle.round_f16(np.zeros(1)); "
             "m = open('/proc/self/maps').read(); "
             "assert %r in m and %r in m and 'libclang_rt.asan' in m, 'sanitized builds not loaded'"
             % (SAN_LIB, SAN_ORACLE))
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *HOST_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-6000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-6000:]
    assert " passed" in r.stdout
