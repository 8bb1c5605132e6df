"""Builds oracle/liboracle.so with gcc (test infrastructure only).

The oracle is plain C compiled without fast-math or FMA contraction so that
its fp64 arithmetic is the arithmetic written in oracle.c.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


# the LLVM C compiler of the ROCm install (its sanitizer runtime is the one the
# HIP library's host code links against, so both share one runtime)
CLANG = "/opt/rocm/llvm/bin/clang"


def build_oracle(force: bool = True, out: str = LIB, sanitize: bool = False) -> str:
    """gcc with OpenMP by default; with sanitize, clang with AddressSanitizer
    and UndefinedBehaviorSanitizer (errors fatal) and no OpenMP."""
    src = os.path.join(HERE, "oracle.c")
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + ".tmp%d" % os.getpid()
    common = ["-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math", "-frounding-math", "-Wall",
              "-Wextra"]
    if sanitize:
        cmd = [CLANG, "-O1", "-g", *common, "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
               "-fno-omit-frame-pointer", "-o", tmp, src, "-lm"]
    else:
        cmd = ["gcc", "-O2", *common, "-fopenmp", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_oracle())
