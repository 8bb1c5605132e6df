"""Builds the HIP library libattn_mi355x.so in-tree for gfx950 with hipcc."""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn_mi355x.so")
SOURCES = ["attn_api.cpp", "attn_kernels.hip", "attn_unfused.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-fp32 VALU instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


# host code only, for the CPU sanitizer run of the host-side tests: AddressSanitizer
# and UndefinedBehaviorSanitizer (errors fatal); device code is built as usual
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer",
                 "-Xarch_host", "-g"]


def build(verbose: bool = False, out: str = LIB, defines=(), sanitize_host: bool = False) -> str:
    """Compile the library to `out`; `defines` are extra -D settings of the
    kernel source (build-time alternatives such as ATTN_FUSED_KQUANT=1);
    sanitize_host instruments the host code (the result then needs the
    sanitizer runtime preloaded)."""
    objs, procs = [], []
    tag = "_".join(d.replace("=", "") for d in defines) + ("_san" if sanitize_host else "")
    bdir = os.path.join(PKG, "_build" if not tag else "_build_" + tag)
    os.makedirs(bdir, exist_ok=True)
    for src in SOURCES:
        obj = os.path.join(bdir, src + ".o")
        cmd = [HIPCC, *FLAGS, *(HOST_SANITIZE if sanitize_host else []), *("-D" + d for d in defines), "-c",
               os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append(subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True))
        objs.append(obj)
    failed = False
    for p in procs:
        _, err = p.communicate()
        err = "\n".join(ln for ln in err.splitlines()
                        if "packed-fp32-ops" not in ln and "is not a recognized feature" not in ln)
        if err.strip():
            sys.stderr.write(err + "\n")
        failed |= p.returncode != 0
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs,
                    "-L/opt/rocm/lib", "-lrocblas"], check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
