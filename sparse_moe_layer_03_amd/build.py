"""Build libmoe355.so (all HIP sources, gfx950) in-tree with hipcc.

    python -m sparse_moe_layer_03_amd.build
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe355.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are kept out of the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


# Host code instrumented with AddressSanitizer and UndefinedBehaviorSanitizer (device code is not):
# the build the CPU tests of the argument checks and the bucket planner run under.
SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                  "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime a process must preload to load the sanitized build."""
    cands = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found")
    return cands[-1]


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Compile every HIP source to an object (in parallel) and link the shared library at ``out``
    (``sanitize``: host code with ASan and UBSan, see SANITIZE_FLAGS)."""
    cc = hipcc()
    extra = SANITIZE_FLAGS if sanitize else []
    with tempfile.TemporaryDirectory(prefix="moe355_build_") as tmp:
        procs = []
        objs = []
        for src in sources():
            obj = os.path.join(tmp, os.path.basename(src) + ".o")
            cmd = [cc, *HIPCC_FLAGS, *extra, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
            objs.append(obj)
        failed = []
        for src, p in procs:
            msg, _ = p.communicate()
            if msg and (verbose or p.returncode):
                lines = [ln for ln in msg.splitlines() if "packed-fp32-ops" not in ln]
                if lines:
                    print("\n".join(lines), file=sys.stderr)
            if p.returncode:
                failed.append(src)
        if failed:
            raise RuntimeError("hipcc failed for: " + ", ".join(os.path.basename(f) for f in failed))
        tmp_lib = os.path.join(tmp, "libmoe355.so")
        cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib]
        subprocess.run(cmd, check=True)
        shutil.copyfile(tmp_lib, out + ".tmp")
        os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
