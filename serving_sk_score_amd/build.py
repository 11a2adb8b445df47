"""Build ``libsk.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m serving_sk_score_amd.build``.  Every source is compiled
every time (objects go to ``_build/`` at the repository root), then linked
into ``serving_sk_score_amd/libsk.so``.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libsk.so")
ARCH = "gfx950"

SOURCES = ["sk_api.cpp", "pack.hip", "select.hip", "score.hip", "importance.hip", "decode.hip"]

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    # packed fp32 VALU ops are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # exact IEEE semantics for the quantizer: no contraction, correctly
    # rounded fp32 division
    "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # MFMA results in architectural VGPRs: the softmax reads them directly
    # instead of copying each element out of an AGPR first
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall",
    "-Wno-unused-function",
    f"-I{INCLUDE}",
]


# Flags for one source only.  The score passes take the iterative ILP
# machine scheduler: it interleaves a unit's softmax with the next unit's
# MFMAs better than the default one does (column pass 3-6% faster on the
# Qwen- and Gemma-shaped layers and at 40K tokens, row pass within +-0.5%,
# the same bits; no spills, two wavefronts per SIMD as before).
SOURCE_FLAGS = {
    "score.hip": ["-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libsk.so)")


def _compile(src, verbose):
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass warns that it does not know the packed-fp32 feature
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    return obj


def build(verbose=False, jobs=4):
    os.makedirs(OBJDIR, exist_ok=True)
    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


# Host-sanitized build: the same sources and device code, with the host C++
# (argument validation, the plan's closed form, workspace sizes, launch-grid
# arithmetic) instrumented by AddressSanitizer and UndefinedBehaviorSanitizer.
# Every sanitizer flag applies to the host pass only.  The result is a test
# artefact under _build/, loaded into a process that preloads the ASan
# runtime (asan_runtime()); it is never the library the package loads.
SAN_DIR = os.path.join(OBJDIR, "host_san")
SAN_LIB = os.path.join(SAN_DIR, "libsk_host_san.so")
_SAN = ["-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=all",
        "-fno-omit-frame-pointer", "-g"]


def _host_only(flags):
    out = []
    for f in flags:
        out += ["-Xarch_host", f]
    return out


def build_host_sanitized(verbose=False, jobs=6):
    """Build (when a source is newer than the last build) and return the path
    of the host-sanitized library."""
    srcs = [os.path.join(CSRC, f) for f in SOURCES + ["sk_kernels.h"]]
    srcs.append(os.path.join(INCLUDE, "sk.h"))
    if os.path.exists(SAN_LIB) and os.path.getmtime(SAN_LIB) >= max(map(os.path.getmtime, srcs)):
        return SAN_LIB
    os.makedirs(SAN_DIR, exist_ok=True)

    def one(src):
        obj = os.path.join(SAN_DIR, src + ".o")
        cmd = [hipcc(), *FLAGS, *_host_only(_SAN), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src} (host-sanitized):\n{r.stderr}")
        return obj

    with ThreadPoolExecutor(max(1, jobs)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = SAN_LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC",
           *_host_only(["-fsanitize=address", "-fsanitize=undefined", "-shared-libsan"]),
           *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (host-sanitized):\n{r.stderr}")
    os.replace(tmp, SAN_LIB)
    return SAN_LIB


def asan_runtime():
    """The shared ASan runtime of the ROCm compiler (preloaded into the
    process that loads the host-sanitized library)."""
    for clang in ("/opt/rocm/llvm/bin/clang", shutil.which("clang")):
        if not clang or not os.path.exists(clang):
            continue
        r = subprocess.run([clang, "-print-resource-dir"], capture_output=True, text=True)
        if r.returncode == 0:
            path = os.path.join(r.stdout.strip(), "lib", "linux", "libclang_rt.asan-x86_64.so")
            if os.path.exists(path):
                return path
    raise RuntimeError("ASan runtime of the ROCm compiler not found")


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
