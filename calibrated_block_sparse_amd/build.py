"""Builds libcalibatt.so in-tree with hipcc for gfx950.

    python -m calibrated_block_sparse_amd.build            # libcalibatt.so
    python -m calibrated_block_sparse_amd.build --sanitize # libcalibatt_asan.so

Every translation unit under csrc/ is compiled to an object file under
_build/ (in parallel), then linked into calibrated_block_sparse_amd/libcalibatt.so.
The sanitized variant instruments the host code only (AddressSanitizer and
UndefinedBehaviorSanitizer; the device code is built as usual) into
_build_asan/ and libcalibatt_asan.so; it is for the CPU tests of the host
side (argument checks, list validation, the mask bank reader) and is loaded
with the sanitizer runtime preloaded (see asan_runtime()).
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcalibatt.so")
BUILD_ASAN = os.path.join(PKG, "_build_asan")
LIB_ASAN = os.path.join(PKG, "libcalibatt_asan.so")
# host-only instrumentation: each sanitizer flag goes to the host compiler
SANITIZE_FLAGS = ["-O1", "-g", "-Xarch_host", "-fno-omit-frame-pointer",
                  "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
ARCH = "gfx950"

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # keep the compiler from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the scores feed VALU softmax code, and
    # the accumulation-register form costs a copy per value
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, extra, out_dir: str = BUILD) -> str:
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{errs}")
    if errs.strip():
        print(errs, file=sys.stderr)
    return obj


def build(extra=(), verbose: bool = False, sanitize: bool = False) -> str:
    out_dir, lib = (BUILD_ASAN, LIB_ASAN) if sanitize else (BUILD, LIB)
    flags = list(extra) + (SANITIZE_FLAGS if sanitize else [])
    os.makedirs(out_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, flags, out_dir), srcs))
    tmp = lib + ".tmp"
    link = ["-shared-libasan", *SANITIZE_FLAGS[2:]] if sanitize else []
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *link, *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime, which a
    process loading libcalibatt_asan.so must preload (LD_PRELOAD)."""
    r = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True)
    p = r.stdout.strip()
    if r.returncode == 0 and os.path.isabs(p) and os.path.exists(p):
        return p
    import glob
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/*/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("AddressSanitizer runtime not found")
    return hits[-1]


if __name__ == "__main__":
    build(verbose=True, sanitize="--sanitize" in sys.argv[1:])
