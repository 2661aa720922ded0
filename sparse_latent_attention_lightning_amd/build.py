"""Builds libdsa.so (the HIP kernels + C ABI) in-tree for gfx950.

    python -m sparse_latent_attention_lightning_amd.build

Each .hip file compiles separately (in parallel) with hipcc, then the objects
link into ``sparse_latent_attention_lightning_amd/libdsa.so``.
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = os.environ.get("DSA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # never emit packed-fp32 VALU ops (v_pk_add/mul/fma_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-munsafe-fp-atomics", "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def _compile(src: str, extra, build_dir: str) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    noisy = [ln for ln in (r.stderr or "").splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noisy:
        sys.stderr.write("\n".join(noisy) + "\n")
    return obj


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer for a CPU check of
# the library's host code (argument checks, workspace sizing, error paths).
# Each -fsanitize= applies to the host pass only; device code is unchanged.
HOST_SANITIZE_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                       "-Xarch_host", "-fno-sanitize-recover=undefined",
                       "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def build(extra=(), jobs: int = 8, out: str = LIB, build_dir: str = BUILD_DIR) -> str:
    """Compile every csrc/*.hip and link them into `out` (default: the
    in-tree libdsa.so the binding loads)."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with ThreadPoolExecutor(max_workers=min(jobs, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra), build_dir), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


DEBUG_LIB = os.path.join(PKG, "libdsa_debug.so")


def build_debug(jobs: int = 8) -> str:
    """libdsa_debug.so: the same sources with -DDSA_DEBUG (LDS filled with
    0xff bytes before first use; index rows checked on the device, with a
    synchronizing read-back, after top-K and before the attention)."""
    return build(extra=["-DDSA_DEBUG"], jobs=jobs, out=DEBUG_LIB, build_dir=os.path.join(BUILD_DIR, "debug"))


if __name__ == "__main__":
    print(build())
    if "--debug" in sys.argv[1:]:
        print(build_debug())
