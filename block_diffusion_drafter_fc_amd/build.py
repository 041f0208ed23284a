"""Compile the HIP sources of the package into libdflash.so (gfx950)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdflash.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = os.environ.get("DFLASH_OFFLOAD_ARCH", "gfx950")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         # keep the compiler from forming packed fp32 instructions
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + INCLUDE, "-I" + CSRC]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# Per-file flags.  skinny.hip: keep single-lane atomics as written (no
# wave-level aggregation), so the LM head's group claim is waited for where
# its result is used, not right after it is issued.
FILE_FLAGS = {"skinny.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (CPU code only:
# the device code is built as usual).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer"]


def _compile(src: str, build_dir: str = BUILD_DIR, extra_flags=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    extra = FILE_FLAGS.get(os.path.basename(src), []) + list(extra_flags)
    r = subprocess.run([HIPCC] + FLAGS + extra + ["-c", src, "-o", obj], capture_output=True,
                       text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, out: str = LIB, sanitize: bool = False) -> str:
    """Build libdflash.so (or, with sanitize, a host-sanitized build at `out`)."""
    build_dir = BUILD_DIR if not sanitize else out + ".objs"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    extra = SANITIZE_HOST if sanitize else []
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, extra), srcs))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] +
                       (["-Xarch_host", "-shared-libsan"] if sanitize else []) + objs,
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
