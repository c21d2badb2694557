"""Build libattn.so (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python -m transformer_self_attention_amd.build [--verbose]``.  Every call recompiles
every source (object files go to ``_build/`` at the repository root, the library next to this
file).  Packed fp32 VALU instructions are disabled for all device code.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libattn.so")
ARCH = "gfx950"

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wextra",
    "-Wno-unused-value",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libattn.so)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str, verbose: bool, obj_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"  # host pass does not know the device-only feature flag
    msgs = "\n".join(line for line in (res.stdout + res.stderr).splitlines() if noise not in line)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    return obj


def _build(out: str, obj_dir: str, extra=(), verbose: bool = False) -> str:
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, obj_dir, extra), srcs))
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """libattn.so, the product build."""
    return _build(LIB_PATH, BUILD_DIR, verbose=verbose)


CHECKED_LIB_PATH = os.path.join(PKG_DIR, "libattn_checked.so")


def build_checked(verbose: bool = False) -> str:
    """libattn_checked.so: the same sources with ATTN_CHECKED defined, so every kernel tests its
    indices before the accesses they guard and reports failures through attn_checked_sites()
    (load it with ATTN_LIBRARY=<path>).  A debugging aid, never the product path."""
    return _build(CHECKED_LIB_PATH, os.path.join(BUILD_DIR, "checked"), extra=("-DATTN_CHECKED",), verbose=verbose)


# Host code of the C ABI (argument validation, dispatch) under AddressSanitizer and UBSan; device
# code is built as usual.  Each sanitizer flag applies to the host pass only.
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str:
    """The shared ASan runtime of the ROCm clang; a process that loads the host-sanitized library
    must preload it (LD_PRELOAD)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    clang = os.path.join(rocm, "lib", "llvm", "lib", "clang")
    for ver in sorted(os.listdir(clang)) if os.path.isdir(clang) else []:
        path = os.path.join(clang, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    raise RuntimeError(f"no libclang_rt.asan-x86_64.so under {clang}")


def build_host_sanitized(verbose: bool = False) -> str:
    """libattn.so with the host code of attn_api.hip under ASan + UBSan (-O1 -g), at
    _build/sanitize/libattn_sanitized.so; load it with ATTN_LIBRARY=<path> and the runtime of
    asan_runtime() preloaded."""
    out_dir = os.path.join(BUILD_DIR, "sanitize")
    os.makedirs(out_dir, exist_ok=True)

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        flags = list(COMMON_FLAGS)
        if os.path.basename(src) == "attn_api.hip":
            flags = [f for f in flags if f != "-O3"] + ["-O1", "-g", *SANITIZE_HOST]
        res = subprocess.run([hipcc(), *flags, "-c", src, "-o", obj], capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}{res.stderr}")
        return obj

    srcs = sources()
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    path = os.path.join(out_dir, "libattn_sanitized.so")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-shared-libasan", *SANITIZE_HOST[:4],
           "-o", path, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    return path


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
