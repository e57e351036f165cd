"""Build libspconv_mi355x.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libspconv_mi355x.so")
SOURCES = ["capi.hip", "nmap.hip", "forward.hip", "wgrad.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


def flags(extra=()):
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # packed fp32 instructions stay off: the compiler must not form them
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"), *extra]


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer (the device code is
# built as usual): every sanitizer flag applies to the host pass only.
SANITIZE = ["-g", "-fno-omit-frame-pointer",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined"]
ASAN_LIB = os.path.join(BUILD, "asan", "libspconv_mi355x_asan.so")


def build(verbose: bool = False, extra=(), sanitize: bool = False) -> str:
    """Compile every source and link the library in the package directory;
    sanitize: a host-sanitized build under _build/asan instead, for a process
    that preloads clang's ASan runtime and sets SPCONV_LIB to it."""
    bdir = os.path.join(BUILD, "asan") if sanitize else BUILD
    os.makedirs(bdir, exist_ok=True)
    cc = hipcc()
    if sanitize:
        extra = (*extra, *SANITIZE)

    def compile_one(src):
        obj = os.path.join(bdir, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *flags(extra), "-c", os.path.join(CSRC, src), "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines()
                         if "packed-fp32-ops" not in l)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{msgs}")
        if verbose and msgs.strip():
            print(msgs)
        return obj

    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    lib = ASAN_LIB if sanitize else LIB
    tmp = lib + ".tmp"
    link = [cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    if sanitize:
        link[1:1] = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libasan"]
    subprocess.check_call(link)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
