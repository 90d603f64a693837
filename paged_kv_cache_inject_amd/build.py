"""Builds libpkv.so in-tree with hipcc for gfx950.

The HIP sources are compiled with contraction of float multiply-add turned
off (the key rotation must be two products and one add, unfused) and with
the packed-fp32 instructions disabled.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpkv.so")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument", "-I", INCLUDE]
SOURCES = [os.path.join(CSRC, "pkv_host.cpp"), os.path.join(CSRC, "pkv_kernels.hip")]
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build of the same
# sources (device code is compiled as usual): for running the CPU tests of the
# allocator and planners with the sanitizer runtime preloaded.
LIB_SAN = os.path.join(HERE, "libpkv_san.so")
SAN_FLAGS = ["-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer"]


def sanitizer_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to LD_PRELOAD)."""
    clang = os.path.join(os.path.dirname(os.path.realpath(HIPCC)), "..", "llvm", "bin", "clang")
    res = subprocess.run([clang, "-print-file-name=libclang_rt.asan-x86_64.so"],
                         capture_output=True, text=True)
    return res.stdout.strip()


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compile every source into libpkv.so (always recompiles); with
    sanitize, into libpkv_san.so with host-side ASan/UBSan."""
    out = LIB_SAN if sanitize else LIB
    tmp = out + ".tmp"
    flags = [f for f in FLAGS if f != "-O3"] + SAN_FLAGS if sanitize else FLAGS
    cmd = [HIPCC] + flags + SOURCES + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + err)
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        print(build(verbose=True, sanitize=True))
        print("runtime to preload:", sanitizer_runtime())
    else:
        print(build(verbose=True))
