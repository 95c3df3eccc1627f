"""Build the fp64 CPU oracle (oracle.c) into liboracle.so next to this file.

Test infrastructure: the oracle is a checker for the GPU library, never part of it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")
LIB_ASAN = os.path.join(HERE, "liboracle_asan.so")
CLANG = "/opt/rocm/llvm/bin/clang"


def build(src: str = SRC, out: str = LIB, quiet: bool = False) -> str:
    """Compile `src` with gcc (-O2, OpenMP, IEEE arithmetic: no fast-math) into `out`."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-fno-fast-math", "-ffp-contract=off", src, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


def build_sanitized(src: str = SRC, out: str = LIB_ASAN, quiet: bool = False) -> str:
    """The same source with AddressSanitizer and UndefinedBehaviorSanitizer (clang, so that one
    preloaded ASan runtime serves it and the sanitized GPU library's host code), without OpenMP
    (the loops run serially), any UB report fatal."""
    cmd = [CLANG, "-O1", "-g", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra", "-fno-fast-math", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           src, "-o", out + ".tmp", "-lm"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("sanitized oracle build failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    os.replace(out + ".tmp", out)
    if not quiet:
        print("built", out)
    return out


if __name__ == "__main__":
    if sys.argv[1:2] == ["--sanitize"]:
        build_sanitized()
    else:
        build(*sys.argv[1:])
