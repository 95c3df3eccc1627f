"""Compile the gfx950 HIP sources under csrc/ into libretention.so (in this package directory).

Every call recompiles. Objects go to _build/ at the repository root; the .so lands next to this
file so that it ships with the source tree. No torch extension machinery is involved: the
library is a plain C-ABI shared object loaded through ctypes.

`build(sanitize=True)` (or `python -m linear_recurrent_sequence_chunkwise_amd.build --sanitize`)
builds libretention_asan.so instead: the same device code, with the host code (argument
validation, workspace layout, dispatch) instrumented by AddressSanitizer and
UndefinedBehaviorSanitizer. It is a CPU test artefact: it loads only with clang's ASan runtime
preloaded (SANITIZER_RUNTIME), and the CPU tests that run under it never launch a kernel.
"""
import glob
import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libretention.so")
LIB_ASAN = os.path.join(PKG, "libretention_asan.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off: hipcc still vectorises scalar fp32 code without them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# host-side instrumentation only (each option applies to the host compilation pass)
SANITIZE = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=undefined".split() + \
    "-Xarch_host -fno-omit-frame-pointer -Xarch_host -g".split()


def sanitizer_runtime() -> str:
    """clang's ASan runtime (with the UBSan handlers), to preload into a process that loads a
    sanitized library."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise RuntimeError("clang's ASan runtime is not installed under /opt/rocm/llvm")
    return found[-1]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src, sanitize=False):
    obj = os.path.join(BUILD, ("asan_" if sanitize else "") + os.path.basename(src) + ".o")
    cmd = [HIPCC, *CFLAGS, *(SANITIZE if sanitize else []), "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "'-packed-fp32-ops' is not a recognized feature"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{err}")
    return obj, err


def build(verbose: bool = True, sanitize: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    out = LIB_ASAN if sanitize else LIB
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _compile(s, sanitize), srcs))
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + " ".join(cmd) + "\n" + res.stderr)
    # every kernel the host code launches must be defined in the library (a host pass that silently
    # drops a kernel template leaves an undefined symbol that only dlopen would report)
    res = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [l.split()[-1] for l in res.stdout.splitlines() if "_ZN3ret" in l]
    if missing:
        raise RuntimeError("library references undefined symbols of its own: " + ", ".join(missing[:4]))
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(sanitize="--sanitize" in sys.argv[1:])
