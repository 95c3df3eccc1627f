"""AddressSanitizer and UndefinedBehaviorSanitizer over the host code.

Both libraries are rebuilt with the sanitizers: the oracle (oracle.c, clang, serial) and the GPU
library with its host side instrumented (argument validation, workspace sizes and layouts,
dispatch: api.hip and the launch code of every source; the device code is the normal build). A
child process with clang's ASan runtime preloaded then runs the CPU tests that exercise that
code: the C ABI's validation paths and workspace queries, the binding's checks and the oracle's
pins. No kernel runs. Any ASan report, or any UBSan report (fatal with -fno-sanitize-recover),
fails the child and so this test.
"""
import importlib
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# the child checks that the sanitized builds are the ones mapped, not the normal libraries
_CHECK = """
import sys
sys.path.insert(0, {root!r})
from linear_recurrent_sequence_chunkwise_amd import retention as R
import oracle
R.load_library()
oracle.get()
maps = open("/proc/self/maps").read()
for name in ("libclang_rt.asan", "libretention_asan.so", "liboracle_asan.so"):
    assert name in maps, name + " is not loaded"
for name in ("/libretention.so", "/liboracle.so"):
    assert name not in maps, name + " is loaded"
print("sanitized libraries loaded")
"""


def test_host_code_under_asan_and_ubsan():
    from linear_recurrent_sequence_chunkwise_amd import build as lib_build
    oracle_build = importlib.import_module("oracle.build")  # the module (the package re-exports its build function)

    lib = lib_build.build(verbose=False, sanitize=True)
    olib = oracle_build.build_sanitized(quiet=True)
    preload = " ".join(p for p in (lib_build.sanitizer_runtime(), os.environ.get("LD_PRELOAD", "")) if p)
    env = dict(os.environ, LD_PRELOAD=preload, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", RETENTION_LIB=lib, RETENTION_ORACLE_LIB=olib)
    r = subprocess.run([sys.executable, "-c", _CHECK.format(root=ROOT)], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "-m", "not gpu",
                        "tests/test_abi.py", "tests/test_binding.py", "tests/test_oracle.py"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    print(r.stdout.strip().splitlines()[-1])
