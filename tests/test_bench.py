"""Host-side checks of bench.py: its counting rules against independent counts and the totals the
workloads are quoted with, and the one-GPU guard. No GPU needed."""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def pairs_bruteforce(N, C):
    """Causal (n, m) pairs with m <= n in the same chunk, counted one by one."""
    return sum(1 for n in range(N) for m in range(n + 1) if n // C == m // C)


def test_chunk_pairs_against_bruteforce():
    b = load_bench()
    for N, C in [(1, 64), (7, 8), (64, 64), (250, 64), (256, 64), (300, 128), (129, 128)]:
        dk, dv = 3, 5
        inter = 4 * N * dk * dv
        assert b.chunk_flops(1, 1, N, dk, dv, C) == 2 * (dk + dv) * pairs_bruteforce(N, C) + inter, (N, C)
        assert b.backward_flops(1, 1, N, dk, dv, C) == 2 * (3 * dk + 2 * dv) * pairs_bruteforce(N, C) + 10 * N * dk * dv


def test_quoted_totals():
    b = load_bench()
    # the N=8192 layer at chunk 128: 81.7 GFLOP algorithmic
    assert b.chunk_flops(1, 16, 8192, 256, 512, 128) == 81_705_041_920
    # N=65536 at chunk 64 / 128 / 256 / 512: 602 / 654 / 757 / 963 GFLOP
    got = [b.chunk_flops(1, 16, 65536, 256, 512, C) / 1e9 for C in (64, 128, 256, 512)]
    assert [round(g) for g in got] == [602, 654, 757, 963], got
    # the decode step of 128 x 16 fp32 256 x 512 states: 2,155,872,256 bytes
    assert b.decode_bytes(128, 16, 256, 512) == 2_155_872_256
    # the layer's bf16 q, k, v read and bf16 out written (384 MiB), plus the fp32 final state written
    # once (8 MiB): 392 MiB
    assert b.chunk_bytes(1, 16, 8192, 256, 512) == 384 * 2 ** 20
    assert b.chunk_bytes(1, 16, 8192, 256, 512) + 16 * 256 * 512 * 4 == 392 * 2 ** 20
    # the parallel form of the layer: every causal pair, 825 GFLOP
    assert round(2 * (256 + 512) * 16 * 8192 * 8193 // 2 / 1e9) == 825


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                         timeout=120)
    assert res.returncode == 2
    assert "exactly one GPU" in res.stderr
    assert res.stdout == ""
