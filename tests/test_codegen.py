"""Code generation of the streaming kernels (CPU: hipcc for gfx950, device assembly only, no GPU).

A buffer access whose resource descriptor the compiler cannot prove wave-uniform gets wrapped in a
readfirstlane loop: per access, v_readfirstlane of the four descriptor words, v_cmp_eq_u64 against
every lane's copy, s_and_saveexec, the access, and a branch back until every lane was served. The
results stay right, so only the speed shows it (the rotated decode step once ran 14% slower that
way). These tests compile the kernels that stream through buffer descriptors and check that no
such loop is left in any instantiation.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_recurrent_sequence_chunkwise_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S"]

pytestmark = pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not found")


def device_asm(src, tmp_path):
    out = os.path.join(str(tmp_path), os.path.basename(src) + ".s")
    r = subprocess.run([HIPCC, *FLAGS, os.path.join(CSRC, src), "-o", out], capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    return open(out).read()


def kernels(asm):
    """(symbol, body) of every kernel in the assembly, from its label to its s_endpgm."""
    out = []
    for m in re.finditer(r"^(_Z\S+):\s*(?:;.*)?$", asm, flags=re.M):
        end = asm.find("s_endpgm", m.end())
        out.append((m.group(1), asm[m.end():end]))
    return out


def readfirstlane_loops(body):
    """Number of buffer accesses issued under an exec mask taken from comparing a readfirstlane
    copy of a 64-bit value with every lane's (the shape of the compiler's readfirstlane loop)."""
    lines = body.splitlines()
    n = 0
    for i, ln in enumerate(lines):
        if re.search(r"\bbuffer_(load|store|atomic)", ln):
            window = "\n".join(lines[max(0, i - 12):i])
            if "v_readfirstlane_b32" in window and "v_cmp_eq_u64" in window and "s_and_saveexec_b64" in window:
                n += 1
    return n


SOURCES = ["chunkwise_bf16.hip", "chunk_seg.hip", "parallel_bf16.hip", "recurrent_step.hip", "backward.hip", "rla.hip",
           "rotation.hip", "fp32_path.hip"]


def test_no_readfirstlane_loops(tmp_path):
    """Every kernel source, compiled four at a time (the largest takes about 40 s)."""
    from concurrent.futures import ThreadPoolExecutor
    with ThreadPoolExecutor(max_workers=4) as ex:
        asms = dict(zip(SOURCES, ex.map(lambda src: device_asm(src, tmp_path), SOURCES)))
    bad = {}
    for src, asm in asms.items():
        ks = kernels(asm)
        assert ks, f"no kernels found in the assembly of {src}"
        bad.update({f"{src}: {name}": c for name, body in ks if (c := readfirstlane_loops(body))})
    assert not bad, f"buffer accesses inside readfirstlane loops: {bad}"


def test_detector_finds_a_loop():
    """The pattern the check looks for, as the compiler emits it around one buffer load."""
    body = """
.LBB0_1:
	v_readfirstlane_b32 s4, v46
	v_readfirstlane_b32 s5, v47
	v_readfirstlane_b32 s6, v44
	v_readfirstlane_b32 s7, v45
	v_cmp_eq_u64_e32 vcc, s[4:5], v[46:47]
	v_cmp_eq_u64_e64 s[0:1], s[6:7], v[44:45]
	s_and_b64 s[0:1], vcc, s[0:1]
	s_and_saveexec_b64 s[0:1], s[0:1]
	buffer_load_dwordx4 v[34:37], v48, s[4:7], 0 offen nt
	s_xor_b64 exec, exec, s[0:1]
	s_cbranch_execnz .LBB0_1
"""
    assert readfirstlane_loops(body) == 1
    assert readfirstlane_loops(body.replace("v_cmp_eq_u64", "v_cmp_eq_u32")) == 0
