"""C-ABI contract on the CPU: the library loads, exports what include/retention.h declares, and
rejects invalid arguments on the host before any HIP call (so no GPU is needed here)."""
import ctypes
import math
import os
import re

import pytest

from linear_recurrent_sequence_chunkwise_amd import retention as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "retention.h")

# fake, 16-byte aligned, far-apart device addresses: validation never dereferences them
Q, K, V, OUT, ST, WS, GW = (ctypes.c_void_p(i << 36) for i in range(1, 8))


@pytest.fixture(scope="module")
def lib():
    return R.load_library()


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"\b(retention_[a-z_]+)\s*\(", txt)))


def test_exports_every_declared_symbol(lib):
    syms = declared_symbols()
    assert set(syms) == set(R.EXPORTED)
    for s in syms:
        assert hasattr(lib, s), s


def test_abi_version_and_strings(lib):
    assert lib.retention_abi_version() == 4
    for s in range(5):
        assert lib.retention_status_string(s).decode().startswith("RET_")
    assert lib.retention_status_string(99).decode() == "unknown status"


def shape(B=1, H=2, N=256, dk=64, dv=64, i=R.RET_BF16, o=R.RET_F32):
    return R.RetShape(B, H, N, dk, dv, i, o)


def gam(vals):
    return (ctypes.c_double * len(vals))(*vals)


def chunk(lib, shp=None, C=64, q=Q, k=K, v=V, g=None, sin=None, gn=None, out=OUT, sout=ST, ws=WS, wsb=1 << 40, rot=None):
    shp = shp if shp is not None else shape()
    g = g if g is not None else gam([0.9] * shp.heads)
    return lib.retention_chunkwise_fwd(ctypes.byref(shp), C, q, k, v, g, rot, sin, gn, out, sout, ws, wsb, None)


def test_null_shape(lib):
    assert lib.retention_chunkwise_fwd(None, 64, Q, K, V, gam([0.9]), None, None, None, OUT, ST, WS, 1 << 40, None) == R.RET_ERR_INVALID_ARG
    assert "shape" in lib.retention_last_error().decode()


@pytest.mark.parametrize("field,val", [("batch", 0), ("heads", -1), ("seq_len", 0), ("d_k", 0), ("d_v", -3)])
def test_bad_dims(lib, field, val):
    s = shape()
    setattr(s, field, val)
    assert chunk(lib, s) == R.RET_ERR_INVALID_ARG


def test_bad_dtype(lib):
    assert chunk(lib, shape(i=7)) == R.RET_ERR_INVALID_ARG
    assert chunk(lib, shape(o=-1)) == R.RET_ERR_INVALID_ARG


def test_too_many_heads(lib):
    s = shape(H=129)
    assert chunk(lib, s, g=gam([0.9] * 129)) == R.RET_ERR_UNSUPPORTED


@pytest.mark.parametrize("which", ["q", "k", "v"])
def test_null_inputs(lib, which):
    kw = {which: None}
    assert chunk(lib, **kw) == R.RET_ERR_INVALID_ARG
    assert which in lib.retention_last_error().decode()


def test_misaligned(lib):
    assert chunk(lib, q=ctypes.c_void_p((1 << 36) + 8)) == R.RET_ERR_INVALID_ARG
    assert "aligned" in lib.retention_last_error().decode()
    assert chunk(lib, sout=ctypes.c_void_p((5 << 36) + 4)) == R.RET_ERR_INVALID_ARG


@pytest.mark.parametrize("g", [0.0, -0.5, 1.5, math.nan, math.inf])
def test_bad_gamma(lib, g):
    assert chunk(lib, g=gam([0.9, g])) == R.RET_ERR_INVALID_ARG
    assert "gamma[1]" in lib.retention_last_error().decode()


def test_null_gamma(lib):
    s = shape()
    assert lib.retention_chunkwise_fwd(ctypes.byref(s), 64, Q, K, V, None, None, None, None, OUT, ST, WS, 1 << 40, None) == R.RET_ERR_INVALID_ARG


def test_no_outputs(lib):
    assert chunk(lib, out=None, sout=None) == R.RET_ERR_INVALID_ARG


@pytest.mark.parametrize("eps", [0.0, -1e-5, math.nan])
def test_bad_eps(lib, eps):
    gn = R.RetGroupNorm(1, eps, None, None)
    assert chunk(lib, gn=ctypes.byref(gn)) == R.RET_ERR_INVALID_ARG


def test_gate_validation(lib):
    # a gate only follows an enabled GroupNorm, and must be 16-byte aligned
    gn = R.RetGroupNorm(0, 1e-5, None, None, ctypes.c_void_p(1 << 36))
    assert chunk(lib, gn=ctypes.byref(gn)) == R.RET_ERR_INVALID_ARG
    assert "gate" in lib.retention_last_error().decode()
    gn = R.RetGroupNorm(1, 1e-5, None, None, ctypes.c_void_p((1 << 36) + 8))
    assert chunk(lib, gn=ctypes.byref(gn)) == R.RET_ERR_INVALID_ARG
    assert "gate" in lib.retention_last_error().decode()


def test_unsupported_chunk_and_dims(lib):
    assert chunk(lib, C=96) == R.RET_ERR_UNSUPPORTED
    assert chunk(lib, C=0) == R.RET_ERR_INVALID_ARG
    assert chunk(lib, shape(dk=48)) == R.RET_ERR_UNSUPPORTED
    assert chunk(lib, shape(i=R.RET_F32), C=256) == R.RET_ERR_UNSUPPORTED
    s = shape(dk=64, dv=64)
    assert lib.retention_parallel_fwd(ctypes.byref(shape(dk=128, dv=64)), Q, K, V, gam([0.9, 0.9]), None, None, OUT, WS, 1 << 40,
                                      None) == R.RET_ERR_UNSUPPORTED
    del s


def test_aliasing(lib):
    assert chunk(lib, out=Q) == R.RET_ERR_INVALID_ARG
    assert "alias" in lib.retention_last_error().decode()
    assert chunk(lib, out=ST, sout=ST) == R.RET_ERR_INVALID_ARG
    partly = ctypes.c_void_p((5 << 36) + 256)
    assert chunk(lib, sin=ST, sout=partly) == R.RET_ERR_INVALID_ARG


def test_workspace(lib):
    s = shape()
    need = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(s), 64, 0)
    assert 0 < need < (1 << 40)
    # bf16 chunkwise holds one bf16 C x C score block per chunk
    assert need >= 1 * 2 * 4 * 64 * 64 * 2
    assert chunk(lib, ws=None, wsb=0) == R.RET_ERR_WORKSPACE
    assert chunk(lib, wsb=need - 1) == R.RET_ERR_WORKSPACE
    assert "workspace" in lib.retention_last_error().decode()
    assert lib.retention_workspace_bytes(R.RET_FN_RECURRENT_STEP, ctypes.byref(shape(N=1)), 0, 1) == 0
    assert lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, None, 64, 0) == ctypes.c_size_t(-1).value
    assert lib.retention_workspace_bytes(9, ctypes.byref(s), 64, 0) == ctypes.c_size_t(-1).value
    gn_need = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(s), 64, 1)
    # GroupNorm adds the fp32 pre-norm rows, normalised by a second kernel
    assert gn_need >= need + s.batch * s.heads * s.seq_len * s.d_v * 4


def test_step_validation(lib):
    def step(shp, state=ST, out=OUT, g=None):
        g = g if g is not None else gam([0.9] * shp.heads)
        return lib.retention_recurrent_step(ctypes.byref(shp), Q, K, V, g, None, state, None, out, None, 0, None)
    assert step(shape(N=2)) == R.RET_ERR_INVALID_ARG
    assert step(shape(N=1), state=None) == R.RET_ERR_INVALID_ARG
    assert step(shape(N=1, dv=6)) == R.RET_ERR_UNSUPPORTED
    assert step(shape(N=1, dv=4 * 3 * 5)) == R.RET_ERR_UNSUPPORTED
    assert step(shape(N=1), out=ST) == R.RET_ERR_INVALID_ARG
    assert step(shape(N=1), g=gam([0.9, 2.0])) == R.RET_ERR_INVALID_ARG


def test_error_is_thread_local(lib):
    import threading
    assert chunk(lib, C=96) == R.RET_ERR_UNSUPPORTED
    seen = {}

    def other():
        seen["msg"] = lib.retention_last_error().decode()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "chunk" in lib.retention_last_error().decode()


def bwd(lib, shp=None, C=64, q=Q, k=K, v=V, dout=GW, sin=None, dq=OUT, dk=ST, dv=WS, ds=None, ws=ctypes.c_void_p(9 << 36),
        wsb=1 << 40, rot=None):
    shp = shp if shp is not None else shape()
    return lib.retention_chunkwise_bwd(ctypes.byref(shp), C, q, k, v, gam([0.9] * shp.heads), rot, sin, dout, dq, dk, dv, ds, ws,
                                       wsb, None)


def test_backward_validation(lib):
    # every check below fails on the host before any HIP call
    assert bwd(lib, dout=None) == R.RET_ERR_INVALID_ARG
    assert "dout" in lib.retention_last_error().decode()
    assert bwd(lib, dq=None, dk=None, dv=None, ds=None) == R.RET_ERR_INVALID_ARG
    assert bwd(lib, shape(o=R.RET_BF16)) == R.RET_ERR_UNSUPPORTED
    assert bwd(lib, C=96) == R.RET_ERR_UNSUPPORTED
    assert bwd(lib, shape(dk=48)) == R.RET_ERR_UNSUPPORTED
    assert bwd(lib, dq=Q) == R.RET_ERR_INVALID_ARG  # aliases q
    assert "alias" in lib.retention_last_error().decode()
    assert bwd(lib, dk=OUT) == R.RET_ERR_INVALID_ARG  # aliases dq
    assert bwd(lib, dq=ctypes.c_void_p((1 << 36) * 3 + 8)) == R.RET_ERR_INVALID_ARG  # misaligned
    assert bwd(lib, ws=None, wsb=0) == R.RET_ERR_WORKSPACE
    need = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE_BWD, ctypes.byref(shape()), 64, 0)
    assert bwd(lib, wsb=need - 1) == R.RET_ERR_WORKSPACE
    # bf16: the forwards read their operands in place; the workspace holds a forward's scores and
    # the blocks of state_in^T. fp32: also reversed copies of q, k, v and dout and an fp32 output.
    s = shape()
    assert need >= lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(s), 64, 0) + s.heads * s.d_k * s.d_v * 4
    s32 = shape(i=R.RET_F32)
    rows = s32.batch * s32.heads * s32.seq_len
    need32 = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE_BWD, ctypes.byref(s32), 64, 0)
    assert need32 >= rows * (2 * s32.d_k + 2 * s32.d_v) * 4 + rows * max(s32.d_k, s32.d_v) * 4
    assert lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE_BWD, ctypes.byref(s), 0, 0) == ctypes.c_size_t(-1).value


def rot(base=10000.0, offset=0, enabled=1):
    return ctypes.byref(R.RetRotation(enabled, base, offset))


@pytest.mark.parametrize("base,offset,err", [(0.0, 0, "base"), (-2.0, 0, "base"), (math.inf, 0, "base"), (math.nan, 0, "base"),
                                             (10000.0, -1, "offset"), (10000.0, 1 << 31, "offset")])
def test_rotation_validation(lib, base, offset, err):
    assert chunk(lib, rot=rot(base, offset)) == R.RET_ERR_INVALID_ARG
    assert err in lib.retention_last_error().decode()


def test_rotation_shapes(lib):
    # odd d_k cannot be paired; d_k above 256 has no constants slot; disabled rotation is ignored
    s = shape(dk=63, i=R.RET_F32)
    assert chunk(lib, s, rot=rot()) == R.RET_ERR_INVALID_ARG
    assert "even" in lib.retention_last_error().decode()
    s = R.RetShape(1, 2, 1, 514, 64, R.RET_F32, R.RET_F32)
    assert lib.retention_recurrent_step(ctypes.byref(s), Q, K, V, gam([0.9, 0.9]), rot(), ST, None, OUT, WS, 1 << 40,
                                        None) == R.RET_ERR_UNSUPPORTED
    assert chunk(lib, shape(dk=48), rot=rot(enabled=0)) == R.RET_ERR_UNSUPPORTED  # the d_k check, not the rotation's
    assert "chunkwise" in lib.retention_last_error().decode()
    assert bwd(lib, rot=rot(offset=-5)) == R.RET_ERR_INVALID_ARG


def test_rotation_workspace(lib):
    al = lambda n: (n + 255) // 256 * 256
    # a rotation stages the rotated q and k (input dtype, each copy 256-byte aligned) in front: one
    # copy each for fp32 inputs
    for fn, C, i in ((R.RET_FN_CHUNKWISE_BWD, 64, R.RET_F32), (R.RET_FN_CHUNKWISE, 64, R.RET_F32), (R.RET_FN_PARALLEL, 0, R.RET_F32)):
        s = shape(i=i)
        base = lib.retention_workspace_bytes(fn, ctypes.byref(s), C, 0)
        with_rot = lib.retention_workspace_bytes(fn, ctypes.byref(s), C, R.RET_WS_ROTATION)
        copy = s.batch * s.heads * s.seq_len * s.d_k * (2 if i == R.RET_BF16 else 4)
        assert with_rot == base + 2 * al(copy), fn
    # the bf16 forward forms keep high and low parts (four planes), then the three calls' fp32
    # partial outputs and second partial state, then the calls' own workspace without a GroupNorm.
    # The parallel form keeps two partial outputs (three with a GroupNorm after their sum or a bf16
    # output); the chunkwise calls add theirs in place, into out or (GroupNorm, bf16 out) one, and
    # keep the scores of the three products (both bf16 parts) that their two calls share.
    s = shape()
    rows = s.batch * s.heads * s.seq_len
    planes = 4 * al(rows * s.d_k * 2)
    o, st = al(rows * s.d_v * 4), al(s.batch * s.heads * s.d_k * s.d_v * 4)
    sc = al(2 * s.batch * s.heads * (s.seq_len // 64) * 64 * 64 * 2)
    for fn, C, n0, n1, extra in ((R.RET_FN_CHUNKWISE, 64, 0, 1, sc), (R.RET_FN_PARALLEL, 0, 2, 3, 0)):
        base = lib.retention_workspace_bytes(fn, ctypes.byref(s), C, 0)
        assert lib.retention_workspace_bytes(fn, ctypes.byref(s), C, R.RET_WS_ROTATION) == planes + n0 * o + st + extra + base, fn
        assert lib.retention_workspace_bytes(fn, ctypes.byref(s), C, R.RET_WS_ROTATION | R.RET_WS_GROUPNORM) == \
            planes + n1 * o + st + extra + base, fn
    # the bf16 backward likewise, with the partial gradients (dq, dk, two dv, dstate_in)
    base = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE_BWD, ctypes.byref(s), 64, 0)
    g = 2 * al(rows * s.d_k * 4) + 2 * al(rows * s.d_v * 4) + st
    assert lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE_BWD, ctypes.byref(s), 64, R.RET_WS_ROTATION) == planes + g + base
    s = shape(N=1)
    # the step turns q and k inside its kernel: no workspace, with or without a rotation
    assert lib.retention_workspace_bytes(R.RET_FN_RECURRENT_STEP, ctypes.byref(s), 0, R.RET_WS_ROTATION) == 0
    assert lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(shape()), 64, 4) == ctypes.c_size_t(-1).value
    need = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(shape()), 64, R.RET_WS_ROTATION)
    assert chunk(lib, wsb=need - 1, rot=rot()) == R.RET_ERR_WORKSPACE


def rla(lib, shp=None, C=64, window=3, fmap=R.RET_FMAP_SOFTMAX, kp=None, vp=None, plen=0, sin=None, out=OUT, sout=ST, ws=WS,
        wsb=1 << 40):
    shp = shp if shp is not None else shape()
    return lib.retention_rla_fwd(ctypes.byref(shp), C, window, fmap, Q, K, V, kp, vp, plen, sin, out, sout, ws, wsb, None)


def test_rla_validation(lib):
    # every check below fails on the host before any HIP call
    assert rla(lib, window=-1) == R.RET_ERR_INVALID_ARG
    assert "window" in lib.retention_last_error().decode()
    assert rla(lib, fmap=2) == R.RET_ERR_INVALID_ARG
    assert rla(lib, plen=5, kp=GW, vp=GW) == R.RET_ERR_INVALID_ARG  # more than window + 1 earlier tokens
    assert rla(lib, plen=2) == R.RET_ERR_INVALID_ARG  # earlier tokens without their rows
    assert "k_prev" in lib.retention_last_error().decode()
    assert rla(lib, out=None, sout=None) == R.RET_ERR_INVALID_ARG
    assert rla(lib, shape(dk=512, i=R.RET_F32)) == R.RET_ERR_UNSUPPORTED
    assert rla(lib, shape(N=1, dk=6)) == R.RET_ERR_UNSUPPORTED  # d_k not a multiple of 4
    assert rla(lib, C=96) == R.RET_ERR_UNSUPPORTED
    assert rla(lib, shape(N=1), sout=None) == R.RET_ERR_INVALID_ARG  # a decode step needs its state
    assert "state_out" in lib.retention_last_error().decode()
    assert rla(lib, shape(N=1, dv=6)) == R.RET_ERR_UNSUPPORTED
    assert rla(lib, shape(N=1, dv=12)) == R.RET_ERR_UNSUPPORTED  # 24-byte bf16 value rows
    assert rla(lib, out=Q) == R.RET_ERR_INVALID_ARG
    assert rla(lib, plen=4, kp=GW, vp=ctypes.c_void_p(9 << 36), out=GW) == R.RET_ERR_INVALID_ARG  # out aliases k_prev
    need = lib.retention_workspace_bytes(R.RET_FN_RLA, ctypes.byref(shape()), 64, 0)
    s = shape()
    rows = s.batch * s.heads * s.seq_len
    assert need >= rows * (2 * s.d_k + s.d_v) * 2
    assert rla(lib, wsb=need - 1) == R.RET_ERR_WORKSPACE
    assert rla(lib, ws=None, wsb=0) == R.RET_ERR_WORKSPACE
    # a decode step needs only the operands: 2 rows x 64 features or values each, in fp32 for bf16
    # inputs with the softmax map (the larger need), so three 512-byte planes
    s1 = shape(N=1)
    assert lib.retention_workspace_bytes(R.RET_FN_RLA, ctypes.byref(s1), 0, 0) == 3 * 512
    assert lib.retention_workspace_bytes(R.RET_FN_RLA, ctypes.byref(shape(N=1, i=R.RET_F32)), 0, 0) == 3 * 512


def test_workspace_query_unsupported_shapes(lib):
    """The query answers (size_t)-1 exactly where the call would return RET_ERR_UNSUPPORTED."""
    bad = ctypes.c_size_t(-1).value
    q = lambda fn, shp, C=64, fl=0: lib.retention_workspace_bytes(fn, ctypes.byref(shp), C, fl)
    assert q(R.RET_FN_CHUNKWISE, shape(dk=128)) == bad  # bf16 chunk kernels: d_k 64 or 256
    assert q(R.RET_FN_CHUNKWISE, shape(dk=128, i=R.RET_F32)) != bad
    assert q(R.RET_FN_CHUNKWISE, shape(), C=96) == bad
    assert q(R.RET_FN_CHUNKWISE_BWD, shape(dv=32)) == bad  # no column split of d_v = 32 for the swapped forwards
    assert q(R.RET_FN_CHUNKWISE_BWD, shape(dv=128)) != bad
    assert q(R.RET_FN_PARALLEL, shape(dk=128, dv=128)) == bad  # bf16 parallel: d_k 64 or 256
    assert q(R.RET_FN_PARALLEL, shape(dk=64, dv=32)) == bad  # d_v in four groups of 16-column tiles
    assert q(R.RET_FN_PARALLEL, shape(dk=256, dv=128)) != bad
    assert q(R.RET_FN_PARALLEL, shape(dk=128, dv=128, i=R.RET_F32)) != bad
    assert q(R.RET_FN_RECURRENT_STEP, shape(N=1, dv=12), 0) == bad
    assert q(R.RET_FN_RECURRENT_STEP, shape(N=1, dv=16), 0) == 0
    assert q(R.RET_FN_CHUNKWISE, shape(dk=64, i=R.RET_F32), 64, R.RET_WS_ROTATION) != bad
    assert q(R.RET_FN_RECURRENT_STEP, shape(N=1, dk=7, dv=16), 0, R.RET_WS_ROTATION) == bad  # odd d_k
    assert q(R.RET_FN_RLA, shape(), 64, R.RET_WS_ROTATION) == bad  # no rotation for residual linear attention
    assert q(R.RET_FN_RLA, shape(N=1, dv=12), 0) == bad
    # each rejected shape is one the call itself rejects
    assert bwd(lib, shape(dv=32)) == R.RET_ERR_UNSUPPORTED
    assert chunk(lib, shape(dk=128)) == R.RET_ERR_UNSUPPORTED


def test_bf16_sequence_length_limit(lib):
    """One head's rows and scores must fit 32-bit offsets in the bf16 chunk kernels: about 1M tokens
    at d_v = 512; longer sequences are refused (not truncated), by the calls and the query alike."""
    bad = ctypes.c_size_t(-1).value
    ok_n, long_n = 1 << 19, 1 << 20  # 2^19 * 512 * 4 = 1 GiB fits; 2^20 * 512 * 4 = 2 GiB does not
    for fn in (R.RET_FN_CHUNKWISE, R.RET_FN_CHUNKWISE_BWD, R.RET_FN_RLA):
        assert lib.retention_workspace_bytes(fn, ctypes.byref(shape(H=1, N=ok_n, dk=256, dv=512)), 128, 0) != bad, fn
        assert lib.retention_workspace_bytes(fn, ctypes.byref(shape(H=1, N=long_n, dk=256, dv=512)), 128, 0) == bad, fn
    # fp32 inputs address through 64-bit pointers: no such bound
    assert lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(shape(H=1, N=long_n, dk=256, dv=512, i=R.RET_F32)), 128,
                                         0) != bad
    s = shape(H=1, N=long_n, dk=256, dv=512)
    assert lib.retention_chunkwise_fwd(ctypes.byref(s), 128, Q, K, V, gam([0.9]), None, None, None, OUT, ST, WS, 1 << 40,
                                       None) == R.RET_ERR_UNSUPPORTED
    assert "2^31" in lib.retention_last_error().decode()
    assert bwd(lib, s, C=128) == R.RET_ERR_UNSUPPORTED
    assert rla(lib, s, C=128) == R.RET_ERR_UNSUPPORTED


def noalloc(lib, shp=None, C=64, q=Q, k=K, v=V, g=None, sin=None, gn=None, out=OUT, sout=ST, rot=None):
    shp = shp if shp is not None else shape()
    g = g if g is not None else gam([0.9] * shp.heads)
    return lib.retention_chunkwise_fwd_noalloc(ctypes.byref(shp), C, q, k, v, g, rot, sin, gn, out, sout, None)


def test_noalloc_validates_like_the_plain_call(lib):
    # the same host validation as retention_chunkwise_fwd, before the scratch array is touched
    assert noalloc(lib, q=None) == R.RET_ERR_INVALID_ARG
    assert "q is NULL" in lib.retention_last_error().decode()
    assert noalloc(lib, out=None, sout=None) == R.RET_ERR_INVALID_ARG
    assert noalloc(lib, g=gam([0.9, 1.5])) == R.RET_ERR_INVALID_ARG
    assert noalloc(lib, C=96) == R.RET_ERR_UNSUPPORTED


def test_noalloc_refuses_beyond_its_array(lib):
    # the N=8192 layer with GroupNorm needs more scratch than the fixed array holds: refused on the
    # host with a message that names both sizes
    s = shape(B=1, H=16, N=8192, dk=256, dv=512, o=R.RET_BF16)
    gn = R.RetGroupNorm(1, 1e-5, None, None, None)
    need = lib.retention_workspace_bytes(R.RET_FN_CHUNKWISE, ctypes.byref(s), 128, R.RET_WS_GROUPNORM)
    assert need > R.NOALLOC_SCRATCH_BYTES
    assert noalloc(lib, s, C=128, g=gam([0.9] * 16), gn=ctypes.byref(gn)) == R.RET_ERR_WORKSPACE
    msg = lib.retention_last_error().decode()
    assert str(need) in msg and str(R.NOALLOC_SCRATCH_BYTES) in msg


def test_noalloc_scratch_size_matches_header():
    txt = open(HEADER).read()
    m = re.search(r"#define RETENTION_NOALLOC_SCRATCH_BYTES \((\d+)ull << (\d+)\)", txt)
    assert m and int(m.group(1)) << int(m.group(2)) == R.NOALLOC_SCRATCH_BYTES
