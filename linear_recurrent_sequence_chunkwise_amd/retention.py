"""Thin ctypes binding of the C ABI in include/retention.h.

Argument marshalling only: every step of the computation runs in the gfx950 kernels of
libretention.so. torch supplies device memory (outputs, workspace) and the current HIP stream.
If the library is missing this module raises; there is no fallback of any kind.
"""
import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# the library (RETENTION_LIB names another build of it, e.g. the host-sanitized one)
LIB_PATH = os.environ.get("RETENTION_LIB", os.path.join(_PKG, "libretention.so"))

RET_OK, RET_ERR_INVALID_ARG, RET_ERR_UNSUPPORTED, RET_ERR_WORKSPACE, RET_ERR_DEVICE = range(5)
RET_F32, RET_BF16 = 0, 1
RET_FN_CHUNKWISE, RET_FN_RECURRENT_STEP, RET_FN_PARALLEL, RET_FN_CHUNKWISE_BWD, RET_FN_RLA = 0, 1, 2, 3, 4
RET_FMAP_IDENTITY, RET_FMAP_SOFTMAX = 0, 1
RET_WS_GROUPNORM, RET_WS_ROTATION = 1, 2

EXPORTED = [
    "retention_chunkwise_fwd", "retention_recurrent_step", "retention_parallel_fwd", "retention_chunkwise_bwd",
    "retention_rla_fwd", "retention_chunkwise_fwd_noalloc",
    "retention_workspace_bytes",
    "retention_status_string", "retention_last_error", "retention_abi_version",
]


class RetShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32), ("in_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32)]


class RetGroupNorm(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("eps", ctypes.c_float), ("weight", ctypes.c_void_p),
                ("bias", ctypes.c_void_p), ("gate", ctypes.c_void_p)]


class RetRotation(ctypes.Structure):
    _fields_ = [("enabled", ctypes.c_int32), ("base", ctypes.c_double), ("offset", ctypes.c_int64)]


class RetentionError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libretention.so and declare its signatures. Raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m linear_recurrent_sequence_chunkwise_amd.build` "
                           "(the retention library has no CPU fallback)")
    lib = ctypes.CDLL(path)
    vp, sz, i32, dp = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)
    sp, gp, rp = ctypes.POINTER(RetShape), ctypes.POINTER(RetGroupNorm), ctypes.POINTER(RetRotation)
    lib.retention_chunkwise_fwd.argtypes = [sp, i32, vp, vp, vp, dp, rp, vp, gp, vp, vp, vp, sz, vp]
    lib.retention_recurrent_step.argtypes = [sp, vp, vp, vp, dp, rp, vp, gp, vp, vp, sz, vp]
    lib.retention_parallel_fwd.argtypes = [sp, vp, vp, vp, dp, rp, gp, vp, vp, sz, vp]
    lib.retention_chunkwise_bwd.argtypes = [sp, i32, vp, vp, vp, dp, rp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.retention_rla_fwd.argtypes = [sp, i32, i32, i32, vp, vp, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.retention_chunkwise_fwd_noalloc.argtypes = [sp, i32, vp, vp, vp, dp, rp, vp, gp, vp, vp, vp]
    for f in (lib.retention_chunkwise_fwd, lib.retention_recurrent_step, lib.retention_parallel_fwd, lib.retention_chunkwise_bwd,
              lib.retention_rla_fwd, lib.retention_chunkwise_fwd_noalloc):
        f.restype = ctypes.c_int
    lib.retention_workspace_bytes.argtypes = [i32, sp, i32, i32]
    lib.retention_workspace_bytes.restype = sz
    lib.retention_status_string.argtypes = [i32]
    lib.retention_status_string.restype = ctypes.c_char_p
    lib.retention_last_error.argtypes = []
    lib.retention_last_error.restype = ctypes.c_char_p
    lib.retention_abi_version.argtypes = []
    lib.retention_abi_version.restype = i32
    if path == LIB_PATH:
        _lib = lib
    return lib


def _check(status):
    if status != RET_OK:
        lib = load_library()
        raise RetentionError(status, f"{lib.retention_status_string(status).decode()}: "
                                     f"{lib.retention_last_error().decode()}")


@dataclass
class GroupNorm:
    """Per-head GroupNorm epilogue: y = (o - mean) / sqrt(var + eps) * weight[h] + bias[h] over d_v,
    then, with a gate, y * swish(gate)."""
    eps: float = 1e-5
    weight: Optional[torch.Tensor] = None  # fp32 [H, d_v] on the device, or None
    bias: Optional[torch.Tensor] = None
    gate: Optional[torch.Tensor] = None  # shaped like the output, in the input dtype, or None

    def as_struct(self, in_dtype, out_shape):
        c = _Checks()
        c.groupnorm(self, in_dtype, out_shape)
        c.done()
        return RetGroupNorm(1, float(self.eps), _ptr(self.weight), _ptr(self.bias), _ptr(self.gate))


@dataclass
class Rotation:
    """Positional rotation of q and k before retention: feature pair (2i, 2i+1) of the row at
    absolute position offset + n turns by (offset + n) * base^(-2i/d_k). offset is the position of
    token 0 of the call (the tokens already processed, e.g. the prefill length for a decode step)."""
    base: float = 10000.0
    offset: int = 0

    def as_struct(self):
        return RetRotation(1, float(self.base), int(self.offset))


def _rot(rotation):
    return ctypes.byref(rotation.as_struct()) if rotation is not None else None


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt):
    if dt == torch.float32:
        return RET_F32
    if dt == torch.bfloat16:
        return RET_BF16
    raise ValueError(f"unsupported dtype {dt}")


def _torch_dtype(code):
    return torch.bfloat16 if code == RET_BF16 else torch.float32


def _gamma(gamma, H):
    g = [float(x) for x in (gamma.tolist() if hasattr(gamma, "tolist") else gamma)]
    if len(g) != H:
        raise ValueError(f"gamma has {len(g)} entries, expected {H}")
    return (ctypes.c_double * H)(*g)


def _stream(dev, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _shape(B, H, N, dk, dv, in_code, out_code):
    return RetShape(B, H, N, dk, dv, in_code, out_code)


_IN_DTYPES = (torch.float32, torch.bfloat16)


class _Checks:
    """The caller-supplied tensors of one call. The C ABI takes bare pointers and cannot see buffer
    sizes, so every tensor is checked here before any pointer crosses it: first the exact shape and
    dtype of every tensor, then that each is contiguous and on the GPU (so the size checks also
    run, and can be tested, on CPU tensors)."""

    def __init__(self):
        self.seen = []

    def tensor(self, name, t, shape, dtypes):
        if t is None:
            return
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {[str(d) for d in dtypes]}")
        self.seen.append((name, t))

    def inputs(self, q, k, v, ndim):
        """q, k, v: q and k [B,H,N,d_k] (decode: [B,H,d_k]), v [B,H,N,d_v] ([B,H,d_v]), one dtype
        (fp32 or bf16). Returns the leading dims, d_k and d_v."""
        for name, t in (("q", q), ("k", k), ("v", v)):
            if not isinstance(t, torch.Tensor) or t.dim() != ndim:
                raise ValueError(f"{name} must be a tensor with {ndim} dimensions")
        lead, dk, dv = tuple(q.shape[:-1]), q.shape[-1], v.shape[-1]
        self.tensor("q", q, q.shape, _IN_DTYPES)
        self.tensor("k", k, lead + (dk,), (q.dtype,))
        self.tensor("v", v, lead + (dv,), (q.dtype,))
        if min(q.shape) <= 0 or dv <= 0:
            raise ValueError(f"q and v need positive dimensions (q {tuple(q.shape)}, v {tuple(v.shape)})")
        return lead, dk, dv

    def state(self, name, t, B, H, dk, dv):
        self.tensor(name, t, (B, H, dk, dv), (torch.float32,))

    def out(self, t, shape):
        self.tensor("out", t, shape, _IN_DTYPES)

    def groupnorm(self, gn, in_dtype, out_shape):
        if gn is None:
            return
        H, dv = out_shape[1], out_shape[-1]
        self.tensor("groupnorm weight", gn.weight, (H, dv), (torch.float32,))
        self.tensor("groupnorm bias", gn.bias, (H, dv), (torch.float32,))
        self.tensor("gate", gn.gate, out_shape, (in_dtype,))

    def done(self):
        for name, t in self.seen:
            if not t.is_contiguous():
                raise ValueError(f"{name} must be contiguous")
        for name, t in self.seen:
            if not t.is_cuda:
                raise ValueError(f"{name} must be a device tensor")


def _flags(groupnorm, rotation):
    return (RET_WS_GROUPNORM if groupnorm else 0) | (RET_WS_ROTATION if rotation else 0)


def workspace_bytes(fn, B, H, N, dk, dv, in_dtype, out_dtype, chunk=0, groupnorm=False, rotation=False):
    lib = load_library()
    shp = _shape(B, H, N, dk, dv, _dtype_code(in_dtype), _dtype_code(out_dtype))
    n = lib.retention_workspace_bytes(fn, ctypes.byref(shp), int(chunk), _flags(groupnorm, rotation))
    if n == ctypes.c_size_t(-1).value:
        raise ValueError("workspace query: invalid arguments, or no kernel for this shape, chunk and flags")
    return n


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or not workspace.is_contiguous() or not workspace.is_cuda:
            raise ValueError("workspace must be a contiguous device tensor")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace, workspace.numel() * workspace.element_size()
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return ws, nbytes


def chunkwise_fwd(q, k, v, gamma: Sequence[float], chunk: int, *, state_in=None, groupnorm: Optional[GroupNorm] = None,
                  rotation: Optional[Rotation] = None, out=None, state_out=None, out_dtype=torch.float32, want_out=True,
                  want_state=True, workspace=None, stream=None):
    """Chunkwise retention forward. q, k: [B,H,N,dk]; v: [B,H,N,dv] (fp32 or bf16, device).
    Returns (out [B,H,N,dv] of out_dtype or None, state_out fp32 [B,H,dk,dv] or None).
    state_out may be passed as the same tensor as state_in (in place)."""
    c = _Checks()
    (B, H, N), dk, dv = c.inputs(q, k, v, 4)
    c.out(out, (B, H, N, dv))
    c.state("state_in", state_in, B, H, dk, dv)
    c.state("state_out", state_out, B, H, dk, dv)
    c.groupnorm(groupnorm, q.dtype, (B, H, N, dv))
    c.done()
    lib = load_library()
    in_code = _dtype_code(q.dtype)
    if out is not None:
        out_dtype = out.dtype
    out_code = _dtype_code(out_dtype)
    if want_out and out is None:
        out = torch.empty((B, H, N, dv), dtype=out_dtype, device=q.device)
    if not want_out:
        out = None
    if want_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if not want_state:
        state_out = None
    gn = groupnorm.as_struct(q.dtype, (B, H, N, dv)) if groupnorm is not None else None
    shp = _shape(B, H, N, dk, dv, in_code, out_code)
    need = lib.retention_workspace_bytes(RET_FN_CHUNKWISE, ctypes.byref(shp), int(chunk),
                                         _flags(gn is not None and out is not None, rotation is not None))
    if need == ctypes.c_size_t(-1).value:
        need = 0  # the call itself reports the invalid argument
    ws, wsb = _workspace(need, q.device, workspace)
    st = lib.retention_chunkwise_fwd(ctypes.byref(shp), int(chunk), _ptr(q), _ptr(k), _ptr(v), _gamma(gamma, H),
                                     _rot(rotation), _ptr(state_in), ctypes.byref(gn) if gn is not None else None, _ptr(out),
                                     _ptr(state_out), _ptr(ws), wsb, _stream(q.device, stream))
    _check(st)
    return out, state_out


NOALLOC_SCRATCH_BYTES = 64 << 20  # RETENTION_NOALLOC_SCRATCH_BYTES


def chunkwise_fwd_noalloc(q, k, v, gamma: Sequence[float], chunk: int, *, state_in=None,
                          groupnorm: Optional[GroupNorm] = None, rotation: Optional[Rotation] = None, out, state_out=None,
                          stream=None):
    """The chunkwise forward through retention_chunkwise_fwd_noalloc: no workspace, the library's own
    fixed scratch array instead. The caller passes every output (out and/or state_out), so this
    call allocates nothing either. Returns (out, state_out)."""
    c = _Checks()
    (B, H, N), dk, dv = c.inputs(q, k, v, 4)
    c.out(out, (B, H, N, dv))
    c.state("state_in", state_in, B, H, dk, dv)
    c.state("state_out", state_out, B, H, dk, dv)
    c.groupnorm(groupnorm, q.dtype, (B, H, N, dv))
    c.done()
    lib = load_library()
    out_code = _dtype_code(out.dtype) if out is not None else RET_F32
    gn = groupnorm.as_struct(q.dtype, (B, H, N, dv)) if groupnorm is not None else None
    shp = _shape(B, H, N, dk, dv, _dtype_code(q.dtype), out_code)
    st = lib.retention_chunkwise_fwd_noalloc(ctypes.byref(shp), int(chunk), _ptr(q), _ptr(k), _ptr(v), _gamma(gamma, H),
                                             _rot(rotation), _ptr(state_in), ctypes.byref(gn) if gn is not None else None,
                                             _ptr(out), _ptr(state_out), _stream(q.device, stream))
    _check(st)
    return out, state_out


def recurrent_step(q, k, v, gamma: Sequence[float], state, *, groupnorm: Optional[GroupNorm] = None,
                   rotation: Optional[Rotation] = None, out=None, out_dtype=torch.float32, want_out=True, workspace=None,
                   stream=None):
    """One recurrent step: state <- g*state + k^T v (in place), o = q state.
    q, k: [B,H,dk]; v: [B,H,dv]; state: fp32 [B,H,dk,dv]. Returns o [B,H,dv] (or None).
    With a rotation, rotation.offset is the position of this token."""
    c = _Checks()
    (B, H), dk, dv = c.inputs(q, k, v, 3)
    if state is None:
        raise ValueError("state is required")
    c.state("state", state, B, H, dk, dv)
    c.out(out, (B, H, dv))
    c.groupnorm(groupnorm, q.dtype, (B, H, dv))
    c.done()
    lib = load_library()
    if out is not None:
        out_dtype = out.dtype
    if want_out and out is None:
        out = torch.empty((B, H, dv), dtype=out_dtype, device=q.device)
    if not want_out:
        out = None
    gn = groupnorm.as_struct(q.dtype, (B, H, dv)) if groupnorm is not None else None
    shp = _shape(B, H, 1, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype))
    need = lib.retention_workspace_bytes(RET_FN_RECURRENT_STEP, ctypes.byref(shp), 0, _flags(False, rotation is not None))
    if need == ctypes.c_size_t(-1).value:
        need = 0
    ws, wsb = _workspace(need, q.device, workspace)
    st = lib.retention_recurrent_step(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _gamma(gamma, H), _rot(rotation),
                                      _ptr(state), ctypes.byref(gn) if gn is not None else None, _ptr(out), _ptr(ws), wsb,
                                      _stream(q.device, stream))
    _check(st)
    return out


def parallel_fwd(q, k, v, gamma: Sequence[float], *, groupnorm: Optional[GroupNorm] = None,
                 rotation: Optional[Rotation] = None, out=None, out_dtype=torch.float32, workspace=None, stream=None):
    """Parallel form O = (Q K^T (.) D) V. Returns out [B,H,N,dv]."""
    c = _Checks()
    (B, H, N), dk, dv = c.inputs(q, k, v, 4)
    c.out(out, (B, H, N, dv))
    c.groupnorm(groupnorm, q.dtype, (B, H, N, dv))
    c.done()
    lib = load_library()
    if out is not None:
        out_dtype = out.dtype
    else:
        out = torch.empty((B, H, N, dv), dtype=out_dtype, device=q.device)
    gn = groupnorm.as_struct(q.dtype, (B, H, N, dv)) if groupnorm is not None else None
    shp = _shape(B, H, N, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype))
    need = lib.retention_workspace_bytes(RET_FN_PARALLEL, ctypes.byref(shp), 0, _flags(gn is not None, rotation is not None))
    if need == ctypes.c_size_t(-1).value:
        need = 0
    ws, wsb = _workspace(need, q.device, workspace)
    st = lib.retention_parallel_fwd(ctypes.byref(shp), _ptr(q), _ptr(k), _ptr(v), _gamma(gamma, H), _rot(rotation),
                                    ctypes.byref(gn) if gn is not None else None, _ptr(out), _ptr(ws), wsb,
                                    _stream(q.device, stream))
    _check(st)
    return out


def chunkwise_bwd(q, k, v, gamma: Sequence[float], dout, chunk: int, *, state_in=None, rotation: Optional[Rotation] = None,
                  want=("dq", "dk", "dv", "dstate_in"), workspace=None, stream=None):
    """Gradients of chunkwise retention for dL/dout = dout (the pre-norm output): fp32 dq, dk, dv
    (shaped like q, k, v) and dstate_in ([B,H,dk,dv]); the names not in `want` come back None.
    dout is laid out like v, in the input dtype. With a rotation, dq and dk are the gradients with
    respect to the unrotated q and k."""
    c = _Checks()
    (B, H, N), dk, dv = c.inputs(q, k, v, 4)
    if dout is None:
        raise ValueError("dout is required")
    c.tensor("dout", dout, (B, H, N, dv), (q.dtype,))
    c.state("state_in", state_in, B, H, dk, dv)
    c.done()
    lib = load_library()
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, H, N, dk), **f32) if "dq" in want else None
    dk_ = torch.empty((B, H, N, dk), **f32) if "dk" in want else None
    dv_ = torch.empty((B, H, N, dv), **f32) if "dv" in want else None
    ds = torch.empty((B, H, dk, dv), **f32) if "dstate_in" in want else None
    shp = _shape(B, H, N, dk, dv, _dtype_code(q.dtype), RET_F32)
    need = lib.retention_workspace_bytes(RET_FN_CHUNKWISE_BWD, ctypes.byref(shp), int(chunk), _flags(False, rotation is not None))
    if need == ctypes.c_size_t(-1).value:
        need = 0
    ws, wsb = _workspace(need, q.device, workspace)
    st = lib.retention_chunkwise_bwd(ctypes.byref(shp), int(chunk), _ptr(q), _ptr(k), _ptr(v), _gamma(gamma, H), _rot(rotation),
                                     _ptr(state_in),
                                     _ptr(dout), _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(ds), _ptr(ws), wsb, _stream(q.device, stream))
    _check(st)
    return dq, dk_, dv_, ds


_FMAPS = {"identity": RET_FMAP_IDENTITY, "softmax": RET_FMAP_SOFTMAX}


def rla_fwd(q, k, v, window: int, chunk: int = 128, *, fmap: str = "softmax", k_prev=None, v_prev=None,
            prev_len: Optional[int] = None, state_in=None, out=None, state_out=None, out_dtype=torch.float32, want_out=True,
            want_state=True, workspace=None, stream=None):
    """Residual linear attention over a segment: o_t = phi(q_t) S_(t-window-1), S_t = S_(t-1) +
    phi(k_t)^T v_t. q, k: [B,H,N,dk]; v: [B,H,N,dv]. k_prev, v_prev: [B,H,window+1,d], the positions
    before the segment, of which the last prev_len (default: all, or none without them) hold tokens.
    state_in / state_out: fp32 [B,H,dk,dv], the sum over the tokens that have left the window
    (state_out may be state_in; a one-token segment needs a state_out). Returns (out, state_out)."""
    c = _Checks()
    (B, H, N), dk, dv = c.inputs(q, k, v, 4)
    if window < 0:
        raise ValueError(f"window must be >= 0 (got {window})")
    if prev_len is None:
        prev_len = 0 if k_prev is None else window + 1
    c.tensor("k_prev", k_prev, (B, H, window + 1, dk), (q.dtype,))
    c.tensor("v_prev", v_prev, (B, H, window + 1, dv), (q.dtype,))
    if not 0 <= prev_len <= window + 1:
        raise ValueError(f"prev_len must be in [0, window + 1] (got {prev_len})")
    if prev_len > 0 and (k_prev is None or v_prev is None):
        raise ValueError("prev_len > 0 needs k_prev and v_prev")
    c.out(out, (B, H, N, dv))
    c.state("state_in", state_in, B, H, dk, dv)
    c.state("state_out", state_out, B, H, dk, dv)
    if fmap not in _FMAPS:
        raise ValueError(f"fmap must be one of {sorted(_FMAPS)} (got {fmap!r})")
    c.done()
    lib = load_library()
    if out is not None:
        out_dtype = out.dtype
    if want_out and out is None:
        out = torch.empty((B, H, N, dv), dtype=out_dtype, device=q.device)
    if not want_out:
        out = None
    if want_state and state_out is None:
        state_out = torch.empty((B, H, dk, dv), dtype=torch.float32, device=q.device)
    if not want_state:
        state_out = None
    shp = _shape(B, H, N, dk, dv, _dtype_code(q.dtype), _dtype_code(out_dtype))
    need = lib.retention_workspace_bytes(RET_FN_RLA, ctypes.byref(shp), int(chunk), 0)
    if need == ctypes.c_size_t(-1).value:
        need = 0
    ws, wsb = _workspace(need, q.device, workspace)
    st = lib.retention_rla_fwd(ctypes.byref(shp), int(chunk), int(window), _FMAPS[fmap], _ptr(q), _ptr(k), _ptr(v), _ptr(k_prev),
                               _ptr(v_prev), int(prev_len), _ptr(state_in), _ptr(out), _ptr(state_out), _ptr(ws), wsb,
                               _stream(q.device, stream))
    _check(st)
    return out, state_out
