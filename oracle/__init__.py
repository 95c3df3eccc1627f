"""fp64 CPU oracle for multi-scale retention (parallel, recurrent and chunkwise forms, GroupNorm).

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the benchmark's CPU-baseline leg
may import this package. The GPU library shares no code with it.

The arithmetic lives in oracle.c (plain C, double precision); this module only marshals numpy
arrays to it. Citations of the pages are in oracle.c beside each function.
"""
import ctypes
import os

import numpy as np

from .build import LIB, SRC, build

_lib = None
_DP = ctypes.POINTER(ctypes.c_double)


def load(path: str = LIB):
    """Load (building first if missing or stale) the oracle shared library."""
    if not os.path.exists(path) or (path == LIB and os.path.getmtime(SRC) > os.path.getmtime(path)):
        build(out=path, quiet=True)
    lib = ctypes.CDLL(path)
    i, d = ctypes.c_int, ctypes.c_double
    lib.oracle_recurrent.argtypes = [i, i, i, i, i, _DP, _DP, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_parallel.argtypes = [i, i, i, i, i, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_chunkwise.argtypes = [i, i, i, i, i, i, _DP, _DP, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_groupnorm.argtypes = [i, i, i, i, d, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_recurrent_bwd.argtypes = [i, i, i, i, i, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP, _DP]
    lib.oracle_recurrent_bwd.restype = None
    lib.oracle_rotate.argtypes = [ctypes.c_long, i, i, d, ctypes.c_longlong, i, _DP, _DP]
    lib.oracle_rotate.restype = None
    lib.oracle_rla.argtypes = [i, i, i, i, i, i, i, _DP, _DP, _DP, _DP, _DP, i, _DP, _DP, _DP]
    lib.oracle_rla.restype = None
    lib.oracle_rla_phi.argtypes = [ctypes.c_long, i, i, _DP, _DP]
    lib.oracle_rla_phi.restype = None
    lib.oracle_threads.restype = i
    lib.oracle_set_threads.argtypes = [i]
    for f in (lib.oracle_recurrent, lib.oracle_parallel, lib.oracle_chunkwise, lib.oracle_groupnorm):
        f.restype = None
    return lib


def _get():
    """The process's oracle library: liboracle.so, or the library that RETENTION_ORACLE_LIB names
    (the sanitized build, under the sanitizer test)."""
    global _lib
    if _lib is None:
        _lib = load(os.environ.get("RETENTION_ORACLE_LIB", LIB))
    return _lib


def _f64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor: widen the exact stored values
        x = x.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_DP)


class Oracle:
    """Callable wrapper around one oracle library (the real one, or a test-built variant)."""

    def __init__(self, lib=None):
        self.lib = lib if lib is not None else _get()

    def threads(self) -> int:
        return int(self.lib.oracle_threads())

    def set_threads(self, n: int) -> None:
        self.lib.oracle_set_threads(int(n))

    @staticmethod
    def _dims(q, v):
        B, H, N, dk = q.shape
        dv = v.shape[-1]
        return B, H, N, dk, dv

    def recurrent(self, q, k, v, gamma, state_in=None, want_out=True, want_state=True):
        """Recurrent form. q, k: [B,H,N,dk]; v: [B,H,N,dv]; gamma: [H]. Returns (out, state)."""
        q, k, v, g, s0 = map(_f64, (q, k, v, gamma, state_in))
        B, H, N, dk, dv = self._dims(q, v)
        out = np.zeros((B, H, N, dv)) if want_out else None
        st = np.zeros((B, H, dk, dv)) if want_state else None
        self.lib.oracle_recurrent(B, H, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(out), _ptr(st))
        return out, st

    def parallel(self, q, k, v, gamma):
        """Parallel form O = (QK^T (.) D) V. Quadratic in N."""
        q, k, v, g = map(_f64, (q, k, v, gamma))
        B, H, N, dk, dv = self._dims(q, v)
        out = np.zeros((B, H, N, dv))
        self.lib.oracle_parallel(B, H, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(out))
        return out

    def chunkwise(self, q, k, v, gamma, chunk, state_in=None, want_state=True):
        """Chunkwise recurrent form with chunk length `chunk`. Returns (out, state)."""
        q, k, v, g, s0 = map(_f64, (q, k, v, gamma, state_in))
        B, H, N, dk, dv = self._dims(q, v)
        out = np.zeros((B, H, N, dv))
        st = np.zeros((B, H, dk, dv)) if want_state else None
        self.lib.oracle_chunkwise(B, H, N, dk, dv, int(chunk), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0),
                                  _ptr(out), _ptr(st))
        return out, st

    def groupnorm(self, x, eps, weight=None, bias=None, gate=None):
        """Per-head GroupNorm over the d_v channels of each (b, h, n) row, then (if gate, laid out
        like x, is given) times swish(gate). x: [B,H,N,dv]."""
        x, w, b, g = map(_f64, (x, weight, bias, gate))
        B, H, N, dv = x.shape
        if g is not None and g.shape != x.shape:
            raise ValueError(f"gate shape {g.shape} != {x.shape}")
        y = np.zeros_like(x)
        self.lib.oracle_groupnorm(B, H, N, dv, float(eps), _ptr(w), _ptr(b), _ptr(g), _ptr(x), _ptr(y))
        return y

    def recurrent_bwd(self, q, k, v, gamma, dout, state_in=None):
        """Gradients of the recurrent form for dL/dout = dout: (dq, dk, dv, dstate_in), fp64.
        q, k: [B,H,N,dk]; v, dout: [B,H,N,dv]; state_in: [B,H,dk,dv] or None."""
        q, k, v, dout, g, s0 = map(_f64, (q, k, v, dout, gamma, state_in))
        B, H, N, dk, dv = self._dims(q, v)
        dq, dkk, dvv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        ds = np.zeros((B, H, dk, dv))
        self.lib.oracle_recurrent_bwd(B, H, N, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(s0), _ptr(dout),
                                      _ptr(dq), _ptr(dkk), _ptr(dvv), _ptr(ds))
        return dq, dkk, dvv, ds

    def rotate(self, x, base=10000.0, offset=0, inverse=False):
        """Positional rotation of x [..., N, d] (d even): row n turned by (offset + n) * theta_i on
        feature pairs (2i, 2i+1), theta_i = base^(-2i/d); inverse=True turns the other way."""
        x = _f64(x)
        *lead, N, d = x.shape
        if d % 2:
            raise ValueError(f"rotation needs an even feature count, got {d}")
        rows = int(np.prod(lead)) if lead else 1
        y = np.zeros_like(x)
        self.lib.oracle_rotate(rows, N, d, float(base), int(offset), -1 if inverse else 1, _ptr(x), _ptr(y))
        return y

    def recurrent_rot(self, q, k, v, gamma, base=10000.0, offset=0, state_in=None, want_out=True, want_state=True):
        """Recurrent form on rotated q and k (the rotation first, then the recurrence)."""
        return self.recurrent(self.rotate(q, base, offset), self.rotate(k, base, offset), v, gamma, state_in,
                              want_out, want_state)

    def recurrent_rot_bwd(self, q, k, v, gamma, dout, base=10000.0, offset=0, state_in=None):
        """Gradients of recurrent_rot with respect to the unrotated q and k (and v, state_in): the
        gradients at the rotated inputs turned back by the inverse rotation (chain rule)."""
        dq, dk, dv, ds = self.recurrent_bwd(self.rotate(q, base, offset), self.rotate(k, base, offset), v, gamma, dout,
                                            state_in)
        return self.rotate(dq, base, offset, inverse=True), self.rotate(dk, base, offset, inverse=True), dv, ds

    FMAPS = {"identity": 0, "softmax": 1}

    def rla_phi(self, x, fmap="softmax"):
        """Feature map of residual linear attention over the last axis (softmax over the features,
        or the identity)."""
        x = _f64(x)
        y = np.zeros_like(x)
        self.lib.oracle_rla_phi(int(np.prod(x.shape[:-1])), x.shape[-1], self.FMAPS[fmap], _ptr(x), _ptr(y))
        return y

    def rla(self, q, k, v, window, fmap="softmax", k_prev=None, v_prev=None, prev_len=None, state_in=None):
        """Residual linear attention over one segment: o_t = phi(q_t) S_(t-w-1), S_t = S_(t-1) +
        phi(k_t)^T v_t. k_prev, v_prev: the window+1 positions before the segment ([B,H,window+1,d]),
        of which the last prev_len (default: all) hold tokens, or None; state_in: the state over every
        earlier token, or None. Returns (out, state_out)."""
        q, k, v, kp, vp, s0 = map(_f64, (q, k, v, k_prev, v_prev, state_in))
        if prev_len is None:
            prev_len = 0 if kp is None else window + 1
        if not 0 <= prev_len <= window + 1 or (prev_len > 0 and kp is None):
            raise ValueError("prev_len must be in [0, window + 1], with k_prev and v_prev when positive")
        B, H, N, dk, dv = self._dims(q, v)
        if (kp is None) != (vp is None):
            raise ValueError("k_prev and v_prev come together")
        if kp is not None and (kp.shape != (B, H, window + 1, dk) or vp.shape != (B, H, window + 1, dv)):
            raise ValueError("k_prev, v_prev must be [B, H, window + 1, d]")
        out = np.zeros((B, H, N, dv))
        st = np.zeros((B, H, dk, dv))
        self.lib.oracle_rla(B, H, N, dk, dv, int(window), self.FMAPS[fmap], _ptr(q), _ptr(k), _ptr(v), _ptr(kp), _ptr(vp),
                            int(prev_len), _ptr(s0), _ptr(out), _ptr(st))
        return out, st

    def step(self, q, k, v, gamma, state):
        """One recurrent decode step. q, k: [B,H,dk]; v: [B,H,dv]; state: [B,H,dk,dv].
        Returns (out [B,H,dv], new_state)."""
        q, k, v, s = map(_f64, (q, k, v, state))
        out, st = self.recurrent(q[:, :, None, :], k[:, :, None, :], v[:, :, None, :], gamma, state_in=s)
        return out[:, :, 0, :], st


def get() -> Oracle:
    return Oracle()
