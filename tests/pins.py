"""Pins for the fp64 oracle: checks against facts the pages and mathematics fix, not against the
oracle itself. Each pin takes an `oracle.Oracle` and raises AssertionError when the oracle is wrong.

They are collected in PINS so that the mutation test can run all of them against oracle builds
with planted mistakes and require that every planted mistake fails at least one pin.

Sources of truth used here:
  - a hand-worked 3-token example (tests/golden/hand_worked.json), derived by hand from the
    recurrence on the abeam.tech RetNet summary ("Training in parallel, generation by state update");
  - closed forms: with q_n = k_m = 1/sqrt(dk) and v = 1, o_n = (1 - g^(n+1)) / (1 - g) and the
    final state is (1 - g^N) / (1 - g) / sqrt(dk) everywhere (geometric series);
  - special cases with textbook answers: g = 1 is causal linear attention O = tril(QK^T) V, a
    tiny g keeps only the diagonal term (q_n . k_n) v_n;
  - brute force: a plain Python double sum over (n, m) on tiny inputs;
  - the pages' claim that the parallel, recurrent and chunkwise forms compute the same result
    (eulerwa.com "3. RetNet in detail", "How does it work?"; abeam.tech summary, FAQ), and the
    state hand-over between chunks / steps (abeam.tech, "Chunk recursion for long-sequence
    training"), checked as split/resume and decode-after-prefill identities;
  - GroupNorm invariants: each normalised row has mean b_h and variance w_h^2 var/(var+eps);
  - the positional rotation: hand-worked rows (tests/golden/rotation_hand_worked.json) and the
    facts a rotation by p * theta_i must satisfy (position 0 is the identity, pair norms are kept,
    turning by a then b is turning by a + b, the inverse undoes it), plus the property the
    rotation is used for: retention scores and outputs depend only on relative positions;
  - residual linear attention: hand-worked segments (tests/golden/rla_hand_worked.json), the
    masked linear attention it equals (numpy's shifted tril, scipy's softmax), and the segment
    and decode identities its window and state hand-over must satisfy.
"""
import json
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _qkv(B, H, N, dk, dv, seed):
    s = 1.0 / np.sqrt(dk)
    return _rand((B, H, N, dk), seed, s), _rand((B, H, N, dk), seed + 1, s), _rand((B, H, N, dv), seed + 2, s)


def _rel(a, b):
    a, b = np.asarray(a, dtype=np.float64), np.asarray(b, dtype=np.float64)
    den = max(np.sqrt(np.mean(b * b)), 1e-300)
    return float(np.max(np.abs(a - b)) / den)


# ---------------------------------------------------------------------------------------------
def pin_hand_worked(o):
    g = json.load(open(os.path.join(HERE, "golden", "hand_worked.json")))
    r = g["retention"]
    q = np.array(r["q"], float)[None, None]
    k = np.array(r["k"], float)[None, None]
    v = np.array(r["v"], float)[None, None]
    gam = [r["gamma"]]
    want_o, want_s = np.array(r["out"], float), np.array(r["state"], float)
    out, st = o.recurrent(q, k, v, gam)
    assert np.array_equal(out[0, 0], want_o), ("recurrent out", out[0, 0])
    assert np.array_equal(st[0, 0], want_s), ("recurrent state", st[0, 0])
    out = o.parallel(q, k, v, gam)
    assert np.array_equal(out[0, 0], want_o), ("parallel out", out[0, 0])
    for C in (1, 2, 3):
        out, st = o.chunkwise(q, k, v, gam, C)
        assert np.array_equal(out[0, 0], want_o), ("chunkwise out", C, out[0, 0])
        assert np.array_equal(st[0, 0], want_s), ("chunkwise state", C, st[0, 0])
    gn = g["groupnorm"]
    x = np.array(gn["x"], float)[None, None]
    y = o.groupnorm(x, gn["eps"], np.array(gn["weight"], float)[None], np.array(gn["bias"], float)[None])
    assert np.allclose(y[0, 0, 0], gn["y_row0"], rtol=0, atol=1e-15), ("groupnorm", y)
    y = o.groupnorm(x, gn["eps"], np.array(gn["weight"], float)[None], np.array(gn["bias"], float)[None],
                    np.array(gn["gate"], float)[None, None, None])
    assert np.allclose(y[0, 0, 0], gn["y_gated_row0"], rtol=0, atol=1e-15), ("gated groupnorm", y)


def pin_closed_form(o):
    for dk, dv in ((64, 48), (8, 3)):
        for gam in (0.5, 0.9, 0.99):
            N = 250
            q = np.full((1, 1, N, dk), 1.0 / np.sqrt(dk))
            k = q.copy()
            v = np.ones((1, 1, N, dv))
            n = np.arange(N, dtype=np.float64)
            want = ((1.0 - gam ** (n + 1)) / (1.0 - gam))[:, None] * np.ones((1, dv))
            want_s = (1.0 - gam ** N) / (1.0 - gam) / np.sqrt(dk)
            out, st = o.recurrent(q, k, v, [gam])
            assert _rel(out[0, 0], want) < 1e-13, ("recurrent closed form", gam, _rel(out[0, 0], want))
            assert abs(st - want_s).max() < 1e-12 * want_s, ("recurrent state", gam)
            out = o.parallel(q, k, v, [gam])
            assert _rel(out[0, 0], want) < 1e-13, ("parallel closed form", gam)
            for C in (8, 64, 128):
                out, st = o.chunkwise(q, k, v, [gam], C)
                assert _rel(out[0, 0], want) < 1e-13, ("chunkwise closed form", gam, C, _rel(out[0, 0], want))
                assert abs(st - want_s).max() < 1e-12 * want_s, ("chunkwise state", gam, C)
            # GroupNorm of a constant row is its bias (zero variance)
            bias = np.linspace(-1, 1, dv)[None]
            y = o.groupnorm(out, 1e-5, np.full((1, dv), 3.0), bias)
            assert np.abs(y[0, 0] - bias).max() < 1e-9, ("groupnorm of constant rows", gam)


def pin_gamma_one(o):
    B, H, N, dk, dv = 1, 2, 40, 5, 7
    q, k, v = _qkv(B, H, N, dk, dv, 11)
    gam = [1.0, 1.0]
    want = np.stack([np.tril(q[0, h] @ k[0, h].T) @ v[0, h] for h in range(H)])[None]
    want_s = np.stack([k[0, h].T @ v[0, h] for h in range(H)])[None]
    out, st = o.recurrent(q, k, v, gam)
    assert _rel(out, want) < 1e-12 and _rel(st, want_s) < 1e-12, "recurrent gamma=1"
    assert _rel(o.parallel(q, k, v, gam), want) < 1e-12, "parallel gamma=1"
    out, st = o.chunkwise(q, k, v, gam, 16)
    assert _rel(out, want) < 1e-12 and _rel(st, want_s) < 1e-12, "chunkwise gamma=1"


def pin_tiny_gamma(o):
    B, H, N, dk, dv = 1, 1, 33, 6, 4
    q, k, v = _qkv(B, H, N, dk, dv, 21)
    gam = [1e-30]
    want = (np.sum(q * k, axis=-1, keepdims=True) * v)
    out, st = o.recurrent(q, k, v, gam)
    assert _rel(out, want) < 1e-12, "recurrent tiny gamma"
    assert _rel(st[0, 0], np.outer(k[0, 0, -1], v[0, 0, -1])) < 1e-12, "recurrent tiny gamma state"
    assert _rel(o.parallel(q, k, v, gam), want) < 1e-12, "parallel tiny gamma"
    out, st = o.chunkwise(q, k, v, gam, 8)
    assert _rel(out, want) < 1e-12, "chunkwise tiny gamma"
    assert _rel(st[0, 0], np.outer(k[0, 0, -1], v[0, 0, -1])) < 1e-12, "chunkwise tiny gamma state"


def _brute(q, k, v, gam, state_in=None):
    B, H, N, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, H, N, dv))
    for b in range(B):
        for h in range(H):
            g = gam[h]
            for n in range(N):
                acc = np.zeros(dv)
                for m in range(n + 1):
                    acc += (g ** (n - m)) * float(np.dot(q[b, h, n], k[b, h, m])) * v[b, h, m]
                if state_in is not None:
                    acc += (g ** (n + 1)) * (q[b, h, n] @ state_in[b, h])
                out[b, h, n] = acc
    return out


def pin_bruteforce(o):
    B, H, N, dk, dv = 2, 3, 21, 4, 5
    q, k, v = _qkv(B, H, N, dk, dv, 31)
    gam = [0.7, 0.95, 1.0]
    want = _brute(q, k, v, gam)
    out, _ = o.recurrent(q, k, v, gam)
    assert _rel(out, want) < 1e-12, "recurrent vs brute force"
    assert _rel(o.parallel(q, k, v, gam), want) < 1e-12, "parallel vs brute force"
    for C in (1, 4, 5, 21, 64):
        out, _ = o.chunkwise(q, k, v, gam, C)
        assert _rel(out, want) < 1e-12, ("chunkwise vs brute force", C)
    # with an initial state: o_n gains g^(n+1) q_n S0
    s0 = _rand((B, H, dk, dv), 35)
    want = _brute(q, k, v, gam, s0)
    out, _ = o.recurrent(q, k, v, gam, state_in=s0)
    assert _rel(out, want) < 1e-12, "recurrent with state_in vs brute force"
    for C in (3, 8):
        out, _ = o.chunkwise(q, k, v, gam, C, state_in=s0)
        assert _rel(out, want) < 1e-12, ("chunkwise with state_in vs brute force", C)


def pin_three_forms(o):
    for N in (1, 7, 64, 250, 256):
        q, k, v = _qkv(1, 2, N, 16, 12, 40 + N)
        gam = [0.9, 1.0 - 2.0 ** -20]
        a, sa = o.recurrent(q, k, v, gam)
        p = o.parallel(q, k, v, gam)
        assert _rel(p, a) < 1e-12, ("parallel vs recurrent", N)
        for C in (8, 16, 64):
            c, sc = o.chunkwise(q, k, v, gam, C)
            assert _rel(c, a) < 1e-12, ("chunkwise vs recurrent", N, C)
            assert _rel(sc, sa) < 1e-12, ("chunkwise state vs recurrent state", N, C)


def pin_split_resume(o):
    B, H, N, dk, dv = 1, 2, 200, 8, 6
    q, k, v = _qkv(B, H, N, dk, dv, 51)
    gam = [0.8, 0.995]
    full, sfull = o.chunkwise(q, k, v, gam, 32)
    for n1 in (1, 64, 77, 199):
        a, sa = o.chunkwise(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], gam, 32)
        b, sb = o.chunkwise(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], gam, 32, state_in=sa)
        assert _rel(np.concatenate([a, b], axis=2), full) < 1e-12, ("split/resume out", n1)
        assert _rel(sb, sfull) < 1e-12, ("split/resume state", n1)
        ra, rsa = o.recurrent(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], gam)
        assert _rel(rsa, sa) < 1e-12, ("recurrent prefill state", n1)


def pin_decode_after_prefill(o):
    B, H, N, dk, dv = 2, 2, 130, 8, 16
    q, k, v = _qkv(B, H, N + 1, dk, dv, 61)
    gam = [0.9, 0.999]
    full, sfull = o.chunkwise(q, k, v, gam, 64)
    _, s = o.chunkwise(q[:, :, :N], k[:, :, :N], v[:, :, :N], gam, 64)
    out, s2 = o.step(q[:, :, N], k[:, :, N], v[:, :, N], gam, s)
    assert _rel(out, full[:, :, N]) < 1e-12, "decode after prefill: output"
    assert _rel(s2, sfull) < 1e-12, "decode after prefill: state"


def pin_linearity(o):
    B, H, N, dk, dv = 1, 2, 50, 6, 5
    q, k, v1 = _qkv(B, H, N, dk, dv, 71)
    v2 = _rand((B, H, N, dv), 75)
    gam = [0.85, 0.97]
    a, sa = o.chunkwise(q, k, v1, gam, 16)
    b, sb = o.chunkwise(q, k, v2, gam, 16)
    c, sc = o.chunkwise(q, k, 2.0 * v1 - 3.0 * v2, gam, 16)
    assert _rel(c, 2.0 * a - 3.0 * b) < 1e-12 and _rel(sc, 2.0 * sa - 3.0 * sb) < 1e-12, "linear in v"
    # the state read-out is linear in the initial state with weight g^(n+1)
    s0 = _rand((B, H, dk, dv), 77)
    d, _ = o.recurrent(q, k, v1, gam, state_in=s0)
    ra, _ = o.recurrent(q, k, v1, gam)
    z = np.zeros_like(v1)
    e, _ = o.recurrent(q, k, z, gam, state_in=s0)
    assert _rel(d, ra + e) < 1e-12, "state_in contribution adds"
    for h, g in enumerate(gam):
        n = np.arange(N)
        want = (g ** (n + 1))[:, None] * (q[0, h] @ s0[0, h])
        assert _rel(e[0, h], want) < 1e-12, ("state_in decays as g^(n+1)", h)


def pin_groupnorm(o):
    B, H, N, dv = 2, 3, 5, 32
    x = _rand((B, H, N, dv), 81) * np.array([0.01, 1.0, 100.0])[None, :, None, None] + 0.3
    w = np.array([0.5, 2.0, -1.0])[:, None] * np.ones((1, dv))
    bias = np.array([1.0, -2.0, 0.25])[:, None] * np.ones((1, dv))
    eps = 1e-3
    y = o.groupnorm(x, eps, w, bias)
    for h in range(H):
        xr = x[:, h]
        var = xr.var(axis=-1)
        yr = y[:, h]
        assert np.allclose(yr.mean(axis=-1), bias[h, 0], atol=1e-12), ("groupnorm mean", h)
        assert np.allclose(yr.var(axis=-1), w[h, 0] ** 2 * var / (var + eps), rtol=1e-10), ("groupnorm var", h)
    # scale invariance up to eps: scaling a row by c changes y only through eps
    y1 = o.groupnorm(x * 1e3, eps * 1e6, w, bias)
    assert _rel(y1, y) < 1e-10, "groupnorm scale invariance"


def pin_swish_gate(o):
    """The gate multiplies the affine GroupNorm output by swish(g) = g * sigmoid(g), checked through
    properties of the logistic function rather than its formula: swish(g) - swish(-g) = g (since
    sigmoid(g) + sigmoid(-g) = 1), swish(0) = 0, swish(g) -> g for large g and -> 0 for very
    negative g, and sigmoid(ln 3) = 3/4."""
    B, H, N, dv = 2, 3, 4, 16
    x = _rand((B, H, N, dv), 91) + 0.2
    w = _rand((H, dv), 92) + 1.0
    bias = _rand((H, dv), 93)
    eps = 1e-5
    y0 = o.groupnorm(x, eps, w, bias)
    g = 4.0 * _rand((B, H, N, dv), 94)
    diff = o.groupnorm(x, eps, w, bias, g) - o.groupnorm(x, eps, w, bias, -g)
    assert _rel(diff, y0 * g) < 1e-12, "swish(g) - swish(-g) = g"
    assert np.all(o.groupnorm(x, eps, w, bias, np.zeros_like(x)) == 0.0), "swish(0) = 0"
    assert _rel(o.groupnorm(x, eps, w, bias, np.full_like(x, 40.0)), 40.0 * y0) < 1e-15, "swish(40) = 40"
    assert np.abs(o.groupnorm(x, eps, w, bias, np.full_like(x, -40.0))).max() < 1e-13 * np.abs(y0).max(), "swish(-40) ~ 0"
    # the gate applies after the affine, bias included: with g = ln 3 everywhere, y = (3/4) ln 3 * y0
    ln3 = np.log(3.0)
    assert _rel(o.groupnorm(x, eps, w, bias, np.full_like(x, ln3)), 0.75 * ln3 * y0) < 1e-14, "sigmoid(ln 3) = 3/4"


def _ip(a, b):
    return float(np.sum(np.asarray(a) * np.asarray(b)))


def pin_backward_adjoint(o):
    """The output is linear in q (k, v and the state fixed), in k and in v (zero state), and in the
    state (q, k fixed, v = 0). For a linear map A with gradient A^T dout the adjoint identity
    <dout, A(d)> = <A^T dout, d> holds for every direction d, so each gradient is fixed by the
    pinned forward oracle alone."""
    B, H, N, dk, dv = 2, 2, 37, 5, 4
    q, k, v = _qkv(B, H, N, dk, dv, 101)
    s0 = _rand((B, H, dk, dv), 102)
    dout = _rand((B, H, N, dv), 103)
    gam = [0.9, 0.5]
    dq, dk_, dv_, ds = o.recurrent_bwd(q, k, v, gam, dout, state_in=s0)
    dq0, dk0, dv0, _ = o.recurrent_bwd(q, k, v, gam, dout)
    d = [_rand(x.shape, 104 + i) for i, x in enumerate((q, k, v, s0))]
    fwd = lambda qq, kk, vv, ss=None: o.recurrent(qq, kk, vv, gam, state_in=ss)[0]
    checks = [("dq", _ip(dout, fwd(d[0], k, v, s0)), _ip(dq, d[0])),
              ("dk", _ip(dout, fwd(q, d[1], v)), _ip(dk0, d[1])),
              ("dv", _ip(dout, fwd(q, k, d[2])), _ip(dv0, d[2])),
              ("dstate_in", _ip(dout, fwd(q, k, 0 * v, d[3])), _ip(ds, d[3]))]
    for name, lhs, rhs in checks:
        assert abs(lhs - rhs) <= 1e-12 * max(abs(lhs), 1.0), (name, lhs, rhs)
    # dk and dv do not depend on the state
    assert _rel(dk_, dk0) < 1e-14 and _rel(dv_, dv0) < 1e-14, "state-independent dk, dv"


def pin_backward_fd(o):
    """Central finite differences of L = <dout, out> in fp64 against single gradient entries."""
    B, H, N, dk, dv = 1, 2, 9, 3, 2
    q, k, v = _qkv(B, H, N, dk, dv, 111)
    s0 = _rand((B, H, dk, dv), 112)
    dout = _rand((B, H, N, dv), 113)
    gam = [0.8, 0.99]
    grads = o.recurrent_bwd(q, k, v, gam, dout, state_in=s0)
    args = [q, k, v, s0]
    L = lambda a: _ip(dout, o.recurrent(a[0], a[1], a[2], gam, state_in=a[3])[0])
    rng = np.random.default_rng(114)
    h = 1e-4
    for t in range(4):
        for _ in range(3):
            idx = tuple(int(rng.integers(0, s)) for s in args[t].shape)
            ap, am = [x.copy() for x in args], [x.copy() for x in args]
            ap[t][idx] += h
            am[t][idx] -= h
            fd = (L(ap) - L(am)) / (2 * h)
            assert abs(fd - grads[t][idx]) <= 1e-8 * max(abs(fd), 1.0), ("finite difference", t, idx, fd, grads[t][idx])


def pin_backward_bruteforce(o):
    """The parallel form's derivatives as Python double sums, for a small case:
    dq_n = sum_{m<=n} g^(n-m) (dout_n . v_m) k_m, dk_m = sum_{n>=m} g^(n-m) (dout_n . v_m) q_n,
    dv_m = sum_{n>=m} g^(n-m) (q_n . k_m) dout_n, plus dq_n += g^(n+1) dout_n S_in^T."""
    B, H, N, dk, dv = 1, 1, 11, 3, 2
    q, k, v = _qkv(B, H, N, dk, dv, 121)
    s0 = _rand((B, H, dk, dv), 122)
    dout = _rand((B, H, N, dv), 123)
    g = 0.7
    dq, dk_, dv_, ds = o.recurrent_bwd(q, k, v, [g], dout, state_in=s0)
    Q, K, V, G, S = q[0, 0], k[0, 0], v[0, 0], dout[0, 0], s0[0, 0]
    for n in range(N):
        want_q = sum(g ** (n - m) * (G[n] @ V[m]) * K[m] for m in range(n + 1)) + g ** (n + 1) * (S @ G[n])
        want_k = sum(g ** (m - n) * (G[m] @ V[n]) * Q[m] for m in range(n, N))
        want_v = sum(g ** (m - n) * (Q[m] @ K[n]) * G[m] for m in range(n, N))
        assert np.allclose(dq[0, 0, n], want_q, rtol=1e-12, atol=1e-12), ("dq", n)
        assert np.allclose(dk_[0, 0, n], want_k, rtol=1e-12, atol=1e-12), ("dk", n)
        assert np.allclose(dv_[0, 0, n], want_v, rtol=1e-12, atol=1e-12), ("dv", n)
    want_s = sum(g ** (n + 1) * np.outer(Q[n], G[n]) for n in range(N))
    assert np.allclose(ds[0, 0], want_s, rtol=1e-12, atol=1e-12), "dstate_in"


def pin_rotation_hand_worked(o):
    import math
    g = json.load(open(os.path.join(HERE, "golden", "rotation_hand_worked.json")))
    env = {"__builtins__": {}, "cos": math.cos, "sin": math.sin}
    for case in g["cases"]:
        x = np.array(case["x"], float)[None, None]
        want = np.array([[eval(e, env) for e in row] for row in case["y"]])
        y = o.rotate(x, case["base"], case["offset"])[0, 0]
        assert np.allclose(y, want, rtol=0, atol=1e-15), ("rotation hand-worked", case["what"], y, want)


def pin_rotation_properties(o):
    rng = np.random.default_rng(131)
    x = rng.standard_normal((2, 3, 50, 16))
    for base, off in ((10000.0, 0), (500.0, 123), (10000.0, 65536)):
        y = o.rotate(x, base, off)
        # pair norms are kept
        nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
        assert _rel(ny, nx) < 1e-14, ("pair norms", base, off)
        # the inverse undoes the rotation
        assert _rel(o.rotate(y, base, off, inverse=True), x) < 1e-13, ("inverse", base, off)
    # position 0 is the identity
    assert np.array_equal(o.rotate(x[:, :, :1], 10000.0, 0), x[:, :, :1]), "position 0"
    # one row: turning by a, then by b, is turning by a + b
    r = x[:, :, :1]
    for a, b in ((1, 2), (37, 1000), (5000, 3)):
        assert _rel(o.rotate(o.rotate(r, 10000.0, a), 10000.0, b), o.rotate(r, 10000.0, a + b)) < 1e-12, ("compose", a, b)
    # the scores of rotated q and k depend only on relative positions
    q, k = rng.standard_normal((1, 1, 40, 16)), rng.standard_normal((1, 1, 40, 16))
    s0 = o.rotate(q, 10000.0, 0)[0, 0] @ o.rotate(k, 10000.0, 0)[0, 0].T
    s1 = o.rotate(q, 10000.0, 911)[0, 0] @ o.rotate(k, 10000.0, 911)[0, 0].T
    assert _rel(s1, s0) < 1e-12, "relative positions"
    # the score of one pair at positions n and m equals q . R((m - n) theta) k, with k turned alone
    for n, m in ((7, 3), (30, 0), (12, 12)):
        want = float(q[0, 0, n] @ o.rotate(k[:, :, m:m + 1], 10000.0, m - n)[0, 0, 0])
        assert abs(s0[n, m] - want) < 1e-12 * max(1.0, abs(want)), ("relative score", n, m)


def pin_rotation_retention(o):
    B, H, N, dk, dv = 1, 2, 90, 8, 5
    q, k, v = _qkv(B, H, N, dk, dv, 141)
    gam = [0.9, 0.995]
    # outputs with zero start state depend only on relative positions
    a, _ = o.recurrent_rot(q, k, v, gam, 10000.0, 0)
    b, _ = o.recurrent_rot(q, k, v, gam, 10000.0, 4097)
    assert _rel(b, a) < 1e-11, "rotated retention: offset invariance"
    # ... and the rotation is not a no-op
    c, _ = o.recurrent(q, k, v, gam)
    assert _rel(c, a) > 1e-3, "rotation changes the output"
    # split and resume with the position offset carried
    full, sfull = o.recurrent_rot(q, k, v, gam, 500.0, 3)
    for n1 in (1, 40, 89):
        x, sx = o.recurrent_rot(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], gam, 500.0, 3)
        y, sy = o.recurrent_rot(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], gam, 500.0, 3 + n1, state_in=sx)
        assert _rel(np.concatenate([x, y], axis=2), full) < 1e-12, ("rotated split/resume out", n1)
        assert _rel(sy, sfull) < 1e-12, ("rotated split/resume state", n1)


def pin_rotation_backward_fd(o):
    """Central finite differences of L = <dout, out> through the rotation, against the gradients
    with respect to the unrotated q and k."""
    B, H, N, dk, dv = 1, 1, 8, 4, 3
    q, k, v = _qkv(B, H, N, dk, dv, 151)
    s0 = _rand((B, H, dk, dv), 152)
    dout = _rand((B, H, N, dv), 153)
    gam, base, off = [0.85], 100.0, 5
    grads = o.recurrent_rot_bwd(q, k, v, gam, dout, base, off, state_in=s0)
    L = lambda qq, kk: _ip(dout, o.recurrent_rot(qq, kk, v, gam, base, off, state_in=s0)[0])
    rng = np.random.default_rng(154)
    h = 1e-4
    for t in range(2):
        for _ in range(4):
            idx = tuple(int(rng.integers(0, s)) for s in q.shape)
            ap, am = [q.copy(), k.copy()], [q.copy(), k.copy()]
            ap[t][idx] += h
            am[t][idx] -= h
            fd = (L(*ap) - L(*am)) / (2 * h)
            assert abs(fd - grads[t][idx]) <= 1e-8 * max(abs(fd), 1.0), ("rotated finite difference", t, idx, fd, grads[t][idx])


def _num(x):
    import math
    return {"ln2": math.log(2.0), "ln3": math.log(3.0)}.get(x, x) if isinstance(x, str) else x


def _arr(rows):
    return np.array([[_num(x) for x in r] for r in rows], float)


def pin_rla_hand_worked(o):
    g = json.load(open(os.path.join(HERE, "golden", "rla_hand_worked.json")))
    for c in g["cases"]:
        ex = lambda key: _arr(c[key])[None, None] if key in c else None
        out, st = o.rla(ex("q"), ex("k"), ex("v"), c["window"], c["fmap"], ex("k_prev"), ex("v_prev"), state_in=ex("state_in"))
        assert np.allclose(out[0, 0], _arr(c["out"]), rtol=0, atol=1e-14), ("rla hand-worked out", c["what"], out[0, 0])
        assert np.allclose(st[0, 0], _arr(c["state_out"]), rtol=0, atol=1e-14), ("rla hand-worked state", c["what"], st[0, 0])
    for r in g["softmax_rows"]:
        y = o.rla_phi(_arr([r["x"]]), "softmax")[0]
        assert np.allclose(y, r["y"], rtol=0, atol=1e-15), ("softmax feature map", r, y)


def pin_rla_masked_attention(o):
    """With no earlier tokens and zero state, o = tril(phi(Q) phi(K)^T, -(w+1)) V: linear attention
    with the diagonal and the w tokens before it masked out."""
    from scipy.special import softmax
    B, H, N, dk, dv = 1, 2, 40, 6, 5
    q, k, v = _qkv(B, H, N, dk, dv, 161)
    q, k = q * 4, k * 4  # a peaked softmax
    for fmap, phi in (("identity", lambda x: x), ("softmax", lambda x: softmax(x, axis=-1))):
        for w in (0, 1, 7, 39, 45):
            out, st = o.rla(q, k, v, w, fmap)
            for h in range(H):
                A = np.tril(phi(q[0, h]) @ phi(k[0, h]).T, -(w + 1))
                assert _rel(out[0, h], A @ v[0, h]) < 1e-12 or np.abs(out[0, h]).max() == 0 == np.abs(A @ v[0, h]).max(), \
                    ("rla masked attention", fmap, w, h)
                n_left = max(N - w - 1, 0)
                want_s = phi(k[0, h, :n_left]).T @ v[0, h, :n_left]
                assert np.allclose(st[0, h], want_s, rtol=1e-12, atol=1e-13), ("rla state out", fmap, w, h)
    # softmax rows are positive, sum to 1, and do not change when a constant is added
    y = o.rla_phi(q, "softmax")
    assert np.all(y > 0) and np.allclose(y.sum(-1), 1.0, rtol=0, atol=1e-14), "softmax rows"
    assert _rel(o.rla_phi(q + 3.25, "softmax"), y) < 1e-14, "softmax shift invariance"


def pin_rla_segments(o):
    """Two segments with the window and state handed over equal one pass, also when the first
    segment is shorter than the window (a partial window, prev_len < w + 1); one-token segments
    (decode steps) equal one pass."""
    B, H, N, dk, dv = 1, 2, 60, 5, 4
    q, k, v = _qkv(B, H, N, dk, dv, 171)
    s0 = _rand((B, H, dk, dv), 172, 0.1)
    for fmap in ("identity", "softmax"):
        for w in (0, 3, 9):
            full, sfull = o.rla(q, k, v, w, fmap, state_in=s0)
            P = w + 1
            for n1 in (2, 9, 30, 59):
                a, sa = o.rla(q[:, :, :n1], k[:, :, :n1], v[:, :, :n1], w, fmap, state_in=s0)
                # rows before the sequence start hold junk, which must not be read
                kp, vp = _rand((B, H, P, dk), 173), _rand((B, H, P, dv), 174)
                L = min(n1, P)
                kp[:, :, P - L:], vp[:, :, P - L:] = k[:, :, n1 - L:n1], v[:, :, n1 - L:n1]
                b, sb = o.rla(q[:, :, n1:], k[:, :, n1:], v[:, :, n1:], w, fmap, kp, vp, L, state_in=sa)
                assert _rel(np.concatenate([a, b], axis=2), full) < 1e-12, ("rla split/resume out", fmap, w, n1)
                assert _rel(sb, sfull) < 1e-12, ("rla split/resume state", fmap, w, n1)
            # decode: one token per call, the window slid by the caller
            st, outs = s0, []
            for t in range(N):
                kp, vp = _rand((B, H, P, dk), 175 + t), _rand((B, H, P, dv), 176 + t)
                L = min(t, P)
                if L:
                    kp[:, :, P - L:], vp[:, :, P - L:] = k[:, :, t - L:t], v[:, :, t - L:t]
                ot, st = o.rla(q[:, :, t:t + 1], k[:, :, t:t + 1], v[:, :, t:t + 1], w, fmap, kp, vp, L, state_in=st)
                outs.append(ot)
            assert _rel(np.concatenate(outs, axis=2), full) < 1e-12, ("rla decode steps out", fmap, w)
            assert _rel(st, sfull) < 1e-12, ("rla decode steps state", fmap, w)


PINS = [pin_hand_worked, pin_closed_form, pin_gamma_one, pin_tiny_gamma, pin_bruteforce, pin_three_forms,
        pin_split_resume, pin_decode_after_prefill, pin_linearity, pin_groupnorm, pin_swish_gate,
        pin_backward_adjoint, pin_backward_fd, pin_backward_bruteforce, pin_rotation_hand_worked,
        pin_rotation_properties, pin_rotation_retention, pin_rotation_backward_fd, pin_rla_hand_worked,
        pin_rla_masked_attention, pin_rla_segments]
