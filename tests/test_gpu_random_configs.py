"""GPU parity over seeded random configurations of the chunkwise forward, against the fp64 oracle.

Each case draws, from one fixed seed, a shape the library supports (input dtype, d_k, d_v, chunk,
B, H, a ragged N), per-head decays (the multi-scale set or uniform in [0.5, 0.999]), and the
options a caller can combine: state_in (in place or not), the GroupNorm epilogue (weight, bias,
gate), the positional rotation (with an offset). The combinations reach every kernel family of the
forward: the (b, h, slice) kernels with two or three stage buffers, the single-group kernel at chunk
512, the segmented kernels (grids of fewer slices than compute units), the two- and three-pass
splits of rotated bf16 inputs and the fp32 kernels. Out and state are compared with the oracle
(recurrent form, rotated first when a rotation is on, then GroupNorm), by max|gpu - oracle| /
RMS(oracle) against 1e-4 (fp32 inputs) or 2e-2 (bf16 inputs), with fp32 outputs; a bf16 output of
the same call must be the fp32 one rounded (within 2^-8 relative, element by element).
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_chunkwise_amd import inputs as I
from linear_recurrent_sequence_chunkwise_amd import retention as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


def _configs(n=32, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 4 == 3 else "bf16"
        if dt == "bf16":
            dk = int(rng.choice([64, 256]))
            dv = int(rng.choice([32, 64, 128, 256, 512]))
            C = int(rng.choice([64, 128, 256, 512]))
        else:
            dk = int(rng.choice([64, 128, 256]))
            dv = int(rng.choice([64, 128, 256, 512]))
            C = int(rng.choice([64, 128]))
        B, H = [(1, 1), (1, 3), (2, 2), (1, 5), (2, 4), (1, 16), (1, 17), (2, 10)][int(rng.integers(0, 8))]
        N = int(rng.integers(1, 800))
        state = bool(rng.random() < 0.6)
        out.append(dict(i=i, dt=dt, dk=dk, dv=dv, C=C, B=B, H=H, N=N, state=state,
                        inplace=state and bool(rng.random() < 0.3), gn=bool(rng.random() < 0.4), gate=bool(rng.random() < 0.5),
                        rot=bool(rng.random() < 0.3), off=int(rng.integers(0, 100000)), multiscale=bool(rng.random() < 0.5),
                        gseed=int(rng.integers(0, 2 ** 31))))
    return out


CONFIGS = _configs()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    R.load_library()
    yield
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def rel_err(gpu, ref):
    g = gpu.detach().double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    return float(np.max(np.abs(g - r)) / np.sqrt(np.mean(r * r)))


def _name(c):
    return (f"{c['i']}-{c['dt']}-dk{c['dk']}-dv{c['dv']}-C{c['C']}-B{c['B']}H{c['H']}-N{c['N']}"
            f"{'-state' if c['state'] else ''}{'-inplace' if c['inplace'] else ''}{'-gn' if c['gn'] else ''}"
            f"{'-gate' if c['gn'] and c['gate'] else ''}{'-rot' if c['rot'] else ''}")


@pytest.mark.parametrize("c", CONFIGS, ids=_name)
def test_random_chunkwise_config(orc, c):
    B, H, N, dk, dv, C, dt = c["B"], c["H"], c["N"], c["dk"], c["dv"], c["C"], c["dt"]
    gen = torch.Generator().manual_seed(c["gseed"])
    q, k, v = I.make_qkv(B, H, N, dk, dv, dt, seed=c["gseed"] % 100003)
    if c["multiscale"]:
        gam = [1.0 - 2.0 ** (-5 - (h % 16)) for h in range(H)]
    else:
        gam = [float(x) for x in 0.5 + 0.499 * torch.rand(H, generator=gen, dtype=torch.float64)]
    s0 = I.make_state(B, H, dk, dv, seed=c["gseed"] % 99991, scale=0.02) if c["state"] else None
    gn = None
    w = b = g = None
    if c["gn"]:
        w = (1.0 + 0.1 * torch.randn(H, dv, generator=gen)).float()
        b = (0.1 * torch.randn(H, dv, generator=gen)).float()
        if c["gate"]:
            g = torch.randn(B, H, N, dv, generator=gen).to(q.dtype)
        gn = R.GroupNorm(1e-5, w.to(DEV), b.to(DEV), g.to(DEV) if g is not None else None)
    rot = R.Rotation(10000.0, c["off"]) if c["rot"] else None

    if rot is not None:
        ref, ref_s = orc.recurrent_rot(q, k, v, gam, 10000.0, c["off"], state_in=s0)
    else:
        ref, ref_s = orc.recurrent(q, k, v, gam, state_in=s0)
    if c["gn"]:
        ref = orc.groupnorm(ref, 1e-5, w, b, g)

    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    s0d = s0.to(DEV) if s0 is not None else None
    st_out = s0d.clone() if c["inplace"] else None
    o, s = R.chunkwise_fwd(qd, kd, vd, gam, C, state_in=st_out if c["inplace"] else s0d, groupnorm=gn, rotation=rot,
                           state_out=st_out)
    tol = TOL[dt]
    e_out, e_state = rel_err(o, ref), rel_err(s, ref_s)
    print(f"  {_name(c)}: out {e_out:.3e}, state {e_state:.3e} (bound {tol:g})", flush=True)
    assert e_out <= tol, f"out {e_out:.3e} > {tol:g}"
    assert e_state <= tol, f"state {e_state:.3e} > {tol:g}"
    if c["inplace"]:
        assert s.data_ptr() == st_out.data_ptr()
    # the bf16 output of the same call is the fp32 output rounded to nearest
    ob, _ = R.chunkwise_fwd(qd, kd, vd, gam, C, state_in=s0d, groupnorm=gn, rotation=rot, out_dtype=torch.bfloat16,
                            want_state=False)
    o64, ob64 = o.double().cpu(), ob.double().cpu()
    rel = float(((ob64 - o64).abs() / o64.abs().clamp_min(1e-30)).max())
    assert rel <= 2.0 ** -8, f"bf16 out vs fp32 out rounded: {rel:.3e}"


def _bwd_configs(n=16, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 4 == 3 else "bf16"
        if dt == "bf16":
            dk, C = int(rng.choice([64, 256])), int(rng.choice([64, 128, 256, 512]))
        else:
            dk, C = int(rng.choice([64, 128, 256])), int(rng.choice([64, 128]))
        dv = int(rng.choice([64, 128, 256, 512]))
        B, H = [(1, 1), (1, 3), (2, 2), (1, 4), (1, 6)][int(rng.integers(0, 5))]
        # N a multiple of the chunk in some cases (bf16: the dk forward then reuses the dq forward's scores)
        N = C * int(rng.integers(1, 4)) if rng.random() < 0.4 else int(rng.integers(1, 500))
        out.append(dict(i=i, dt=dt, dk=dk, dv=dv, C=C, B=B, H=H, N=N, state=bool(rng.random() < 0.5),
                        rot=bool(rng.random() < 0.3), off=int(rng.integers(0, 100000)), gseed=int(rng.integers(0, 2 ** 31))))
    return out


def _bname(c):
    return (f"{c['i']}-{c['dt']}-dk{c['dk']}-dv{c['dv']}-C{c['C']}-B{c['B']}H{c['H']}-N{c['N']}"
            f"{'-state' if c['state'] else ''}{'-rot' if c['rot'] else ''}")


# The chunkwise backward over seeded random configurations: dq, dk, dv and dstate_in against the
# oracle's gradients of the recurrent form (rotated inputs: with respect to the unrotated q and k).
@pytest.mark.parametrize("c", _bwd_configs(), ids=_bname)
def test_random_backward_config(orc, c):
    B, H, N, dk, dv, C, dt = c["B"], c["H"], c["N"], c["dk"], c["dv"], c["C"], c["dt"]
    gen = torch.Generator().manual_seed(c["gseed"])
    q, k, v = I.make_qkv(B, H, N, dk, dv, dt, seed=c["gseed"] % 100003)
    dout = torch.randn(B, H, N, dv, generator=gen).to(q.dtype)
    gam = [float(x) for x in 0.5 + 0.499 * torch.rand(H, generator=gen, dtype=torch.float64)]
    s0 = I.make_state(B, H, dk, dv, seed=c["gseed"] % 99991, scale=0.02) if c["state"] else None
    if c["rot"]:
        ref = orc.recurrent_rot_bwd(q, k, v, gam, dout, 10000.0, c["off"], state_in=s0)
    else:
        ref = orc.recurrent_bwd(q, k, v, gam, dout, state_in=s0)
    got = R.chunkwise_bwd(q.to(DEV), k.to(DEV), v.to(DEV), gam, dout.to(DEV), C,
                          state_in=s0.to(DEV) if s0 is not None else None,
                          rotation=R.Rotation(10000.0, c["off"]) if c["rot"] else None)
    tol = TOL[dt]
    for name, g_, r_ in zip(("dq", "dk", "dv", "dstate_in"), got, ref):
        e = rel_err(g_, r_)
        print(f"  {_bname(c)} {name}: {e:.3e} (bound {tol:g})", flush=True)
        assert e <= tol, f"{name} {e:.3e} > {tol:g}"


def _par_configs(n=12, seed=20261205):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dt = "f32" if i % 3 == 2 else "bf16"
        dk = int(rng.choice([64, 256])) if dt == "bf16" else int(rng.choice([32, 64, 128, 256]))
        dv = int(rng.choice([64, 128, 256, 512]))
        B, H = [(1, 1), (1, 3), (2, 2), (1, 5), (1, 16)][int(rng.integers(0, 5))]
        out.append(dict(i=i, dt=dt, dk=dk, dv=dv, B=B, H=H, N=int(rng.integers(1, 700)), gn=bool(rng.random() < 0.5),
                        rot=bool(rng.random() < 0.3), off=int(rng.integers(0, 100000)), gseed=int(rng.integers(0, 2 ** 31))))
    return out


def _pname(c):
    return f"{c['i']}-{c['dt']}-dk{c['dk']}-dv{c['dv']}-B{c['B']}H{c['H']}-N{c['N']}{'-gn' if c['gn'] else ''}{'-rot' if c['rot'] else ''}"


# The parallel form over seeded random configurations, against the oracle's recurrent form.
@pytest.mark.parametrize("c", _par_configs(), ids=_pname)
def test_random_parallel_config(orc, c):
    B, H, N, dk, dv, dt = c["B"], c["H"], c["N"], c["dk"], c["dv"], c["dt"]
    gen = torch.Generator().manual_seed(c["gseed"])
    q, k, v = I.make_qkv(B, H, N, dk, dv, dt, seed=c["gseed"] % 100003)
    gam = [float(x) for x in 0.5 + 0.499 * torch.rand(H, generator=gen, dtype=torch.float64)]
    if c["rot"]:
        ref, _ = orc.recurrent_rot(q, k, v, gam, 10000.0, c["off"])
    else:
        ref, _ = orc.recurrent(q, k, v, gam)
    gn = None
    if c["gn"]:
        w = (1.0 + 0.1 * torch.randn(H, dv, generator=gen)).float()
        b = (0.1 * torch.randn(H, dv, generator=gen)).float()
        ref = orc.groupnorm(ref, 1e-5, w, b)
        gn = R.GroupNorm(1e-5, w.to(DEV), b.to(DEV))
    o = R.parallel_fwd(q.to(DEV), k.to(DEV), v.to(DEV), gam, groupnorm=gn,
                       rotation=R.Rotation(10000.0, c["off"]) if c["rot"] else None)
    e = rel_err(o, ref)
    print(f"  {_pname(c)}: out {e:.3e} (bound {TOL[dt]:g})", flush=True)
    assert e <= TOL[dt], f"out {e:.3e} > {TOL[dt]:g}"
