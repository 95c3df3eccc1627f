"""The library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

Every call only enqueues kernels on the caller's stream (no allocation, copy, memset or
synchronisation inside the library), so a captured call must replay to the same bits as the eager
call. Each graph is replayed several times, with eager library work and synchronisations in
between, and every replay is compared with the eager result bitwise; one replay is also checked
against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
from linear_recurrent_sequence_chunkwise_amd import inputs as I
from linear_recurrent_sequence_chunkwise_amd import retention as R

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    R.load_library()


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


def rel_err(gpu, ref):
    g = gpu.double().cpu().numpy()
    r = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(g - r)) / np.sqrt(np.mean(r * r)))


def capture(fn):
    """Warm the call up eagerly (first-call set-up), then capture it on a side stream."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        res = fn()
    torch.cuda.synchronize()
    return g, res


def eager_noise(x):
    """Unrelated eager library work between replays, so that a replay cannot lean on leftovers."""
    y = R.chunkwise_fwd(x[0], x[1], x[2], [0.5] * x[0].shape[1], 64, want_state=False)[0]
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("H", [4, 16])  # 4 heads: the segmented kernels; 16: the (b, h, slice) chunk kernels
def test_graph_chunkwise_groupnorm(orc, H):
    B, N, dk, dv = 1, 1000, 256, 512
    q, k, v = I.make_qkv(B, H, N, dk, dv, "bf16", seed=950)
    s0 = I.make_state(B, H, dk, dv, seed=951, scale=0.02)
    gam = I.multiscale_gammas(16)[::16 // H]
    qd, kd, vd, s0d = (t.to(DEV) for t in (q, k, v, s0))
    gn = R.GroupNorm(1e-5)
    call = lambda: R.chunkwise_fwd(qd, kd, vd, gam, 128, state_in=s0d, groupnorm=gn, out_dtype=torch.bfloat16)
    eo, es = call()
    torch.cuda.synchronize()
    eo, es = eo.clone(), es.clone()
    g, (go, gs) = capture(call)
    noise = I.make_qkv(1, 2, 300, 64, 64, "bf16", seed=952)
    noise = [t.to(DEV) for t in noise]
    for r in range(REPLAYS):
        go.zero_()
        gs.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(go, eo) and torch.equal(gs, es), f"replay {r} differs from the eager call"
        eager_noise(noise)
    ref, ref_s = orc.recurrent(q, k, v, gam, state_in=s0)
    assert rel_err(go, orc.groupnorm(ref, 1e-5)) <= 2e-2
    assert rel_err(gs, ref_s) <= 2e-2


def test_graph_decode_steps_advance_the_state(orc):
    """A captured decode step updates the state in place: n replays are n steps."""
    B, H, dk, dv = 8, 4, 256, 512
    q, k, v = I.make_qkv(B, H, 1, dk, dv, "bf16", seed=960)
    s0 = I.make_state(B, H, dk, dv, seed=961, scale=0.05)
    gam = I.multiscale_gammas(16)[::4]
    qd, kd, vd = (t[:, :, 0].contiguous().to(DEV) for t in (q, k, v))
    state_e = s0.to(DEV)
    state_g = s0.to(DEV)
    out_g = torch.empty((B, H, dv), dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    # warm-up on a scratch state, so the graph's state has seen no step before the replays
    scratch = s0.to(DEV)
    R.recurrent_step(qd, kd, vd, gam, scratch)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        R.recurrent_step(qd, kd, vd, gam, state_g, out=out_g)
    torch.cuda.synchronize()
    ref_state = s0.double().numpy()
    for r in range(REPLAYS):
        eo = R.recurrent_step(qd, kd, vd, gam, state_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, eo) and torch.equal(state_g, state_e), f"replay {r} differs from eager step {r}"
        ro, ref_state = orc.step(q[:, :, 0], k[:, :, 0], v[:, :, 0], gam, ref_state)
        assert rel_err(out_g, ro) <= 2e-2 and rel_err(state_g, ref_state) <= 2e-2


def test_graph_backward_with_rotation(orc):
    """The backward (scores, chunk, block-sum, transpose, scale and rotation kernels) as one graph."""
    B, H, N, dk, dv = 1, 2, 700, 256, 512
    q, k, v = I.make_qkv(B, H, N, dk, dv, "bf16", seed=970)
    dout = torch.randn((B, H, N, dv), generator=torch.Generator().manual_seed(971)).to(torch.bfloat16)
    s0 = I.make_state(B, H, dk, dv, seed=972, scale=0.02)
    gam = [0.9, 0.999]
    rot = R.Rotation(10000.0, 37)
    qd, kd, vd, dod, s0d = (t.to(DEV) for t in (q, k, v, dout, s0))
    call = lambda: R.chunkwise_bwd(qd, kd, vd, gam, dod, 128, state_in=s0d, rotation=rot)
    eager = [t.clone() for t in call()]
    torch.cuda.synchronize()
    g, got = capture(call)
    noise = [t.to(DEV) for t in I.make_qkv(1, 2, 300, 64, 64, "bf16", seed=973)]
    for r in range(REPLAYS):
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv", "dstate_in"), got, eager):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
        eager_noise(noise)
    # the oracle's gradients at the rotated q and k rounded to bf16 (the operands the kernels see),
    # turned back by the inverse rotation in fp64
    rq, rk = (torch.from_numpy(orc.rotate(x, 10000.0, 37)).float().to(torch.bfloat16) for x in (q, k))
    gq, gk, gv, gs = orc.recurrent_bwd(rq, rk, v, gam, dout, state_in=s0)
    ref = (orc.rotate(gq, 10000.0, 37, inverse=True), orc.rotate(gk, 10000.0, 37, inverse=True), gv, gs)
    for name, a, b in zip(("dq", "dk", "dv", "dstate_in"), got, ref):
        assert rel_err(a, b) <= 2e-2, name


def test_graph_parallel_and_rla(orc):
    B, H, N, dk, dv = 1, 3, 600, 64, 64
    q, k, v = I.make_qkv(B, H, N, dk, dv, "bf16", seed=980)
    gam = [0.5, 0.9, 0.999]
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    par = lambda: R.parallel_fwd(qd, kd, vd, gam, groupnorm=R.GroupNorm(1e-5))
    rla = lambda: R.rla_fwd(qd, kd, vd, 40, 64)
    e_par = par().clone()
    e_rla = [t.clone() for t in rla()]
    torch.cuda.synchronize()
    gp, o_par = capture(par)
    gr, o_rla = capture(rla)
    noise = [t.to(DEV) for t in I.make_qkv(1, 2, 300, 64, 64, "bf16", seed=981)]
    for r in range(REPLAYS):
        o_par.zero_()
        for t in o_rla:
            t.zero_()
        torch.cuda.synchronize()
        gp.replay()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_par, e_par), f"replay {r}: parallel differs"
        assert all(torch.equal(a, b) for a, b in zip(o_rla, e_rla)), f"replay {r}: residual linear attention differs"
        eager_noise(noise)
    assert rel_err(o_par, orc.groupnorm(orc.parallel(q, k, v, gam), 1e-5)) <= 2e-2


def test_graph_rotated_chunkwise(orc):
    """The rotated bf16 chunkwise forward with GroupNorm and a state: the scores kernel that turns q
    and k and writes their high and low parts, the two chunk passes adding into one fp32 buffer, the
    state sum and the GroupNorm pass, as one graph (16 heads: the (b, h, slice) chunk kernels)."""
    B, H, N, dk, dv = 1, 16, 1000, 256, 512
    q, k, v = I.make_qkv(B, H, N, dk, dv, "bf16", seed=990)
    s0 = I.make_state(B, H, dk, dv, seed=991, scale=0.02)
    gam = I.multiscale_gammas(16)
    rot = R.Rotation(10000.0, 321)
    gn = R.GroupNorm(1e-5)
    qd, kd, vd, s0d = (t.to(DEV) for t in (q, k, v, s0))
    call = lambda: R.chunkwise_fwd(qd, kd, vd, gam, 128, state_in=s0d, groupnorm=gn, rotation=rot, out_dtype=torch.bfloat16)
    eager = [t.clone() for t in call()]
    torch.cuda.synchronize()
    g, got = capture(call)
    noise = [t.to(DEV) for t in I.make_qkv(1, 2, 300, 64, 64, "bf16", seed=992)]
    for r in range(REPLAYS):
        for t in got:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "state"), got, eager):
            assert torch.equal(a, b), f"replay {r}: {name} differs from the eager call"
        eager_noise(noise)
    ro, rs = orc.recurrent_rot(q, k, v, gam, 10000.0, 321, state_in=s0)
    assert rel_err(got[0], orc.groupnorm(ro, 1e-5)) <= 2e-2
    assert rel_err(got[1], rs) <= 2e-2
