"""retention_chunkwise_fwd_noalloc on the GPU: the library's fixed scratch array in place of a caller
workspace. Two calls in a row, the second smaller, each bitwise equal to retention_chunkwise_fwd with
a workspace (same kernels, same inputs) and within the bf16 bound of the oracle. Runs alone or after
every other test: whatever the array holds from earlier calls must not matter."""
import numpy as np
import pytest
import torch

from linear_recurrent_sequence_chunkwise_amd import inputs as I
from linear_recurrent_sequence_chunkwise_amd import retention as R

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    R.load_library()


def rel_err(gpu, ref):
    g = gpu.double().cpu().numpy()
    return float(np.max(np.abs(g - ref)) / np.sqrt(np.mean(ref * ref)))


# (B, H, N, d_k, d_v, chunk, GroupNorm): the first needs several MiB of scratch (scores and pre-norm
# rows), the second far less at another layout of the array
CASES = [(1, 4, 1100, 256, 512, 128, True), (2, 3, 300, 64, 64, 64, False)]


def test_noalloc_two_calls_match_workspace_call(orc):
    dev = torch.device("cuda:0")
    for i, (B, H, N, dk, dv, C, use_gn) in enumerate(CASES):
        print(f"noalloc case {i}: B={B} H={H} N={N} dk={dk} dv={dv} C={C} gn={use_gn}", flush=True)
        q, k, v = I.make_qkv(B, H, N, dk, dv, "bf16", seed=900 + i)
        gam = I.multiscale_gammas(16)[:H]
        s0 = I.make_state(B, H, dk, dv, seed=910 + i, scale=0.05)
        qd, kd, vd, s0d = (t.to(dev) for t in (q, k, v, s0))
        gn = R.GroupNorm(1e-5) if use_gn else None
        odt = torch.bfloat16 if use_gn else torch.float32
        need = R.workspace_bytes(R.RET_FN_CHUNKWISE, B, H, N, dk, dv, torch.bfloat16, odt, C, use_gn)
        assert 0 < need <= R.NOALLOC_SCRATCH_BYTES
        o_ws, s_ws = R.chunkwise_fwd(qd, kd, vd, gam, C, state_in=s0d, groupnorm=gn, out_dtype=odt)
        out = torch.full((B, H, N, dv), float("nan"), dtype=odt, device=dev)
        st = torch.full((B, H, dk, dv), float("nan"), dtype=torch.float32, device=dev)
        o_na, s_na = R.chunkwise_fwd_noalloc(qd, kd, vd, gam, C, state_in=s0d, groupnorm=gn, out=out, state_out=st)
        torch.cuda.synchronize()
        assert torch.equal(o_na, o_ws) and torch.equal(s_na, s_ws), f"case {i}: differs from the workspace call"
        ref, ref_s = orc.recurrent(q, k, v, gam, state_in=s0)
        if use_gn:
            ref = orc.groupnorm(ref, 1e-5)
        e_o, e_s = rel_err(o_na, ref), rel_err(s_na, ref_s)
        print(f"  noalloc vs oracle: out {e_o:.3e}, state {e_s:.3e} (bound 2e-2)", flush=True)
        assert e_o <= 2e-2 and e_s <= 2e-2
