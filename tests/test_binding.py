"""The Python binding checks every caller-supplied tensor before a pointer reaches the C ABI (which
cannot see buffer sizes): shape, dtype, contiguity and device. These run on the CPU: the shape and
dtype checks come first, and a correctly shaped CPU tensor is rejected as not being on the GPU."""
import pytest
import torch

from linear_recurrent_sequence_chunkwise_amd import retention as R

B, H, N, DK, DV = 2, 3, 10, 8, 16
BF = torch.bfloat16
F32 = torch.float32


def qkv(dtype=BF, n=N):
    return (torch.zeros(B, H, n, DK, dtype=dtype), torch.zeros(B, H, n, DK, dtype=dtype),
            torch.zeros(B, H, n, DV, dtype=dtype))


def expect(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


G = [0.9] * H


def test_chunkwise_mismatched_inputs():
    q, k, v = qkv()
    expect("k has shape", R.chunkwise_fwd, q, k[:, :, :5], v, G, 64)
    expect("v has shape", R.chunkwise_fwd, q, k, v[:1], G, 64)
    expect("k has shape", R.chunkwise_fwd, q, torch.zeros(B, H, N, DK + 1, dtype=BF), v, G, 64)
    expect("k has dtype", R.chunkwise_fwd, q, k.float(), v, G, 64)
    expect("q has dtype", R.chunkwise_fwd, q.half(), k.half(), v.half(), G, 64)
    expect("4 dimensions", R.chunkwise_fwd, q[0], k, v, G, 64)


def test_chunkwise_caller_buffers():
    q, k, v = qkv()
    expect("out has shape", R.chunkwise_fwd, q, k, v, G, 64, out=torch.zeros(B, H, N, DV - 1))
    expect("out has dtype", R.chunkwise_fwd, q, k, v, G, 64, out=torch.zeros(B, H, N, DV, dtype=torch.float16))
    expect("state_in has shape", R.chunkwise_fwd, q, k, v, G, 64, state_in=torch.zeros(B, H, DK, DV + 4))
    expect("state_in has dtype", R.chunkwise_fwd, q, k, v, G, 64, state_in=torch.zeros(B, H, DK, DV, dtype=BF))
    expect("state_out has shape", R.chunkwise_fwd, q, k, v, G, 64, state_out=torch.zeros(B, H, DV, DK))
    st = torch.zeros(B, H, DV, DK).transpose(-1, -2)  # right shape, not contiguous
    expect("state_in must be contiguous", R.chunkwise_fwd, q, k, v, G, 64, state_in=st)
    expect("groupnorm weight has shape", R.chunkwise_fwd, q, k, v, G, 64, groupnorm=R.GroupNorm(1e-5, weight=torch.ones(H * DV)))
    expect("groupnorm bias has dtype", R.chunkwise_fwd, q, k, v, G, 64,
           groupnorm=R.GroupNorm(1e-5, bias=torch.zeros(H, DV, dtype=BF)))
    expect("gate has shape", R.chunkwise_fwd, q, k, v, G, 64, groupnorm=R.GroupNorm(1e-5, gate=torch.zeros(B, H, N, DK, dtype=BF)))
    expect("gate has dtype", R.chunkwise_fwd, q, k, v, G, 64, groupnorm=R.GroupNorm(1e-5, gate=torch.zeros(B, H, N, DV)))


def test_cpu_tensors_rejected():
    q, k, v = qkv()
    expect("must be a device tensor", R.chunkwise_fwd, q, k, v, G, 64)
    expect("must be a device tensor", R.parallel_fwd, q, k, v, G)
    expect("must be a device tensor", R.chunkwise_bwd, q, k, v, G, torch.zeros(B, H, N, DV, dtype=BF), 64)


def test_recurrent_step_shapes():
    q, k, v = (t[:, :, 0] for t in qkv())
    st = torch.zeros(B, H, DK, DV)
    expect("state has shape", R.recurrent_step, q, k, v, G, torch.zeros(B, H, DK, DV - 1))
    expect("state has dtype", R.recurrent_step, q, k, v, G, st.double())
    expect("out has shape", R.recurrent_step, q, k, v, G, st, out=torch.zeros(B, H, DK))
    expect("k has shape", R.recurrent_step, q, k[:1], v, G, st)
    expect("3 dimensions", R.recurrent_step, q[:, :, None], k, v, G, st)


def test_parallel_and_backward_shapes():
    q, k, v = qkv()
    expect("out has shape", R.parallel_fwd, q, k, v, G, out=torch.zeros(B, H, N + 1, DV))
    expect("dout has shape", R.chunkwise_bwd, q, k, v, G, torch.zeros(B, H, N, DK, dtype=BF), 64)
    expect("dout has dtype", R.chunkwise_bwd, q, k, v, G, torch.zeros(B, H, N, DV), 64)
    expect("state_in has shape", R.chunkwise_bwd, q, k, v, G, torch.zeros(B, H, N, DV, dtype=BF), 64,
           state_in=torch.zeros(B, H, DK, DK))


def test_rla_shapes():
    q, k, v = qkv()
    w = 4
    expect("k_prev has shape", R.rla_fwd, q, k, v, w, 64, k_prev=torch.zeros(B, H, w, DK, dtype=BF),
           v_prev=torch.zeros(B, H, w + 1, DV, dtype=BF))
    expect("v_prev has dtype", R.rla_fwd, q, k, v, w, 64, k_prev=torch.zeros(B, H, w + 1, DK, dtype=BF),
           v_prev=torch.zeros(B, H, w + 1, DV))
    expect("needs k_prev", R.rla_fwd, q, k, v, w, 64, prev_len=2)
    expect("window must be", R.rla_fwd, q, k, v, -1, 64)
    expect("fmap must be", R.rla_fwd, q, k, v, w, 64, fmap="relu")
    expect("state_out has shape", R.rla_fwd, q, k, v, w, 64, state_out=torch.zeros(B, H, DK, DK))


def test_workspace_must_be_device_tensor():
    with pytest.raises(ValueError, match="workspace must be"):
        R._workspace(100, "cpu", torch.zeros(200, dtype=torch.uint8))
