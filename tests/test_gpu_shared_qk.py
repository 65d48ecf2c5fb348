"""GPU parity with one query/key shared by all value heads (the notes' multi-value layout §2.4,
N_q = N_k = 1) and the pages' head shape K = 64, V = 16: forward, backward (dq, dk summed over
the heads, §2.7) and the decode step, against the fp64 oracle with q, k broadcast to every head."""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import TOL, gpu_bwd, gpu_fwd, max_abs, oracle_bwd, oracle_fwd, oracle_units, rel_l2, say, to_device, \
    torch_cuda

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,T,N,K,V,dtype,math", [
    (2, 100, 8, 64, 16, "bf16", "f16x3"),   # the pages' head shape
    (1, 37, 3, 32, 64, "f32", "f16x3"),
    (2, 50, 4, 64, 16, "bf16", "f32"),
    (1, 20, 2, 16, 128, "bf16", "bf16"),
])
def test_forward_shared_qk(B, T, N, K, V, dtype, math):
    torch_cuda()
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=2000 + T + V, with_H0=True, shared_qk=True)
    say("fwd shared qk", B, T, N, K, V, dtype, math)
    y, H = gpu_fwd(to_device(d, dtype), math)
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y, yr), max_abs(H, Hr)
    say("errors", ey, eh)
    assert ey <= TOL[math] and eh <= TOL[math], (ey, eh)


@pytest.mark.parametrize("B,T,N,K,V,dtype", [
    (2, 70, 4, 64, 16, "bf16"),
    (1, 130, 3, 32, 32, "f32"),
    (1, 64, 1, 16, 64, "f32"),     # one head: the shared gradient is the per-head one
])
def test_backward_shared_qk(B, T, N, K, V, dtype):
    torch_cuda()
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=3000 + T + V, with_H0=True, with_dy=True,
                           with_dHT=True, shared_qk=True)
    say("bwd shared qk", B, T, N, K, V, dtype)
    got = gpu_bwd(to_device(d, dtype))
    ref = oracle_bwd(d)
    assert got["dq"].shape == (B, T, 1, K) and got["dk"].shape == (B, T, 1, K)
    errs = {n: rel_l2(got[n], ref[n]) for n in ("dq", "dk", "dv", "df", "dW", "dw_r", "dH0")}
    say("rel-L2", errs)
    for n, e in errs.items():
        assert e <= 1e-3, (n, e)


def test_decode_shared_qk():
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    B, N, K, V = 6, 8, 64, 16
    d = inputs.make_inputs(B, 1, N, K, V, qkv_dtype="bf16", seed=4040, with_H0=True, shared_qk=True)
    say("decode shared qk", B, N, K, V)
    dd = to_device(d, "bf16")
    y, Hn = m2.m2rnn_decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(), dd["v"][:, 0].contiguous(),
                                 dd["f"][:, 0].contiguous(), dd["W"], dd["w_r"], dd["H0"])
    torch.cuda.synchronize()
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y.cpu().numpy(), yr[:, 0]), max_abs(Hn.cpu().numpy(), Hr)
    say("errors", ey, eh)
    assert ey <= TOL["f16x3"] and eh <= TOL["f16x3"], (ey, eh)


def test_paper_shape_workload_sampled_units():
    # B4 N128 T4096 K=64 V=16 with a shared query/key, launched as the benchmark launches it;
    # the oracle recomputes sampled (batch, head) units.
    torch_cuda()
    name = "paper_b4_h128_t4096_k64_v16"
    w = inputs.WORKLOADS[name]
    d = inputs.workload_inputs(name)
    units = [(0, 0), (3, 127), (1, 64), (2, 5)]
    say(name, units)
    y, H = gpu_fwd(to_device(d, w.qkv_dtype), "f16x3")
    assert np.all(np.abs(H) <= 1.0 + 1e-6)
    for (b, n), (yr, Hr) in oracle_units(d, units).items():
        ey, eh = max_abs(y[b, :, n], yr), max_abs(H[b, n], Hr)
        say((b, n), ey, eh)
        assert ey <= TOL["f16x3"] and eh <= TOL["f16x3"], ((b, n), ey, eh)
