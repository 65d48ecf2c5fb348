"""GPU parity of the backward (BPTT, checkpoints every 64 steps) against the oracle's manual
backward: relative L2 error <= 1e-3 per gradient tensor."""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import gpu_bwd, oracle_bwd, rel_l2, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "df", "dW", "dw_r", "dH0")
TOL = 1e-3


def check(got, ref, names=GRADS):
    errs = {n: rel_l2(got[n], ref[n]) for n in names}
    say("rel-L2", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= TOL, (n, e)


@pytest.mark.parametrize("B,T,N,K,V,dtype", [
    (1, 70, 2, 16, 16, "f32"),     # tiny, ragged second segment
    (2, 130, 3, 32, 64, "bf16"),   # three segments, two row blocks per state
    (1, 64, 2, 48, 32, "f32"),     # exactly one segment, three row blocks
    (1, 65, 1, 16, 128, "bf16"),   # largest V, one step into the second segment
    (2, 1, 2, 16, 64, "f32"),      # a single step
])
def test_small_shapes_with_H0_and_dHT(B, T, N, K, V, dtype):
    torch_cuda()
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=500 + T + K + V, with_H0=True, with_dy=True,
                           with_dHT=True)
    say("bwd", B, T, N, K, V, dtype)
    got = gpu_bwd(to_device(d, dtype))
    check(got, oracle_bwd(d))


def test_without_H0_and_dHT():
    torch_cuda()
    d = inputs.make_inputs(2, 100, 2, 64, 64, qkv_dtype="bf16", seed=17, with_dy=True)
    got = gpu_bwd(to_device(d, "bf16"))
    check(got, oracle_bwd(d))


def test_bwd_workload_sampled_heads():
    # The full B4 N16 T4096 K=V=64 fp32 workload on the GPU; the oracle recomputes every batch
    # entry of two heads (dW and dw_r sum over the batch).
    torch_cuda()
    name = "bwd_b4_h16_t4096_kv64"
    w = inputs.WORKLOADS[name]
    d = inputs.workload_inputs(name)
    say(name)
    got = gpu_bwd(to_device(d, w.qkv_dtype))
    for n in (0, 15):
        sub = dict(q=d["q"][:, :, n:n + 1], k=d["k"][:, :, n:n + 1], v=d["v"][:, :, n:n + 1], f=d["f"][:, :, n:n + 1],
                   W=d["W"][n:n + 1], w_r=d["w_r"][n:n + 1], H0=None, dy=d["dy"][:, :, n:n + 1], dH_T=None)
        ref = oracle_bwd(sub)
        part = {"dq": got["dq"][:, :, n:n + 1], "dk": got["dk"][:, :, n:n + 1], "dv": got["dv"][:, :, n:n + 1],
                "df": got["df"][:, :, n:n + 1], "dW": got["dW"][n:n + 1], "dw_r": got["dw_r"][n:n + 1],
                "dH0": got["dH0"][:, n:n + 1]}
        say("head", n)
        check(part, ref)


def test_zero_steps():
    torch_cuda()
    d = inputs.make_inputs(2, 0, 2, 16, 32, qkv_dtype="f32", seed=3, with_H0=True, with_dy=True, with_dHT=True)
    got = gpu_bwd(to_device(d, "f32"))
    assert np.all(got["dW"] == 0.0) and np.all(got["dw_r"] == 0.0)
    assert np.array_equal(got["dH0"], d["dH_T"].astype(np.float64))


def test_deterministic():
    torch_cuda()
    d = inputs.make_inputs(2, 150, 2, 32, 64, qkv_dtype="bf16", seed=23, with_dy=True)
    dd = to_device(d, "bf16")
    a = gpu_bwd(dd)
    b = gpu_bwd(dd)
    for n in GRADS:
        assert np.array_equal(a[n], b[n]), n


@pytest.mark.parametrize("B,T,N,K,V,dtype,clip", [
    (1, 70, 2, 16, 16, "f32", 0.3),
    (2, 130, 2, 32, 64, "bf16", 0.6),
    (1, 65, 1, 16, 128, "bf16", 0.3),
])
def test_clipped_recurrent_gradient(B, T, N, K, V, dtype, clip):
    # Per-step clipping of the gradient sent back to each step's input state (elementwise bound);
    # the clamp is 1-Lipschitz, so the kernel's rounding cannot grow through it.
    torch_cuda()
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=700 + T + V, with_H0=True, with_dy=True,
                           with_dHT=True)
    say("bwd clip", B, T, N, K, V, dtype, clip)
    ref = oracle_bwd(d, clip=clip)
    exact = oracle_bwd(d)
    assert rel_l2(ref["dW"], exact["dW"]) > 10 * TOL  # the bound changes the result
    got = gpu_bwd(to_device(d, dtype), grad_clip=clip)
    check(got, ref)
    assert np.max(np.abs(got["dH0"])) <= np.float32(clip)  # the bound as the kernel holds it
