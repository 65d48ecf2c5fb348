"""GPU parity of the single-step (decode) kernel, m2rnn_decode_step, against the fp64 oracle.

One decode step is the recurrence over one step started from the given state (M²RNN notes §2.1,
Eq. 10-12), so the oracle's forward with T = 1 and H0 = the state is its reference.  Budget:
max-abs <= 5e-4 on y and on the new state (fp32 state, split-fp16 contraction).
"""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import TOL, max_abs, oracle_fwd, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu
TOL_DEC = TOL["f16x3"]


def gpu_decode(dd, H=None, H_out=None):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    y, Hn = m2.m2rnn_decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(), dd["v"][:, 0].contiguous(),
                                 dd["f"][:, 0].contiguous(), dd["W"], dd["w_r"], H, H_out=H_out)
    torch.cuda.synchronize()
    return y, Hn


@pytest.mark.parametrize("B,N,K,V,dtype,with_H", [
    (3, 2, 16, 16, "f32", True),
    (5, 3, 48, 32, "bf16", True),
    (6, 2, 64, 64, "bf16", False),
    (9, 2, 64, 64, "f32", True),      # a batch that is not a multiple of the four entries per workgroup
    (4, 2, 128, 128, "f32", True),
    (2, 3, 32, 128, "bf16", True),
    (1, 1, 160, 16, "bf16", True),
])
def test_decode_matches_oracle(B, N, K, V, dtype, with_H):
    torch_cuda()
    d = inputs.make_inputs(B, 1, N, K, V, qkv_dtype=dtype, seed=900 + K + V + B, with_H0=with_H)
    say("decode", B, N, K, V, dtype, with_H)
    dd = to_device(d, dtype)
    y, Hn = gpu_decode(dd, dd["H0"])
    yr, Hr = oracle_fwd(d)
    ey = max_abs(y.cpu().numpy(), yr[:, 0])
    eh = max_abs(Hn.cpu().numpy(), Hr)
    say("errors", ey, eh)
    assert ey <= TOL_DEC and eh <= TOL_DEC, (ey, eh)


def test_decode_in_place_equals_out_of_place():
    torch = torch_cuda()
    d = inputs.make_inputs(6, 1, 4, 64, 64, qkv_dtype="bf16", seed=77, with_H0=True)
    say("decode in place")
    dd = to_device(d, "bf16")
    y1, H1 = gpu_decode(dd, dd["H0"])
    H = dd["H0"].clone()
    y2, H2 = gpu_decode(dd, H, H_out=H)
    assert H2.data_ptr() == H.data_ptr()
    assert torch.equal(y1, y2) and torch.equal(H1, H2)


def test_decode_chain_matches_oracle_over_many_steps():
    # T decode steps, each feeding the state to the next, against the oracle's T-step forward.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    B, T, N, K, V = 3, 40, 2, 64, 32
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="bf16", seed=4711, with_H0=True)
    say("decode chain", B, T, N, K, V)
    dd = to_device(d, "bf16")
    H = dd["H0"].clone()
    ys = []
    for t in range(T):
        y, _ = m2.m2rnn_decode_step(dd["q"][:, t].contiguous(), dd["k"][:, t].contiguous(),
                                    dd["v"][:, t].contiguous(), dd["f"][:, t].contiguous(), dd["W"], dd["w_r"], H,
                                    H_out=H)
        ys.append(y.clone())
    torch.cuda.synchronize()
    y = torch.stack(ys, dim=1).cpu().numpy()
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y, yr), max_abs(H.cpu().numpy(), Hr)
    say("errors", ey, eh)
    assert ey <= TOL_DEC and eh <= TOL_DEC, (ey, eh)


def test_decode_workload_full():
    # The batch-128 decode step exactly as the benchmark launches it, every unit checked.
    torch_cuda()
    w = inputs.WORKLOADS["decode_b128_h32_kv64"]
    d = inputs.workload_inputs(w.name)
    say(w.name)
    dd = to_device(d, w.qkv_dtype)
    y, Hn = gpu_decode(dd, dd["H0"])
    Hn = Hn.cpu().numpy()
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y.cpu().numpy(), yr[:, 0]), max_abs(Hn, Hr)
    say("errors", ey, eh)
    assert ey <= TOL_DEC and eh <= TOL_DEC, (ey, eh)
    assert np.all(np.abs(Hn) <= 1.0 + 1e-6)


def test_decode_f_one_holds_state_exactly():
    # f = 1 keeps the state bit for bit (the blend is fma(-0, r, fma(1, H, 0))).
    torch = torch_cuda()
    d = inputs.make_inputs(4, 1, 3, 32, 64, qkv_dtype="bf16", seed=5, with_H0=True)
    d["f"][:] = 1.0
    say("decode f == 1")
    dd = to_device(d, "bf16")
    _, Hn = gpu_decode(dd, dd["H0"])
    assert torch.equal(Hn, dd["H0"])
