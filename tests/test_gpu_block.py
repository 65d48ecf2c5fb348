"""GPU parity of the steps on either side of the recurrence (M²RNN notes §2.2, §2.3, Appendix C)
against the fp64 oracle (oracle/block.py): the gate, the output gate + RMSNorm and the causal
conv4 + SiLU, forward and backward.

Budgets: these are fp32 streams, so outputs match to a few fp32 ulps (rtol 1e-5); a bf16 output
adds its own rounding (2^-8 relative); sums over batch and time (dalpha, dbeta, dgamma, dw, dbias)
are checked by relative L2 error <= 1e-5."""
import numpy as np
import pytest

from oracle import block

from _gpu import rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu


def rng(seed):
    return np.random.default_rng(seed)


def bf16_round(a):
    from matrix_state_nonlinear_m2rnn_amd import inputs
    return inputs.round_to_bf16(np.asarray(a, dtype=np.float32)).astype(np.float64)


def dev(a, dtype="f32"):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(torch.bfloat16).contiguous() if dtype == "bf16" else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def close(got, ref, rtol=1e-5, atol=1e-6):
    err = np.max(np.abs(got - ref) / (atol + rtol * np.abs(ref))) if np.size(ref) else 0.0
    return err <= 1.0, err


@pytest.mark.parametrize("B,T,N", [(2, 37, 5), (4, 2048, 16), (1, 1, 1)])
def test_gate_forward_and_backward(B, T, N):
    import matrix_state_nonlinear_m2rnn_amd as m2
    r = rng(B * T + N)
    a = r.normal(0, 2, (B, T, N)).astype(np.float32)
    alpha = r.uniform(0.1, 4, N).astype(np.float32)
    beta = r.normal(0, 1, N).astype(np.float32)
    df = r.normal(0, 1, (B, T, N)).astype(np.float32)
    say("gate", B, T, N)
    f = host(m2.m2rnn_gate_fwd(dev(a), dev(alpha), dev(beta)))
    ok, err = close(f, block.gate_fwd(a, alpha, beta))
    assert ok, err
    g = m2.m2rnn_gate_bwd(dev(a), dev(alpha), dev(beta), dev(df))
    ref = block.gate_bwd(a, alpha, beta, df)
    ok, err = close(host(g["da"]), ref["da"])
    assert ok, ("da", err)
    for n in ("dalpha", "dbeta"):
        e = rel_l2(host(g[n]), ref[n])
        say(n, e)
        assert e <= 1e-5, (n, e)


# D = N V features per row: 48, 1024, 512 and 2048 take the narrow register layouts; 2304 (a ragged
# last group) and 8192 (the widest row the library takes) the wide ones.
@pytest.mark.parametrize("B,T,N,V,gz_dtype", [(2, 9, 3, 16, "f32"), (4, 2048, 16, 64, "bf16"), (1, 130, 4, 128, "f32"),
                                              (2, 5, 128, 16, "bf16"), (2, 4, 36, 64, "f32"), (1, 3, 64, 128, "bf16")])
def test_out_norm_forward_and_backward(B, T, N, V, gz_dtype):
    import matrix_state_nonlinear_m2rnn_amd as m2
    r = rng(N * V + T)
    y = r.normal(0, 1, (B, T, N, V)).astype(np.float32)
    gz = r.normal(0, 2, (B, T, N, V)).astype(np.float32)
    if gz_dtype == "bf16":
        gz = bf16_round(gz)
    gamma = r.normal(1, 0.2, (N, V)).astype(np.float32)
    dout = r.normal(0, 1, (B, T, N, V)).astype(np.float32)
    eps = 1e-6
    say("out_norm", B, T, N, V, gz_dtype)
    out = host(m2.m2rnn_out_norm_fwd(dev(y), dev(gz, gz_dtype), dev(gamma), eps))
    ok, err = close(out, block.out_norm_fwd(y, gz, gamma, eps))
    assert ok, err
    g = m2.m2rnn_out_norm_bwd(dev(y), dev(gz, gz_dtype), dev(gamma), dev(dout), eps)
    ref = block.out_norm_bwd(y, gz, gamma, eps, dout)
    for n in ("dy", "dgz"):
        got = host(g[n])
        ok, err = close(got, ref[n], rtol=1e-4, atol=1e-5 * float(np.max(np.abs(ref[n]))))
        assert ok, (n, err)
    e = rel_l2(host(g["dgamma"]), ref["dgamma"])
    say("dgamma", e)
    assert e <= 1e-5, e


# Ragged cases: C = 12 fills part of a wave; C = 328 spans two waves per row, the second partly;
# T = 70, 129 and 300 end inside a chunk of the forward (64 steps) and of the backward (128 steps).
@pytest.mark.parametrize("B,T,C,dtype,with_bias", [(2, 70, 12, "f32", True), (4, 2048, 1024, "bf16", True),
                                                   (1, 3, 4, "f32", False), (3, 129, 64, "bf16", False),
                                                   (2, 300, 328, "bf16", True)])
def test_conv4_silu_forward_and_backward(B, T, C, dtype, with_bias):
    import matrix_state_nonlinear_m2rnn_amd as m2
    r = rng(T + C)
    x = r.normal(0, 1, (B, T, C)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_round(x)
    w = r.normal(0, 0.5, (C, 4)).astype(np.float32)
    bias = r.normal(0, 0.2, C).astype(np.float32) if with_bias else None
    du = r.normal(0, 1, (B, T, C)).astype(np.float32)
    say("conv4_silu", B, T, C, dtype, with_bias)
    u = host(m2.m2rnn_conv4_silu_fwd(dev(x, dtype), dev(w), dev(bias) if with_bias else None))
    uref = block.conv4_silu_fwd(x, w, bias)
    if dtype == "bf16":
        ok, err = close(u, uref, rtol=2.0 ** -8, atol=1e-6)
    else:
        ok, err = close(u, uref)
    assert ok, err
    g = m2.m2rnn_conv4_silu_bwd(dev(x, dtype), dev(w), dev(bias) if with_bias else None, dev(du))
    ref = block.conv4_silu_bwd(x, w, bias, du)
    ok, err = close(host(g["dx"]), ref["dx"], rtol=1e-5, atol=1e-6)
    assert ok, ("dx", err)
    names = ("dw", "dbias") if with_bias else ("dw",)
    for n in names:
        e = rel_l2(host(g[n]), ref[n])
        say(n, e)
        assert e <= 1e-5, (n, e)
    if not with_bias:
        assert g["dbias"] is None


def test_block_ops_are_deterministic():
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    r = rng(11)
    y, gz, dout = (dev(r.normal(0, 1, (3, 100, 8, 32))) for _ in range(3))
    gamma = dev(r.normal(1, 0.1, (8, 32)))
    g1 = m2.m2rnn_out_norm_bwd(y, gz, gamma, dout)
    g2 = m2.m2rnn_out_norm_bwd(y, gz, gamma, dout)
    for n in g1:
        assert torch.equal(g1[n], g2[n]), n
