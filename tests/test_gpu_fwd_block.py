"""GPU parity of the fused block forward (m2rnn_fwd_block): the gate, the recurrence, and the output
gate + RMSNorm applied by the pass that sums the readouts (M²RNN notes §2.2, §2.3, Appendix C).

Two checks per case:
  * bit-identity with the unfused calls on the same device inputs (m2rnn_gate_fwd, m2rnn_fwd,
    m2rnn_out_norm_fwd), which takes the same operations in the same order;
  * the fp64 oracle's composition (oracle/block.py's gate and norm around oracle.ref_fwd), within
    the recurrence's budget of 5e-4 on y carried through the norm: |d out_j| <= |gamma_j SiLU(gz_j)|
    s |d y_j| plus the change of s, bounded here by twice the first term, s = 1 / rms(x) per token.
"""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs
from oracle import block

from _gpu import TOL, oracle_fwd, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu

EPS = 1e-6


def block_inputs(B, T, N, K, V, qkv_dtype, shared_qk=False, with_H0=False, seed=11):
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=qkv_dtype, shared_qk=shared_qk, with_H0=with_H0, seed=seed)
    r = np.random.default_rng(seed + 1000 * T + N)
    d["a"] = r.normal(0.0, 2.0, (B, T, N)).astype(np.float32)
    d["alpha"] = r.uniform(0.1, 3.0, N).astype(np.float32)
    d["beta"] = r.normal(0.0, 1.0, N).astype(np.float32)
    d["gz"] = r.normal(0.0, 2.0, (B, T, N, V)).astype(np.float32)
    d["gamma"] = (1.0 + 0.1 * r.normal(0.0, 1.0, (N, V))).astype(np.float32)
    return d


def run_both(d, qkv_dtype, gz_dtype, math, row_blocks=0):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    dd = to_device({x: d[x] for x in ("q", "k", "v", "W", "w_r", "H0", "a", "alpha", "beta", "gamma")}, qkv_dtype)
    gz = torch.from_numpy(d["gz"]).to("cuda")
    if gz_dtype == "bf16":
        gz = gz.to(torch.bfloat16).contiguous()
    out, H_T = m2.m2rnn_fwd_block(dd["q"], dd["k"], dd["v"], dd["a"], dd["alpha"], dd["beta"], dd["W"], dd["w_r"], gz,
                                  dd["gamma"], dd["H0"], eps=EPS, math=math, row_blocks=row_blocks)
    f = m2.m2rnn_gate_fwd(dd["a"], dd["alpha"], dd["beta"])
    y, H2 = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], f, dd["W"], dd["w_r"], dd["H0"], math=math,
                         row_blocks=row_blocks)
    ref = m2.m2rnn_out_norm_fwd(y, gz, dd["gamma"], EPS)
    torch.cuda.synchronize()
    return out, H_T, ref, H2, gz


def oracle_out(d, gz_host, budget):
    """The oracle's out and H_T, and the per-element tolerance that the budget on y gives out."""
    e = dict(d)
    e["f"] = block.gate_fwd(d["a"], d["alpha"], d["beta"])
    y, H = oracle_fwd(e)
    B, T, N, V = y.shape
    out = block.out_norm_fwd(y, gz_host, d["gamma"], EPS)
    x = (y * block.silu(gz_host)).reshape(B, T, N * V)
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)
    tol = 2.0 * budget * np.abs(d["gamma"].reshape(1, 1, N * V) * block.silu(gz_host.reshape(B, T, N * V))) * s
    return out, H, tol.reshape(B, T, N, V)


CASES = [
    # B, T, N, K, V, qkv dtype, gz dtype, math, row_blocks, shared q/k, H0
    (2, 70, 4, 64, 64, "bf16", "bf16", "f16x3", 0, False, False),    # rows split over workgroups (S > 1)
    (2, 70, 4, 64, 64, "bf16", "f32", "f16x3", 4, False, True),      # one workgroup per pair (S = 1), H0
    (1, 33, 3, 16, 16, "f32", "f32", "f32", 0, False, False),
    (2, 40, 8, 64, 16, "bf16", "bf16", "f16x3", 0, True, False),     # shared q/k, V = 16 (the pages' shape)
    (1, 21, 64, 16, 64, "bf16", "bf16", "f16x3", 0, False, False),   # N V = 4096 features: the wide epilogue
    (2, 17, 5, 128, 128, "bf16", "bf16", "f16x3", 0, False, False),  # K = V = 128
    (1, 4100, 8, 64, 64, "bf16", "bf16", "f16x3", 0, False, False),   # time segments (as m2rnn_fwd's)
]


@pytest.mark.parametrize("B,T,N,K,V,qkv,gzd,math,rb,shared,h0", CASES)
def test_fused_block_forward(B, T, N, K, V, qkv, gzd, math, rb, shared, h0):
    torch = torch_cuda()
    say("fwd_block", B, T, N, K, V, qkv, gzd, math, rb, shared, h0)
    d = block_inputs(B, T, N, K, V, qkv, shared_qk=shared, with_H0=h0)
    out, H_T, ref, H2, gz = run_both(d, qkv, gzd, math, rb)
    assert torch.equal(out, ref), float((out - ref).abs().max())
    assert torch.equal(H_T, H2)
    gz_host = gz.float().cpu().numpy().astype(np.float64)
    o_ref, H_ref, tol = oracle_out(d, gz_host, TOL[math])
    err = np.abs(out.cpu().numpy().astype(np.float64) - o_ref)
    worst = float(np.max(err / (tol + 1e-6)))
    say("oracle", float(err.max()), "worst/tol", worst)
    assert worst <= 1.0, worst
    assert float(np.max(np.abs(H_T.cpu().numpy() - H_ref))) <= TOL[math]


def test_fused_block_forward_without_steps():
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    say("fwd_block T=0")
    d = block_inputs(2, 0, 3, 16, 16, "f32", with_H0=True)
    dd = to_device({x: d[x] for x in ("q", "k", "v", "W", "w_r", "H0", "a", "alpha", "beta", "gamma")}, "f32")
    gz = torch.zeros((2, 0, 3, 16), dtype=torch.float32, device="cuda")
    out, H_T = m2.m2rnn_fwd_block(dd["q"], dd["k"], dd["v"], dd["a"], dd["alpha"], dd["beta"], dd["W"], dd["w_r"], gz,
                                  dd["gamma"], dd["H0"])
    torch.cuda.synchronize()
    assert out.shape == (2, 0, 3, 16)
    assert torch.equal(H_T, dd["H0"])
