"""GPU parity of the training pair: m2rnn_fwd_ckpt (the forward keeping the state that enters every
64-step segment) and m2rnn_bwd_ckpt (the backward from those checkpoints, without re-running the
recurrence), against the fp64 oracle and against m2rnn_fwd / m2rnn_bwd."""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import TOL, max_abs, oracle_bwd, oracle_fwd, rel_l2, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu
GRADS = ("dq", "dk", "dv", "df", "dW", "dw_r", "dH0")


def fwd_ckpt(dd, math="auto"):
    import matrix_state_nonlinear_m2rnn_amd as m2
    return m2.m2rnn_fwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd.get("H0"), math=math)


@pytest.mark.parametrize("B,T,N,K,V,dtype,shared", [
    (2, 200, 3, 32, 64, "bf16", False),   # four segments, the last one ragged
    (1, 64, 2, 64, 16, "f32", True),      # exactly one segment, shared q/k
    (2, 129, 2, 16, 128, "bf16", False),
])
def test_forward_checkpoints(B, T, N, K, V, dtype, shared):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=700 + T, with_H0=True, shared_qk=shared)
    say("fwd ckpt", B, T, N, K, V, dtype, shared)
    dd = to_device(d, dtype)
    y, H_T, ck = fwd_ckpt(dd)
    y0, H0T = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"])
    torch.cuda.synchronize()
    # Keeping checkpoints changes nothing else.
    assert torch.equal(y, y0) and torch.equal(H_T, H0T)
    ck = ck.cpu().numpy()
    I = m2.m2rnn_checkpoint_interval(m2.Dims(B, T, N, K, V))
    assert ck.shape == (B, N, (T + I - 1) // I, K, V)
    assert np.array_equal(ck[:, :, 0], d["H0"])
    for s in range(1, ck.shape[2]):
        sub = {x: (a[:, :I * s] if x in ("q", "k", "v", "f") else a) for x, a in d.items() if a is not None}
        _, Hs = oracle_fwd(sub)
        e = max_abs(ck[:, :, s], Hs)
        say("segment", s, e)
        assert e <= TOL["bf16x3"], (s, e)


@pytest.mark.parametrize("B,T,N,K,V,dtype,shared", [
    (2, 130, 3, 32, 64, "bf16", False),
    (1, 70, 4, 64, 16, "bf16", True),
    (1, 65, 1, 16, 128, "f32", False),
])
def test_backward_from_checkpoints(B, T, N, K, V, dtype, shared):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=800 + T, with_H0=True, with_dy=True, with_dHT=True,
                           shared_qk=shared)
    say("bwd ckpt", B, T, N, K, V, dtype, shared)
    dd = to_device(d, dtype)
    # The same checkpoints as the backward's own pass (the forwards' default contraction for AUTO,
    # F16X3 when asked for): the same gradients, bit for bit.
    for math in ("auto", "f16x3"):
        _, _, ck = fwd_ckpt(dd, math)
        g = m2.m2rnn_bwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], ck, dd["dy"], dd["dH_T"],
                              math=math)
        g0 = m2.m2rnn_bwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"], dd["dy"], dd["dH_T"],
                          math=math)
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(g[n], g0[n]), (math, n)
    ref = oracle_bwd(d)
    errs = {n: rel_l2(g[n].cpu().numpy(), ref[n]) for n in GRADS}
    say("rel-L2", errs)
    for n, e in errs.items():
        assert e <= 1e-3, (n, e)


def test_clipped_backward_from_checkpoints():
    # The clipping option reaches the checkpoint form of the backward too.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(1, 70, 4, 64, 16, qkv_dtype="bf16", seed=870, with_H0=True, with_dy=True, with_dHT=True,
                           shared_qk=True)
    dd = to_device(d, "bf16")
    _, _, ck = fwd_ckpt(dd)
    g = m2.m2rnn_bwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], ck, dd["dy"], dd["dH_T"],
                          grad_clip=0.4)
    g0 = m2.m2rnn_bwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"], dd["dy"], dd["dH_T"],
                      grad_clip=0.4)
    torch.cuda.synchronize()
    for n in GRADS:
        assert torch.equal(g[n], g0[n]), n
    ref = oracle_bwd(d, clip=0.4)
    errs = {n: rel_l2(g[n].cpu().numpy(), ref[n]) for n in GRADS}
    say("rel-L2", errs)
    for n, e in errs.items():
        assert e <= 1e-3, (n, e)


def test_backward_from_fp32_contraction_checkpoints():
    # Checkpoints from another contraction mode differ within that mode's error; the gradients
    # still meet the budget.
    torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(2, 150, 2, 64, 64, qkv_dtype="bf16", seed=99, with_dy=True)
    dd = to_device(d, "bf16")
    _, _, ck = fwd_ckpt(dd, "f32")
    g = m2.m2rnn_bwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], ck, dd["dy"])
    ref = oracle_bwd(d)
    for n in GRADS:
        e = rel_l2(g[n].cpu().numpy(), ref[n])
        assert e <= 1e-3, (n, e)


def test_training_pair_on_the_bwd_workload():
    # B4 N16 T4096 K=V=64 fp32.  The checkpoint-keeping forward runs in time segments there (their
    # second passes on a side stream); its checkpoints are the single pass's bit for bit, so the pair
    # gives exactly m2rnn_bwd's gradients, and sampled heads meet the oracle.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.workload_inputs("bwd_b4_h16_t4096_kv64")
    say("bwd_b4_h16_t4096_kv64 training pair")
    dd = to_device(d, "f32")
    y, H_T, ck = fwd_ckpt(dd)
    y1, H1, ck1 = m2.m2rnn_fwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], None, overlap=None)
    g = m2.m2rnn_bwd_ckpt(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], ck, dd["dy"])
    g0 = m2.m2rnn_bwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], None, dd["dy"])
    torch.cuda.synchronize()
    assert torch.equal(y, y1) and torch.equal(H_T, H1) and torch.equal(ck, ck1)
    for n in GRADS:
        assert torch.equal(g[n], g0[n]), n
    got = {n: g[n].cpu().numpy().astype(np.float64) for n in GRADS}
    for n in (0, 15):
        sub = dict(q=d["q"][:, :, n:n + 1], k=d["k"][:, :, n:n + 1], v=d["v"][:, :, n:n + 1], f=d["f"][:, :, n:n + 1],
                   W=d["W"][n:n + 1], w_r=d["w_r"][n:n + 1], H0=None, dy=d["dy"][:, :, n:n + 1], dH_T=None)
        ref = oracle_bwd(sub)
        part = {"dq": got["dq"][:, :, n:n + 1], "dk": got["dk"][:, :, n:n + 1], "dv": got["dv"][:, :, n:n + 1],
                "df": got["df"][:, :, n:n + 1], "dW": got["dW"][n:n + 1], "dw_r": got["dw_r"][n:n + 1],
                "dH0": got["dH0"][:, n:n + 1]}
        errs = {x: rel_l2(part[x], ref[x]) for x in GRADS}
        say("head", n, errs)
        for x, e in errs.items():
            assert e <= 1e-3, (n, x, e)


def test_scan_and_finish_equal_the_checkpoint_backward():
    # m2rnn_scan_bwd then m2rnn_scan_bwd_finish on one stream and workspace is m2rnn_bwd_ckpt, bit for
    # bit (split rows and a shared q/k, whose partials go through the workspace).
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    for B, T, N, K, V, shared in ((2, 130, 3, 32, 64, False), (1, 70, 4, 64, 16, True)):
        d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="bf16", seed=880 + T, with_H0=True, with_dy=True,
                               with_dHT=True, shared_qk=shared)
        dd = to_device(d, "bf16")
        say("scan + finish", B, T, N, K, V, shared)
        _, _, ck = fwd_ckpt(dd, "f16x3")
        args = (dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], ck, dd["dy"], dd["dH_T"])
        g0 = m2.m2rnn_bwd_ckpt(*args)
        dims = m2.Dims(B, T, N, K, V, 1 if shared else N)
        ws = torch.empty(m2.m2rnn_bwd_ckpt_workspace_size(dims, m2.DTYPE_BF16), dtype=torch.uint8, device="cuda")
        g = m2.m2rnn_scan_bwd(*args, workspace=ws)
        m2.m2rnn_scan_bwd_finish(*args, workspace=ws, out=g)
        torch.cuda.synchronize()
        for n in GRADS:
            assert torch.equal(g[n], g0[n]), n
