"""One training step of the whole M²RNN layer, every piece on the GPU through the C ABI, against
the same composition of the fp64 oracle's pieces (M²RNN notes §2.2, §2.3, §2.7, Appendix C):

    q, k, v = conv4+SiLU of x_q, x_k, x_v          f = exp(-alpha softplus(a + beta))
    y, H_T  = M2RNN(q, k, v, f; W, w_r)             out = RMSNorm(y (.) SiLU(gz)) * gamma
    loss    = <dout, out>

and back: RMSNorm backward -> recurrence backward (from the forward's checkpoints) -> gate and
conv backward.  Each piece has its own parity tests; this one checks that they compose: the conv's
[B,T,C] channels are the scan's [B,T,N,K] heads, the gradients flow into the right slots, and the
errors stay in budget end to end.  Budgets: out within 5e-4 carried through the norm (as in
test_gpu_fwd_block.py); every gradient within relative L2 1e-3 (the backward's budget).
"""
import numpy as np
import pytest

import oracle
from oracle import block

from _gpu import rel_l2, say, torch_cuda

pytestmark = pytest.mark.gpu

EPS = 1e-6


def layer_inputs(B, T, N, K, V, seed):
    r = np.random.default_rng(seed)
    f32 = lambda a: np.asarray(a, dtype=np.float32)  # noqa: E731
    d = {
        "xq": f32(r.normal(0, 0.7, (B, T, N * K))), "xk": f32(r.normal(0, 0.7, (B, T, N * K))),
        "xv": f32(r.normal(0, 1.0, (B, T, N * V))),
        "wq": f32(r.normal(0, 0.5, (N * K, 4))), "wk": f32(r.normal(0, 0.5, (N * K, 4))),
        "wv": f32(r.normal(0, 0.5, (N * V, 4))),
        "bq": f32(r.normal(0, 0.1, N * K)), "bk": f32(r.normal(0, 0.1, N * K)), "bv": f32(r.normal(0, 0.1, N * V)),
        "a": f32(r.normal(0, 2.0, (B, T, N))), "alpha": f32(r.uniform(0.1, 3.0, N)), "beta": f32(r.normal(0, 1, N)),
        "w_r": f32(r.normal(0, 0.3, (N, V))),
        "gz": f32(r.normal(0, 2.0, (B, T, N, V))), "gamma": f32(1.0 + 0.1 * r.normal(0, 1, (N, V))),
        "dout": f32(r.normal(0, 1.0, (B, T, N, V))),
    }
    W = np.stack([np.linalg.qr(r.normal(0, 1, (V, V)))[0] for _ in range(N)]) * 0.9
    d["W"] = f32(W)
    return d


def oracle_layer(d, B, T, N, K, V):
    uq = block.conv4_silu_fwd(d["xq"], d["wq"], d["bq"]).reshape(B, T, N, K)
    uk = block.conv4_silu_fwd(d["xk"], d["wk"], d["bk"]).reshape(B, T, N, K)
    uv = block.conv4_silu_fwd(d["xv"], d["wv"], d["bv"]).reshape(B, T, N, V)
    f = block.gate_fwd(d["a"], d["alpha"], d["beta"])
    y, _ = oracle.ref_fwd(uq, uk, uv, f, d["W"], d["w_r"], None)
    out = block.out_norm_fwd(y, d["gz"], d["gamma"], EPS)
    gn = block.out_norm_bwd(y, d["gz"], d["gamma"], EPS, d["dout"])
    gs = oracle.ref_bwd(uq, uk, uv, f, d["W"], d["w_r"], None, gn["dy"])
    gg = block.gate_bwd(d["a"], d["alpha"], d["beta"], gs["df"])
    g = {"out": out, "y": y, "dgz": gn["dgz"], "dgamma": gn["dgamma"], "dW": gs["dW"], "dw_r": gs["dw_r"],
         "da": gg["da"], "dalpha": gg["dalpha"], "dbeta": gg["dbeta"]}
    for x, du in (("q", gs["dq"]), ("k", gs["dk"]), ("v", gs["dv"])):
        c = block.conv4_silu_bwd(d["x" + x], d["w" + x], d["b" + x], du.reshape(B, T, -1))
        g["dx" + x], g["dw" + x], g["db" + x] = c["dx"], c["dw"], c["dbias"]
    return g


def gpu_layer(d, B, T, N, K, V):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    t = {n: torch.from_numpy(a).to("cuda") for n, a in d.items()}
    uq = m2.m2rnn_conv4_silu_fwd(t["xq"], t["wq"], t["bq"]).view(B, T, N, K)
    uk = m2.m2rnn_conv4_silu_fwd(t["xk"], t["wk"], t["bk"]).view(B, T, N, K)
    uv = m2.m2rnn_conv4_silu_fwd(t["xv"], t["wv"], t["bv"]).view(B, T, N, V)
    f = m2.m2rnn_gate_fwd(t["a"], t["alpha"], t["beta"])
    y, _, ckpt = m2.m2rnn_fwd_ckpt(uq, uk, uv, f, t["W"], t["w_r"])
    out = m2.m2rnn_out_norm_fwd(y, t["gz"], t["gamma"], EPS)
    gn = m2.m2rnn_out_norm_bwd(y, t["gz"], t["gamma"], t["dout"], EPS)
    gs = m2.m2rnn_bwd_ckpt(uq, uk, uv, f, t["W"], t["w_r"], ckpt, gn["dy"])
    gg = m2.m2rnn_gate_bwd(t["a"], t["alpha"], t["beta"], gs["df"])
    g = {"out": out, "y": y, "dgz": gn["dgz"], "dgamma": gn["dgamma"], "dW": gs["dW"], "dw_r": gs["dw_r"],
         "da": gg["da"], "dalpha": gg["dalpha"], "dbeta": gg["dbeta"]}
    for x, du in (("q", gs["dq"]), ("k", gs["dk"]), ("v", gs["dv"])):
        c = m2.m2rnn_conv4_silu_bwd(t["x" + x], t["w" + x], t["b" + x], du.reshape(B, T, -1).contiguous())
        g["dx" + x], g["dw" + x], g["db" + x] = c["dx"], c["dw"], c["dbias"]
    torch.cuda.synchronize()
    return {n: v.cpu().numpy().astype(np.float64) for n, v in g.items()}


@pytest.mark.parametrize("B,T,N,K,V", [(2, 37, 4, 16, 16), (1, 33, 2, 64, 64), (2, 20, 3, 32, 32)])
def test_layer_training_step(B, T, N, K, V):
    torch_cuda()
    say("layer", B, T, N, K, V)
    d = layer_inputs(B, T, N, K, V, seed=100 + T + K)
    ref = oracle_layer(d, B, T, N, K, V)
    got = gpu_layer(d, B, T, N, K, V)
    ey = float(np.max(np.abs(got["y"] - ref["y"])))
    say("y max-abs", ey)
    assert ey <= 5e-4, ey
    # out: the budget on y carried through the norm (see test_gpu_fwd_block.py)
    x = (ref["y"] * block.silu(d["gz"])).reshape(B, T, N * V)
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)
    tol = 2.0 * 5e-4 * np.abs(d["gamma"].reshape(1, 1, -1) * block.silu(d["gz"].reshape(B, T, -1))) * s
    worst = float(np.max(np.abs(got["out"] - ref["out"]).reshape(B, T, -1) / (tol + 1e-6)))
    say("out worst/tol", worst)
    assert worst <= 1.0, worst
    for n in ("dgz", "dgamma", "dW", "dw_r", "da", "dalpha", "dbeta", "dxq", "dxk", "dxv", "dwq", "dwk", "dwv",
              "dbq", "dbk", "dbv"):
        e = rel_l2(got[n], ref[n])
        say(n, e)
        assert e <= 1e-3, (n, e)
