"""The entry points enqueue only kernels (no memset or copy nodes), so they can be captured in a
HIP graph: captured forward, backward and decode replays equal the eager calls bit for bit, on
every replay, with other work and synchronisations between the replays; and calls on a side
stream equal calls on the default stream."""
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import say, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_eager_calls():
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(2, 150, 4, 64, 64, qkv_dtype="bf16", seed=31337, with_H0=True, with_dy=True)
    dd = to_device(d, "bf16")
    say("graph capture: fwd, bwd, decode")
    B, T, N, K, V = 2, 150, 4, 64, 64
    dims = m2.Dims(B, T, N, K, V)
    y = torch.empty((B, T, N, V), device="cuda")
    H_T = torch.empty((B, N, K, V), device="cuda")
    fws = torch.empty(max(m2.m2rnn_fwd_workspace_size(dims, m2.DTYPE_BF16), 1), dtype=torch.uint8, device="cuda")
    bws = torch.empty(m2.m2rnn_bwd_workspace_size(dims, m2.DTYPE_BF16), dtype=torch.uint8, device="cuda")
    Hd = dd["H0"].clone()
    yd = torch.empty((B, N, V), device="cuda")

    def work():
        m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"], y=y, H_T=H_T, workspace=fws)
        g = m2.m2rnn_bwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"], dd["dy"], workspace=bws)
        m2.m2rnn_decode_step(dd["q"][:, 0].contiguous(), dd["k"][:, 0].contiguous(), dd["v"][:, 0].contiguous(),
                             dd["f"][:, 0].contiguous(), dd["W"], dd["w_r"], dd["H0"], H_out=Hd, y=yd)
        return g

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g_eager = work()
    torch.cuda.synchronize()
    ref = {"y": y.clone(), "H_T": H_T.clone(), "Hd": Hd.clone(), "yd": yd.clone()}
    ref.update({k: v.clone() for k, v in g_eager.items() if v is not None})

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        g_cap = work()
    torch.cuda.synchronize()
    for rep in range(3):
        # clobber the outputs with eager work between replays
        for t in (y, H_T, Hd, yd):
            t.fill_(float("nan"))
        for t in g_cap.values():
            if t is not None:
                t.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = {"y": y, "H_T": H_T, "Hd": Hd, "yd": yd}
        got.update({k: v for k, v in g_cap.items() if v is not None})
        for name, r in ref.items():
            assert torch.equal(got[name], r), (rep, name)


def test_side_stream_equals_default_stream():
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(1, 77, 3, 32, 64, qkv_dtype="f32", seed=99, with_H0=True)
    dd = to_device(d, "f32")
    y0, H0 = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        y1, H1 = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"])
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(H0, H1)


def test_graph_capture_of_a_long_forward_takes_the_single_pass():
    # At T >= 4096 with split rows m2rnn_fwd runs time segments on a side stream; under graph
    # capture it takes the single pass instead, so replays equal the eager scan + finish bit for bit.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    B, T, N, K, V = 1, 4100, 8, 64, 64
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="bf16", seed=4242)
    dd = to_device(d, "bf16")
    say("graph capture of a long forward")
    args = (dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], None)
    y = torch.empty((B, T, N, V), device="cuda")
    H_T = torch.empty((B, N, K, V), device="cuda")
    ws = torch.empty(m2.m2rnn_fwd_workspace_size(m2.Dims(B, T, N, K, V), m2.DTYPE_BF16), dtype=torch.uint8,
                     device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        m2.m2rnn_scan_fwd(*args, y=y, H_T=H_T, workspace=ws)
        m2.m2rnn_scan_fwd_finish(*args, y=y, H_T=H_T, workspace=ws)
    torch.cuda.synchronize()
    ref_y, ref_H = y.clone(), H_T.clone()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        m2.m2rnn_fwd(*args, y=y, H_T=H_T, workspace=ws)
    torch.cuda.synchronize()
    for rep in range(3):
        y.fill_(float("nan"))
        H_T.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref_y) and torch.equal(H_T, ref_H), rep


def test_graph_replays_of_a_layer_training_step():
    # The whole layer's training step (conv4+SiLU, gate, the checkpoint-keeping forward, output gate
    # + RMSNorm, and the backward of each) captured once and replayed: every output and gradient of
    # every replay equals the eager step bit for bit.
    torch = torch_cuda()
    import numpy as np
    import matrix_state_nonlinear_m2rnn_amd as m2
    B, T, N, K, V = 2, 100, 4, 32, 64
    r = np.random.default_rng(4242)
    f32 = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float32)).cuda()  # noqa: E731
    t = {"xq": f32(r.normal(0, 0.7, (B, T, N * K))), "xk": f32(r.normal(0, 0.7, (B, T, N * K))),
         "xv": f32(r.normal(0, 1.0, (B, T, N * V))), "wq": f32(r.normal(0, 0.5, (N * K, 4))),
         "wk": f32(r.normal(0, 0.5, (N * K, 4))), "wv": f32(r.normal(0, 0.5, (N * V, 4))),
         "bq": f32(r.normal(0, 0.1, N * K)), "bk": f32(r.normal(0, 0.1, N * K)), "bv": f32(r.normal(0, 0.1, N * V)),
         "a": f32(r.normal(0, 2.0, (B, T, N))), "alpha": f32(r.uniform(0.1, 3.0, N)), "beta": f32(r.normal(0, 1, N)),
         "W": f32(np.stack([np.linalg.qr(r.normal(0, 1, (V, V)))[0] for _ in range(N)]) * 0.9),
         "w_r": f32(r.normal(0, 0.3, (N, V))), "gz": f32(r.normal(0, 2.0, (B, T, N, V))),
         "gamma": f32(1.0 + 0.1 * r.normal(0, 1, (N, V))), "dout": f32(r.normal(0, 1.0, (B, T, N, V)))}
    say("graph capture: layer training step", B, T, N, K, V)

    def step():
        uq = m2.m2rnn_conv4_silu_fwd(t["xq"], t["wq"], t["bq"]).view(B, T, N, K)
        uk = m2.m2rnn_conv4_silu_fwd(t["xk"], t["wk"], t["bk"]).view(B, T, N, K)
        uv = m2.m2rnn_conv4_silu_fwd(t["xv"], t["wv"], t["bv"]).view(B, T, N, V)
        f = m2.m2rnn_gate_fwd(t["a"], t["alpha"], t["beta"])
        y, H_T, ckpt = m2.m2rnn_fwd_ckpt(uq, uk, uv, f, t["W"], t["w_r"])
        out = m2.m2rnn_out_norm_fwd(y, t["gz"], t["gamma"], 1e-6)
        gn = m2.m2rnn_out_norm_bwd(y, t["gz"], t["gamma"], t["dout"], 1e-6)
        gs = m2.m2rnn_bwd_ckpt(uq, uk, uv, f, t["W"], t["w_r"], ckpt, gn["dy"])
        gg = m2.m2rnn_gate_bwd(t["a"], t["alpha"], t["beta"], gs["df"])
        res = {"out": out, "H_T": H_T, "dgz": gn["dgz"], "dgamma": gn["dgamma"], "dW": gs["dW"], "dw_r": gs["dw_r"],
               "da": gg["da"], "dalpha": gg["dalpha"], "dbeta": gg["dbeta"]}
        for x in ("q", "k", "v"):
            c = m2.m2rnn_conv4_silu_bwd(t["x" + x], t["w" + x], t["b" + x],
                                        gs["d" + x].reshape(B, T, -1).contiguous())
            res["dx" + x], res["dw" + x], res["db" + x] = c["dx"], c["dw"], c["dbias"]
        return res

    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        eager = {k: v.clone() for k, v in step().items()}
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        cap = step()
    torch.cuda.synchronize()
    for rep in range(3):
        for v in cap.values():
            v.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, ref in eager.items():
            assert torch.equal(cap[name], ref), (rep, name)
