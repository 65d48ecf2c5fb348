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
