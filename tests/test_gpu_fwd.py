"""GPU parity of the forward scan (HIP path through the C ABI) against the fp64 oracle.

Tolerances are the stated budgets: max-abs <= 5e-4 on y and H_T when the state is fp32 (f32,
f16x3 and bf16x3 contractions) and <= 2e-2 for the single-pass bf16 contraction.
"""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import TOL, gpu_fwd, max_abs, oracle_fwd, oracle_units, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu

MATHS = ["f32", "f16x3", "bf16x3", "bf16"]


@pytest.mark.parametrize("math", MATHS)
def test_tiny_f32_workload(math):
    torch_cuda()
    d = inputs.workload_inputs("tiny_f32")
    say("tiny_f32", math)
    y, H = gpu_fwd(to_device(d, "f32"), math)
    yr, Hr = oracle_fwd(d)
    assert max_abs(y, yr) <= TOL[math] and max_abs(H, Hr) <= TOL[math], (max_abs(y, yr), max_abs(H, Hr))
    assert np.all(np.abs(H) <= 1.0 + 1e-6)


@pytest.mark.parametrize("math", MATHS)
def test_b4_h16_t2048_kv64_full(math):
    torch_cuda()
    d = inputs.workload_inputs("b4_h16_t2048_kv64")
    say("b4_h16_t2048_kv64", math)
    y, H = gpu_fwd(to_device(d, "bf16"), math)
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y, yr), max_abs(H, Hr)
    say("errors", ey, eh)
    assert ey <= TOL[math] and eh <= TOL[math], (ey, eh)


@pytest.mark.parametrize("name,units,math", [
    ("long_b2_h32_t16384_kv64", [(0, 0), (1, 31), (0, 17), (1, 5)], "f16x3"),
    ("long_b2_h32_t16384_kv64", [(0, 0), (1, 31), (0, 17), (1, 5)], "bf16x3"),
    ("long_b2_h32_t16384_kv64", [(0, 3), (1, 20)], "f32"),
    ("b8_h16_t4096_kv128", [(0, 0), (7, 15)], "f16x3"),
    ("b8_h16_t4096_kv128", [(0, 0), (7, 15)], "bf16x3"),
    ("b1_h16_t4096_kv128", [(0, 0), (0, 9)], "f16x3"),
])
def test_full_size_sampled_units(name, units, math):
    # Full-size launch exactly as the benchmark runs it; the oracle re-computes sampled units.
    torch_cuda()
    w = inputs.WORKLOADS[name]
    d = inputs.workload_inputs(name)
    say(name, math, "units", units)
    y, H = gpu_fwd(to_device(d, w.qkv_dtype), math)
    assert np.all(np.abs(H) <= 1.0 + 1e-6)
    assert np.isfinite(y).all()
    ref = oracle_units(d, units)
    for (b, n), (yr, Hr) in ref.items():
        ey, eh = max_abs(y[b, :, n], yr), max_abs(H[b, n], Hr)
        say((b, n), ey, eh)
        assert ey <= TOL[math] and eh <= TOL[math], ((b, n), ey, eh)


@pytest.mark.parametrize("K,V", [(16, 16), (32, 32), (48, 64), (64, 32), (16, 128), (128, 64)])
@pytest.mark.parametrize("T", [1, 31, 33, 70])
def test_shapes_and_ragged_steps(K, V, T):
    torch_cuda()
    d = inputs.make_inputs(2, T, 3, K, V, qkv_dtype="bf16", seed=1000 + K + V + T, with_H0=True)
    dd = to_device(d, "bf16")
    yr, Hr = oracle_fwd(d)
    for math in ("f32", "f16x3", "bf16x3"):
        say("shape", K, V, T, math)
        y, H = gpu_fwd(dd, math)
        assert max_abs(y, yr) <= TOL[math] and max_abs(H, Hr) <= TOL[math], (math, max_abs(y, yr), max_abs(H, Hr))


@pytest.mark.parametrize("rb", [1, 2, 4])
def test_row_split_matches(rb):
    # The rows of one state may be spread over K/(16*rb) workgroups; all splits agree.
    torch_cuda()
    d = inputs.make_inputs(2, 100, 2, 64, 64, qkv_dtype="bf16", seed=77)
    dd = to_device(d, "bf16")
    say("row_blocks", rb)
    y, H = gpu_fwd(dd, "f16x3", row_blocks=rb)
    y1, H1 = gpu_fwd(dd, "f16x3", row_blocks=4)
    assert np.array_equal(H, H1)  # rows evolve identically whatever the split
    assert max_abs(y, y1) <= 1e-5
    yr, Hr = oracle_fwd(d)
    assert max_abs(y, yr) <= 5e-4 and max_abs(H, Hr) <= 5e-4


def test_hold_when_f_is_one_is_bit_exact():
    torch_cuda()
    d = inputs.make_inputs(2, 40, 2, 32, 64, qkv_dtype="f32", seed=5, with_H0=True)
    d["f"][:] = 1.0
    dd = to_device(d, "f32")
    for math in ("f32", "f16x3"):
        say("hold", math)
        y, H = gpu_fwd(dd, math)
        assert np.array_equal(H, d["H0"].astype(np.float64))
        yr, _ = oracle_fwd(d)
        assert max_abs(y, yr) <= 1e-5


def test_zero_steps_and_empty_batch():
    torch = torch_cuda()
    d = inputs.make_inputs(2, 0, 2, 16, 16, qkv_dtype="f32", seed=6, with_H0=True)
    dd = to_device(d, "f32")
    y, H = gpu_fwd(dd, "f16x3")
    assert y.shape == (2, 0, 2, 16) and np.array_equal(H, d["H0"].astype(np.float64))
    d = inputs.make_inputs(2, 0, 2, 16, 16, qkv_dtype="f32", seed=6)
    y, H = gpu_fwd(to_device(d, "f32"), "f16x3")
    assert np.all(H == 0.0)
    d = inputs.make_inputs(0, 5, 2, 16, 16, qkv_dtype="f32", seed=6)
    y, H = gpu_fwd(to_device(d, "f32"), "f16x3")
    assert y.shape == (0, 5, 2, 16)
    torch.cuda.synchronize()


def test_deterministic_across_runs():
    torch_cuda()
    d = inputs.make_inputs(2, 300, 4, 64, 64, qkv_dtype="bf16", seed=8)
    dd = to_device(d, "bf16")
    for math in ("f32", "f16x3"):
        y1, H1 = gpu_fwd(dd, math)
        y2, H2 = gpu_fwd(dd, math)
        assert np.array_equal(y1, y2) and np.array_equal(H1, H2)


def test_state_bound_under_saturation():
    torch_cuda()
    d = inputs.make_inputs(1, 200, 2, 64, 64, qkv_dtype="f32", seed=9)
    d["k"] *= 20.0
    d["v"] *= 20.0
    d["f"][:, ::4] = 0.0
    y, H = gpu_fwd(to_device(d, "f32"), "f16x3")
    assert np.all(np.abs(H) <= 1.0 + 1e-6)
    yr, Hr = oracle_fwd(d)
    assert max_abs(H, Hr) <= 5e-4


@pytest.mark.parametrize("K,V,T,math", [
    (64, 16, 37, "f16x3"),    # four row groups in a workgroup, one readout plane
    (128, 16, 70, "f16x3"),   # four row groups, two workgroups per state
    (32, 16, 5, "bf16x3"),    # two row groups, a single partial chunk
    (64, 32, 16, "f16x3"),    # two row groups of two waves each, exactly one chunk
    (32, 32, 33, "bf16"),     # two row groups, one plane
    (48, 16, 1, "f16x3"),     # three row blocks: one group per workgroup
    (16, 16, 50, "f32"),      # the fp32 contraction keeps one group
])
def test_row_groups_in_a_workgroup(K, V, T, math):
    # Narrow states (V < 64) put several 16-row blocks side by side in one workgroup and sum their
    # readouts there.
    torch_cuda()
    d = inputs.make_inputs(2, T, 3, K, V, qkv_dtype="bf16", seed=6000 + K + V + T, with_H0=True)
    say("row groups", K, V, T, math)
    y, H = gpu_fwd(to_device(d, "bf16"), math)
    yr, Hr = oracle_fwd(d)
    ey, eh = max_abs(y, yr), max_abs(H, Hr)
    say("errors", ey, eh)
    assert ey <= TOL[math] and eh <= TOL[math], (ey, eh)


def test_long_sequence_time_segments():
    # T >= 4096 with split rows: m2rnn_fwd scans time segments, each from the state the previous one
    # ended in, with each segment's readout finish overlapping the next scan.  H_t depends on H_{t-1}
    # and the inputs only (Eq. 10-12), so the result must equal the single pass (scan + finish over
    # the whole sequence) bit for bit, and the oracle within tolerance.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(1, 4100, 8, 64, 64, qkv_dtype="bf16", seed=31)  # the last segment is ragged
    dd = to_device(d, "bf16")
    say("time segments", 1, 4100, 8, 64, 64)
    args = (dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], None)
    y, H = m2.m2rnn_fwd(*args, math="f16x3")
    y1, H1, ws = m2.m2rnn_scan_fwd(*args, math="f16x3")
    m2.m2rnn_scan_fwd_finish(*args, math="f16x3", y=y1, H_T=H1, workspace=ws)
    torch.cuda.synchronize()
    ey, eh = float((y - y1).abs().max()), float((H - H1).abs().max())
    say("segments vs single pass", ey, eh)
    assert torch.equal(y, y1) and torch.equal(H, H1), (ey, eh)
    y, H = y.cpu().numpy().astype(np.float64), H.cpu().numpy().astype(np.float64)
    for (b, n), (yr, Hr) in oracle_units(d, [(0, 0), (0, 7)]).items():
        ey, eh = max_abs(y[b, :, n], yr), max_abs(H[b, n], Hr)
        say((b, n), ey, eh)
        assert ey <= TOL["f16x3"] and eh <= TOL["f16x3"], ((b, n), ey, eh)



@pytest.mark.parametrize("B,N,T1,T2", [(1, 8, 96, 70), (2, 32, 256, 131), (1, 8, 1, 33)])
@pytest.mark.parametrize("math", ["f16x3", "f32", "bf16x3"])
def test_chained_calls_equal_one_pass(B, N, T1, T2, math):
    # Eq. 10-12 carry the state from H_{t-1} only: a forward over T1 steps, then one over the next T2
    # steps started from its H_T, must give the bits of one forward over T1 + T2 steps (y and H_T),
    # for every row split.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    d = inputs.make_inputs(B, T1 + T2, N, 64, 64, qkv_dtype="bf16", seed=900 + B * N + T1, with_H0=True)
    dd = to_device(d, "bf16")
    for rb in (1, 2, 4):
        say("chained", B, N, T1, T2, math, "row_blocks", rb)
        seq = [dd[x] for x in ("q", "k", "v", "f")]
        y, H = m2.m2rnn_fwd(*seq, dd["W"], dd["w_r"], dd["H0"], math=math, row_blocks=rb)
        first = [x[:, :T1].contiguous() for x in seq]
        second = [x[:, T1:].contiguous() for x in seq]
        ya, Ha = m2.m2rnn_fwd(*first, dd["W"], dd["w_r"], dd["H0"], math=math, row_blocks=rb)
        yb, Hb = m2.m2rnn_fwd(*second, dd["W"], dd["w_r"], Ha, math=math, row_blocks=rb)
        torch.cuda.synchronize()
        assert torch.equal(H, Hb), float((H - Hb).abs().max())
        assert torch.equal(y[:, :T1], ya) and torch.equal(y[:, T1:], yb), (
            float((y[:, :T1] - ya).abs().max()), float((y[:, T1:] - yb).abs().max()))


def test_two_streams_with_their_own_overlap_objects():
    # Two segmented forwards issued at once on two streams, each with its own side stream (the
    # caller's m2rnn_overlap): no shared queue and no cross-stream dependence, and each result is
    # its solo run bit for bit.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    runs = []
    for B, T, N, seed in ((1, 4160, 8, 41), (2, 4100, 4, 42)):
        dd = to_device(inputs.make_inputs(B, T, N, 64, 64, qkv_dtype="bf16", seed=seed), "bf16")
        args = (dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], None)
        y, H = m2.m2rnn_fwd(*args, math="f16x3", overlap=None)
        runs.append((args, y, H))
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    overlaps = [m2.Overlap(), m2.Overlap()]
    out = []
    for (args, _, _), s, ov in zip(runs, streams, overlaps):
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            out.append(m2.m2rnn_fwd(*args, math="f16x3", overlap=ov))
    torch.cuda.synchronize()
    for (_, y, H), (y2, H2) in zip(runs, out):
        assert torch.equal(y, y2) and torch.equal(H, H2)
    for ov in overlaps:
        ov.close()


def test_batch_16_at_16k_tokens_beyond_2_gib():
    # The 16K-token context at batch 16 (B16 N32 T16384 K=V=64, bf16 q/k/v, f = sigmoid(N(3, 1))):
    # y is 2 GiB and the split-row readout planes 8 GiB, past 32-bit offsets from the tensors'
    # starts.  Inputs are eight seeded B2 draws side by side (W and w_r from the first); sampled
    # units from the first and last batch entries are checked against the oracle, with split rows
    # (four readout planes, time segments) and with all rows in one workgroup.
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    B, T, N, K, V = 16, 16384, 32, 64, 64
    q = torch.empty((B, T, N, K), dtype=torch.bfloat16, device="cuda")
    k = torch.empty_like(q)
    v = torch.empty((B, T, N, V), dtype=torch.bfloat16, device="cuda")
    f = torch.empty((B, T, N), dtype=torch.float32, device="cuda")
    units = {(0, 0): None, (1, 31): None, (9, 17): None, (15, 31): None, (14, 2): None}
    W = w_r = None
    for i in range(B // 2):
        d = inputs.make_inputs(2, T, N, K, V, qkv_dtype="bf16", f_mean=3.0, seed=4400 + i)
        if W is None:
            W, w_r = d["W"], d["w_r"]
        dd = to_device(d, "bf16")
        for name, dst in (("q", q), ("k", k), ("v", v), ("f", f)):
            dst[2 * i:2 * i + 2].copy_(dd[name])
        for (b, n) in units:
            if b // 2 == i:
                bb = b - 2 * i
                units[(b, n)] = dict(q=d["q"][bb:bb + 1, :, n:n + 1], k=d["k"][bb:bb + 1, :, n:n + 1],
                                     v=d["v"][bb:bb + 1, :, n:n + 1], f=d["f"][bb:bb + 1, :, n:n + 1],
                                     W=W[n:n + 1], w_r=w_r[n:n + 1], H0=None)
        del dd, d
    Wd = torch.from_numpy(W).cuda()
    wrd = torch.from_numpy(w_r).cuda()
    refs = {u: oracle_fwd(sub) for u, sub in units.items()}
    for rb in (1, 4):
        say("B16 N32 T16384 K=V=64, row_blocks", rb)
        y, H = m2.m2rnn_fwd(q, k, v, f, Wd, wrd, None, math="f16x3", row_blocks=rb)
        torch.cuda.synchronize()
        for (b, n), (yr, Hr) in refs.items():
            ey = max_abs(y[b, :, n].cpu().numpy(), yr[0, :, 0])
            eh = max_abs(H[b, n].cpu().numpy(), Hr[0, 0])
            say((b, n), ey, eh)
            assert ey <= TOL["f16x3"] and eh <= TOL["f16x3"], ((b, n), ey, eh)
        del y, H
        torch.cuda.empty_cache()


@pytest.mark.parametrize("math", ["f16x3", "bf16x3", "bf16"])
def test_readout_waves_give_the_single_role_kernels_bits(math, monkeypatch):
    # The forward with its readout and staging in waves of their own computes every operation of
    # the single-role kernel in the same order: y, H_T and the checkpoints are the same bits, for
    # every row split and a ragged tail (K = V = 128: 32-step chunks, one row block per wave).
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    for B, T, N, KV, seed in ((2, 300, 8, 64, 61), (1, 70, 3, 64, 62), (1, 33, 2, 64, 63), (2, 130, 4, 128, 64),
                              (1, 31, 1, 128, 65)):
        d = inputs.make_inputs(B, T, N, KV, KV, qkv_dtype="bf16", seed=seed, with_H0=True)
        dd = to_device(d, "bf16")
        args = (dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd["H0"])
        for rb in ((1, 2, 4) if KV == 64 else (1,)):
            say("readout waves", B, T, N, KV, math, "row_blocks", rb)
            monkeypatch.delenv("M2RNN_FWD_READOUT_WAVES", raising=False)
            y1, H1, c1 = m2.m2rnn_fwd_ckpt(*args, math=math, row_blocks=rb)
            monkeypatch.setenv("M2RNN_FWD_READOUT_WAVES", "0")
            y0, H0, c0 = m2.m2rnn_fwd_ckpt(*args, math=math, row_blocks=rb)
            monkeypatch.delenv("M2RNN_FWD_READOUT_WAVES", raising=False)
            torch.cuda.synchronize()
            assert torch.equal(y1, y0) and torch.equal(H1, H0) and torch.equal(c1, c0), (
                float((y1 - y0).abs().max()), float((H1 - H0).abs().max()))


@pytest.mark.parametrize("B,N,K,V", [(12, 32, 64, 64), (8, 16, 128, 128), (16, 128, 64, 16), (2, 32, 64, 64)])
def test_automatic_plan_takes_one_row_block(B, N, K, V):
    # The automatic plan takes one 16-row block per wave wherever that kernel keeps its state in
    # registers, also where that needs several rounds of resident workgroups: the readout planes it
    # sizes the workspace for (one per workgroup of a pair) are then those of row_blocks = 1.
    torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    dims = m2.Dims(B, 4096, N, K, V)
    for math in ("bf16x3", "f16x3"):
        auto = m2.m2rnn_fwd_workspace_size(dims, m2.DTYPE_BF16, math, 0)
        one = m2.m2rnn_fwd_workspace_size(dims, m2.DTYPE_BF16, math, 1)
        say("plan", B, N, K, V, math, auto, one)
        assert auto == one, (auto, one)
