"""GPU parity of the backward (BPTT, checkpoints every 64 steps) against the oracle's manual
backward: relative L2 error <= 1e-3 per gradient tensor."""
import numpy as np
import pytest

from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import gpu_bwd, oracle_bwd, rel_l2, say, to_device, torch_cuda

pytestmark = pytest.mark.gpu

GRADS = ("dq", "dk", "dv", "df", "dW", "dw_r", "dH0")
TOL = 1e-3


# Per-step guard: the error of one step's dq (a K-vector per (b, t, n)) or df, relative to the larger
# of that step's own size and a hundredth of the typical step size, stays within ten times the
# whole-tensor budget.  A few wrong steps of a long sequence barely move the whole-tensor rel-L2;
# this bound catches them.
STEP_TOL = 1e-2


def step_rel(got, ref):
    """max over steps of |got - ref| / max(|ref|, 0.01 rms(ref)), with |.| the L2 norm over the
    trailing K axis (dq) or the scalar itself (df)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.ndim == 4:  # [B, T, N, K]
        e = np.linalg.norm(got - ref, axis=-1)
        r = np.linalg.norm(ref, axis=-1)
    else:
        e, r = np.abs(got - ref), np.abs(ref)
    if r.size == 0:
        return 0.0
    floor = 0.01 * np.sqrt(np.mean(r * r))
    if floor == 0.0:
        return float(np.max(e))
    return float(np.max(e / np.maximum(r, floor)))


def check(got, ref, names=GRADS):
    errs = {n: rel_l2(got[n], ref[n]) for n in names}
    say("rel-L2", {n: f"{e:.2e}" for n, e in errs.items()})
    for n, e in errs.items():
        assert e <= TOL, (n, e)
    steps = {n: step_rel(got[n], ref[n]) for n in ("dq", "df") if n in names}
    say("per-step", {n: f"{e:.2e}" for n, e in steps.items()})
    for n, e in steps.items():
        assert e <= STEP_TOL, (n, e)


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


@pytest.mark.parametrize("e", [0, -20])
def test_bwd_workload_sampled_heads(e):
    # The full B4 N16 T4096 K=V=64 fp32 workload on the GPU; the oracle recomputes every batch
    # entry of two heads (dW and dw_r sum over the batch).  Also with dy scaled by 2^-20, the
    # magnitude of activation gradients in bf16 training without loss scaling (§3.1).
    torch_cuda()
    name = "bwd_b4_h16_t4096_kv64"
    w = inputs.WORKLOADS[name]
    d = inputs.workload_inputs(name)
    d["dy"] = (d["dy"] * np.float32(2.0 ** e)).astype(np.float32)
    say(name, "dy scale 2 **", e)
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


@pytest.mark.parametrize("e", [-20, -14, 10])
@pytest.mark.parametrize("B,T,N,K,V,dtype", [
    (1, 70, 2, 16, 16, "f32"),
    (2, 130, 3, 32, 64, "bf16"),
    (1, 65, 1, 16, 128, "bf16"),
    (1, 64, 1, 64, 64, "f32"),
])
def test_gradient_scale(B, T, N, K, V, dtype, e):
    # Every gradient is linear in (dy, dH_T) jointly (§2.7), and bf16 training without loss scaling
    # (§3.1) meets activation gradients far from unit scale.  With both scaled by 2^e the oracle's
    # gradients scale exactly; the GPU must hold the budget at every scale.  The kernel runs each
    # (b, n) at a power-of-two scale taken from its own largest |dy|, |dH_T|, so its result is
    # also exactly 2^e times its unit-scale result.
    torch_cuda()
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype=dtype, seed=800 + T + K + V, with_H0=True, with_dy=True,
                           with_dHT=True)
    s = np.float32(2.0 ** e)
    ds = dict(d)
    ds["dy"] = (d["dy"] * s).astype(np.float32)
    ds["dH_T"] = (d["dH_T"] * s).astype(np.float32)
    say("bwd scale 2 **", e, B, T, N, K, V, dtype)
    got = gpu_bwd(to_device(ds, dtype))
    check(got, oracle_bwd(ds))
    unit = gpu_bwd(to_device(d, dtype))
    for n in GRADS:
        assert np.array_equal(got[n], unit[n] * float(s)), n


def test_gradient_scale_clipped():
    # The clip bound is scaled with the chain: clamping at 2^e c the chain of 2^e dy is 2^e times
    # clamping at c.
    torch_cuda()
    d = inputs.make_inputs(2, 130, 2, 32, 64, qkv_dtype="bf16", seed=811, with_H0=True, with_dy=True, with_dHT=True)
    s = np.float32(2.0 ** -16)
    ds = dict(d)
    ds["dy"] = (d["dy"] * s).astype(np.float32)
    ds["dH_T"] = (d["dH_T"] * s).astype(np.float32)
    clip = 0.6 * float(s)
    got = gpu_bwd(to_device(ds, "bf16"), grad_clip=clip)
    check(got, oracle_bwd(ds, clip=clip))
    unit = gpu_bwd(to_device(d, "bf16"), grad_clip=0.6)
    for n in GRADS:
        assert np.array_equal(got[n], unit[n] * float(s)), n


@pytest.mark.parametrize("B,T,N,dtype,clip,scale", [
    (2, 300, 3, "bf16", 0.0, 0),     # five pairs of sub-segments and a ragged tail
    (1, 70, 2, "f32", 0.6, 0),       # clipped recurrent gradient
    (2, 9, 2, "bf16", 0.0, -20),     # two sub-segments, dy at 2^-20
    (1, 1, 1, "f32", 0.0, 0),        # a single step
])
def test_roles_give_the_one_role_kernels_bits(B, T, N, dtype, clip, scale, monkeypatch):
    # The reverse kernel at V = 64 with the walk and the recompute in waves of their own computes
    # every operation of the one-role kernel in the same order: all seven gradients are the same
    # bits.  (Both are also checked against the oracle.)
    torch_cuda()
    d = inputs.make_inputs(B, T, N, 64, 64, qkv_dtype=dtype, seed=900 + T + N, with_H0=True, with_dy=True,
                           with_dHT=True)
    s = np.float32(2.0 ** scale)
    d["dy"] = (d["dy"] * s).astype(np.float32)
    d["dH_T"] = (d["dH_T"] * s).astype(np.float32)
    dd = to_device(d, dtype)
    say("bwd roles", B, T, N, dtype, clip, scale)
    monkeypatch.delenv("M2RNN_BWD_ROLES", raising=False)
    g1 = gpu_bwd(dd, grad_clip=clip * float(s))
    monkeypatch.setenv("M2RNN_BWD_ROLES", "0")
    g0 = gpu_bwd(dd, grad_clip=clip * float(s))
    monkeypatch.delenv("M2RNN_BWD_ROLES", raising=False)
    for n in GRADS:
        assert np.array_equal(g1[n], g0[n]), n
    check(g1, oracle_bwd(d, clip=clip * float(s)))
