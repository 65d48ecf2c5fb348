"""Pins of the fp64 oracle for the gate, the output gate + RMSNorm and the causal conv4 + SiLU
(M²RNN notes §2.2, §2.3, Appendix C) against closed forms, identities the notes state, library
routines (scipy's expit, torch's conv1d and silu, torch autograd in fp64) and central differences."""
import numpy as np
import pytest
import scipy.special

from oracle import block


def rng(seed):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------ gate

def test_gate_with_alpha_one_is_the_logistic_of_minus_a_minus_beta():
    # §2.2: for alpha = 1 the gate equals sigma(-a - beta).
    r = rng(1)
    a = r.normal(0, 3, (2, 7, 5))
    beta = r.normal(0, 1, 5)
    f = block.gate_fwd(a, np.ones(5), beta)
    np.testing.assert_allclose(f, scipy.special.expit(-(a + beta)), rtol=1e-14, atol=1e-300)


def test_gate_matches_its_power_form_and_range():
    # (1 + e^{a+beta})^{-alpha}: the notes' first form of the same gate; alpha = 0 keeps f = 1.
    r = rng(2)
    a = r.normal(0, 2, (3, 4, 6))
    alpha = r.uniform(0, 4, 6)
    beta = r.normal(0, 1, 6)
    f = block.gate_fwd(a, alpha, beta)
    np.testing.assert_allclose(f, np.power(1.0 + np.exp(a + beta), -alpha), rtol=1e-13)
    assert np.all(f > 0) and np.all(f <= 1)
    assert np.all(block.gate_fwd(a, np.zeros(6), beta) == 1.0)
    # decreasing in a for alpha > 0
    assert np.all(np.diff(block.gate_fwd(np.linspace(-5, 5, 50)[None, :, None], alpha[:1], beta[:1]), axis=1) < 0)


def test_gate_backward_matches_central_differences():
    r = rng(3)
    a = r.normal(0, 2, (2, 3, 4))
    alpha = r.uniform(0.2, 3, 4)
    beta = r.normal(0, 1, 4)
    df = r.normal(0, 1, a.shape)
    g = block.gate_bwd(a, alpha, beta, df)
    L = lambda a_, al_, be_: float(np.sum(block.gate_fwd(a_, al_, be_) * df))  # noqa: E731
    h = 1e-6
    for name, x in (("da", a), ("dalpha", alpha), ("dbeta", beta)):
        num = np.zeros_like(x)
        for i in range(x.size):
            keep = x.flat[i]
            x.flat[i] = keep + h
            lp = L(a, alpha, beta)
            x.flat[i] = keep - h
            lm = L(a, alpha, beta)
            x.flat[i] = keep
            num.flat[i] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g[name], num, rtol=1e-6, atol=1e-9, err_msg=name)


# ------------------------------------------------------------------ output gate + RMSNorm

def test_silu_is_the_library_silu():
    torch = pytest.importorskip("torch")
    x = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(block.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14,
                               atol=1e-300)


def test_rmsnorm_output_has_unit_rms_and_is_scale_invariant():
    r = rng(4)
    y = r.normal(0, 1, (2, 3, 4, 8))
    gz = r.normal(0, 2, y.shape)
    out = block.out_norm_fwd(y, gz, np.ones((4, 8)), 0.0)
    np.testing.assert_allclose(np.mean(out.reshape(2, 3, 32) ** 2, axis=-1), 1.0, rtol=1e-13)
    np.testing.assert_allclose(block.out_norm_fwd(7.5 * y, gz, np.ones((4, 8)), 0.0), out, rtol=1e-12)
    # the gate multiplies before the norm: a gate of all ones leaves y's own normalisation
    big = np.full(y.shape, 60.0)  # SiLU(60) = 60 to fp64 precision: a constant factor, cancelled by the norm
    ref = y.reshape(2, 3, 32) / np.sqrt(np.mean(y.reshape(2, 3, 32) ** 2, axis=-1, keepdims=True))
    np.testing.assert_allclose(block.out_norm_fwd(y, big, np.ones((4, 8)), 0.0), ref.reshape(y.shape), rtol=1e-12)


def test_rmsnorm_forward_matches_torch_rms_norm_with_gamma_and_eps():
    # The per-feature scale and the epsilon against torch's own RMSNorm (a library routine), on the
    # gated row x = y (.) SiLU(gz) over all N V features of a token.
    torch = pytest.importorskip("torch")
    r = rng(6)
    B, T, N, V = 3, 5, 4, 8
    y = r.normal(0, 1, (B, T, N, V))
    gz = r.normal(0, 1.5, y.shape)
    gamma = r.normal(1, 0.4, (N, V))
    for eps in (1e-6, 1e-2, 0.7):
        out = block.out_norm_fwd(y, gz, gamma, eps)
        x = torch.from_numpy(y) * torch.nn.functional.silu(torch.from_numpy(gz))
        ref = torch.nn.functional.rms_norm(x.reshape(B, T, N * V), (N * V,), weight=torch.from_numpy(gamma).reshape(-1),
                                           eps=eps)
        np.testing.assert_allclose(out, ref.reshape(B, T, N, V).numpy(), rtol=1e-12, atol=1e-14)
    # and eps matters: a large eps shrinks the output where the mean square is small
    small = 1e-3 * y
    assert np.all(np.abs(block.out_norm_fwd(small, gz, gamma, 0.7)) < np.abs(block.out_norm_fwd(small, gz, gamma, 0.0)))


def test_rmsnorm_backward_matches_torch_autograd_and_differences():
    torch = pytest.importorskip("torch")
    r = rng(5)
    B, T, N, V = 2, 3, 2, 4
    y = r.normal(0, 1, (B, T, N, V))
    gz = r.normal(0, 1.5, y.shape)
    gamma = r.normal(1, 0.3, (N, V))
    dout = r.normal(0, 1, y.shape)
    eps = 1e-3
    g = block.out_norm_bwd(y, gz, gamma, eps, dout)
    ty, tg, tw = (torch.tensor(a, requires_grad=True) for a in (y, gz, gamma))
    x = (ty * torch.nn.functional.silu(tg)).reshape(B, T, N * V)
    out = tw.reshape(-1) * x * torch.rsqrt(torch.mean(x * x, dim=-1, keepdim=True) + eps)
    (out.reshape(B, T, N, V) * torch.from_numpy(dout)).sum().backward()
    np.testing.assert_allclose(g["dy"], ty.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dgz"], tg.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dgamma"], tw.grad.numpy(), rtol=1e-11, atol=1e-13)
    # and a few central differences of the oracle's own forward
    h = 1e-6
    for idx in [(0, 0, 0, 0), (1, 2, 1, 3), (0, 1, 1, 2)]:
        for name, arr in (("dy", y), ("dgz", gz)):
            keep = arr[idx]
            arr[idx] = keep + h
            lp = np.sum(block.out_norm_fwd(y, gz, gamma, eps) * dout)
            arr[idx] = keep - h
            lm = np.sum(block.out_norm_fwd(y, gz, gamma, eps) * dout)
            arr[idx] = keep
            assert abs((lp - lm) / (2 * h) - g[name][idx]) < 1e-6, (name, idx)


# ------------------------------------------------------------------ causal conv4 + SiLU

def test_conv4_silu_matches_the_library_conv1d():
    torch = pytest.importorskip("torch")
    r = rng(6)
    B, T, C = 2, 9, 5
    x = r.normal(0, 1, (B, T, C))
    w = r.normal(0, 0.5, (C, 4))
    bias = r.normal(0, 0.2, C)
    u = block.conv4_silu_fwd(x, w, bias)
    xt = torch.from_numpy(x).transpose(1, 2)                       # [B, C, T]
    pre = torch.nn.functional.conv1d(xt, torch.from_numpy(w)[:, None, :], torch.from_numpy(bias), padding=3,
                                     groups=C)[:, :, :T]           # causal: keep the first T outputs
    ref = torch.nn.functional.silu(pre).transpose(1, 2).numpy()
    np.testing.assert_allclose(u, ref, rtol=1e-12, atol=1e-14)
    # causality: the output at t does not see x after t
    x2 = x.copy()
    x2[:, 5:] += 10.0
    np.testing.assert_array_equal(block.conv4_silu_fwd(x2, w, bias)[:, :5], u[:, :5])


def test_conv4_silu_backward_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    r = rng(7)
    B, T, C = 2, 7, 3
    x = r.normal(0, 1, (B, T, C))
    w = r.normal(0, 0.5, (C, 4))
    bias = r.normal(0, 0.2, C)
    du = r.normal(0, 1, x.shape)
    g = block.conv4_silu_bwd(x, w, bias, du)
    tx, tw, tb = (torch.tensor(a, requires_grad=True) for a in (x, w, bias))
    pre = torch.nn.functional.conv1d(tx.transpose(1, 2), tw[:, None, :], tb, padding=3, groups=C)[:, :, :T]
    (torch.nn.functional.silu(pre).transpose(1, 2) * torch.from_numpy(du)).sum().backward()
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dw"], tw.grad.numpy(), rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(g["dbias"], tb.grad.numpy(), rtol=1e-11, atol=1e-13)
