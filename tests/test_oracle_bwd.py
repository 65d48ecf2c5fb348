"""Pins of the fp64 oracle's BPTT (M²RNN notes §2.7) against central finite differences of the
oracle's own forward (an independent code path), and against the closed form at f = 1."""
import numpy as np
import pytest

import oracle
from matrix_state_nonlinear_m2rnn_amd import inputs


def loss(d, dy, dHT):
    y, H_T = oracle.ref_fwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"])
    return float(np.sum(y * dy) + np.sum(H_T * dHT))


@pytest.mark.parametrize("B,T,N,K,V", [(1, 5, 2, 3, 2), (2, 4, 1, 2, 3)])
def test_gradients_match_central_differences(B, T, N, K, V):
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="f32", seed=31 + K, with_H0=True, with_dy=True,
                           with_dHT=True)
    d = {x: (a.astype(np.float64) if a is not None else None) for x, a in d.items()}
    d["W"] *= 1.5  # leave the near-linear regime
    d["k"] *= 3.0
    dy, dHT = d.pop("dy"), d.pop("dH_T")
    g = oracle.ref_bwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], dy, dHT)
    names = {"q": "dq", "k": "dk", "v": "dv", "f": "df", "W": "dW", "w_r": "dw_r", "H0": "dH0"}
    h = 1e-6
    for x, gx in names.items():
        a = d[x]
        num = np.empty_like(a)
        flat = a.reshape(-1)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = loss(d, dy, dHT)
            flat[i] = keep - h
            lm = loss(d, dy, dHT)
            flat[i] = keep
            num.reshape(-1)[i] = (lp - lm) / (2 * h)
        err = np.max(np.abs(num - g[gx])) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (x, err)


def test_closed_form_when_f_is_one():
    # f = 1 freezes the state at H_0 and blocks the tanh branch (1 - f = 0), so D = 0:
    # dk = 0, dW = 0, dv_t = w_r (.) u_t, dq_t = H_0 u_t, dw_r = sum_t u_t (.) v_t,
    # dH_0 = dH_T + sum_t q_t u_t^T, and df_t = <R_t, H_0 - Z_t> with R_t = dH_T + sum_{s>=t} q_s u_s^T.
    B, T, N, K, V = 2, 6, 2, 3, 4
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="f32", seed=77, with_H0=True, with_dy=True, with_dHT=True)
    d = {x: (a.astype(np.float64) if a is not None else None) for x, a in d.items()}
    d["f"][:] = 1.0
    g = oracle.ref_bwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], d["dy"], d["dH_T"])
    u, q, v, k = d["dy"], d["q"], d["v"], d["k"]
    assert np.all(g["dk"] == 0.0) and np.all(g["dW"] == 0.0)
    np.testing.assert_allclose(g["dv"], d["w_r"][None, None] * u, rtol=0, atol=1e-14)
    np.testing.assert_allclose(g["dq"], np.einsum("bnkv,btnv->btnk", d["H0"], u), rtol=0, atol=1e-13)
    np.testing.assert_allclose(g["dw_r"], np.einsum("btnv,btnv->nv", u, v), rtol=0, atol=1e-12)
    np.testing.assert_allclose(g["dH0"], d["dH_T"] + np.einsum("btnk,btnv->bnkv", q, u), rtol=0, atol=1e-12)
    for b in range(B):
        for n in range(N):
            R = d["dH_T"][b, n].copy()
            for t in range(T - 1, -1, -1):
                R = R + np.outer(q[b, t, n], u[b, t, n])
                Z = np.tanh(d["H0"][b, n] @ d["W"][n] + np.outer(k[b, t, n], v[b, t, n]))
                np.testing.assert_allclose(g["df"][b, t, n], np.sum(R * (d["H0"][b, n] - Z)), rtol=1e-12,
                                           atol=1e-12)


def test_zero_upstream_gives_zero_gradients():
    d = inputs.make_inputs(2, 5, 2, 4, 4, qkv_dtype="f32", seed=3, with_dy=True)
    dy = np.zeros_like(d["dy"])
    g = oracle.ref_bwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], None, dy, None)
    for x in g.values():
        assert np.all(x == 0.0)


def test_shared_query_key_gradient_is_the_sum_over_heads():
    # One query/key shared by all heads (the notes' multi-value layout, N_q = N_k = 1): the
    # gradient of the shared q (k) is the sum over heads of the per-head gradients (§2.7).  Pinned
    # by central differences of the loss with the shared q (k) broadcast to every head.
    B, T, N, K, V = 1, 4, 3, 3, 2
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="f32", seed=123, with_H0=True, with_dy=True,
                           with_dHT=True, shared_qk=True)
    d = {x: (a.astype(np.float64) if a is not None else None) for x, a in d.items()}
    d["k"] *= 3.0
    dy, dHT = d.pop("dy"), d.pop("dH_T")
    assert d["q"].shape == (B, T, 1, K)

    def per_head(dd):
        e = dict(dd)
        e["q"] = np.ascontiguousarray(np.broadcast_to(dd["q"], (B, T, N, K)))
        e["k"] = np.ascontiguousarray(np.broadcast_to(dd["k"], (B, T, N, K)))
        return e

    e = per_head(d)
    g = oracle.ref_bwd(e["q"], e["k"], e["v"], e["f"], e["W"], e["w_r"], e["H0"], dy, dHT)
    h = 1e-6
    for x, gx in (("q", "dq"), ("k", "dk")):
        flat = d[x].reshape(-1)
        num = np.empty(flat.size)
        for i in range(flat.size):
            keep = flat[i]
            flat[i] = keep + h
            lp = loss(per_head(d), dy, dHT)
            flat[i] = keep - h
            lm = loss(per_head(d), dy, dHT)
            flat[i] = keep
            num[i] = (lp - lm) / (2 * h)
        summed = g[gx].sum(axis=2, keepdims=True)
        err = np.max(np.abs(num.reshape(summed.shape) - summed)) / max(1e-3, np.max(np.abs(num)))
        assert err < 1e-6, (x, err)


def _autograd_clipped(d, dy, dHT, clip):
    """The same loss through torch autograd (fp64, CPU): the state entering each step passes an
    identity whose backward clamps its gradient elementwise to [-clip, clip], so what a step sends
    back to H_{t-1} is clamped while the readout of H_{t-1} and dH_T reach it unclamped.  Returns
    the gradients and the fraction of clamped elements."""
    import torch
    seen = {"n": 0, "clamped": 0}

    class ClampGrad(torch.autograd.Function):
        @staticmethod
        def forward(ctx, x):
            return x.view_as(x)

        @staticmethod
        def backward(ctx, g):
            seen["n"] += g.numel()
            seen["clamped"] += int((g.abs() > clip).sum())
            return g.clamp(-clip, clip)

    t = {x: torch.tensor(a, dtype=torch.float64, requires_grad=True) for x, a in d.items()}
    q, k, v, f, W, w_r, H = t["q"], t["k"], t["v"], t["f"], t["W"], t["w_r"], t["H0"]
    T = q.shape[1]
    L = torch.zeros((), dtype=torch.float64)
    for s in range(T):
        Hin = ClampGrad.apply(H)
        P = torch.matmul(Hin, W) + k[:, s, :, :, None] * v[:, s, :, None, :]
        fs = f[:, s, :, None, None]
        H = fs * Hin + (1 - fs) * torch.tanh(P)
        y = (H * q[:, s, :, :, None]).sum(dim=2) + w_r * v[:, s]
        L = L + (y * torch.from_numpy(dy[:, s])).sum()
    L = L + (H * torch.from_numpy(dHT)).sum()
    grads = torch.autograd.grad(L, [t[x] for x in ("q", "k", "v", "f", "W", "w_r", "H0")])
    names = ("dq", "dk", "dv", "df", "dW", "dw_r", "dH0")
    return {n: g.numpy() for n, g in zip(names, grads)}, seen["clamped"] / max(1, seen["n"])


@pytest.mark.parametrize("B,T,N,K,V,clip", [(2, 7, 2, 3, 4, 0.6), (1, 9, 3, 4, 2, 1.5)])
def test_clipped_gradients_match_autograd_with_a_clamping_identity(B, T, N, K, V, clip):
    d = inputs.make_inputs(B, T, N, K, V, qkv_dtype="f32", seed=91 + T, with_H0=True, with_dy=True, with_dHT=True)
    d = {x: (a.astype(np.float64) if a is not None else None) for x, a in d.items()}
    d["W"] *= 1.5
    d["k"] *= 3.0
    dy, dHT = 4.0 * d.pop("dy"), d.pop("dH_T")
    g = oracle.ref_bwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], dy, dHT, clip=clip)
    ref, frac = _autograd_clipped(d, dy, dHT, clip)
    assert 0.05 < frac < 0.95, frac  # the bound binds on some elements, not all
    for n in ref:
        scale = max(1e-3, float(np.max(np.abs(ref[n]))))
        assert np.max(np.abs(g[n] - ref[n])) <= 1e-12 * scale, n
    assert np.max(np.abs(g["dH0"])) <= clip
    exact = oracle.ref_bwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], dy, dHT)
    assert not np.allclose(exact["dW"], g["dW"])


def test_clip_above_every_gradient_is_exact():
    d = inputs.make_inputs(2, 6, 2, 3, 4, qkv_dtype="f32", seed=5, with_H0=True, with_dy=True, with_dHT=True)
    d = {x: (a.astype(np.float64) if a is not None else None) for x, a in d.items()}
    args = (d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], d["H0"], d["dy"], d["dH_T"])
    exact = oracle.ref_bwd(*args)
    loose = oracle.ref_bwd(*args, clip=1e30)
    for n in exact:
        assert np.array_equal(exact[n], loose[n]), n
    with pytest.raises(ValueError):
        oracle.ref_bwd(*args, clip=-1.0)
