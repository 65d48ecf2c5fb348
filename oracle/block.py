"""fp64 CPU oracle for the steps on either side of the M²RNN recurrence — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this module; the GPU product path never imports it and shares no code with it.

Source: the reading notes "M²RNN：矩阵状态非线性 RNN 的容量、表达力与系统代价" (arXiv:2603.14360v2),
cited as "M²RNN notes".  Plain numpy in fp64, in the order the notes write each formula:

* gate (§2.2, Eq. 13/17):       f = (1 + e^{a + beta})^{-alpha} = exp(-alpha * softplus(a + beta)),
                                per (batch, step, head) with alpha, beta per head;
* output gate + RMSNorm (§2.3 step 4, Appendix C, Eq. 26-33):
                                x = y (.) SiLU(gz);  s = (mean_j x_j^2 + eps)^{-1/2};  out = gamma (.) x s,
                                normalised over the D = N V features of one (batch, step) — the
                                gate multiplies before the norm; eps is the caller's (the notes
                                leave it out);
* causal depthwise Conv1D of kernel size 4 + SiLU (§2.3 step 1):
                                u_t[c] = SiLU(sum_{i<4} w[c][i] x_{t-3+i}[c] + bias[c]), with
                                x_t = 0 for t < 0.

Each backward is the chain rule of its forward written out by hand; the RMSNorm backward is the
Appendix C expression grad_x_i = s p_i - r s^3 x_i / D with p = gamma (.) grad_out and
r = sum_j p_j x_j.  Pins: ``tests/test_oracle_block.py``.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def softplus(x):
    # log(1 + e^x), evaluated without overflow: max(x, 0) + log(1 + e^{-|x|}).
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def silu(x):
    return x * sigmoid(x)


def silu_grad(x):
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


# ------------------------------------------------------------------ gate (§2.2)

def gate_fwd(a, alpha, beta):
    """f [B,T,N] from the pre-activation a [B,T,N] and the per-head alpha, beta [N]."""
    a, alpha, beta = map(_f64, (a, alpha, beta))
    return np.exp(-alpha * softplus(a + beta))


def gate_bwd(a, alpha, beta, df) -> Dict[str, np.ndarray]:
    """da [B,T,N], dalpha [N], dbeta [N] for the loss sum <df, f>."""
    a, alpha, beta, df = map(_f64, (a, alpha, beta, df))
    z = a + beta
    f = np.exp(-alpha * softplus(z))
    da = df * f * (-alpha * sigmoid(z))        # d softplus(z) / dz = sigmoid(z)
    dalpha = np.sum(df * f * (-softplus(z)), axis=(0, 1))
    dbeta = np.sum(da, axis=(0, 1))
    return {"da": da, "dalpha": dalpha, "dbeta": dbeta}


# ------------------------------------------------------------------ output gate + RMSNorm (§2.3, App. C)

def out_norm_fwd(y, gz, gamma, eps):
    """out [B,T,N,V] = RMSNorm over the N V features of y (.) SiLU(gz), scaled by gamma [N,V]."""
    y, gz, gamma = map(_f64, (y, gz, gamma))
    B, T, N, V = y.shape
    x = (y * silu(gz)).reshape(B, T, N * V)
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return (gamma.reshape(1, 1, N * V) * x * s).reshape(B, T, N, V)


def out_norm_bwd(y, gz, gamma, eps, dout) -> Dict[str, np.ndarray]:
    """dy, dgz [B,T,N,V] and dgamma [N,V] for the loss sum <dout, out> (Appendix C)."""
    y, gz, gamma, dout = map(_f64, (y, gz, gamma, dout))
    B, T, N, V = y.shape
    D = N * V
    g = silu(gz).reshape(B, T, D)
    yy = y.reshape(B, T, D)
    x = yy * g
    s = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    do = dout.reshape(B, T, D)
    p = gamma.reshape(1, 1, D) * do
    r = np.sum(p * x, axis=-1, keepdims=True)
    dx = s * p - r * s ** 3 * x / D
    dgamma = np.sum(do * x * s, axis=(0, 1)).reshape(N, V)
    dy = (dx * g).reshape(B, T, N, V)
    dgz = (dx * yy * silu_grad(gz.reshape(B, T, D))).reshape(B, T, N, V)
    return {"dy": dy, "dgz": dgz, "dgamma": dgamma}


# ------------------------------------------------------------------ causal conv4 + SiLU (§2.3)

def conv4_silu_fwd(x, w, bias: Optional[np.ndarray] = None):
    """u [B,T,C] from x [B,T,C], w [C,4] (tap i multiplies x_{t-3+i}) and bias [C] or None."""
    x, w, bias = map(_f64, (x, w, bias))
    B, T, C = x.shape
    pre = np.zeros((B, T, C))
    for t in range(T):
        for i in range(4):
            src = t - 3 + i
            if src >= 0:
                pre[:, t, :] += w[:, i] * x[:, src, :]
    if bias is not None:
        pre += bias
    return silu(pre)


def conv4_silu_bwd(x, w, bias, du) -> Dict[str, np.ndarray]:
    """dx [B,T,C], dw [C,4], dbias [C] for the loss sum <du, u>."""
    x, w, bias, du = map(_f64, (x, w, bias, du))
    B, T, C = x.shape
    pre = np.zeros((B, T, C))
    for t in range(T):
        for i in range(4):
            src = t - 3 + i
            if src >= 0:
                pre[:, t, :] += w[:, i] * x[:, src, :]
    if bias is not None:
        pre += bias
    dpre = du * silu_grad(pre)
    dx = np.zeros((B, T, C))
    dw = np.zeros((C, 4))
    for t in range(T):
        for i in range(4):
            src = t - 3 + i
            if src >= 0:
                dx[:, src, :] += w[:, i] * dpre[:, t, :]
                dw[:, i] += np.sum(dpre[:, t, :] * x[:, src, :], axis=0)
    return {"dx": dx, "dw": dw, "dbias": np.sum(dpre, axis=(0, 1))}
