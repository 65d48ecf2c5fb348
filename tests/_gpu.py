"""Shared helpers of the GPU parity tests: move seeded inputs to the device, run the HIP path
through the C ABI, and run the fp64 oracle on the same inputs (whole tensors or single units)."""
import sys

import numpy as np
import pytest

import oracle
from matrix_state_nonlinear_m2rnn_amd import inputs

TOL = {"f32": 5e-4, "f16x3": 5e-4, "bf16x3": 5e-4, "bf16": 2e-2}


def torch_cuda():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch


def say(*msg):
    print("[case]", *msg, flush=True)
    sys.stdout.flush()


def to_device(d, qkv_dtype):
    torch = torch_cuda()
    out = {}
    for name, a in d.items():
        if a is None:
            out[name] = None
            continue
        t = torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
        if name in ("q", "k", "v") and qkv_dtype == "bf16":
            t = t.to(torch.bfloat16)  # exact: the generator already rounded to bf16
        out[name] = t.contiguous()
    return out


def gpu_fwd(dd, math, row_blocks=0, H0=None):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    y, H_T = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], H0 if H0 is not None else dd.get("H0"),
                          math=math, row_blocks=row_blocks)
    torch.cuda.synchronize()
    return y.cpu().numpy().astype(np.float64), H_T.cpu().numpy().astype(np.float64)


def per_head_qk(d):
    """q, k broadcast to every head when one query/key is shared ([B,T,1,K] -> [B,T,N,K]): the
    oracle takes per-head q and k."""
    N = d["v"].shape[2]
    if d["q"].shape[2] == N:
        return d
    e = dict(d)
    for x in ("q", "k"):
        e[x] = np.ascontiguousarray(np.broadcast_to(d[x], d[x].shape[:2] + (N, d[x].shape[3])))
    return e


def oracle_fwd(d, H0=None):
    d = per_head_qk(d)
    return oracle.ref_fwd(d["q"], d["k"], d["v"], d["f"], d["W"], d["w_r"], H0 if H0 is not None else d.get("H0"))


def oracle_units(d, units):
    """Oracle outputs for a list of (b, n) units: dict (b, n) -> (y [T,V], H_T [K,V])."""
    out = {}
    nq = lambda n: 0 if d["q"].shape[2] == 1 else n  # noqa: E731
    for b, n in units:
        sub = dict(q=d["q"][b:b + 1, :, nq(n):nq(n) + 1], k=d["k"][b:b + 1, :, nq(n):nq(n) + 1], v=d["v"][b:b + 1, :, n:n + 1],
                   f=d["f"][b:b + 1, :, n:n + 1], W=d["W"][n:n + 1], w_r=d["w_r"][n:n + 1],
                   H0=None if d.get("H0") is None else d["H0"][b:b + 1, n:n + 1])
        y, H = oracle_fwd(sub)
        out[(b, n)] = (y[0, :, 0], H[0, 0])
    return out


def max_abs(a, b):
    return float(np.max(np.abs(np.asarray(a, dtype=np.float64) - np.asarray(b, dtype=np.float64)))) if np.size(a) else 0.0


def gpu_bwd(dd, math="auto", dH_T=None, want_dH0=True, grad_clip=0.0):
    torch = torch_cuda()
    import matrix_state_nonlinear_m2rnn_amd as m2
    g = m2.m2rnn_bwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], dd.get("H0"), dd["dy"],
                     dH_T if dH_T is not None else dd.get("dH_T"), math=math, want_dH0=want_dH0, grad_clip=grad_clip)
    torch.cuda.synchronize()
    return {name: (t.cpu().numpy().astype(np.float64) if t is not None else None) for name, t in g.items()}


def oracle_bwd(d, clip=0.0):
    """Oracle gradients; with a shared query/key, dq and dk are summed over the heads (§2.7)."""
    shared = d["q"].shape[2] != d["v"].shape[2]
    e = per_head_qk(d)
    g = oracle.ref_bwd(e["q"], e["k"], e["v"], e["f"], e["W"], e["w_r"], e.get("H0"), e["dy"], e.get("dH_T"),
                       clip=clip)
    if shared:
        g["dq"] = g["dq"].sum(axis=2, keepdims=True)
        g["dk"] = g["dk"].sum(axis=2, keepdims=True)
    return g


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    if den == 0.0:
        return float(np.linalg.norm(a))
    return float(np.linalg.norm(a - b) / den)
