"""The allocation-free forward, m2rnn_fwd_noalloc, called through the C ABI: it must give m2rnn_fwd's
bits (y and H_T) on two calls in a row, the second smaller, and refuse a size beyond its fixed
device array."""
import ctypes

import numpy as np
import pytest

import matrix_state_nonlinear_m2rnn_amd as m2
from matrix_state_nonlinear_m2rnn_amd import inputs

from _gpu import say, to_device, torch_cuda

pytestmark = pytest.mark.gpu


def noalloc(dd, dtype, math="f16x3", H0=None):
    torch = torch_cuda()
    q, v = dd["q"], dd["v"]
    B, T, Nqk, K = q.shape
    N, V = v.shape[2], v.shape[3]
    y = torch.empty((B, T, N, V), dtype=torch.float32, device="cuda")
    H_T = torch.empty((B, N, K, V), dtype=torch.float32, device="cuda")
    dims = m2.Dims(B, T, N, K, V, Nqk)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = m2.lib().m2rnn_fwd_noalloc(ctypes.byref(dims), m2.DTYPE_BF16 if dtype == "bf16" else m2.DTYPE_F32,
                                   m2.MATH[math], 0, p(q), p(dd["k"]), p(v), p(dd["f"]), p(dd["W"]), p(dd["w_r"]),
                                   p(H0), p(y), p(H_T), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, y, H_T


def test_noalloc_equals_the_workspace_forward():
    torch = torch_cuda()
    # 1. The 16K-token workload: B2 N32 T16384 K=V=64 (rows split over four workgroups), many time
    #    segments through the fixed array; 2. a smaller call right after it (one segment, a supplied
    #    H0, ragged T); 3. one workgroup per pair (the array unused).
    cases = [("long_b2_h32_t16384_kv64", None), ((1, 300, 8, 64, 64, 12), "H0"), ((2, 77, 3, 16, 32, 13), None)]
    for spec, h0 in cases:
        if isinstance(spec, str):
            w = inputs.WORKLOADS[spec]
            d, dtype = inputs.workload_inputs(spec), w.qkv_dtype
        else:
            B, T, N, K, V, seed = spec
            d, dtype = inputs.make_inputs(B, T, N, K, V, qkv_dtype="bf16", seed=seed, with_H0=h0 is not None), "bf16"
        say("noalloc", spec)
        dd = to_device(d, dtype)
        H0 = dd.get("H0")
        st, y, H_T = noalloc(dd, dtype, H0=H0)
        assert st == m2.M2RNN_OK, m2.status_string(st)
        y0, H0T = m2.m2rnn_fwd(dd["q"], dd["k"], dd["v"], dd["f"], dd["W"], dd["w_r"], H0, math="f16x3")
        torch.cuda.synchronize()
        say("max diff", float((y - y0).abs().max()), float((H_T - H0T).abs().max()))
        assert torch.equal(y, y0) and torch.equal(H_T, H0T)


def test_noalloc_refuses_sizes_beyond_its_array():
    torch_cuda()
    n = ctypes.c_size_t(0)
    assert m2.lib().m2rnn_fwd_noalloc_max_bytes(ctypes.byref(n)) == m2.M2RNN_OK
    # two states of B N K V floats beyond the array: B64 N32 K=V=128 (256 MiB each)
    dims = m2.Dims(64, 32, 32, 128, 128)
    p = ctypes.c_void_p(256)
    st = m2.lib().m2rnn_fwd_noalloc(ctypes.byref(dims), m2.DTYPE_BF16, m2.MATH["f16x3"], 0, p, p, p, p, p, p, None, p,
                                   p, None)
    assert st == m2.M2RNN_EUNSUPPORTED
    assert 2 * 64 * 32 * 128 * 128 * 4 > n.value
