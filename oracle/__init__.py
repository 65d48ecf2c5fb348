"""fp64 CPU oracle for the M²RNN recurrence — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may import
this package.  The GPU product path (``matrix_state_nonlinear_m2rnn_amd``) never imports it and
shares no code with it; the only common module is the seeded input generator.

The arithmetic lives in ``m2rnn_ref.c`` (plain fp64 loops in the order of the M²RNN reading notes'
§2.1 Eq. (10)-(12) for the forward and §2.7's corrected BPTT for the backward); this file only
builds that library with gcc and marshals numpy arrays into it.

The steps on either side of the recurrence (the gate of §2.2, the output gate + RMSNorm and the
causal conv4 + SiLU of §2.3) are plain numpy fp64 in ``oracle/block.py``.

Pins: every function here is pinned by ``tests/test_oracle_*.py`` against facts that do not come
from the oracle itself (closed forms, invariants, a library tanh-RNN, finite differences).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "m2rnn_ref.c")
_LIB_PATH = os.path.join(_HERE, "libm2rnn_ref.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (portable -O2, no -march=native, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, dp, ci = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_int
        lib.m2rnn_ref_fwd.argtypes = [i64] * 5 + [dp] * 9 + [ci]
        lib.m2rnn_ref_fwd.restype = ci
        lib.m2rnn_ref_bwd.argtypes = [i64] * 5 + [dp] * 9 + [ctypes.c_double] + [dp] * 7 + [ci]
        lib.m2rnn_ref_bwd.restype = ci
        _lib = lib
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _d(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q, v):
    B, T, N, K = q.shape
    V = v.shape[3]
    return B, T, N, K, V


def ref_fwd(q, k, v, f, W, w_r, H0=None, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """Forward recurrence in fp64: returns (y [B,T,N,V], H_T [B,N,K,V])."""
    q, k, v, f, W, w_r, H0 = map(_d, (q, k, v, f, W, w_r, H0))
    B, T, N, K, V = _dims(q, v)
    _check(q, k, v, f, W, w_r, H0, B, T, N, K, V)
    y = np.empty((B, T, N, V), dtype=np.float64)
    H_T = np.empty((B, N, K, V), dtype=np.float64)
    rc = _load().m2rnn_ref_fwd(B, T, N, K, V, _p(q), _p(k), _p(v), _p(f), _p(W), _p(w_r), _p(H0),
                               _p(y), _p(H_T), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"m2rnn_ref_fwd failed with status {rc}")
    return y, H_T


def ref_bwd(q, k, v, f, W, w_r, H0, dy, dH_T=None, nthreads: int = 0, clip: float = 0.0) -> Dict[str, np.ndarray]:
    """BPTT in fp64 for L = sum <dy, y> + <dH_T, H_T>: returns dq, dk, dv, df, dW, dw_r, dH0.

    clip > 0 clamps every element of the gradient each step sends back to its input state,
    C_{t-1} = f_t R_t + D_t W^T, to [-clip, clip] (the per-step recurrent-gradient clipping of the
    M²RNN notes §2.3, read as an elementwise bound); clip = 0 gives the exact gradient."""
    if not clip >= 0.0:
        raise ValueError("clip must be >= 0")
    q, k, v, f, W, w_r, H0, dy, dH_T = map(_d, (q, k, v, f, W, w_r, H0, dy, dH_T))
    B, T, N, K, V = _dims(q, v)
    _check(q, k, v, f, W, w_r, H0, B, T, N, K, V)
    if dy.shape != (B, T, N, V):
        raise ValueError("dy must be [B,T,N,V]")
    if dH_T is not None and dH_T.shape != (B, N, K, V):
        raise ValueError("dH_T must be [B,N,K,V]")
    out = {
        "dq": np.empty((B, T, N, K)), "dk": np.empty((B, T, N, K)), "dv": np.empty((B, T, N, V)),
        "df": np.empty((B, T, N)), "dW": np.empty((N, V, V)), "dw_r": np.empty((N, V)),
        "dH0": np.empty((B, N, K, V)),
    }
    rc = _load().m2rnn_ref_bwd(B, T, N, K, V, _p(q), _p(k), _p(v), _p(f), _p(W), _p(w_r), _p(H0), _p(dy),
                               _p(dH_T), float(clip), _p(out["dq"]), _p(out["dk"]), _p(out["dv"]), _p(out["df"]),
                               _p(out["dW"]), _p(out["dw_r"]), _p(out["dH0"]), nthreads or default_threads())
    if rc != 0:
        raise RuntimeError(f"m2rnn_ref_bwd failed with status {rc}")
    return out


def _check(q, k, v, f, W, w_r, H0, B, T, N, K, V):
    if k.shape != (B, T, N, K):
        raise ValueError("k must match q [B,T,N,K]")
    if v.shape[:3] != (B, T, N):
        raise ValueError("v must be [B,T,N,V]")
    if f.shape != (B, T, N):
        raise ValueError("f must be [B,T,N]")
    if W.shape != (N, V, V):
        raise ValueError("W must be [N,V,V]")
    if w_r.shape != (N, V):
        raise ValueError("w_r must be [N,V]")
    if H0 is not None and H0.shape != (B, N, K, V):
        raise ValueError("H0 must be [B,N,K,V]")
