"""Seeded synthetic inputs for the M²RNN recurrence.

This module only draws random tensors; it holds none of the recurrence's arithmetic and is the
one piece shared by the fp64 oracle's tests and by the GPU path's tests, smoke run and bench.

Random stream
-------------
Every tensor has its own counter-based SplitMix64 stream (Steele, Lea & Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): draw ``i`` (0-based) of the stream with key ``s``
is ``mix64(s + (i + 1) * 0x9E3779B97F4A7C15)`` where ``mix64`` is SplitMix64's finaliser
(xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift 27, multiply 0x94D049BB133111EB,
xor-shift 31), all mod 2**64.  The key of tensor ``id`` under seed ``S`` is
``S xor (id * 0x9E3779B97F4A7C15)``.  A uniform in (0, 1) is ``((x >> 11) + 0.5) * 2**-53``;
normals come from Box–Muller on consecutive pairs of uniforms.  Tensors are filled in
row-major order, so a tensor's contents do not depend on how it is later sliced.

Value distributions (``N(mu, s2)`` names the *variance* s2)
-----------------------------------------------------------
* q, k ~ N(0, 1/K); v ~ N(0, 1) — stored in fp32, or rounded to bf16 (round to nearest even)
  when the workload keeps q/k/v in bf16.  The arrays returned here already hold the rounded
  values, so every consumer reads the very same numbers.
* f = sigmoid(N(mu_f, 1)) per (batch, step, head): mu_f = 1.5, or 3 for the long-retention
  16K-token workload.
* W per head = 0.9 x a Haar-random orthogonal V x V matrix (Householder QR of a Gaussian
  matrix, columns sign-fixed by diag(R)), so its spectral norm is 0.9.
* w_r ~ N(0, 0.1); H0 = 0 unless asked for (then uniform in [-1, 1]); dy ~ N(0, 1).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Optional

import numpy as np

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK64 = (1 << 64) - 1
_BLOCK = 1 << 21  # draws per vectorised block (bounds each thread's temporaries to ~50 MB)

TENSOR_IDS = {"q": 1, "k": 2, "v": 3, "f": 4, "W": 5, "w_r": 6, "H0": 7, "dy": 8, "dH_T": 9}
BASE_SEED = 0x4D32524E


def stream_key(seed: int, tensor_id: int) -> int:
    return (seed ^ ((tensor_id * _GAMMA) & _MASK64)) & _MASK64


def splitmix64(key: int, start: int, count: int) -> np.ndarray:
    """Draws ``start .. start+count-1`` of the SplitMix64 stream with the given key (uint64)."""
    out = np.empty(count, dtype=np.uint64)
    g = np.uint64(_GAMMA)
    m1 = np.uint64(_M1)
    m2 = np.uint64(_M2)
    s30, s27, s31 = np.uint64(30), np.uint64(27), np.uint64(31)
    kk = np.uint64(key)
    for b0 in range(0, count, _BLOCK):
        n = min(_BLOCK, count - b0)
        z = np.arange(start + b0 + 1, start + b0 + 1 + n, dtype=np.uint64)
        with np.errstate(over="ignore"):
            z *= g
            z += kk
            z ^= z >> s30
            z *= m1
            z ^= z >> s27
            z *= m2
            z ^= z >> s31
        out[b0:b0 + n] = z
    return out


def uniform01(key: int, start: int, count: int) -> np.ndarray:
    x = splitmix64(key, start, count)
    return ((x >> np.uint64(11)).astype(np.float64) + 0.5) * (2.0 ** -53)


def _threads() -> int:
    try:
        return max(1, min(16, len(os.sched_getaffinity(0))))
    except AttributeError:  # pragma: no cover
        return max(1, min(16, os.cpu_count() or 1))


def normal(key: int, count: int, mean: float = 0.0, var: float = 1.0) -> np.ndarray:
    """``count`` fp64 normals N(mean, var) from stream ``key`` (Box–Muller on uniform pairs).

    The stream is counter-based, so blocks are drawn in parallel threads; the result does not
    depend on the thread count."""
    out = np.empty(count, dtype=np.float64)
    npairs = (count + 1) // 2
    sd = float(np.sqrt(var))

    def block(p0: int) -> None:
        p = min(_BLOCK // 2, npairs - p0)
        u = uniform01(key, 2 * p0, 2 * p)
        u1, u2 = u[0::2], u[1::2]
        r = np.sqrt(-2.0 * np.log(u1))
        ang = (2.0 * np.pi) * u2
        z = np.empty(2 * p, dtype=np.float64)
        z[0::2] = r * np.cos(ang)
        z[1::2] = r * np.sin(ang)
        lo = 2 * p0
        hi = min(count, lo + 2 * p)
        out[lo:hi] = z[: hi - lo] * sd + mean

    starts = list(range(0, npairs, _BLOCK // 2))
    if len(starts) <= 1:
        for p0 in starts:
            block(p0)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=_threads()) as ex:
            list(ex.map(block, starts))
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as fp32 holding the bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    # No carry leaves 32 bits for finite inputs (largest: 0xFF7FFFFF + 0x8000).
    out = (bits >> np.uint32(16)) & np.uint32(1)
    out += np.uint32(0x7FFF)
    out += bits
    out &= np.uint32(0xFFFF0000)
    return out.view(np.float32)


def haar_orthogonal(g: np.ndarray) -> np.ndarray:
    """Haar-distributed orthogonal matrix from a square Gaussian matrix (QR, sign-fixed)."""
    qm, rm = np.linalg.qr(g)
    d = np.sign(np.diag(rm))
    d[d == 0] = 1.0
    return qm * d[None, :]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    N: int
    K: int
    V: int
    qkv_dtype: str  # "f32" or "bf16"
    f_mean: float
    seed: int
    backward: bool = False
    decode: bool = False  # one step with a given state (H0 drawn), the token-by-token form
    shared_qk: bool = False  # one query/key shared by all heads (q, k drawn as [B, T, 1, K])
    note: str = ""

    @property
    def head_steps(self) -> int:
        return self.B * self.N * self.T


WORKLOADS: Dict[str, Workload] = {
    "tiny_f32": Workload("tiny_f32", 1, 64, 2, 16, 16, "f32", 1.5, BASE_SEED + 0,
                         note="B1 N2 T64 K=V=16, fp32 q/k/v, forward only"),
    "b4_h16_t2048_kv64": Workload("b4_h16_t2048_kv64", 4, 2048, 16, 64, 64, "bf16", 1.5, BASE_SEED + 1,
                                  note="B4 N16 T2048 K=V=64, bf16 q/k/v, fp32 state"),
    "long_b2_h32_t16384_kv64": Workload("long_b2_h32_t16384_kv64", 2, 16384, 32, 64, 64, "bf16", 3.0,
                                        BASE_SEED + 2,
                                        note="16K-token context, B2 N32 K=V=64, f=sigmoid(N(3,1))"),
    "b8_h16_t4096_kv128": Workload("b8_h16_t4096_kv128", 8, 4096, 16, 128, 128, "bf16", 1.5, BASE_SEED + 3,
                                   note="larger state, B8 N16 T4096 K=V=128"),
    "b1_h16_t4096_kv128": Workload("b1_h16_t4096_kv128", 1, 4096, 16, 128, 128, "bf16", 1.5, BASE_SEED + 3,
                                   note="larger state at batch 1 (row split across workgroups)"),
    "bwd_b4_h16_t4096_kv64": Workload("bwd_b4_h16_t4096_kv64", 4, 4096, 16, 64, 64, "f32", 1.5, BASE_SEED + 4,
                                      backward=True,
                                      note="forward + BPTT, B4 N16 T4096 K=V=64, fp32 q/k/v"),
    "paper_b4_h128_t4096_k64_v16": Workload("paper_b4_h128_t4096_k64_v16", 4, 4096, 128, 64, 16, "bf16", 1.5,
                                            BASE_SEED + 6, shared_qk=True,
                                            note="the pages' head shape K=64, V=16 with one query/key shared "
                                                 "by all 128 value heads, 4K context, bf16 q/k/v"),
    "decode_b128_h32_kv64": Workload("decode_b128_h32_kv64", 128, 1, 32, 64, 64, "bf16", 1.5, BASE_SEED + 5,
                                     decode=True,
                                     note="one decode step at batch 128, N32 K=V=64, bf16 q/k/v, state in HBM"),
}


def make_inputs(B: int, T: int, N: int, K: int, V: int, *, qkv_dtype: str = "f32", f_mean: float = 1.5,
                seed: int = BASE_SEED, with_H0: bool = False, with_dy: bool = False,
                with_dHT: bool = False, w_scale: float = 0.9,
                shared_qk: bool = False) -> Dict[str, Optional[np.ndarray]]:
    """All inputs of one workload as fp32 numpy arrays (bf16-exact where q/k/v are bf16).

    With ``shared_qk`` q and k are [B, T, 1, K]: one query/key for all N heads."""
    if qkv_dtype not in ("f32", "bf16"):
        raise ValueError(f"qkv_dtype must be 'f32' or 'bf16', got {qkv_dtype!r}")
    key = lambda name: stream_key(seed, TENSOR_IDS[name])  # noqa: E731

    def qkv(name, count, var, shape):
        a = normal(key(name), count, 0.0, var).astype(np.float32)
        if qkv_dtype == "bf16":
            a = round_to_bf16(a)
        return a.reshape(shape)

    out: Dict[str, Optional[np.ndarray]] = {}
    Nqk = 1 if shared_qk else N
    out["q"] = qkv("q", B * T * Nqk * K, 1.0 / K, (B, T, Nqk, K))
    out["k"] = qkv("k", B * T * Nqk * K, 1.0 / K, (B, T, Nqk, K))
    out["v"] = qkv("v", B * T * N * V, 1.0, (B, T, N, V))
    z = normal(key("f"), B * T * N, f_mean, 1.0)
    out["f"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32).reshape(B, T, N)
    g = normal(key("W"), N * V * V).reshape(N, V, V)
    out["W"] = np.stack([w_scale * haar_orthogonal(g[n]) for n in range(N)]).astype(np.float32)
    out["w_r"] = normal(key("w_r"), N * V, 0.0, 0.1).astype(np.float32).reshape(N, V)
    if with_H0:
        out["H0"] = (2.0 * uniform01(key("H0"), 0, B * N * K * V) - 1.0).astype(np.float32).reshape(B, N, K, V)
    else:
        out["H0"] = None
    out["dy"] = normal(key("dy"), B * T * N * V).astype(np.float32).reshape(B, T, N, V) if with_dy else None
    out["dH_T"] = (normal(key("dH_T"), B * N * K * V).astype(np.float32).reshape(B, N, K, V)
                   if with_dHT else None)
    return out


def workload_inputs(name: str, **overrides) -> Dict[str, Optional[np.ndarray]]:
    """Inputs of a named workload; ``overrides`` may change B, T, N (same seed and recipe)."""
    w = WORKLOADS[name]
    dims = dict(B=w.B, T=w.T, N=w.N, K=w.K, V=w.V)
    dims.update({k: v for k, v in overrides.items() if k in dims})
    extra = {k: v for k, v in overrides.items() if k not in dims}
    extra.setdefault("with_dy", w.backward)
    extra.setdefault("with_H0", w.decode)
    extra.setdefault("shared_qk", w.shared_qk)
    return make_inputs(dims["B"], dims["T"], dims["N"], dims["K"], dims["V"], qkv_dtype=w.qkv_dtype,
                       f_mean=w.f_mean, seed=w.seed, **extra)
