"""MI355X (gfx950) M²RNN recurrence: thin Python binding of libm2rnn.so.

The functions here carry the names of the C entry points in ``include/m2rnn.h`` and only marshal
arguments: they check devices, dtypes and shapes of torch tensors, allocate outputs and the
workspace with torch (device memory and streams are all torch is used for), and pass raw device
pointers plus the current HIP stream to the library.  Every step of the recurrence runs in the
library's HIP kernels.  There is no fallback: if ``libm2rnn.so`` is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
import sys
from typing import Dict, Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libm2rnn.so")

M2RNN_OK = 0
M2RNN_EINVAL = -1
M2RNN_EUNSUPPORTED = -2
M2RNN_EWORKSPACE = -3
M2RNN_EHIP = -4

DTYPE_F32 = 0
DTYPE_BF16 = 1
MATH = {"auto": -1, "f32": 0, "f16x3": 1, "bf16x3": 2, "bf16": 3}
BWD_CHECKPOINT = 64

EXPORTED = (
    "m2rnn_version", "m2rnn_status_string", "m2rnn_last_hip_error", "m2rnn_fwd_workspace_size", "m2rnn_fwd",
    "m2rnn_scan_fwd", "m2rnn_scan_fwd_finish", "m2rnn_bwd_workspace_size", "m2rnn_bwd", "m2rnn_decode_step",
    "m2rnn_fwd_ckpt", "m2rnn_bwd_ckpt_workspace_size", "m2rnn_bwd_ckpt", "m2rnn_checkpoint_interval",
    "m2rnn_gate_fwd", "m2rnn_gate_bwd_workspace_size", "m2rnn_gate_bwd",
    "m2rnn_out_norm_fwd", "m2rnn_out_norm_bwd_workspace_size", "m2rnn_out_norm_bwd",
    "m2rnn_conv4_silu_fwd", "m2rnn_conv4_silu_bwd_workspace_size", "m2rnn_conv4_silu_bwd",
    "m2rnn_fwd_block_workspace_size", "m2rnn_fwd_block", "m2rnn_overlap_create", "m2rnn_overlap_destroy",
    "m2rnn_fwd_noalloc", "m2rnn_fwd_noalloc_max_bytes", "m2rnn_scan_bwd", "m2rnn_scan_bwd_finish",
)


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int64), ("T", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("V", ctypes.c_int64), ("Nqk", ctypes.c_int64)]


class M2RNNError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str, hip_error: int = 0):
        extra = f" (hipError {hip_error})" if status == M2RNN_EHIP else ""
        super().__init__(f"{fn} failed: {msg} [status {status}]{extra}")
        self.status = status


_lib = None

# The C ABI version these bindings are written for (M2RNN_VERSION in include/m2rnn.h).
ABI_VERSION = 400


def lib() -> ctypes.CDLL:
    """Loads libm2rnn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                               "g.build()'` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, sz, ci = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        dp = ctypes.POINTER(Dims)
        L.m2rnn_version.restype = ci
        L.m2rnn_version.argtypes = []
        if L.m2rnn_version() != ABI_VERSION:
            raise RuntimeError(f"{LIB_PATH} has ABI version {L.m2rnn_version()}, these bindings expect {ABI_VERSION}: "
                               "rebuild it with `python -c 'import __graft_entry__ as g; g.build()'`")
        L.m2rnn_status_string.restype = ctypes.c_char_p
        L.m2rnn_status_string.argtypes = [ci]
        L.m2rnn_last_hip_error.restype = ci
        L.m2rnn_last_hip_error.argtypes = []
        L.m2rnn_fwd_workspace_size.restype = ci
        L.m2rnn_fwd_workspace_size.argtypes = [dp, ci, ci, ci, ctypes.POINTER(sz)]
        fwd_args = [dp, ci, ci, ci] + [vp] * 3 + [vp] * 4 + [vp, vp] + [vp, sz, vp]
        for name in ("m2rnn_scan_fwd", "m2rnn_scan_fwd_finish"):
            fn = getattr(L, name)
            fn.restype = ci
            fn.argtypes = fwd_args
        L.m2rnn_fwd.restype = ci
        L.m2rnn_fwd.argtypes = fwd_args + [vp]
        L.m2rnn_fwd_noalloc.restype = ci
        L.m2rnn_fwd_noalloc.argtypes = [dp, ci, ci, ci] + [vp] * 3 + [vp] * 4 + [vp, vp] + [vp]
        L.m2rnn_fwd_noalloc_max_bytes.restype = ci
        L.m2rnn_fwd_noalloc_max_bytes.argtypes = [ctypes.POINTER(sz)]
        L.m2rnn_overlap_create.restype = ci
        L.m2rnn_overlap_create.argtypes = [ctypes.POINTER(vp)]
        L.m2rnn_overlap_destroy.restype = ci
        L.m2rnn_overlap_destroy.argtypes = [vp]
        if hasattr(L, "m2rnn_bwd"):
            L.m2rnn_bwd_workspace_size.restype = ci
            L.m2rnn_bwd_workspace_size.argtypes = [dp, ci, ci, ctypes.POINTER(sz)]
            L.m2rnn_bwd.restype = ci
            L.m2rnn_bwd.argtypes = ([dp, ci, ci] + [vp] * 3 + [vp] * 4 + [vp, vp] + [ctypes.c_float] + [vp] * 7
                                    + [vp, sz, vp])
        L.m2rnn_checkpoint_interval.restype = ci
        L.m2rnn_checkpoint_interval.argtypes = [dp, ctypes.POINTER(ctypes.c_int64)]
        L.m2rnn_fwd_ckpt.restype = ci
        L.m2rnn_fwd_ckpt.argtypes = [dp, ci, ci, ci] + [vp] * 3 + [vp] * 4 + [vp, vp, vp] + [vp, sz, vp, vp]
        L.m2rnn_bwd_ckpt_workspace_size.restype = ci
        L.m2rnn_bwd_ckpt_workspace_size.argtypes = [dp, ci, ci, ctypes.POINTER(sz)]
        for name in ("m2rnn_bwd_ckpt", "m2rnn_scan_bwd", "m2rnn_scan_bwd_finish"):
            fn = getattr(L, name)
            fn.restype = ci
            fn.argtypes = ([dp, ci, ci] + [vp] * 3 + [vp] * 3 + [vp] + [vp, vp] + [ctypes.c_float] + [vp] * 7
                           + [vp, sz, vp])
        i64, cf = ctypes.c_int64, ctypes.c_float
        for name, args in (
            ("m2rnn_gate_fwd", [i64] * 3 + [vp] * 4 + [vp]),
            ("m2rnn_gate_bwd_workspace_size", [i64] * 3 + [ctypes.POINTER(sz)]),
            ("m2rnn_gate_bwd", [i64] * 3 + [vp] * 7 + [vp, sz, vp]),
            ("m2rnn_out_norm_fwd", [i64, i64, vp, vp, ci, vp, cf, vp, vp]),
            ("m2rnn_out_norm_bwd_workspace_size", [i64, i64, ctypes.POINTER(sz)]),
            ("m2rnn_out_norm_bwd", [i64, i64, vp, vp, ci, vp, cf, vp, vp, vp, vp, vp, sz, vp]),
            ("m2rnn_conv4_silu_fwd", [i64] * 3 + [ci] + [vp] * 4 + [vp]),
            ("m2rnn_conv4_silu_bwd_workspace_size", [i64] * 3 + [ctypes.POINTER(sz)]),
            ("m2rnn_conv4_silu_bwd", [i64] * 3 + [ci] + [vp] * 7 + [vp, sz, vp]),
        ):
            fn = getattr(L, name)
            fn.restype = ci
            fn.argtypes = args
        L.m2rnn_fwd_block_workspace_size.restype = ci
        L.m2rnn_fwd_block_workspace_size.argtypes = [dp, ci, ci, ci, ctypes.POINTER(sz)]
        L.m2rnn_fwd_block.restype = ci
        L.m2rnn_fwd_block.argtypes = ([dp, ci, ci, ci] + [vp] * 3 + [vp] * 3 + [vp] * 3 + [vp, ci, vp, cf]
                                      + [vp, vp] + [vp, sz, vp, vp])
        L.m2rnn_decode_step.restype = ci
        L.m2rnn_decode_step.argtypes = [dp, ci, ci] + [vp] * 3 + [vp] * 3 + [vp, vp, vp, vp]
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().m2rnn_status_string(status).decode()


def _check(fn: str, status: int) -> None:
    if status != M2RNN_OK:
        raise M2RNNError(fn, status, status_string(status), lib().m2rnn_last_hip_error())


def _math(math) -> int:
    if isinstance(math, int):
        return math
    if math not in MATH:
        raise ValueError(f"math must be one of {sorted(MATH)}, got {math!r}")
    return MATH[math]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _require(t, name, dtype, shape, device):
    import torch
    if t is None:
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _fwd_prepare(q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, return_state):
    import torch
    if q.dim() != 4 or v.dim() != 4:
        raise ValueError("q must be [B,T,Nqk,K] and v [B,T,N,V]")
    B, T, Nqk, K = q.shape
    N, V = v.shape[2], v.shape[3]
    if Nqk not in (1, N):
        raise ValueError(f"q and k carry {Nqk} heads: expected {N} (one per head) or 1 (shared by all heads)")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU (HIP) device")
    qkv_dtype = q.dtype
    if qkv_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v must be float32 or bfloat16")
    _require(q, "q", qkv_dtype, (B, T, Nqk, K), dev)
    _require(k, "k", qkv_dtype, (B, T, Nqk, K), dev)
    _require(v, "v", qkv_dtype, (B, T, N, V), dev)
    _require(f, "f", torch.float32, (B, T, N), dev)
    _require(W, "W", torch.float32, (N, V, V), dev)
    _require(w_r, "w_r", torch.float32, (N, V), dev)
    if H0 is not None:
        _require(H0, "H0", torch.float32, (B, N, K, V), dev)
    if y is None:
        y = torch.empty((B, T, N, V), dtype=torch.float32, device=dev)
    _require(y, "y", torch.float32, (B, T, N, V), dev)
    if H_T is None and return_state:
        H_T = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
    if H_T is not None:
        _require(H_T, "H_T", torch.float32, (B, N, K, V), dev)
    dims = Dims(B, T, N, K, V, Nqk)
    dt = DTYPE_BF16 if qkv_dtype == torch.bfloat16 else DTYPE_F32
    return dims, dt, _math(math), int(row_blocks), y, H_T


def m2rnn_fwd_workspace_size(dims: Dims, qkv_dtype: int, math="auto", row_blocks: int = 0) -> int:
    n = ctypes.c_size_t(0)
    _check("m2rnn_fwd_workspace_size",
           lib().m2rnn_fwd_workspace_size(ctypes.byref(dims), qkv_dtype, _math(math), int(row_blocks), ctypes.byref(n)))
    return int(n.value)


def _workspace(nbytes: int, device, workspace):
    import torch
    if nbytes == 0:
        return None
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


class Overlap:
    """An m2rnn_overlap of the current device: a side stream (default priority) and its events, on
    which the forward calls overlap the second pass of a long sequence with the scan.  One object
    serves one call at a time: give each stream that issues calls its own."""

    def __init__(self):
        h = ctypes.c_void_p()
        _check("m2rnn_overlap_create", lib().m2rnn_overlap_create(ctypes.byref(h)))
        self._h = h.value

    @property
    def handle(self) -> Optional[int]:
        return self._h

    def close(self) -> None:
        if self._h:
            h, self._h = self._h, None
            _check("m2rnn_overlap_destroy", lib().m2rnn_overlap_destroy(h))

    def __del__(self, _finalizing=sys.is_finalizing):
        if not _finalizing():  # the HIP runtime may already be gone at interpreter exit
            try:
                self.close()
            except Exception:
                pass


# overlap="auto": one Overlap per (device, stream) that issues forward calls, made on first use and
# kept for the life of the process.
_overlaps: Dict[Tuple[int, int], Overlap] = {}


def _overlap(overlap, device, stream) -> Optional[int]:
    if overlap is None:
        return None
    if isinstance(overlap, Overlap):
        return overlap.handle
    if overlap != "auto":
        raise ValueError("overlap must be 'auto', None or an Overlap")
    import torch
    if torch.cuda.is_current_stream_capturing():
        return None  # a captured call runs the single pass anyway (and may not create streams)
    key = (device.index if device.index is not None else torch.cuda.current_device(), _stream(stream) or 0)
    ov = _overlaps.get(key)
    if ov is None:
        with torch.cuda.device(key[0]):
            ov = Overlap()
        _overlaps[key] = ov
    return ov.handle


def _call_fwd(name, q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, workspace, stream, return_state,
              overlap=None):
    dims, dt, m, rb, y, H_T = _fwd_prepare(q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, return_state)
    nbytes = m2rnn_fwd_workspace_size(dims, dt, m, rb)
    ws = _workspace(nbytes, q.device, workspace)
    fn = getattr(lib(), name)
    args = [ctypes.byref(dims), dt, m, rb, _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0),
            _ptr(y), _ptr(H_T), _ptr(ws), nbytes, _stream(stream)]
    if name == "m2rnn_fwd":
        args.append(_overlap(overlap, q.device, stream))
    _check(name, fn(*args))
    return y, H_T, ws


def m2rnn_checkpoint_interval(dims: Dims) -> int:
    """Steps between the checkpoints that m2rnn_fwd_ckpt keeps for the backward."""
    n = ctypes.c_int64(0)
    _check("m2rnn_checkpoint_interval", lib().m2rnn_checkpoint_interval(ctypes.byref(dims), ctypes.byref(n)))
    return int(n.value)


def checkpoint_count(T: int, V: int) -> int:
    """Checkpoints per (batch, head) that a forward keeps for the backward."""
    I = m2rnn_checkpoint_interval(Dims(1, T, 1, 16, V))
    return (T + I - 1) // I


def m2rnn_fwd_ckpt(q, k, v, f, W, w_r, H0=None, *, math="auto", row_blocks: int = 0, y=None, H_T=None, ckpt=None,
                   workspace=None, stream=None, overlap="auto"):
    """m2rnn_fwd that also keeps the backward's checkpoints: returns (y, H_T, ckpt) with ckpt
    [B,N,ceil(T/I),K,V] fp32, the state entering every I-th step, I = m2rnn_checkpoint_interval
    (for m2rnn_bwd_ckpt)."""
    import torch
    dims, dt, m, rb, y, H_T = _fwd_prepare(q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, True)
    shape = (dims.B, dims.N, checkpoint_count(dims.T, dims.V), dims.K, dims.V)
    if ckpt is None:
        ckpt = torch.empty(shape, dtype=torch.float32, device=q.device)
    _require(ckpt, "ckpt", torch.float32, shape, q.device)
    nbytes = m2rnn_fwd_workspace_size(dims, dt, m, rb)
    ws = _workspace(nbytes, q.device, workspace)
    _check("m2rnn_fwd_ckpt", lib().m2rnn_fwd_ckpt(
        ctypes.byref(dims), dt, m, rb, _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), _ptr(y),
        _ptr(H_T), _ptr(ckpt), _ptr(ws), nbytes, _stream(stream), _overlap(overlap, q.device, stream)))
    return y, H_T, ckpt


def m2rnn_fwd(q, k, v, f, W, w_r, H0=None, *, math="auto", row_blocks: int = 0, y=None, H_T=None, workspace=None,
              stream=None, return_state: bool = True, overlap="auto") -> Tuple[object, Optional[object]]:
    """Forward recurrence (M²RNN notes §2.1, Eq. 10-12) on the current HIP stream.

    q, k: [B,T,Nqk,K] with Nqk = N, or 1 for one query/key shared by all heads (§2.4); v: [B,T,N,V]
    (all float32 or all bfloat16); f: [B,T,N] fp32; W: [N,V,V] fp32; w_r: [N,V] fp32; H0: [B,N,K,V]
    fp32 or None.  Returns (y [B,T,N,V] fp32, H_T [B,N,K,V] fp32).  overlap: "auto" (one side stream
    per calling stream, made on first use), None (everything on the call's stream) or an Overlap.
    """
    y, H_T, _ = _call_fwd("m2rnn_fwd", q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, workspace, stream,
                          return_state, overlap)
    return y, H_T


def m2rnn_fwd_noalloc(q, k, v, f, W, w_r, H0=None, *, math="auto", row_blocks: int = 0, y=None, H_T=None,
                      stream=None, return_state: bool = True) -> Tuple[object, Optional[object]]:
    """m2rnn_fwd without a workspace: the library's fixed device array holds the partial readouts
    and the states between time segments (for callers that cannot allocate; pass y and H_T to
    allocate nothing here either).  Calls that overlap in time on one device race."""
    dims, dt, m, rb, y, H_T = _fwd_prepare(q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, return_state)
    _check("m2rnn_fwd_noalloc", lib().m2rnn_fwd_noalloc(
        ctypes.byref(dims), dt, m, rb, _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), _ptr(y),
        _ptr(H_T), _stream(stream)))
    return y, H_T


def m2rnn_fwd_block(q, k, v, a, alpha, beta, W, w_r, gz, gamma, H0=None, *, eps: float = 1e-6, math="auto",
                    row_blocks: int = 0, out=None, H_T=None, workspace=None, stream=None,
                    return_state: bool = True, overlap="auto") -> Tuple[object, Optional[object]]:
    """The block forward from the gate pre-activation to the normalised output (M²RNN notes §2.2,
    §2.3, Appendix C): f = exp(-alpha softplus(a + beta)), the recurrence, then
    out = gamma (.) x / sqrt(mean x^2 + eps) with x = y (.) SiLU(gz) over the N V features of a
    token, formed by the pass that sums the readouts (y never goes to HBM).  a [B,T,N] fp32; alpha, beta [N] fp32;
    gz [B,T,N,V] fp32 or bf16; gamma [N,V] fp32; the rest as m2rnn_fwd.  Returns (out, H_T)."""
    import torch
    dims, dt, m, rb, out, H_T = _fwd_prepare(q, k, v, a, W, w_r, H0, out, H_T, math, row_blocks, return_state)
    dev = q.device
    _require(alpha, "alpha", torch.float32, (dims.N,), dev)
    _require(beta, "beta", torch.float32, (dims.N,), dev)
    _require(gz, "gz", (torch.float32, torch.bfloat16), (dims.B, dims.T, dims.N, dims.V), dev)
    _require(gamma, "gamma", torch.float32, (dims.N, dims.V), dev)
    n = ctypes.c_size_t(0)
    _check("m2rnn_fwd_block_workspace_size",
           lib().m2rnn_fwd_block_workspace_size(ctypes.byref(dims), dt, m, rb, ctypes.byref(n)))
    ws = _workspace(int(n.value), dev, workspace)
    _check("m2rnn_fwd_block", lib().m2rnn_fwd_block(
        ctypes.byref(dims), dt, m, rb, _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(alpha), _ptr(beta), _ptr(W),
        _ptr(w_r), _ptr(H0), _ptr(gz), _dtype_code(gz), _ptr(gamma), float(eps), _ptr(out), _ptr(H_T), _ptr(ws),
        int(n.value), _stream(stream), _overlap(overlap, dev, stream)))
    return out, H_T


def m2rnn_scan_fwd(q, k, v, f, W, w_r, H0=None, *, math="auto", row_blocks: int = 0, y=None, H_T=None,
                   workspace=None, stream=None, return_state: bool = True):
    """The scan launch of m2rnn_fwd alone; returns (y, H_T, workspace) for m2rnn_scan_fwd_finish."""
    return _call_fwd("m2rnn_scan_fwd", q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, workspace, stream,
                     return_state)


def m2rnn_scan_fwd_finish(q, k, v, f, W, w_r, H0=None, *, math="auto", row_blocks: int = 0, y=None, H_T=None,
                          workspace=None, stream=None):
    """The second launch of m2rnn_fwd (sums partial readouts when the rows were split)."""
    y, H_T, _ = _call_fwd("m2rnn_scan_fwd_finish", q, k, v, f, W, w_r, H0, y, H_T, math, row_blocks, workspace,
                          stream, False)
    return y


def m2rnn_bwd_workspace_size(dims: Dims, qkv_dtype: int, math="auto") -> int:
    n = ctypes.c_size_t(0)
    _check("m2rnn_bwd_workspace_size",
           lib().m2rnn_bwd_workspace_size(ctypes.byref(dims), qkv_dtype, _math(math), ctypes.byref(n)))
    return int(n.value)


def m2rnn_bwd_ckpt_workspace_size(dims: Dims, qkv_dtype: int, math="auto") -> int:
    n = ctypes.c_size_t(0)
    _check("m2rnn_bwd_ckpt_workspace_size",
           lib().m2rnn_bwd_ckpt_workspace_size(ctypes.byref(dims), qkv_dtype, _math(math), ctypes.byref(n)))
    return int(n.value)


def _call_bwd_ckpt(name, q, k, v, f, W, w_r, ckpt, dy, dH_T, math, grad_clip, want_dH0, workspace, stream, out):
    import torch
    dims, dt, m, _, _, _ = _fwd_prepare(q, k, v, f, W, w_r, None, None, None, math, 0, False)
    B, T, N, K, V, Nqk = dims.B, dims.T, dims.N, dims.K, dims.V, dims.Nqk
    dev = q.device
    _require(ckpt, "ckpt", torch.float32, (B, N, checkpoint_count(T, V), K, V), dev)
    _require(dy, "dy", torch.float32, (B, T, N, V), dev)
    if dH_T is not None:
        _require(dH_T, "dH_T", torch.float32, (B, N, K, V), dev)
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    if out is None:
        out = {"dq": e(B, T, Nqk, K), "dk": e(B, T, Nqk, K), "dv": e(B, T, N, V), "df": e(B, T, N),
               "dW": e(N, V, V), "dw_r": e(N, V), "dH0": e(B, N, K, V) if want_dH0 else None}
    shapes = {"dq": (B, T, Nqk, K), "dk": (B, T, Nqk, K), "dv": (B, T, N, V), "df": (B, T, N), "dW": (N, V, V),
              "dw_r": (N, V), "dH0": (B, N, K, V)}
    for g, shape in shapes.items():
        if out.get(g) is not None or g != "dH0":
            _require(out.get(g), g, torch.float32, shape, dev)
    nbytes = m2rnn_bwd_ckpt_workspace_size(dims, dt, m)
    ws = _workspace(nbytes, dev, workspace)
    _check(name, getattr(lib(), name)(
        ctypes.byref(dims), dt, m, _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(ckpt), _ptr(dy),
        _ptr(dH_T), float(grad_clip), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["df"]), _ptr(out["dW"]),
        _ptr(out["dw_r"]), _ptr(out.get("dH0")), _ptr(ws), nbytes, _stream(stream)))
    return out


def m2rnn_bwd_ckpt(q, k, v, f, W, w_r, ckpt, dy, dH_T=None, *, math="auto", grad_clip: float = 0.0,
                   want_dH0: bool = True, workspace=None, stream=None, out=None) -> Dict[str, object]:
    """m2rnn_bwd from the checkpoints that m2rnn_fwd_ckpt kept (no forward re-run).  `out` may hold
    the gradient tensors to write (a dict as returned)."""
    return _call_bwd_ckpt("m2rnn_bwd_ckpt", q, k, v, f, W, w_r, ckpt, dy, dH_T, math, grad_clip, want_dH0, workspace,
                          stream, out)


def m2rnn_scan_bwd(q, k, v, f, W, w_r, ckpt, dy, dH_T=None, *, math="auto", grad_clip: float = 0.0,
                   want_dH0: bool = True, workspace=None, stream=None, out=None) -> Dict[str, object]:
    """The scale pass and the reverse scan of m2rnn_bwd_ckpt alone; m2rnn_scan_bwd_finish with the
    same workspace and outputs completes it."""
    return _call_bwd_ckpt("m2rnn_scan_bwd", q, k, v, f, W, w_r, ckpt, dy, dH_T, math, grad_clip, want_dH0, workspace,
                          stream, out)


def m2rnn_scan_bwd_finish(q, k, v, f, W, w_r, ckpt, dy, dH_T=None, *, math="auto", grad_clip: float = 0.0,
                          workspace=None, stream=None, out=None) -> Dict[str, object]:
    """The fixed-order sums of m2rnn_bwd_ckpt's per-workgroup partials (after m2rnn_scan_bwd)."""
    return _call_bwd_ckpt("m2rnn_scan_bwd_finish", q, k, v, f, W, w_r, ckpt, dy, dH_T, math, grad_clip,
                          out.get("dH0") is not None, workspace, stream, out)


def m2rnn_bwd(q, k, v, f, W, w_r, H0, dy, dH_T=None, *, math="auto", grad_clip: float = 0.0, want_dH0: bool = True,
              workspace=None, stream=None) -> Dict[str, object]:
    """BPTT (M²RNN notes §2.7) for L = sum <dy, y> + <dH_T, H_T>; returns dq, dk, dv, df, dW, dw_r, dH0.

    dq, dk have q's shape [B,T,Nqk,K]: with a shared query/key (Nqk = 1) they are summed over heads.
    grad_clip > 0 clamps, at every step, each element of the gradient sent back to the step's input
    state to [-grad_clip, grad_clip] (§2.3's per-step clipping); 0 gives the exact gradient."""
    import torch
    dims, dt, m, _, _, _ = _fwd_prepare(q, k, v, f, W, w_r, H0, None, None, math, 0, False)
    B, T, N, K, V, Nqk = dims.B, dims.T, dims.N, dims.K, dims.V, dims.Nqk
    dev = q.device
    _require(dy, "dy", torch.float32, (B, T, N, V), dev)
    if dH_T is not None:
        _require(dH_T, "dH_T", torch.float32, (B, N, K, V), dev)
    e = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)  # noqa: E731
    out = {"dq": e(B, T, Nqk, K), "dk": e(B, T, Nqk, K), "dv": e(B, T, N, V), "df": e(B, T, N), "dW": e(N, V, V),
           "dw_r": e(N, V), "dH0": e(B, N, K, V) if want_dH0 else None}
    nbytes = m2rnn_bwd_workspace_size(dims, dt, m)
    ws = _workspace(nbytes, dev, workspace)
    _check("m2rnn_bwd", lib().m2rnn_bwd(
        ctypes.byref(dims), dt, m, _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(H0), _ptr(dy),
        _ptr(dH_T), float(grad_clip), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["df"]), _ptr(out["dW"]),
        _ptr(out["dw_r"]), _ptr(out["dH0"]), _ptr(ws), nbytes, _stream(stream)))
    return out


def m2rnn_decode_step(q, k, v, f, W, w_r, H=None, *, H_out=None, y=None, math="auto",
                      stream=None) -> Tuple[object, object]:
    """One recurrence step (M²RNN notes §2.1, Eq. 10-12) with the state in device memory (decode).

    q, k: [B,Nqk,K] (Nqk = N, or 1 when shared by all heads); v: [B,N,V] (float32 or bfloat16,
    all alike); f: [B,N] fp32; W: [N,V,V];
    w_r: [N,V]; H: the state [B,N,K,V] fp32 or None (zeros).  Returns (y [B,N,V], H_out
    [B,N,K,V]).  Pass ``H_out=H`` to update the state in place.
    """
    import torch
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q must be [B,Nqk,K] and v [B,N,V]")
    B, Nqk, K = q.shape
    N, V = v.shape[1], v.shape[2]
    if Nqk not in (1, N):
        raise ValueError(f"q and k carry {Nqk} heads: expected {N} (one per head) or 1 (shared by all heads)")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("inputs must be on a GPU (HIP) device")
    qkv_dtype = q.dtype
    if qkv_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("q, k, v must be float32 or bfloat16")
    _require(q, "q", qkv_dtype, (B, Nqk, K), dev)
    _require(k, "k", qkv_dtype, (B, Nqk, K), dev)
    _require(v, "v", qkv_dtype, (B, N, V), dev)
    _require(f, "f", torch.float32, (B, N), dev)
    _require(W, "W", torch.float32, (N, V, V), dev)
    _require(w_r, "w_r", torch.float32, (N, V), dev)
    if H is not None:
        _require(H, "H", torch.float32, (B, N, K, V), dev)
    if H_out is None:
        H_out = torch.empty((B, N, K, V), dtype=torch.float32, device=dev)
    _require(H_out, "H_out", torch.float32, (B, N, K, V), dev)
    if y is None:
        y = torch.empty((B, N, V), dtype=torch.float32, device=dev)
    _require(y, "y", torch.float32, (B, N, V), dev)
    dims = Dims(B, 1, N, K, V, Nqk)
    dt = DTYPE_BF16 if qkv_dtype == torch.bfloat16 else DTYPE_F32
    _check("m2rnn_decode_step", lib().m2rnn_decode_step(
        ctypes.byref(dims), dt, _math(math), _ptr(q), _ptr(k), _ptr(v), _ptr(f), _ptr(W), _ptr(w_r), _ptr(H),
        _ptr(H_out), _ptr(y), _stream(stream)))
    return y, H_out


# ---------------------------------------------------------------- the steps around the recurrence

def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_F32
    raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")


def _size_query(name, *args) -> int:
    n = ctypes.c_size_t(0)
    _check(name, getattr(lib(), name)(*args, ctypes.byref(n)))
    return int(n.value)


def m2rnn_gate_fwd(a, alpha, beta, *, f=None, stream=None):
    """Gate of the notes' §2.2 (Eq. 13/17): f = exp(-alpha softplus(a + beta)); a [B,T,N], alpha, beta [N]."""
    import torch
    B, T, N = a.shape
    for name, t, shape in (("a", a, (B, T, N)), ("alpha", alpha, (N,)), ("beta", beta, (N,))):
        _require(t, name, torch.float32, shape, a.device)
    if f is None:
        f = torch.empty_like(a)
    _require(f, "f", torch.float32, (B, T, N), a.device)
    _check("m2rnn_gate_fwd", lib().m2rnn_gate_fwd(B, T, N, _ptr(a), _ptr(alpha), _ptr(beta), _ptr(f), _stream(stream)))
    return f


def m2rnn_gate_bwd(a, alpha, beta, df, *, workspace=None, stream=None) -> Dict[str, object]:
    """da [B,T,N], dalpha, dbeta [N] of the gate for the upstream df."""
    import torch
    B, T, N = a.shape
    for name, t, shape in (("a", a, (B, T, N)), ("alpha", alpha, (N,)), ("beta", beta, (N,)), ("df", df, (B, T, N))):
        _require(t, name, torch.float32, shape, a.device)
    out = {"da": torch.empty_like(a), "dalpha": torch.empty_like(alpha), "dbeta": torch.empty_like(beta)}
    nbytes = _size_query("m2rnn_gate_bwd_workspace_size", B, T, N)
    ws = _workspace(nbytes, a.device, workspace)
    _check("m2rnn_gate_bwd", lib().m2rnn_gate_bwd(B, T, N, _ptr(a), _ptr(alpha), _ptr(beta), _ptr(df), _ptr(out["da"]),
                                                  _ptr(out["dalpha"]), _ptr(out["dbeta"]), _ptr(ws), nbytes,
                                                  _stream(stream)))
    return out


def _norm_dims(y, gamma):
    D = gamma.numel()
    if tuple(y.shape[y.dim() - gamma.dim():]) != tuple(gamma.shape):
        raise ValueError(f"y {tuple(y.shape)} must end with gamma's shape {tuple(gamma.shape)}")
    return y.numel() // max(D, 1), D


def m2rnn_out_norm_fwd(y, gz, gamma, eps: float = 1e-6, *, out=None, stream=None):
    """Output gate + RMSNorm (§2.3, step 4): gamma (.) x / sqrt(mean x^2 + eps), x = y (.) SiLU(gz),
    normalised over gamma's features (for y [B,T,N,V] and gamma [N,V]: all heads of a token)."""
    import torch
    rows, D = _norm_dims(y, gamma)
    _require(y, "y", torch.float32, tuple(y.shape), y.device)
    _require(gz, "gz", (torch.float32, torch.bfloat16), tuple(y.shape), y.device)
    _require(gamma, "gamma", torch.float32, tuple(gamma.shape), y.device)
    if out is None:
        out = torch.empty_like(y)
    _require(out, "out", torch.float32, tuple(y.shape), y.device)
    _check("m2rnn_out_norm_fwd", lib().m2rnn_out_norm_fwd(rows, D, _ptr(y), _ptr(gz), _dtype_code(gz), _ptr(gamma),
                                                          float(eps), _ptr(out), _stream(stream)))
    return out


def m2rnn_out_norm_bwd(y, gz, gamma, dout, eps: float = 1e-6, *, workspace=None, stream=None) -> Dict[str, object]:
    """dy, dgz (fp32, shaped like y) and dgamma of the output gate + RMSNorm (Appendix C)."""
    import torch
    rows, D = _norm_dims(y, gamma)
    _require(y, "y", torch.float32, tuple(y.shape), y.device)
    _require(gz, "gz", (torch.float32, torch.bfloat16), tuple(y.shape), y.device)
    _require(gamma, "gamma", torch.float32, tuple(gamma.shape), y.device)
    _require(dout, "dout", torch.float32, tuple(y.shape), y.device)
    out = {"dy": torch.empty_like(y), "dgz": torch.empty_like(y), "dgamma": torch.empty_like(gamma)}
    nbytes = _size_query("m2rnn_out_norm_bwd_workspace_size", rows, D)
    ws = _workspace(nbytes, y.device, workspace)
    _check("m2rnn_out_norm_bwd", lib().m2rnn_out_norm_bwd(
        rows, D, _ptr(y), _ptr(gz), _dtype_code(gz), _ptr(gamma), float(eps), _ptr(dout), _ptr(out["dy"]),
        _ptr(out["dgz"]), _ptr(out["dgamma"]), _ptr(ws), nbytes, _stream(stream)))
    return out


def m2rnn_conv4_silu_fwd(x, w, bias=None, *, u=None, stream=None):
    """Causal depthwise conv (kernel 4) + SiLU (§2.3, step 1): x [B,T,C] fp32/bf16, w [C,4], bias [C] or None."""
    import torch
    B, T, C = x.shape
    _require(x, "x", (torch.float32, torch.bfloat16), (B, T, C), x.device)
    _require(w, "w", torch.float32, (C, 4), x.device)
    if bias is not None:
        _require(bias, "bias", torch.float32, (C,), x.device)
    if u is None:
        u = torch.empty_like(x)
    _require(u, "u", x.dtype, (B, T, C), x.device)
    _check("m2rnn_conv4_silu_fwd", lib().m2rnn_conv4_silu_fwd(B, T, C, _dtype_code(x), _ptr(x), _ptr(w), _ptr(bias),
                                                              _ptr(u), _stream(stream)))
    return u


def m2rnn_conv4_silu_bwd(x, w, bias, du, *, workspace=None, stream=None) -> Dict[str, object]:
    """dx [B,T,C] fp32, dw [C,4] and dbias [C] (None without a bias) of the causal conv4 + SiLU."""
    import torch
    B, T, C = x.shape
    _require(x, "x", (torch.float32, torch.bfloat16), (B, T, C), x.device)
    _require(w, "w", torch.float32, (C, 4), x.device)
    if bias is not None:
        _require(bias, "bias", torch.float32, (C,), x.device)
    _require(du, "du", torch.float32, (B, T, C), x.device)
    out = {"dx": torch.empty((B, T, C), dtype=torch.float32, device=x.device), "dw": torch.empty_like(w),
           "dbias": torch.empty_like(bias) if bias is not None else None}
    nbytes = _size_query("m2rnn_conv4_silu_bwd_workspace_size", B, T, C)
    ws = _workspace(nbytes, x.device, workspace)
    _check("m2rnn_conv4_silu_bwd", lib().m2rnn_conv4_silu_bwd(
        B, T, C, _dtype_code(x), _ptr(x), _ptr(w), _ptr(bias), _ptr(du), _ptr(out["dx"]), _ptr(out["dw"]),
        _ptr(out["dbias"]), _ptr(ws), nbytes, _stream(stream)))
    return out
