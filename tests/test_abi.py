"""The C ABI on the CPU: the library loads, exports every entry point that include/m2rnn.h
declares, and rejects invalid calls with the documented status before enqueuing anything."""
import ctypes
import os
import re

import pytest

import matrix_state_nonlinear_m2rnn_amd as m2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "m2rnn.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(m2rnn_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_function():
    L = m2.lib()
    names = declared_functions()
    assert "m2rnn_fwd" in names and "m2rnn_bwd" in names
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(m2.EXPORTED)


def test_header_and_bindings_agree_on_the_abi_version():
    text = open(os.path.join(ROOT, "include", "m2rnn.h")).read()
    assert int(re.search(r"#define M2RNN_VERSION (\d+)", text).group(1)) == m2.ABI_VERSION


def test_version_and_status_strings():
    assert m2.lib().m2rnn_version() == m2.ABI_VERSION
    assert m2.status_string(0) == "ok"
    assert "workspace" in m2.status_string(m2.M2RNN_EWORKSPACE)


def fwd(dims, dtype=0, math=-1, rb=0, ptr=16, ws=None, nbytes=0, y=True, q=True, f=True):
    L = m2.lib()
    p = ctypes.c_void_p(ptr)
    return L.m2rnn_fwd(ctypes.byref(dims) if dims is not None else None, dtype, math, rb, p if q else None, p, p,
                       p if f else None, p, p, None, p if y else None, None, ws, nbytes, None, None)


def test_invalid_arguments_are_rejected_on_the_host():
    D = m2.Dims
    assert fwd(None) == m2.M2RNN_EINVAL
    assert fwd(D(-1, 4, 2, 16, 16)) == m2.M2RNN_EINVAL
    assert fwd(D(1, 4, 2, 16, 16), dtype=7) == m2.M2RNN_EINVAL
    assert fwd(D(1, 4, 2, 16, 16), math=9) == m2.M2RNN_EINVAL
    assert fwd(D(1, 4, 2, 16, 48)) == m2.M2RNN_EUNSUPPORTED      # V not in {16,32,64,128}
    assert fwd(D(1, 4, 2, 24, 16)) == m2.M2RNN_EUNSUPPORTED      # K not a multiple of 16
    assert fwd(D(1, 4, 2, 16, 16), y=False) == m2.M2RNN_EINVAL    # missing output
    assert fwd(D(1, 4, 2, 16, 16), q=False) == m2.M2RNN_EINVAL
    assert fwd(D(1, 4, 2, 16, 16), f=False) == m2.M2RNN_EINVAL
    assert fwd(D(1, 4, 2, 16, 16), ptr=18) == m2.M2RNN_EINVAL     # misaligned
    assert fwd(D(1, 4, 2, 48, 16), rb=2) == m2.M2RNN_EINVAL       # rb must divide K/16
    # K = 128, V = 16 with one 16-row block per wave: a workgroup carries four row blocks (one per
    # SIMD), so each state spans two workgroups whose partial readouts need a workspace.
    assert fwd(D(1, 4, 2, 128, 16), rb=1) == m2.M2RNN_EWORKSPACE
    # The fp32 contraction keeps one row block per workgroup: four partial planes at K = 64.
    assert fwd(D(1, 4, 2, 64, 16), rb=1, math=0) == m2.M2RNN_EWORKSPACE


def test_workspace_size_query():
    # V = 32: two row groups of two waves per workgroup, so K = 64 spans two workgroups (two planes)
    n = m2.m2rnn_fwd_workspace_size(m2.Dims(2, 10, 3, 64, 32), 1, "f16x3", 1)
    assert n >= 2 * 2 * 10 * 3 * 32 * 4
    # the fp32 contraction: one row block per workgroup, four planes
    assert m2.m2rnn_fwd_workspace_size(m2.Dims(2, 10, 3, 64, 32), 1, "f32", 1) >= 4 * 2 * 10 * 3 * 32 * 4
    # V = 16, K = 64: the four row blocks share one workgroup, so no partial planes at all
    assert m2.m2rnn_fwd_workspace_size(m2.Dims(2, 10, 3, 64, 16), 1, "f16x3", 1) == 0
    assert m2.m2rnn_fwd_workspace_size(m2.Dims(2, 10, 3, 64, 32), 1, "f16x3", 4) == 0
    with pytest.raises(m2.M2RNNError):
        m2.m2rnn_fwd_workspace_size(m2.Dims(2, 10, 3, 64, 40), 1, "f16x3", 0)


def decode(dims, dtype=0, math=-1, ptr=16, H_in=16, H_out=16, y=True, f=True):
    L = m2.lib()
    p = ctypes.c_void_p(ptr)
    return L.m2rnn_decode_step(ctypes.byref(dims), dtype, math, p, p, p, p if f else None, p, p,
                               ctypes.c_void_p(H_in) if H_in else None, ctypes.c_void_p(H_out) if H_out else None,
                               p if y else None, None)


def test_decode_step_invalid_arguments_are_rejected_on_the_host():
    D = m2.Dims
    assert decode(D(2, 2, 3, 16, 16)) == m2.M2RNN_EINVAL              # T must be 1
    assert decode(D(2, 0, 3, 16, 16)) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 48)) == m2.M2RNN_EUNSUPPORTED         # V not in {16,32,64,128}
    assert decode(D(2, 1, 3, 16, 16), math=0) == m2.M2RNN_EUNSUPPORTED  # only the split-fp16 contraction
    assert decode(D(2, 1, 3, 16, 16), math=9) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 16), y=False) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 16), f=False) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 16), H_out=0) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 16), ptr=24) == m2.M2RNN_EINVAL       # misaligned
    # H_out may be H_in (in place) but must not overlap it otherwise.
    assert decode(D(2, 1, 3, 16, 16), H_in=1 << 20, H_out=(1 << 20) + 256) == m2.M2RNN_EINVAL
    assert decode(D(0, 1, 3, 16, 16)) == m2.M2RNN_OK                   # nothing to do


def test_shared_query_key_head_count_is_checked():
    D = m2.Dims
    assert fwd(D(1, 4, 3, 16, 16, 2)) == m2.M2RNN_EINVAL      # Nqk must be 0, 1 or N
    assert fwd(D(1, 4, 3, 16, 16, -1)) == m2.M2RNN_EINVAL
    assert decode(D(2, 1, 3, 16, 16, 2)) == m2.M2RNN_EINVAL


def test_checkpoint_entry_points_check_their_arguments():
    L = m2.lib()
    D = m2.Dims
    p = ctypes.c_void_p(16)
    dims = D(1, 4, 2, 16, 16)
    # forward that keeps checkpoints: the checkpoint buffer is required when there are steps
    assert L.m2rnn_fwd_ckpt(ctypes.byref(dims), 0, -1, 0, p, p, p, p, p, p, None, p, None, None, None, 0,
                            None, None) == m2.M2RNN_EINVAL
    # backward from checkpoints: likewise
    assert L.m2rnn_bwd_ckpt(ctypes.byref(dims), 0, -1, p, p, p, p, p, p, None, p, None, 0.0, p, p, p, p, p, p, None,
                            p, 1 << 30, None) == m2.M2RNN_EINVAL
    # the gradient clip must be >= 0 (0 = exact gradient); NaN is rejected too
    for bad in (-1.0, float("nan")):
        assert L.m2rnn_bwd(ctypes.byref(dims), 0, -1, p, p, p, p, p, p, None, p, None, bad, p, p, p, p, p, p, None,
                           p, 1 << 30, None) == m2.M2RNN_EINVAL
        assert L.m2rnn_bwd_ckpt(ctypes.byref(dims), 0, -1, p, p, p, p, p, p, p, p, None, bad, p, p, p, p, p, p,
                                None, p, 1 << 30, None) == m2.M2RNN_EINVAL
    # its workspace excludes the checkpoints
    big = m2.Dims(4, 4096, 16, 64, 64)
    assert m2.m2rnn_bwd_ckpt_workspace_size(big, 0) + 4 * 16 * 64 * 64 * 64 * 4 <= m2.m2rnn_bwd_workspace_size(big, 0)


def test_block_entry_points_check_their_arguments():
    L = m2.lib()
    p = ctypes.c_void_p(16)
    n = ctypes.c_size_t(0)
    assert L.m2rnn_gate_fwd(-1, 2, 3, p, p, p, p, None) == m2.M2RNN_EINVAL
    assert L.m2rnn_gate_fwd(1, 2, 3, None, p, p, p, None) == m2.M2RNN_EINVAL
    assert L.m2rnn_gate_fwd(0, 2, 3, None, None, None, None, None) == m2.M2RNN_OK
    assert L.m2rnn_gate_bwd(1, 2, 3, p, p, p, p, p, p, p, None, 0, None) == m2.M2RNN_EWORKSPACE
    assert L.m2rnn_out_norm_fwd(4, 6, p, p, 0, p, ctypes.c_float(1e-6), p, None) == m2.M2RNN_EUNSUPPORTED  # D % 4
    assert L.m2rnn_out_norm_fwd(4, 16, p, p, 5, p, ctypes.c_float(1e-6), p, None) == m2.M2RNN_EINVAL     # dtype
    assert L.m2rnn_out_norm_fwd(4, 16, p, p, 0, p, ctypes.c_float(-1.0), p, None) == m2.M2RNN_EINVAL     # eps
    assert L.m2rnn_out_norm_fwd(4, 16, ctypes.c_void_p(20), p, 0, p, ctypes.c_float(0), p, None) == m2.M2RNN_EINVAL
    assert L.m2rnn_out_norm_fwd(4, 8196, p, p, 0, p, ctypes.c_float(0), p, None) == m2.M2RNN_EUNSUPPORTED
    assert L.m2rnn_out_norm_bwd_workspace_size(130, 64, ctypes.byref(n)) == m2.M2RNN_OK and n.value >= 3 * 64 * 4
    assert L.m2rnn_conv4_silu_fwd(1, 8, 6, 0, p, p, None, p, None) == m2.M2RNN_EUNSUPPORTED             # C % 4
    assert L.m2rnn_conv4_silu_fwd(1, 8, 8, 3, p, p, None, p, None) == m2.M2RNN_EINVAL
    assert L.m2rnn_conv4_silu_fwd(1, 8, 8, 0, p, None, None, p, None) == m2.M2RNN_EINVAL                # no weights
    assert L.m2rnn_conv4_silu_bwd(1, 8, 8, 0, p, p, None, p, p, p, None, None, 0, None) == m2.M2RNN_EWORKSPACE


def test_fused_block_forward_checks_its_arguments():
    L = m2.lib()
    D = m2.Dims
    p = ctypes.c_void_p(16)

    def call(dims, alpha=True, gz_dtype=0, eps=1e-6, ws=None, nbytes=0, gz=True):
        return L.m2rnn_fwd_block(ctypes.byref(dims), 0, -1, 0, p, p, p, p, p if alpha else None, p, p, p, None,
                                 p if gz else None, gz_dtype, p, ctypes.c_float(eps), p, None, ws, nbytes, None,
                                 None)
    assert call(D(1, 4, 2, 16, 16), alpha=False) == m2.M2RNN_EINVAL
    assert call(D(1, 4, 2, 16, 16), gz=False) == m2.M2RNN_EINVAL
    assert call(D(1, 4, 2, 16, 16), gz_dtype=5) == m2.M2RNN_EINVAL
    assert call(D(1, 4, 2, 16, 16), eps=-1.0) == m2.M2RNN_EINVAL
    assert call(D(1, 4, 128, 16, 128)) == m2.M2RNN_EUNSUPPORTED          # N V = 16384 features
    assert call(D(1, 4, 2, 16, 16)) == m2.M2RNN_EWORKSPACE                # y goes through the workspace
    assert call(D(1, 4, 2, 16, 16), ws=p, nbytes=256 + 4 * 2 * 16 * 4 - 4) == m2.M2RNN_EWORKSPACE
    n = ctypes.c_size_t(0)
    # the gate f [B,T,N], then y [B,T,N,V] (one workgroup per pair) or the partial planes (rows split:
    # K = 64, V = 32)
    f_bytes = (2 * 10 * 3 * 4 + 255) // 256 * 256
    assert L.m2rnn_fwd_block_workspace_size(ctypes.byref(D(2, 10, 3, 16, 16)), 0, -1, 0, ctypes.byref(n)) == 0
    assert n.value >= f_bytes + 2 * 10 * 3 * 16 * 4
    assert L.m2rnn_fwd_block_workspace_size(ctypes.byref(D(2, 10, 3, 64, 32)), 1, 1, 1, ctypes.byref(n)) == 0
    assert n.value == f_bytes + m2.m2rnn_fwd_workspace_size(D(2, 10, 3, 64, 32), 1, "f16x3", 1)
    assert L.m2rnn_fwd_block_workspace_size(ctypes.byref(D(2, 0, 3, 16, 16)), 0, -1, 0, ctypes.byref(n)) == 0
    assert n.value == 0


def test_checkpoint_interval():
    # every sub-segment of the backward for V <= 64, every 64-step segment at V = 128
    assert [m2.m2rnn_checkpoint_interval(m2.Dims(1, 100, 1, 16, V)) for V in (16, 32, 64, 128)] == [8, 8, 8, 64]
    assert m2.checkpoint_count(4096, 64) == 512 and m2.checkpoint_count(70, 16) == 9


def test_overlap_object_arguments():
    L = m2.lib()
    assert L.m2rnn_overlap_create(None) == m2.M2RNN_EINVAL
    assert L.m2rnn_overlap_destroy(None) == m2.M2RNN_OK


def test_tensors_beyond_2_gib_are_accepted_per_batch_slice():
    # The 16K-token context at batch 16 (B16 N32 T16384 K=V=64): y is 2 GiB and the split-row
    # readout planes 8 GiB; only one batch entry's slice must stay below 2 GiB.
    n = ctypes.c_size_t(0)
    dims = m2.Dims(16, 16384, 32, 64, 64)
    assert m2.lib().m2rnn_fwd_workspace_size(ctypes.byref(dims), m2.DTYPE_BF16, -1, 1, ctypes.byref(n)) == m2.M2RNN_OK
    assert n.value >= 4 * 16 * 16384 * 32 * 64 * 4  # four planes of [B,T,N,V] fp32
    assert m2.lib().m2rnn_bwd_workspace_size(ctypes.byref(dims), m2.DTYPE_BF16, -1, ctypes.byref(n)) == m2.M2RNN_OK
    # one batch entry's slice of 2 GiB or more is refused
    big = m2.Dims(1, 1 << 20, 32, 64, 64)
    assert m2.lib().m2rnn_fwd_workspace_size(ctypes.byref(big), m2.DTYPE_BF16, -1, 0, ctypes.byref(n)) == \
        m2.M2RNN_EUNSUPPORTED
