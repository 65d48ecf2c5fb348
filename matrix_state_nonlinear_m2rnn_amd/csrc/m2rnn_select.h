// Kernel selection: each contraction mode is compiled in its own translation unit, which
// exports one function mapping (V, RB, input dtype, mode) to the kernel's host stub.
#pragma once

#include "m2rnn_fwd_kernel.h"

namespace m2rnn {

template <int MATH, int V, int RB, int RW>
const void* pick_fwd_vrb(bool bf16, int mode) {
  if (mode == MODE_FWD_RO) {
    // readout waves: the split contractions at V = 64, and at V = 128 with one row block per wave
    // (two would spill in a 16-wave workgroup), one row group
    if constexpr (MATH != MATH_F32 && RW == 1 && (V == 64 || (V == 128 && RB == 1)))
      return bf16 ? (const void*)&m2rnn_scan_fwd_ro_kernel<V, RB, MATH, true>
                  : (const void*)&m2rnn_scan_fwd_ro_kernel<V, RB, MATH, false>;
    return nullptr;
  }
  if (mode == MODE_FWD)
    return bf16 ? (const void*)&m2rnn_scan_fwd_kernel<V, RB, MATH, true, MODE_FWD, RW>
                : (const void*)&m2rnn_scan_fwd_kernel<V, RB, MATH, false, MODE_FWD, RW>;
  if constexpr (MATH != MATH_BF16 && RW == 1) {
    if (mode == MODE_CKPT)
      return bf16 ? (const void*)&m2rnn_scan_fwd_kernel<V, RB, MATH, true, MODE_CKPT>
                  : (const void*)&m2rnn_scan_fwd_kernel<V, RB, MATH, false, MODE_CKPT>;
  }
  return nullptr;
}

// Row groups (rw) are built for one row block per wave and V < 64, up to four waves per workgroup.
template <int MATH, int V>
const void* pick_fwd_v(int rb, int rw, bool bf16, int mode) {
  if (rw == 1) {
    switch (rb) {
      case 1: return pick_fwd_vrb<MATH, V, 1, 1>(bf16, mode);
      case 2: return pick_fwd_vrb<MATH, V, 2, 1>(bf16, mode);
      case 4: return pick_fwd_vrb<MATH, V, 4, 1>(bf16, mode);
      default: return nullptr;
    }
  }
  if (rb != 1) return nullptr;
  if constexpr (V == 16) {
    if (rw == 2) return pick_fwd_vrb<MATH, V, 1, 2>(bf16, mode);
    if (rw == 4) return pick_fwd_vrb<MATH, V, 1, 4>(bf16, mode);
  } else if constexpr (V == 32) {
    if (rw == 2) return pick_fwd_vrb<MATH, V, 1, 2>(bf16, mode);
  }
  return nullptr;
}

template <int MATH>
const void* pick_fwd(int V, int rb, int rw, bool bf16, int mode) {
  switch (V) {
    case 16: return pick_fwd_v<MATH, 16>(rb, rw, bf16, mode);
    case 32: return pick_fwd_v<MATH, 32>(rb, rw, bf16, mode);
    case 64: return pick_fwd_v<MATH, 64>(rb, rw, bf16, mode);
    case 128: return pick_fwd_v<MATH, 128>(rb, rw, bf16, mode);
    default: return nullptr;
  }
}

// One per contraction mode (defined in m2rnn_fwd_<mode>.hip).
const void* fwd_kernel_f32(int V, int rb, int rw, bool bf16, int mode);
const void* fwd_kernel_f16x3(int V, int rb, int rw, bool bf16, int mode);
const void* fwd_kernel_bf16x3(int V, int rb, int rw, bool bf16, int mode);
const void* fwd_kernel_bf16(int V, int rb, int rw, bool bf16, int mode);

// Single-step (decode) kernel for value size V (defined in m2rnn_decode.hip).
const void* decode_kernel(int V, bool bf16);

}  // namespace m2rnn
