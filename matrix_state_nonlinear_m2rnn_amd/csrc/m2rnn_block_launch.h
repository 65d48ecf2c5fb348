// Launchers of block kernels that the recurrence's entry points use (defined in m2rnn_block.hip,
// so that the block kernels are compiled in one translation unit only).
#pragma once

#include <hip/hip_runtime.h>

namespace m2rnn {

// Widest token row (N V features) of the output gate + RMSNorm.
constexpr long kNormMaxFeatures = 8192;

// The block forward's output epilogue over the tokens t0 .. t0 + len - 1 of every batch entry of
// a [B, T] sequence of D features: y from the S readout planes part[S][B*T][D] (+ w_r (.) v when
// w_r is set), then out = RMSNorm(y (.) SiLU(gz)) * gamma.  Returns a hipError_t.
int launch_fwd_finish_norm(const float* part, int S, const void* v, bool v_bf16, const float* w_r, const void* gz,
                           bool gz_bf16, const float* gamma, long B, long T, long t0, long len, int D, float eps,
                           float* out, hipStream_t stream);

}  // namespace m2rnn
