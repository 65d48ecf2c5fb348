// Forward scan kernels with the BF16X3 contraction.
#include "m2rnn_select.h"

namespace m2rnn {
const void* fwd_kernel_bf16x3(int V, int rb, int rw, bool bf16, int mode) { return pick_fwd<MATH_BF16X3>(V, rb, rw, bf16, mode); }
}  // namespace m2rnn
