// Single-step (decode) kernels, one instantiation per value size and input dtype.
#include "m2rnn_decode_kernel.h"
#include "m2rnn_select.h"

namespace m2rnn {
const void* decode_kernel(int V, bool bf16) {
  switch (V) {
    case 16: return bf16 ? (const void*)&m2rnn_decode_kernel<16, true> : (const void*)&m2rnn_decode_kernel<16, false>;
    case 32: return bf16 ? (const void*)&m2rnn_decode_kernel<32, true> : (const void*)&m2rnn_decode_kernel<32, false>;
    case 64: return bf16 ? (const void*)&m2rnn_decode_kernel<64, true> : (const void*)&m2rnn_decode_kernel<64, false>;
    case 128: return bf16 ? (const void*)&m2rnn_decode_kernel<128, true> : (const void*)&m2rnn_decode_kernel<128, false>;
    default: return nullptr;
  }
}
}  // namespace m2rnn
