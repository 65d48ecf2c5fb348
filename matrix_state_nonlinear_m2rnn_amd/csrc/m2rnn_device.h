// Device-side building blocks for the gfx950 M²RNN kernels: MFMA operand types, the
// split-precision conversions, wave-level DPP reductions and an LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace m2rnn {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Contraction modes (values match the public M2RNN_MATH_* enum).
enum { MATH_F32 = 0, MATH_F16X3 = 1, MATH_BF16X3 = 2, MATH_BF16 = 3 };

// 2*log2(e): the kernels keep c*P instead of P so that exp(2P) is a single v_exp_f32 (2^x).
constexpr float kTwoLog2e = 2.88539008177792681472f;

// Word 3 of a gfx9 buffer resource for raw (unformatted, stride 0) dword access: 32-bit data
// format, no swizzle.  With stride 0 the buffer unit checks each access's byte offset against the
// resource's size and drops out-of-range stores (and returns 0 for out-of-range loads).
constexpr int kBufferRsrcWord3 = 0x00020000;
// A byte offset past the end of every buffer resource built here (sizes stay below 2^31 bytes).
constexpr uint32_t kBufferDrop = 0x80000000u;

// Workgroup barrier whose fences cover LDS only: it waits for this wave's LDS traffic
// (lgkmcnt(0)) but not for its outstanding global loads/stores, so input prefetches and output
// stores stay in flight across the per-step barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_amdgcn_update_dpp(0.0f, x, CTRL, 0xF, 0xF, false);
}

// DPP lane permutation with all lanes written (no `old` value), so that the compiler can fold
// the permutation into the consuming VALU instruction's first operand.
template <int CTRL>
__device__ __forceinline__ float dpp_all(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kDppRowMirror = 0x140;      // lane i <- lane 15-i within each row of 16
constexpr int kDppRowHalfMirror = 0x141;  // lane i <- lane 7-i within each half-row of 8
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppQuadBcast0 = 0x00;      // quad_perm [0,0,0,0]
constexpr int kDppQuadBcast1 = 0x55;      // quad_perm [1,1,1,1]
constexpr int kDppQuadBcast2 = 0xAA;      // quad_perm [2,2,2,2]
constexpr int kDppQuadBcast3 = 0xFF;      // quad_perm [3,3,3,3]

// Sums four per-lane values over the 16 lanes of each DPP row at once: on return, lane n of a
// row holds sum_{lanes m of the row} x_{(n >> 2) & 3}(m).  Lanes xor 15 and xor 7 exchange the
// halves that each keeps, then two quad swaps finish the sum (11 VALU ops for 4 row sums).
__device__ __forceinline__ float row16_sum4(float x0, float x1, float x2, float x3, int lane) {
  const bool b3 = (lane & 8) != 0;
  const bool b2 = (lane & 4) != 0;
  const float s0 = b3 ? x0 : x2, s1 = b3 ? x1 : x3;
  const float k0 = b3 ? x2 : x0, k1 = b3 ? x3 : x1;
  const float a0 = k0 + dpp<kDppRowMirror>(s0);
  const float a1 = k1 + dpp<kDppRowMirror>(s1);
  const float s = b2 ? a0 : a1, k = b2 ? a1 : a0;
  float c = k + dpp<kDppRowHalfMirror>(s);
  c += dpp<kDppQuadXor1>(c);
  c += dpp<kDppQuadXor2>(c);
  return c;
}

__device__ __forceinline__ float bf16_lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 p;
  p[0] = (__bf16)a;  // round to nearest even (v_cvt_pk_bf16_f32)
  p[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  fp16x2 p;
  p[0] = (__fp16)a;  // round to nearest even (v_cvt_pk_f16_f32)
  p[1] = (__fp16)b;
  return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float f16_lo_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(fp16x2, w)[0];
}
__device__ __forceinline__ float f16_hi_to_f32(uint32_t w) {
  return (float)__builtin_bit_cast(fp16x2, w)[1];
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                0, 0, 0);
}
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short bf16x4_bits __attribute__((ext_vector_type(4)));
// 16x16x16 variants: K = 16, four 16-bit values per lane (2 dwords).
__device__ __forceinline__ f32x4 mfma16_f16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16_bf16(uint2 a, uint2 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_bits, a), __builtin_bit_cast(bf16x4_bits, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16(uint4 a, uint4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                 c, 0, 0, 0);
}

// Makes four values opaque to the compiler at this point (an empty asm that "modifies" them in
// place), so that a later fp16 conversion rounds the fp32 values themselves.  Without it the
// compiler may fold the FMA that produced a value into the conversion (v_fma_mix with an fp16
// result), which rounds the unrounded FMA once instead of the fp32 value: the split of a state
// would then depend on how the value was produced, and a scan restarted from a stored fp32 state
// would differ from a continuous one.
__device__ __forceinline__ void opaque4(float (&x)[4]) {
  asm("" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));
}

// x rounded to fp32 at this point: an empty asm that "modifies" it, so that the compiler cannot fuse
// the multiply that produced it into a later operation.  The split of c W into fp16 hi/lo parts
// needs it: with the product fused into the remainder's v_fma_mix, lo = fp16(c W - hi) would be
// taken from the exact product in some kernels and from the fp32 one in others, and kernels that
// should agree bit for bit would not.
__device__ __forceinline__ float opaque1(float x) {
  asm("" : "+v"(x));
  return x;
}

// fma(h, b, c) in fp32 with h one fp16 half of a packed pair (HI: the high half), widened exactly
// inside the instruction: one v_fma_mix_f32 in place of a conversion and an FMA.
template <bool HI>
__device__ __forceinline__ float fma_mix_f16(uint32_t h, float b, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(b), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(b), "v"(c));
  return d;
}
// h + c in fp32 with h one fp16 half of a packed pair (HI: the high half): one v_fma_mix_f32.
template <bool HI>
__device__ __forceinline__ float add_mix_f16(uint32_t h, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
  return d;
}

// h - c in fp32 with h one fp16 half of a packed pair (HI: the high half): one v_fma_mix_f32 with
// the negation as a source modifier.
template <bool HI>
__device__ __forceinline__ float sub_mix_f16(uint32_t h, float c) {
  float d;
  if constexpr (HI)
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
  else
    asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(c));
  return d;
}

// tanh(x/c) from x = c*P, c = 2 log2 e:  tanh(P) = 1 - 2 / (1 + 2^x).  Returns r = 1/(1 + 2^x)
// so that callers fold "1 - 2r" into the gate blend.  2^x overflowing to +inf gives r = 0
// (tanh = 1); underflowing to 0 gives r = 1 (tanh = -1).
__device__ __forceinline__ float tanh_recip(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

}  // namespace m2rnn
