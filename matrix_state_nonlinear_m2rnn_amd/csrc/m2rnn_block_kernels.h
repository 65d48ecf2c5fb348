// Kernels for the steps on either side of the recurrence in the M²RNN block (M²RNN notes §2.2,
// §2.3, Appendix C): the gate f = exp(-alpha softplus(a + beta)), the output gate + RMSNorm over
// the N V features of a token, and the causal depthwise conv of kernel size 4 + SiLU on q, k, v.
// All of them are HBM-bound streams; every reduction runs in a fixed order, so results are
// bit-reproducible.
#pragma once

#include "m2rnn_device.h"

namespace m2rnn {

constexpr int kBlkThreads = 256;

// e^x and ln x from the hardware's 2^x and log2 x (v_exp_f32, v_log_f32), about 1 ulp each plus the
// rounding of the base change; 1/x from v_rcp_f32.
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float exp_(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }
__device__ __forceinline__ float log_(float x) { return __builtin_amdgcn_logf(x) * kLn2; }
__device__ __forceinline__ float sigmoidf_(float x) { return __builtin_amdgcn_rcpf(1.0f + exp_(-x)); }
// log(1 + e^x) without overflow.
__device__ __forceinline__ float softplusf_(float x) { return fmaxf(x, 0.0f) + log_(1.0f + exp_(-fabsf(x))); }
__device__ __forceinline__ float siluf_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float silu_gradf_(float x) {
  const float s = sigmoidf_(x);
  return s * (1.0f + x * (1.0f - s));
}
// The forget gate of the M2RNN block (notes §2.2): f = exp(-alpha softplus(a + beta)) from the
// pre-activation a and the head's alpha, beta.
__device__ __forceinline__ float gate_f(float a, float alpha, float beta) {
  return exp_(-alpha * softplusf_(a + beta));
}

template <bool BF16>
__device__ __forceinline__ float4 load4(const void* base, long i) {
  if constexpr (BF16) {
    const uint2 r = *(const uint2*)((const uint16_t*)base + i);
    return make_float4(bf16_lo_to_f32(r.x), bf16_hi_to_f32(r.x), bf16_lo_to_f32(r.y), bf16_hi_to_f32(r.y));
  }
  return *(const float4*)((const float*)base + i);
}

// load4 as a non-temporal load, for streams read once.  (It helps the RMSNorm and the conv
// backward by 2-4%; the conv forward, whose x rows are also read by the neighbouring chunk's
// window, runs slower with it.)
template <bool BF16>
__device__ __forceinline__ float4 load4_nt(const void* base, long i) {
  if constexpr (BF16) {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const u2v r = __builtin_nontemporal_load((const u2v*)((const uint16_t*)base + i));
    return make_float4(bf16_lo_to_f32(r[0]), bf16_hi_to_f32(r[0]), bf16_lo_to_f32(r[1]), bf16_hi_to_f32(r[1]));
  }
  const f32x4 t = __builtin_nontemporal_load((const f32x4*)((const float*)base + i));
  return make_float4(t[0], t[1], t[2], t[3]);
}

template <bool BF16>
__device__ __forceinline__ void store4(void* base, long i, float4 v) {
  if constexpr (BF16) {
    *(uint2*)((uint16_t*)base + i) = make_uint2(pack_bf16(v.x, v.y), pack_bf16(v.z, v.w));
  } else {
    *(float4*)((float*)base + i) = v;
  }
}

// store4 as a non-temporal store: the caches need not keep a stream written once and not read
// back by the kernel.
template <bool BF16>
__device__ __forceinline__ void store4_nt(void* base, long i, const float (&o)[4]) {
  if constexpr (BF16) {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const u2v v = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
    __builtin_nontemporal_store(v, (u2v*)((uint16_t*)base + i));
  } else {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = {o[0], o[1], o[2], o[3]};
    __builtin_nontemporal_store(v, (f4v*)((float*)base + i));
  }
}

// Sum over the workgroup (kBlkThreads threads) of a pair of values, in a fixed order; every
// thread receives the totals.  `red` holds 2 * (kBlkThreads / 64) floats.
__device__ __forceinline__ float2 block_sum2(float a, float b, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    a += __shfl_xor(a, o);
    b += __shfl_xor(b, o);
  }
  const int w = threadIdx.x >> 6;
  __syncthreads();  // `red` may still be read by the previous call
  if ((threadIdx.x & 63) == 0) {
    red[2 * w] = a;
    red[2 * w + 1] = b;
  }
  __syncthreads();
  float2 s = make_float2(0.0f, 0.0f);
#pragma unroll
  for (int i = 0; i < kBlkThreads / 64; ++i) {
    s.x += red[2 * i];
    s.y += red[2 * i + 1];
  }
  return s;
}

// ------------------------------------------------------------------ gate (§2.2, Eq. 13/17)

// f[i] = exp(-alpha[n] softplus(a[i] + beta[n])), i over [B*T, N] (n = i % N).
__global__ void __launch_bounds__(kBlkThreads) m2rnn_gate_fwd_kernel(const float* __restrict__ a,
                                                                      const float* __restrict__ alpha,
                                                                      const float* __restrict__ beta, long count, int N,
                                                                      float* __restrict__ f) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (long)gridDim.x * blockDim.x) {
    const int n = (int)(i % N);
    f[i] = gate_f(a[i], alpha[n], beta[n]);
  }
}

// da[i] = df f (-alpha sigmoid(z)), z = a + beta; ga[i] = df f (-softplus(z)) (dalpha's terms).
__global__ void __launch_bounds__(kBlkThreads) m2rnn_gate_bwd_kernel(const float* __restrict__ a,
                                                                      const float* __restrict__ alpha,
                                                                      const float* __restrict__ beta,
                                                                      const float* __restrict__ df, long count, int N,
                                                                      float* __restrict__ da, float* __restrict__ ga) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += (long)gridDim.x * blockDim.x) {
    const int n = (int)(i % N);
    const float z = a[i] + beta[n];
    const float sp = softplusf_(z);
    const float g = df[i] * exp_(-alpha[n] * sp);
    da[i] = -alpha[n] * sigmoidf_(z) * g;
    ga[i] = -sp * g;
  }
}

// The same with the sums over (b, t) taken per workgroup: the workgroup has a multiple of N
// threads, so thread t meets only column n = t % N of the [B*T, N] elements i0 + t + m * blockDim
// it handles; its partials are then added in the order of t into part[blockIdx][2][N]
// (0: dbeta, 1: dalpha).
__global__ void __launch_bounds__(kBlkThreads) m2rnn_gate_bwd_part_kernel(const float* __restrict__ a,
                                                                           const float* __restrict__ alpha,
                                                                           const float* __restrict__ beta,
                                                                           const float* __restrict__ df, long count,
                                                                           int N, long per_block, float* __restrict__ da,
                                                                           float* __restrict__ part) {
  __shared__ float red[2][kBlkThreads];
  const int tb = blockDim.x;
  const int t = threadIdx.x;
  const int n = t % N;
  const float al = alpha[n], be = beta[n];
  const long i0 = (long)blockIdx.x * per_block;
  const long i1 = i0 + per_block < count ? i0 + per_block : count;
  float s0 = 0.0f, s1 = 0.0f;
  for (long i = i0 + t; i < i1; i += tb) {
    const float z = a[i] + be;
    const float sp = softplusf_(z);
    const float g = df[i] * exp_(-al * sp);
    const float d = -al * sigmoidf_(z) * g;
    da[i] = d;
    s0 += d;
    s1 += -sp * g;
  }
  red[0][t] = s0;
  red[1][t] = s1;
  __syncthreads();
  if (t < N) {
    float r0 = 0.0f, r1 = 0.0f;
    for (int k = t; k < tb; k += N) {
      r0 += red[0][k];
      r1 += red[1][k];
    }
    part[((long)blockIdx.x * 2 + 0) * N + t] = r0;
    part[((long)blockIdx.x * 2 + 1) * N + t] = r1;
  }
}

// out0[n] = sum over r of in0[r * N + n], out1 likewise (one workgroup per n, fixed order).
__global__ void __launch_bounds__(kBlkThreads) m2rnn_col_sum2_kernel(const float* __restrict__ in0,
                                                                      const float* __restrict__ in1, long rows, int N,
                                                                      float* __restrict__ out0,
                                                                      float* __restrict__ out1) {
  __shared__ float red[2 * kBlkThreads / 64];
  const int n = blockIdx.x;
  float s0 = 0.0f, s1 = 0.0f;
  for (long r = threadIdx.x; r < rows; r += kBlkThreads) {
    s0 += in0[r * N + n];
    s1 += in1[r * N + n];
  }
  const float2 s = block_sum2(s0, s1, red);
  if (threadIdx.x == 0) {
    out0[n] = s.x;
    out1[n] = s.y;
  }
}

// ------------------------------------------------------------------ output gate + RMSNorm (§2.3, App. C)

// One workgroup per row (token) of D features: x = y (.) SiLU(gz), out = gamma (.) x / sqrt(mean x^2 + eps).
// Thread t owns the 4-feature groups t, t + 256, ... (QMAX of them at most; D is a multiple of 4)
// and keeps their x in registers between the sum of squares and the scaling.
template <bool BF16, int QMAX>
__global__ void __launch_bounds__(kBlkThreads) m2rnn_out_norm_fwd_kernel(const float* __restrict__ y,
                                                                          const void* __restrict__ gz,
                                                                          const float* __restrict__ gamma, int D,
                                                                          float eps, float* __restrict__ out) {
  __shared__ float red[2 * kBlkThreads / 64];
  const long row = blockIdx.x;
  const long base = row * D;
  float ss = 0.0f;
  float4 xk[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * ((int)threadIdx.x + kBlkThreads * q);
    if (j < D) {
      const float4 yv = load4_nt<false>(y, base + j);
      const float4 g = load4_nt<BF16>(gz, base + j);
      xk[q] = make_float4(yv.x * siluf_(g.x), yv.y * siluf_(g.y), yv.z * siluf_(g.z), yv.w * siluf_(g.w));
      ss += xk[q].x * xk[q].x + xk[q].y * xk[q].y + xk[q].z * xk[q].z + xk[q].w * xk[q].w;
    }
  }
  const float s = 1.0f / sqrtf(block_sum2(ss, 0.0f, red).x / (float)D + eps);
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * ((int)threadIdx.x + kBlkThreads * q);
    if (j < D) {
      const float4 gm = *(const float4*)(gamma + j);
      const float o[4] = {gm.x * xk[q].x * s, gm.y * xk[q].y * s, gm.z * xk[q].z * s, gm.w * xk[q].w * s};
      store4_nt<false>(out, base + j, o);
    }
  }
}

// The block forward's output epilogue, one workgroup per token: y = the sum of the scan's S
// readout planes + w_r (.) v (w_r null: the single plane already holds y), then the output gate
// and RMSNorm exactly as m2rnn_out_norm_fwd_kernel takes them (same operations in the same
// order, so the result is bit-identical to the two passes).  y itself never goes to HBM.  Token
// (b = blockIdx.y, t = t0 + blockIdx.x) of a [B, T] sequence.
template <bool BF16V, bool BF16G, int QMAX>
__global__ void __launch_bounds__(kBlkThreads) m2rnn_fwd_finish_norm_kernel(
    const float* __restrict__ part, int S, long plane, const void* __restrict__ v, const float* __restrict__ w_r,
    const void* __restrict__ gz, const float* __restrict__ gamma, int D, float eps, float* __restrict__ out, long T,
    long t0) {
  __shared__ float red[2 * kBlkThreads / 64];
  const long base = ((long)blockIdx.y * T + t0 + blockIdx.x) * D;
  float ss = 0.0f;
  float4 xk[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * ((int)threadIdx.x + kBlkThreads * q);
    if (j < D) {
      // the planes are read once: non-temporal loads
      f32x4 ys = __builtin_nontemporal_load((const f32x4*)(part + base + j));
      for (int s = 1; s < S; ++s) ys += __builtin_nontemporal_load((const f32x4*)(part + (long)s * plane + base + j));
      float4 yv = make_float4(ys[0], ys[1], ys[2], ys[3]);
      if (w_r) {
        const float4 wr = *(const float4*)(w_r + j);
        const float4 vv = load4_nt<BF16V>(v, base + j);
        yv.x = __builtin_fmaf(wr.x, vv.x, yv.x);
        yv.y = __builtin_fmaf(wr.y, vv.y, yv.y);
        yv.z = __builtin_fmaf(wr.z, vv.z, yv.z);
        yv.w = __builtin_fmaf(wr.w, vv.w, yv.w);
      }
      const float4 g = load4_nt<BF16G>(gz, base + j);
      xk[q] = make_float4(yv.x * siluf_(g.x), yv.y * siluf_(g.y), yv.z * siluf_(g.z), yv.w * siluf_(g.w));
      ss += xk[q].x * xk[q].x + xk[q].y * xk[q].y + xk[q].z * xk[q].z + xk[q].w * xk[q].w;
    }
  }
  const float s = 1.0f / sqrtf(block_sum2(ss, 0.0f, red).x / (float)D + eps);
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * ((int)threadIdx.x + kBlkThreads * q);
    if (j < D) {
      const float4 gm = *(const float4*)(gamma + j);
      const float o[4] = {gm.x * xk[q].x * s, gm.y * xk[q].y * s, gm.z * xk[q].z * s, gm.w * xk[q].w * s};
      store4_nt<false>(out, base + j, o);
    }
  }
}

// Backward (Appendix C), one workgroup per `rows_per` consecutive rows, in the forward's layout:
// p = gamma (.) dout, r = sum p x, dx = s p - r s^3 x / D; dy = dx (.) SiLU(gz);
// dgz = dx (.) y (.) SiLU'(gz).  The workgroup's partial of dgamma = sum over its rows of
// dout (.) x s goes to dgamma_part[workgroup][D].  With at most 2 groups per thread the next row's
// loads are in flight while the current row is reduced and written.
template <bool BF16, int QMAX>
__global__ void __launch_bounds__(kBlkThreads) m2rnn_out_norm_bwd_kernel(
    const float* __restrict__ y, const void* __restrict__ gz, const float* __restrict__ gamma, int D, float eps,
    const float* __restrict__ dout, long rows, int rows_per, float* __restrict__ dy, float* __restrict__ dgz,
    float* __restrict__ dgamma_part) {
  __shared__ float red[2 * kBlkThreads / 64];
  constexpr bool PIPE = QMAX <= 2;
  const int tid = threadIdx.x;
  const long r0 = (long)blockIdx.x * rows_per;
  const long r1 = min(rows, r0 + rows_per);
  struct Row {
    float4 y[QMAX], g[QMAX], d[QMAX];
  };
  auto load = [&](long r, Row& o) {
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int j = 4 * (tid + kBlkThreads * q);
      if (j < D) {
        o.y[q] = load4_nt<false>(y, r * D + j);
        o.g[q] = load4_nt<BF16>(gz, r * D + j);
        o.d[q] = load4_nt<false>(dout, r * D + j);
      }
    }
  };
  float4 gm[QMAX], acc[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * (tid + kBlkThreads * q);
    gm[q] = j < D ? *(const float4*)(gamma + j) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    acc[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  Row cur;
  load(r0, cur);
  for (long r = r0; r < r1; ++r) {
    Row nxt;
    if constexpr (PIPE) load(min(r + 1, r1 - 1), nxt);
    float ss = 0.0f, rp = 0.0f;
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int j = 4 * (tid + kBlkThreads * q);
      if (j < D) {
        const float4 yv = cur.y[q], g = cur.g[q], d = cur.d[q];
        const float x0 = yv.x * siluf_(g.x), x1 = yv.y * siluf_(g.y), x2 = yv.z * siluf_(g.z),
                    x3 = yv.w * siluf_(g.w);
        ss += x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
        rp += gm[q].x * d.x * x0 + gm[q].y * d.y * x1 + gm[q].z * d.z * x2 + gm[q].w * d.w * x3;
      }
    }
    const float2 t = block_sum2(ss, rp, red);
    const float s = 1.0f / sqrtf(t.x / (float)D + eps);
    const float c = t.y * s * s * s / (float)D;
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
      const int j = 4 * (tid + kBlkThreads * q);
      if (j < D) {
        const float gs[4] = {cur.g[q].x, cur.g[q].y, cur.g[q].z, cur.g[q].w};
        const float ys[4] = {cur.y[q].x, cur.y[q].y, cur.y[q].z, cur.y[q].w};
        const float ds[4] = {cur.d[q].x, cur.d[q].y, cur.d[q].z, cur.d[q].w};
        const float gms[4] = {gm[q].x, gm[q].y, gm[q].z, gm[q].w};
        float oy[4], og[4], ag[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float sg = siluf_(gs[e]);
          const float x = ys[e] * sg;
          const float dx = s * gms[e] * ds[e] - c * x;
          oy[e] = dx * sg;
          og[e] = dx * ys[e] * silu_gradf_(gs[e]);
          ag[e] = ds[e] * x * s;
        }
        store4_nt<false>(dy, r * D + j, oy);
        store4_nt<false>(dgz, r * D + j, og);
        acc[q].x += ag[0];
        acc[q].y += ag[1];
        acc[q].z += ag[2];
        acc[q].w += ag[3];
      }
    }
    if constexpr (PIPE)
      cur = nxt;
    else if (r + 1 < r1)
      load(r + 1, cur);
  }
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int j = 4 * (tid + kBlkThreads * q);
    if (j < D) *(float4*)(dgamma_part + (long)blockIdx.x * D + j) = acc[q];
  }
}

// One level of a fixed-order reduction of `parts` rows of M columns (row p at part + p * stride):
// slice y of `per` consecutive rows is summed into output row y; output row y, column j goes to
// out0[y * M + j] when j < M0, else to out1[y * M + j - M0] (out1 may be null: those are dropped).
__global__ void __launch_bounds__(kBlkThreads) m2rnn_sum_slices_kernel(const float* __restrict__ part, int parts,
                                                                        long M, long stride, int per,
                                                                        float* __restrict__ out0, long M0,
                                                                        float* __restrict__ out1) {
  const long j = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= M) return;
  const int p0 = blockIdx.y * per;
  const int p1 = p0 + per < parts ? p0 + per : parts;
  float acc = 0.0f;
#pragma unroll 8
  for (int p = p0; p < p1; ++p) acc += part[(long)p * stride + j];
  if (j < M0) out0[(long)blockIdx.y * M + j] = acc;
  else if (out1) out1[(long)blockIdx.y * M + j - M0] = acc;
}

// ------------------------------------------------------------------ causal conv4 + SiLU (§2.3)

// Steps per thread (a sliding window over time).  The backward takes longer chunks: half the
// partial sums of dw and dbias, and fewer re-read steps at the chunk edges.
// (The host halves them, down to kConvChunkMin, while the grid would hold fewer than
// kConvMinWaves waves: short or narrow inputs then still fill the chip.)
constexpr int kConvChunkFwd = 64;
constexpr int kConvChunkBwd = 128;
constexpr int kConvChunkMin = 16;
constexpr long kConvMinWaves = 2048;
constexpr int kConvBatch = 4;  // steps whose loads are issued together

// The threads of a wave share one (b, chunk) and take 64 consecutive groups of 4 channels; a row
// of C/4 groups spans ceil(C/256) waves.  b, chunk and the step range are then uniform over the
// wave (scalar registers and branches).  False for a lane with nothing to do.
__device__ __forceinline__ bool conv_pos(int B, int T, int C, int CHUNK, int& b, int& chunk, int& c4) {
  const int C4 = C / 4;
  const int nchunk = (T + CHUNK - 1) / CHUNK;
  const int wpr = (C4 + 63) / 64;
  const int gw = (int)blockIdx.x * (kBlkThreads / 64) + __builtin_amdgcn_readfirstlane((int)threadIdx.x / 64);
  const int bc = gw / wpr;
  c4 = (gw - bc * wpr) * 64 + (int)(threadIdx.x & 63);
  chunk = bc % nchunk;
  b = bc / nchunk;
  return b < B && c4 < C4;
}

// Thread (b, chunk of CHUNK steps, 4 channels c4): pre_t = sum_i w[c][i] x_{t-3+i} + bias[c],
// u_t = SiLU(pre_t), with x_t = 0 for t < 0.  Layout [B, T, C]; C is a multiple of 4.
template <bool BF16>
__global__ void __launch_bounds__(kBlkThreads) m2rnn_conv4_silu_fwd_kernel(const void* __restrict__ x,
                                                                            const float* __restrict__ w,
                                                                            const float* __restrict__ bias, int B,
                                                                            int T, int C, int CHUNK,
                                                                            void* __restrict__ u) {
  int b, chunk, c4;
  if (!conv_pos(B, T, C, CHUNK, b, chunk, c4)) return;
  const int c = 4 * c4;
  float wk[4][4];  // [channel][tap]
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 t4 = *(const float4*)(w + (long)(c + e) * 4);
    wk[e][0] = t4.x; wk[e][1] = t4.y; wk[e][2] = t4.z; wk[e][3] = t4.w;
  }
  const float4 bv = bias ? *(const float4*)(bias + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float bs[4] = {bv.x, bv.y, bv.z, bv.w};
  const int t0 = chunk * CHUNK;
  const int t1 = min(T, t0 + CHUNK);
  const long row = (long)b * T;
  // window: xs[0..2] = x_{t-3..t-1}
  float xs[3][4];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    const int src = t0 - 3 + i;
    const float4 v = src >= 0 ? load4<BF16>(x, (row + src) * C + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    xs[i][0] = v.x; xs[i][1] = v.y; xs[i][2] = v.z; xs[i][3] = v.w;
  }
  // The loads run one batch of kConvBatch steps ahead of the arithmetic, so a wave always has a
  // batch in flight.  A step past the thread's last one re-reads the last (no branch, no extra
  // HBM traffic).
  auto issue = [&](int tb, float4(&o)[kConvBatch]) {
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) o[k] = load4<BF16>(x, (row + min(tb + k, t1 - 1)) * C + c);
  };
  float4 xv[kConvBatch];
  issue(t0, xv);
  for (int tb = t0; tb < t1; tb += kConvBatch) {
    float4 xn[kConvBatch];
    issue(tb + kConvBatch, xn);
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) {
      if (tb + k < t1) {
        const float xc[4] = {xv[k].x, xv[k].y, xv[k].z, xv[k].w};
        float o[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pre =
              wk[e][0] * xs[0][e] + wk[e][1] * xs[1][e] + wk[e][2] * xs[2][e] + wk[e][3] * xc[e] + bs[e];
          o[e] = siluf_(pre);
          xs[0][e] = xs[1][e];
          xs[1][e] = xs[2][e];
          xs[2][e] = xc[e];
        }
        store4_nt<BF16>(u, (row + tb + k) * C + c, o);
      }
    }
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) xv[k] = xn[k];
  }
}

// Backward, same layout (its chunks start at kConvChunkBwd steps).  dpre_t = du_t SiLU'(pre_t),
// dx_s = sum_i w[c][i] dpre_{s+3-i}; the thread's partials of dw[c][i] = sum dpre_t x_{t-3+i} and
// dbias[c] = sum dpre_t go to part[(b * nchunk + chunk)] as [C][4] taps followed by C biases.
template <bool BF16>
__global__ void __launch_bounds__(kBlkThreads) m2rnn_conv4_silu_bwd_kernel(const void* __restrict__ x,
                                                                            const float* __restrict__ w,
                                                                            const float* __restrict__ bias,
                                                                            const float* __restrict__ du, int B, int T,
                                                                            int C, int CHUNK, float* __restrict__ dx,
                                                                            float* __restrict__ part) {
  int b, chunk, c4;
  if (!conv_pos(B, T, C, CHUNK, b, chunk, c4)) return;
  const int c = 4 * c4;
  float wk[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float4 t4 = *(const float4*)(w + (long)(c + e) * 4);
    wk[e][0] = t4.x; wk[e][1] = t4.y; wk[e][2] = t4.z; wk[e][3] = t4.w;
  }
  const float4 bv = bias ? *(const float4*)(bias + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  const float bs[4] = {bv.x, bv.y, bv.z, bv.w};
  const int t0 = chunk * CHUNK;
  const int t1 = min(T, t0 + CHUNK);
  const long row = (long)b * T;
  auto xat = [&](int t, float (&o)[4]) {
    const float4 v = (t >= 0 && t < T) ? load4<BF16>(x, (row + t) * C + c) : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  };
  // dpre at step t (0 outside [0, T)).
  auto dpre_at = [&](int t, const float (&xw)[4][4], float (&o)[4]) {
    // xw[i] = x_{t-3+i}
    if (t < 0 || t >= T) {
      o[0] = o[1] = o[2] = o[3] = 0.0f;
      return;
    }
    const float4 d = *(const float4*)(du + (row + t) * C + c);
    const float ds[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float pre = wk[e][0] * xw[0][e] + wk[e][1] * xw[1][e] + wk[e][2] * xw[2][e] + wk[e][3] * xw[3][e] + bs[e];
      o[e] = ds[e] * silu_gradf_(pre);
    }
  };
  // Sliding window over t = t0 .. t1 + 2 of x_{t-3 .. t} and of dpre_{t-3 .. t}: dx_s for s = t - 3
  // needs dpre_{s .. s+3} = dpre_{t-3 .. t}.
  float xw[4][4];
  for (int i = 0; i < 3; ++i) xat(t0 - 3 + i, xw[i]);
  float dp[4][4];  // dp[i] = dpre_{t-3+i}
  {
    float xx[4][4];
    for (int i = 0; i < 3; ++i) {
      // dpre_{t0-3+i}: its window is x_{t0-6+i .. t0-3+i}
      for (int k = 0; k < 4; ++k) xat(t0 - 6 + i + k, xx[k]);
      dpre_at(t0 - 3 + i, xx, dp[i]);
    }
  }
  float aw[4][4] = {}, ab[4] = {};
  const int tend = t1 + 3;
  // x and du loads run one batch of kConvBatch steps ahead of the arithmetic.  A step at or past
  // min(tend, T) re-reads the last one below it; such values only meet dpre = 0 (selected, so
  // they cannot leak) and take no part in dw.
  const int tlast = min(tend, T) - 1;
  auto issue = [&](int tb, float4(&xo)[kConvBatch], float4(&dvo)[kConvBatch]) {
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) {
      const long i = (row + min(tb + k, tlast)) * C + c;
      xo[k] = load4_nt<BF16>(x, i);
      dvo[k] = load4_nt<false>(du, i);
    }
  };
  float4 xv[kConvBatch], dv[kConvBatch];
  issue(t0, xv, dv);
  for (int tb = t0; tb < tend; tb += kConvBatch) {
    float4 xn[kConvBatch], dn[kConvBatch];
    issue(tb + kConvBatch, xn, dn);
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) {
      const int t = tb + k;
      if (t < tend) {
        xw[3][0] = xv[k].x; xw[3][1] = xv[k].y; xw[3][2] = xv[k].z; xw[3][3] = xv[k].w;
        const float ds[4] = {dv[k].x, dv[k].y, dv[k].z, dv[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float pre =
              wk[e][0] * xw[0][e] + wk[e][1] * xw[1][e] + wk[e][2] * xw[2][e] + wk[e][3] * xw[3][e] + bs[e];
          dp[3][e] = t < T ? ds[e] * silu_gradf_(pre) : 0.0f;
        }
        if (t < t1) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int i = 0; i < 4; ++i) aw[e][i] += dp[3][e] * xw[i][e];
            ab[e] += dp[3][e];
          }
        }
        const int sidx = t - 3;
        if (sidx >= t0) {
          float o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            o[e] = wk[e][3] * dp[0][e] + wk[e][2] * dp[1][e] + wk[e][1] * dp[2][e] + wk[e][0] * dp[3][e];
          store4_nt<false>(dx, (row + sidx) * C + c, o);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            xw[i][e] = xw[i + 1][e];
            dp[i][e] = dp[i + 1][e];
          }
      }
    }
#pragma unroll
    for (int k = 0; k < kConvBatch; ++k) {
      xv[k] = xn[k];
      dv[k] = dn[k];
    }
  }
  // [4C: dw as [C][4] | C: dbias]
  float* pp = part + ((long)b * ((T + CHUNK - 1) / CHUNK) + chunk) * C * 5;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    *(float4*)(pp + (c + e) * 4) = make_float4(aw[e][0], aw[e][1], aw[e][2], aw[e][3]);
    pp[4 * C + c + e] = ab[e];
  }
}

}  // namespace m2rnn
