// One step of the M²RNN recurrence (M²RNN notes §2.1, Eq. 10-12) with the state in HBM: the
// decode form of the layer, where each call advances every (b, n) state by one token.  The notes
// stress that inference keeps a fixed-size recurrent state (§2.6); this kernel reads that state,
// applies Eq. 10-12 once and writes it back, so it is bound by HBM traffic (8 K V bytes of state
// per (b, n)), not by the contraction.
//
// Work decomposition
//   One wave carries one (b, n) pair: all K rows (in 16-row blocks, the next block's loads in
//   flight while the current one is computed) and all V columns.  A workgroup holds four waves,
//   the batch entries 4j .. 4j+3 of one head, which share W'^T = (c W)^T (c = 2 log2 e) as split
//   fp16 MFMA operands in LDS, converted once per workgroup.  Because a wave reads each row block
//   whole before it writes it, and no other wave touches that pair, the state may be updated in
//   place (H_out == H_in).
//
// Register layout (as in the forward scan): the contraction computes P^T = W'^T H^T with
// 16x16x32 fp16 MFMAs, so lane (g = lane/16, n = lane%16), register r of output tile t holds
// P[row n][col 16t + 4g + r].  The state block is loaded in that same layout (one 16-byte load per
// lane per tile), so the blend needs no data movement, and the contraction index of chunk c is
// permuted to v = 16(2c + i/4) + 4g + i%4 for k-slot i of lane group g, in both operands.
#pragma once

#include "m2rnn_device.h"

namespace m2rnn {

struct DecArgs {
  const void* q;      // [B, Nqk, K]
  const void* k;      // [B, Nqk, K]
  const void* v;      // [B, N, V]
  const float* f;     // [B, N]
  const float* W;     // [N, V, V]
  const float* w_r;   // [N, V]
  const float* H_in;  // [B, N, K, V] or null (zeros)
  float* H_out;       // [B, N, K, V] (may equal H_in)
  float* y;           // [B, N, V]
  int B, N, K;
  int Nqk;            // heads of q and k: N, or 1 when one query/key is shared by all heads
};

constexpr int kDecWaves = 4;  // batch entries (one wave each) per workgroup

template <bool BF16>
__device__ __forceinline__ float load_scalar(const void* base, long idx) {
  if constexpr (BF16) return bf16_lo_to_f32((uint32_t)((const uint16_t*)base)[idx]);
  return ((const float*)base)[idx];
}

// Four consecutive elements starting at idx (a multiple of 4).
template <bool BF16>
__device__ __forceinline__ float4 load_vec4(const void* base, long idx) {
  if constexpr (BF16) {
    const uint2 r = *(const uint2*)((const uint16_t*)base + idx);
    return make_float4(bf16_lo_to_f32(r.x), bf16_hi_to_f32(r.x), bf16_lo_to_f32(r.y), bf16_hi_to_f32(r.y));
  }
  return *(const float4*)((const float*)base + idx);
}

// Splits x (>= 4 values) into packed fp16 high parts and fp16 rounding remainders: x ~ hi + lo
// with about 22 significant bits (the remainder x - hi is exact in fp32).
__device__ __forceinline__ void split4_f16(const float* x, uint32_t& h01, uint32_t& h23, uint32_t& l01, uint32_t& l23) {
  h01 = pack_f16(x[0], x[1]);
  h23 = pack_f16(x[2], x[3]);
  l01 = pack_f16(x[0] - f16_lo_to_f32(h01), x[1] - f16_hi_to_f32(h01));
  l23 = pack_f16(x[2] - f16_lo_to_f32(h23), x[3] - f16_hi_to_f32(h23));
}

template <int V, bool BF16IN>
__global__ void __launch_bounds__(64 * kDecWaves) m2rnn_decode_kernel(const DecArgs a) {
  constexpr int NT = V / 16;          // 16-column tiles
  constexpr int NCH = (NT + 1) / 2;   // 32-wide contraction chunks
  // A operands W'^T, [tile][chunk][hi|lo][lane] x 16 bytes: each MFMA's operand is one
  // conflict-free 16-byte read per lane.
  __shared__ uint4 wop[NT * NCH * 2 * 64];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;
  const int nh = blockIdx.x % a.N;
  const int b = (blockIdx.x / a.N) * kDecWaves + w;

  // This wave's pair (a wave past the batch only helps to stage W).
  const bool active = b < a.B;
  const long unit = (long)(active ? b : 0) * a.N + nh;
  const long KV = (long)a.K * V;
  const float* Hin = a.H_in ? a.H_in + unit * KV : nullptr;
  float* Hout = a.H_out + unit * KV;

  auto load_block = [&](int rb, float (&Hb)[NT][4]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      f32x4 x = {0.0f, 0.0f, 0.0f, 0.0f};
      if (Hin) x = *((const f32x4*)(Hin + (long)(16 * rb + n) * V + 16 * t + 4 * g));
      Hb[t][0] = x[0]; Hb[t][1] = x[1]; Hb[t][2] = x[2]; Hb[t][3] = x[3];
    }
  };

  // The first state block and the per-pair inputs are requested before W is staged, so that their
  // latency overlaps the staging.
  const int KB = a.K / 16;
  float Hc[NT][4];
  load_block(0, Hc);
  const float fv = a.f[unit];
  const float gf = 1.0f - fv, m2g = -2.0f * gf;
  // v at this lane's columns 16t + 4g + r.
  float vv[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float4 x = load_vec4<BF16IN>(a.v, unit * V + 16 * t + 4 * g);
    vv[t][0] = x.x; vv[t][1] = x.y; vv[t][2] = x.z; vv[t][3] = x.w;
  }

  // ---- W'^T operands, split once per workgroup ----
  const float* Wn = a.W + (long)nh * V * V;
  for (int e = tid; e < NT * NCH * 64; e += 64 * kDecWaves) {
    const int l = e & 63, tc = e >> 6;
    const int tile = tc / NCH, c = tc % NCH;
    const int gg = l >> 4, m = l & 15;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int vin = 16 * (2 * c + (i >> 2)) + 4 * gg + (i & 3);
      x[i] = vin < V ? opaque1(kTwoLog2e * Wn[vin * V + 16 * tile + m]) : 0.0f;
    }
    uint32_t h[4], lo[4];
    split4_f16(x, h[0], h[1], lo[0], lo[1]);
    split4_f16(x + 4, h[2], h[3], lo[2], lo[3]);
    wop[(tc * 2 + 0) * 64 + l] = make_uint4(h[0], h[1], h[2], h[3]);
    wop[(tc * 2 + 1) * 64 + l] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
  // LDS-only barrier: the state loads above stay in flight across it.
  lds_barrier();
  if (!active) return;  // no barrier follows

  float yacc[NT][4];
#pragma unroll
  for (int t = 0; t < NT; ++t) yacc[t][0] = yacc[t][1] = yacc[t][2] = yacc[t][3] = 0.0f;

  for (int rb = 0; rb < KB; ++rb) {
    // Next block in flight while this one is computed.
    float Hn[NT][4];
    if (rb + 1 < KB) load_block(rb + 1, Hn);
    const long row = ((long)b * a.Nqk + (a.Nqk == 1 ? 0 : nh)) * a.K + 16 * rb + n;
    const float qv = load_scalar<BF16IN>(a.q, row);
    const float ck = kTwoLog2e * load_scalar<BF16IN>(a.k, row);

    // B operands H^T (split), chunk c = tiles 2c (k-slots 0..3) and 2c+1 (k-slots 4..7).
    uint4 bh[NCH], bl[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      uint32_t h0, h1, l0, l1, h2 = 0, h3 = 0, l2 = 0, l3 = 0;
      split4_f16(Hc[2 * c], h0, h1, l0, l1);
      if (2 * c + 1 < NT) split4_f16(Hc[2 * c + 1], h2, h3, l2, l3);
      bh[c] = make_uint4(h0, h1, h2, h3);
      bl[c] = make_uint4(l0, l1, l2, l3);
    }

    // The A operands are read from LDS again for every block (an opaque offset keeps the compiler
    // from hoisting all of them into registers, which would cost occupancy: this kernel needs
    // many waves in flight to cover HBM latency).
    int wofs = lane;
    asm volatile("" : "+v"(wofs));
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      // acc = (c k) v^T + W'^T H^T for output tile t.
      f32x4 acc = {ck * vv[t][0], ck * vv[t][1], ck * vv[t][2], ck * vv[t][3]};
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint4 Ah = wop[((t * NCH + c) * 2 + 0) * 64 + wofs];
        const uint4 Al = wop[((t * NCH + c) * 2 + 1) * 64 + wofs];
        acc = mfma_f16(Ah, bh[c], acc);
        acc = mfma_f16(Al, bh[c], acc);
        acc = mfma_f16(Ah, bl[c], acc);
      }
      // tanh + gate blend: H = f H + (1-f)(1 - 2r) = fma(-2(1-f), r, fma(f, H, 1-f)).
      float hn[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        hn[r] = __builtin_fmaf(m2g, tanh_recip(acc[r]), __builtin_fmaf(fv, Hc[t][r], gf));
        yacc[t][r] = __builtin_fmaf(qv, hn[r], yacc[t][r]);
      }
      const f32x4 hv = {hn[0], hn[1], hn[2], hn[3]};
      *(f32x4*)(Hout + (long)(16 * rb + n) * V + 16 * t + 4 * g) = hv;
    }
    if (rb + 1 < KB) {
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) Hc[t][r] = Hn[t][r];
    }
  }

  // Readout y = H^T q + w_r (.) v: sum the lanes' q-weighted partials over the 16 rows of a DPP
  // row; lane (g, n) then holds column 16t + 4g + n/4, and the lanes with n % 4 == 0 store it.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const float s = row16_sum4(yacc[t][0], yacc[t][1], yacc[t][2], yacc[t][3], lane);
    if ((n & 3) == 0) {
      const int col = 16 * t + 4 * g + (n >> 2);
      const float vc = load_scalar<BF16IN>(a.v, unit * V + col);
      a.y[unit * V + col] = __builtin_fmaf(a.w_r[(long)nh * V + col], vc, s);
    }
  }
}

}  // namespace m2rnn
