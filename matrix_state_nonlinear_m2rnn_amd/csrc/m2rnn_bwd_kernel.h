// Backward (BPTT) of the M²RNN recurrence for gfx950: the chain-rule equations of the M²RNN notes
// §2.7 (written there in place of the paper's Algorithm 2):
//     R_t = C_t + q_t u_t^T                      u_t = dL/dy_t
//     D_t = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t)
//     C_{t-1} = f_t R_t + D_t W^T                (serial chain, C_T = dL/dH_T)
//     dq_t = H_t u_t,  dk_t = D_t v_t,  dv_t = D_t^T k_t + w_r (.) u_t,  df_t = <R_t, H_{t-1} - Z_t>
//     dW = sum_t H_{t-1}^T D_t,  dw_r = sum_t u_t (.) v_t,  dH_0 = C_0.
//
// Work decomposition (one 16-row block of one (b, n) pair per workgroup, wave w owns value
// columns [16w, 16w+16), same register layout as the forward scan):
//   for every 64-step segment, last to first:
//     1. stage the segment's q, k, v, f, dy in LDS;
//     2. recompute the segment forward from its checkpoint, writing each step's H_{t-1} (split
//        fp16 hi/lo, the form that is exchanged anyway) and Z_t (fp32) to a per-workgroup
//        workspace slice;
//     3. walk the segment backwards: R, D and the row/column reductions in registers; D is
//        published through LDS exactly like H in the forward, and the chain's D W^T runs on the
//        split-precision MFMA; every wave transposes the D tiles it has just read (one MFMA per
//        tile) and accumulates dW[own columns of H_{t-1}][all columns of D] with split-fp16 MFMAs.
//   Per-workgroup partials of dv, df and dW are summed by separate, deterministic passes.
#pragma once

#include "m2rnn_fwd_kernel.h"

namespace m2rnn {

constexpr int kBwdSeg = 64;  // checkpoint interval (steps)

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* f;
  const float* W;
  const float* w_r;
  const float* dy;
  const float* dH_T;
  const float* ckpt;   // [B][N][nseg][K][V] states entering each segment
  float* seg_ws;       // per-workgroup segment store
  float* dq;
  float* dk;
  float* dv;           // final dv (S == 1) or partials [S][B*T*N*V]
  float* df;           // final df (S == 1) or partials [S][B*T*N]
  float* dW_part;      // [B*S][N][V][V]
  float* dwr_part;     // [B][N][V] (written by the workgroups with s == 0)
  float* dH0;          // may be null
  int B, T, N, K;
  int S;
};

// Per-step stage record of the backward (fp32):
//   [f, 1-f, -2(1-f), 0 | q (16) | c*k (16) | k (16) | v (V) | u (V)]
template <int V>
struct BwdStage {
  static constexpr int OQ = 4;
  static constexpr int OCK = 20;
  static constexpr int OK = 36;
  static constexpr int OV = 52;
  static constexpr int OU = 52 + V;
  static constexpr int STEP = 52 + 2 * V;
};

// Loads the (up to) kBwdSeg steps [t0, t0 + n_steps) of one 16-row block into the stage.
template <int V, bool BF16IN>
__device__ __forceinline__ void bwd_stage_segment(const BwdArgs& a, int b, int nh, int row0, int t0, int n_steps,
                                                  float* stage, int tid, int nth) {
  using St = BwdStage<V>;
  const int esz = BF16IN ? 2 : 4;
  constexpr int VEC = BF16IN ? 8 : 4;
  // q, k: 16 values per step, VEC per load.
  constexpr int QV = 16 / VEC;
  for (int i = tid; i < kBwdSeg * QV * 2; i += nth) {
    const int which = i / (kBwdSeg * QV);  // 0 = q, 1 = k
    const int r = i % (kBwdSeg * QV);
    const int step = r / QV, cv = r % QV;
    if (step >= n_steps) continue;
    const long off = ((((long)b * a.T + t0 + step) * a.N + nh) * a.K + row0 + cv * VEC);
    const void* src = which == 0 ? a.q : a.k;
    const uint4 raw = *(const uint4*)((const char*)src + off * esz);
    float vals[VEC];
    if constexpr (BF16IN) {
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vals[2 * e] = bf16_lo_to_f32(wds[e]);
        vals[2 * e + 1] = bf16_hi_to_f32(wds[e]);
      }
    } else {
      vals[0] = __uint_as_float(raw.x); vals[1] = __uint_as_float(raw.y);
      vals[2] = __uint_as_float(raw.z); vals[3] = __uint_as_float(raw.w);
    }
    float* d = stage + step * St::STEP;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      if (which == 0) {
        d[St::OQ + cv * VEC + e] = vals[e];
      } else {
        d[St::OCK + cv * VEC + e] = kTwoLog2e * vals[e];
        d[St::OK + cv * VEC + e] = vals[e];
      }
    }
  }
  // v (dtype of the inputs) and u = dy (fp32): V values per step.
  constexpr int VV = V / VEC;
  for (int i = tid; i < kBwdSeg * VV; i += nth) {
    const int step = i / VV, cv = i % VV;
    if (step >= n_steps) continue;
    const long off = (((long)b * a.T + t0 + step) * a.N + nh) * V + cv * VEC;
    const uint4 raw = *(const uint4*)((const char*)a.v + off * esz);
    float* d = stage + step * St::STEP + St::OV + cv * VEC;
    if constexpr (BF16IN) {
      const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        d[2 * e] = bf16_lo_to_f32(wds[e]);
        d[2 * e + 1] = bf16_hi_to_f32(wds[e]);
      }
    } else {
      *(uint4*)d = raw;
    }
  }
  constexpr int UV = V / 4;
  for (int i = tid; i < kBwdSeg * UV; i += nth) {
    const int step = i / UV, cv = i % UV;
    if (step >= n_steps) continue;
    const long off = (((long)b * a.T + t0 + step) * a.N + nh) * V + cv * 4;
    *(float4*)(stage + step * St::STEP + St::OU + cv * 4) = *(const float4*)(a.dy + off);
  }
  for (int i = tid; i < kBwdSeg; i += nth) {
    if (i >= n_steps) continue;
    const float fv = a.f[((long)b * a.T + t0 + i) * a.N + nh];
    const float g = 1.0f - fv;
    *(float4*)(stage + i * St::STEP) = make_float4(fv, g, -2.0f * g, 0.0f);
  }
}

template <int V, bool BF16IN>
__global__ void __launch_bounds__(64 * (V / 16)) m2rnn_scan_bwd_kernel(const BwdArgs a) {
  constexpr int NT = V / 16;
  constexpr int NTH = 64 * NT;
  constexpr int NCH = (NT + 1) / 2;
  using St = BwdStage<V>;
  constexpr int XWORDS = NCH * 2 * 64 * 4;

  __shared__ __attribute__((aligned(16))) float stage[kBwdSeg * St::STEP];
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2][XWORDS];
  // Cross-wave partial sums of dq, dk (per row) and df, by step parity.
  __shared__ float red_q[2][NT][16], red_k[2][NT][16], red_f[2][NT];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;

  const int U = a.B * a.N;
  int u, s;
  if ((U & 7) == 0 && a.S > 1) {
    const int slot = blockIdx.x >> 3;
    s = slot % a.S;
    u = (slot / a.S) * 8 + (blockIdx.x & 7);
  } else {
    u = blockIdx.x / a.S;
    s = blockIdx.x % a.S;
  }
  const int b = u / a.N;
  const int nh = u % a.N;
  const int row0 = s * 16;
  const long KV = (long)a.K * V;
  const int nseg = (a.T + kBwdSeg - 1) / kBwdSeg;
  const int wg = blockIdx.x;

  // ---- operands of W ----
  // forward contraction: A = (c W)^T, A[m][k] = c W[k][16w + m]   (as in the forward scan)
  // backward chain:      A = W,       A[m][k] = W[16w + m][k]
  const float* Wn = a.W + (long)nh * V * V;
  const int col = 16 * w + n;
  uint4 fHi[NCH], fLo[NCH], bHi[NCH], bLo[NCH];
#pragma unroll
  for (int cc = 0; cc < NCH; ++cc) {
    float fv[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tile = 2 * cc + (i >> 2);
      const int vin = 16 * tile + 4 * g + (i & 3);
      fv[i] = tile < NT ? kTwoLog2e * Wn[vin * V + col] : 0.0f;
      bv[i] = tile < NT ? Wn[col * V + vin] : 0.0f;
    }
    uint32_t fh[4], fl[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      fh[i] = pack_f16(fv[2 * i], fv[2 * i + 1]);
      fl[i] = pack_f16(fv[2 * i] - f16_lo_to_f32(fh[i]), fv[2 * i + 1] - f16_hi_to_f32(fh[i]));
      bh[i] = pack_f16(bv[2 * i], bv[2 * i + 1]);
      bl[i] = pack_f16(bv[2 * i] - f16_lo_to_f32(bh[i]), bv[2 * i + 1] - f16_hi_to_f32(bh[i]));
    }
    fHi[cc] = make_uint4(fh[0], fh[1], fh[2], fh[3]);
    fLo[cc] = make_uint4(fl[0], fl[1], fl[2], fl[3]);
    bHi[cc] = make_uint4(bh[0], bh[1], bh[2], bh[3]);
    bLo[cc] = make_uint4(bl[0], bl[1], bl[2], bl[3]);
  }
  // Transposing-MFMA selector (see the forward readout).
  uint4 bsel;
  {
    uint32_t e16[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) e16[e] = (n == 4 * g + (e & 3)) ? 0x3C00u : 0u;
    bsel = make_uint4(e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16), e16[4] | (e16[5] << 16),
                      e16[6] | (e16[7] << 16));
  }
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  if constexpr (NT & 1) {
    for (int i = tid; i < 2 * XWORDS; i += NTH) (&xbuf[0][0])[i] = 0u;
  }

  // Publishes a split tile (hi01, hi23, lo01, lo23) into exchange buffer `buf`.
  auto publish = [&](int buf, const uint32_t (&hs)[4]) {
    const int base = ((w >> 1) * 2) * 64 * 4 + lane * 4 + 2 * (w & 1);
    *(uint2*)&xbuf[buf][base] = make_uint2(hs[0], hs[1]);
    *(uint2*)&xbuf[buf][base + 64 * 4] = make_uint2(hs[2], hs[3]);
  };
  auto split4 = [&](const float (&x)[4], uint32_t (&hs)[4]) {
    split_pair<MATH_F16X3>(x[0], x[1], hs[0], hs[2]);
    split_pair<MATH_F16X3>(x[2], x[3], hs[1], hs[3]);
  };

  // State of the chain, and H_t for dq (the state after the step being processed).
  float C[4], Hc[4];
  const long own_off = ((long)b * a.N + nh) * KV + (long)(row0 + n) * V + 16 * w + 4 * g;
  if (a.dH_T) {
    const float4 c4 = *(const float4*)(a.dH_T + own_off);
    C[0] = c4.x; C[1] = c4.y; C[2] = c4.z; C[3] = c4.w;
  } else {
    C[0] = C[1] = C[2] = C[3] = 0.0f;
  }
  Hc[0] = Hc[1] = Hc[2] = Hc[3] = 0.0f;
  f32x4 dWacc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) dWacc[tt] = zero4;

  // Per-workgroup segment store: [kBwdSeg][NT waves][64 lanes][8 words] = (H_{t-1} split, Z).
  float* segs = a.seg_ws + (long)wg * kBwdSeg * NT * 64 * 8 + ((long)w * 64 + lane) * 8;
  constexpr long SEG_STEP = (long)NT * 64 * 8;

  const long plane = (long)a.B * a.T * a.N * V;
  float* dv_dst = a.dv + (a.S > 1 ? (long)s * plane : 0);
  float* df_dst = a.df + (a.S > 1 ? (long)s * a.B * a.T * a.N : 0);
  const float wr_col = a.S == 1 ? a.w_r[(long)nh * V + 16 * w + n] : 0.0f;  // for dv's w_r (.) u term
  float dwr = 0.0f;  // dw_r[16w + n] partial over this batch entry (workgroups with s == 0, lanes g == 0)

  for (int seg = nseg - 1; seg >= 0; --seg) {
    const int t0 = seg * kBwdSeg;
    const int nst = min(kBwdSeg, a.T - t0);
    lds_barrier();  // the previous segment's readers are done with the stage
    bwd_stage_segment<V, BF16IN>(a, b, nh, row0, t0, nst, stage, tid, NTH);

    // ---------------- 1. recompute the segment forward ----------------
    float H[4];
    {
      const float4 h4 = *(const float4*)(a.ckpt + ((long)u * nseg + seg) * KV + (long)(row0 + n) * V + 16 * w + 4 * g);
      H[0] = h4.x; H[1] = h4.y; H[2] = h4.z; H[3] = h4.w;
    }
    uint32_t hs[4];
    split4(H, hs);
    publish(0, hs);
    lds_barrier();
    for (int j = 0; j < nst; ++j) {
      const float* st = stage + j * St::STEP;
      const float4 fg = *(const float4*)st;
      const float av = g == 0 ? st[St::OV + 16 * w + n] : 0.0f;
      const float bk = g == 0 ? st[St::OCK + n] : 0.0f;
      f32x4 acc = mfma_f32(av, bk, zero4);
      const uint32_t* xr = xbuf[j & 1];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const uint4 bh = *(const uint4*)&xr[(cc * 2) * 64 * 4 + lane * 4];
        const uint4 bl = *(const uint4*)&xr[(cc * 2 + 1) * 64 * 4 + lane * 4];
        acc = mfma_f16(fHi[cc], bh, acc);
        acc = mfma_f16(fLo[cc], bh, acc);
        acc = mfma_f16(fHi[cc], bl, acc);
      }
      float Z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float rr = tanh_recip(acc[r]);
        Z[r] = __builtin_fmaf(-2.0f, rr, 1.0f);
        H[r] = __builtin_fmaf(fg.z, rr, __builtin_fmaf(fg.x, H[r], fg.y));
      }
      // Store H_{t-1} (split) and Z_t for the reverse walk.
      *(uint4*)(segs + j * SEG_STEP) = make_uint4(hs[0], hs[1], hs[2], hs[3]);
      *(float4*)(segs + j * SEG_STEP + 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
      split4(H, hs);
      publish((j + 1) & 1, hs);
      lds_barrier();
    }
    if (seg == nseg - 1) {
      // H_T: the state after the last step, for dq_{T-1}.
      Hc[0] = H[0]; Hc[1] = H[1]; Hc[2] = H[2]; Hc[3] = H[3];
    }
    __threadfence_block();  // the segment store is read back by the same lanes below

    // ---------------- 2. walk the segment backwards ----------------
    // The segment store is read two steps ahead of use (its latency is that of L2 / HBM).
    uint4 nh0 = *(const uint4*)(segs + (nst - 1) * SEG_STEP);
    float4 nz0 = *(const float4*)(segs + (nst - 1) * SEG_STEP + 4);
    uint4 nh1 = make_uint4(0, 0, 0, 0);
    float4 nz1 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (nst >= 2) {
      nh1 = *(const uint4*)(segs + (nst - 2) * SEG_STEP);
      nz1 = *(const float4*)(segs + (nst - 2) * SEG_STEP + 4);
    }
    for (int j = nst - 1; j >= 0; --j) {
      const int t = t0 + j;
      const float* st = stage + j * St::STEP;
      const float4 fg = *(const float4*)st;
      const float qn = st[St::OQ + n];
      const float4 u4 = *(const float4*)(st + St::OU + 16 * w + 4 * g);
      const float4 v4 = *(const float4*)(st + St::OV + 16 * w + 4 * g);
      const uint4 hsp = nh0;  // H_{t-1} split
      const float4 z4 = nz0;
      nh0 = nh1;
      nz0 = nz1;
      if (j >= 2) {
        nh1 = *(const uint4*)(segs + (j - 2) * SEG_STEP);
        nz1 = *(const float4*)(segs + (j - 2) * SEG_STEP + 4);
      }
      if (s == 0 && g == 0) dwr = __builtin_fmaf(st[St::OU + 16 * w + n], st[St::OV + 16 * w + n], dwr);
      const float Z[4] = {z4.x, z4.y, z4.z, z4.w};
      const float uu[4] = {u4.x, u4.y, u4.z, u4.w};
      const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
      float Hp[4];
      Hp[0] = f16_lo_to_f32(hsp.x) + f16_lo_to_f32(hsp.z);
      Hp[1] = f16_hi_to_f32(hsp.x) + f16_hi_to_f32(hsp.z);
      Hp[2] = f16_lo_to_f32(hsp.y) + f16_lo_to_f32(hsp.w);
      Hp[3] = f16_hi_to_f32(hsp.y) + f16_hi_to_f32(hsp.w);

      float R[4], D[4], cinit[4];
      float dq_l = 0.0f, dk_l = 0.0f, df_l = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        R[r] = __builtin_fmaf(qn, uu[r], C[r]);
        D[r] = (fg.y * R[r]) * __builtin_fmaf(-Z[r], Z[r], 1.0f);
        df_l = __builtin_fmaf(R[r], Hp[r] - Z[r], df_l);
        dq_l = __builtin_fmaf(Hc[r], uu[r], dq_l);
        dk_l = __builtin_fmaf(D[r], vv[r], dk_l);
        cinit[r] = fg.x * R[r];
      }
      // Row sums over this wave's 16 columns (the four lane rows), then one slot per wave.
      dq_l = sum_rows4(dq_l);
      dk_l = sum_rows4(dk_l);
      df_l = sum_rows4(df_l);
      // df also sums over the 16 rows (lanes of a row).
      df_l += dpp<kDppRowMirror>(df_l);
      df_l += dpp<kDppRowHalfMirror>(df_l);
      df_l += dpp<kDppQuadXor1>(df_l);
      df_l += dpp<kDppQuadXor2>(df_l);
      const int par = j & 1;
      if (g == 0) {
        red_q[par][w][n] = dq_l;
        red_k[par][w][n] = dk_l;
        if (n == 0) red_f[par][w] = df_l;
      }
      uint32_t ds[4];
      split4(D, ds);
      publish(par, ds);
      lds_barrier();

      // Completed row sums of dq, dk and the step's df.
      if (w == 0 && g == 0) {
        float sq = 0.0f, sk = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) {
          sq += red_q[par][ww][n];
          sk += red_k[par][ww][n];
        }
        const long qk = (((long)b * a.T + t) * a.N + nh) * a.K + row0 + n;
        a.dq[qk] = sq;
        a.dk[qk] = sk;
        if (n == 0) {
          float sf = 0.0f;
#pragma unroll
          for (int ww = 0; ww < NT; ++ww) sf += red_f[par][ww];
          df_dst[((long)b * a.T + t) * a.N + nh] = sf;
        }
      }

      // Chain: C_{t-1} = f R + D W^T, on the split-precision MFMA; and the transposes of the
      // D tiles for dW and dv.
      const uint32_t* xr = xbuf[par];
      f32x4 acc = {cinit[0], cinit[1], cinit[2], cinit[3]};
      f32x4 dT[NT];
#pragma unroll
      for (int cc = 0; cc < NCH; ++cc) {
        const uint4 bh = *(const uint4*)&xr[(cc * 2) * 64 * 4 + lane * 4];
        const uint4 bl = *(const uint4*)&xr[(cc * 2 + 1) * 64 * 4 + lane * 4];
        acc = mfma_f16(bHi[cc], bh, acc);
        acc = mfma_f16(bLo[cc], bh, acc);
        acc = mfma_f16(bHi[cc], bl, acc);
        dT[2 * cc] = mfma_f16(make_uint4(bh.x, bh.y, bl.x, bl.y), bsel, zero4);
        if (2 * cc + 1 < NT) dT[2 * cc + 1] = mfma_f16(make_uint4(bh.z, bh.w, bl.z, bl.w), bsel, zero4);
      }
      // Transposed own H_{t-1} tile: hT at lane (g, m) reg r = H_{t-1}[row 4g + r][col 16w + m].
      const f32x4 hT = mfma_f16(hsp, bsel, zero4);
      // dW[16w + m][16tt + j] += sum_rows H_{t-1}[row][16w + m] D[row][16tt + j]: one 16x16x16
      // MFMA per split term, A = hT (k = row), B = dT[tt] (k = row), both re-split to fp16 hi/lo.
      uint32_t th[4];
      split_pair<MATH_F16X3>(hT[0], hT[1], th[0], th[2]);
      split_pair<MATH_F16X3>(hT[2], hT[3], th[1], th[3]);
      const uint2 hThi = make_uint2(th[0], th[1]), hTlo = make_uint2(th[2], th[3]);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        uint32_t dd[4];
        split_pair<MATH_F16X3>(dT[tt][0], dT[tt][1], dd[0], dd[2]);
        split_pair<MATH_F16X3>(dT[tt][2], dT[tt][3], dd[1], dd[3]);
        const uint2 dhi = make_uint2(dd[0], dd[1]), dlo = make_uint2(dd[2], dd[3]);
        dWacc[tt] = mfma16_f16(hThi, dhi, dWacc[tt]);
        dWacc[tt] = mfma16_f16(hTlo, dhi, dWacc[tt]);
        dWacc[tt] = mfma16_f16(hThi, dlo, dWacc[tt]);
      }
      // dv[col 16w + j] = sum_rows D[row][col] k[row] (+ w_r u when this workgroup holds all rows).
      {
        const float4 k4 = *(const float4*)(st + St::OK + 4 * g);
        const f32x4 dTo = dT[w];
        float x = k4.x * dTo[0];
        x = __builtin_fmaf(k4.y, dTo[1], x);
        x = __builtin_fmaf(k4.z, dTo[2], x);
        x = __builtin_fmaf(k4.w, dTo[3], x);
        x = sum_rows4(x);
        if (g == 0) {
          const float ucol = st[St::OU + 16 * w + n];
          dv_dst[(((long)b * a.T + t) * a.N + nh) * V + 16 * w + n] = __builtin_fmaf(wr_col, ucol, x);
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        C[r] = acc[r];
        Hc[r] = Hp[r];
      }
    }
  }

  if (a.dH0) *(float4*)(a.dH0 + own_off) = make_float4(C[0], C[1], C[2], C[3]);
  if (s == 0 && g == 0) a.dwr_part[((long)b * a.N + nh) * V + 16 * w + n] = dwr;
  // dW partial of this workgroup: dWacc[tt] at lane (g, j) reg r = dW[16w + 4g + r][16tt + j].
  float* dWp = a.dW_part + ((long)(b * a.S + s) * a.N + nh) * V * V;
#pragma unroll
  for (int tt = 0; tt < NT; ++tt)
#pragma unroll
    for (int r = 0; r < 4; ++r) dWp[(long)(16 * w + 4 * g + r) * V + 16 * tt + n] = dWacc[tt][r];
}

// df = sum_s df_s  (S > 1).
__global__ void __launch_bounds__(256) m2rnn_bwd_sum_df_kernel(const float* __restrict__ part, int S, long count,
                                                                float* __restrict__ df) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int s = 1; s < S; ++s) acc += part[(long)s * count + i];
  df[i] = acc;
}

// dW[n] = sum over (b, s) of the workgroup partials, in a fixed order.
__global__ void __launch_bounds__(256) m2rnn_bwd_sum_dW_kernel(const float* __restrict__ part, int BS, int N,
                                                                int VV, float* __restrict__ dW) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;  // index into [N][V][V]
  if (i >= (long)N * VV) return;
  float acc = 0.0f;
  for (int p = 0; p < BS; ++p) acc += part[(long)p * N * VV + i];
  dW[i] = acc;
}

// dw_r[n][j] = sum over b of the per-batch-entry partials (each already summed over t).
__global__ void __launch_bounds__(256) m2rnn_bwd_sum_dwr_kernel(const float* __restrict__ part, int B, int NV,
                                                                 float* __restrict__ dw_r) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= NV) return;
  float acc = 0.0f;
  for (int b = 0; b < B; ++b) acc += part[(long)b * NV + i];
  dw_r[i] = acc;
}

}  // namespace m2rnn
