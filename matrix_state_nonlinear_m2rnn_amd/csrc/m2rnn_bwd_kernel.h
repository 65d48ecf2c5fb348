// Backward (BPTT) of the M²RNN recurrence for gfx950: the chain-rule equations of the M²RNN notes
// §2.7 (written there in place of the paper's Algorithm 2):
//     R_t = C_t + q_t u_t^T                      u_t = dL/dy_t
//     D_t = ((1 - f_t) R_t) (.) (1 - Z_t (.) Z_t)
//     C_{t-1} = f_t R_t + D_t W^T                (serial chain, C_T = dL/dH_T)
//     dq_t = H_t u_t,  dk_t = D_t v_t,  dv_t = D_t^T k_t + w_r (.) u_t,  df_t = <R_t, H_{t-1} - Z_t>
//     dW = sum_t H_{t-1}^T D_t,  dw_r = sum_t u_t (.) v_t,  dH_0 = C_0.
//
// Work decomposition (one 16-row block of one (b, n) pair per workgroup, wave w owns value
// columns [16w, 16w+16), same register layout as the forward scan).  Time is walked last to first
// in sub-segments of SUB steps (8 for V <= 64, 2 for V = 128).  For each sub-segment:
//   1. its q, k, v, f, dy records are in LDS (a ragged tail is padded with f = 1 and zero inputs,
//      steps that leave the state and the chain exactly unchanged);
//   2. recompute: the forward from the sub-segment's entry state, keeping each step's H_{t-1}
//      (split fp16 hi/lo tiles) and Z_t in LDS;
//   3. walk it backwards: R, D and the row/column partial sums in registers; D is published
//      through LDS like H in the forward and the chain's D W^T runs on the split-precision MFMA;
//      dW and dv read the H_{t-1} and D tiles transposed straight from LDS (ds_read_b64_tr_b16).
// Entry states: with checkpoints at every sub-segment (V <= 64) they are read from the checkpoint
// array, prefetched with the records one sub-segment ahead; with checkpoints every 64 steps
// (V = 128) a segment is staged whole and a forward pass over it (pass A) keeps them in scratch.
// At V = 64 the walk of sub-segment p runs interleaved with the recompute of sub-segment p - 1.
// Per-workgroup partials of dv, df and dW are summed by separate, deterministic passes.
//
// Range: every gradient is linear in (dy, dH_T) jointly (§2.7), and the walk holds D_t in split
// fp16, whose accurate range is narrow (the remainder becomes subnormal below about 6e-5 and the
// high part overflows above 65504).  So each (b, n) pair runs at a power-of-two scale 2^e chosen
// from the largest |dy| and |dH_T| of the pair (m2rnn_bwd_absmax_kernel): u = 2^e dy and
// C_T = 2^e dH_T (with the clip bound scaled alike), which puts the largest |u| in [1, 2), and every
// gradient is multiplied by 2^-e before it is stored.  Both multiplications are exact, so the
// gradients do not depend on the scale of dy except through rounding at unit scale.
#pragma once

#include "m2rnn_fwd_kernel.h"

namespace m2rnn {

constexpr int kBwdSeg = 64;  // segment (checkpoint interval at V = 128), a multiple of every SUB

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* f;
  const float* W;
  const float* w_r;
  const float* dy;
  const float* dH_T;
  const float* ckpt;   // [B][N][ncheck][K][V]: states entering each segment, or (SUBCK) each sub-segment
  float* subck;        // per-workgroup states entering each sub-segment (without SUBCK)
  float* dq;           // per head [B][T][N][K] (summed over heads afterwards when q is shared)
  float* dk;           // per head [B][T][N][K]
  float* dv;           // final dv (S == 1) or partials [S][B*T*N*V]
  float* df;           // final df (S == 1) or partials [S][B*T*N]
  float* dW_part;      // [B*S][N][V][V]
  float* dwr_part;     // [B][N][V] (written by the workgroups with s == 0)
  float* dH0;          // may be null
  const float* umax;   // [B*N][umax_parts]: partial maxima of |dy| and |dH_T| per (b, n)
  int umax_parts;      // 1 .. 64
  int B, T, N, K;
  int Nqk;             // heads of q and k: N, or 1 when one query/key is shared by all heads
  int S;
  float clip;          // > 0: the gradient each step sends back to its input state is clamped to [-clip, clip]
};

// Per-step stage record of the backward (fp32):
//   [f, 0, 0, 0 | q (16) | c*k (16) | k (16) | v (V) | u (V)]   (slot 3 is a zero)
template <int V>
struct BwdStage {
  static constexpr int OQ = 4;
  static constexpr int OCK = 20;
  static constexpr int OK = 36;
  static constexpr int OV = 52;
  static constexpr int OU = 52 + V;
  static constexpr int STEP = 52 + 2 * V;
};

// Steps of a segment whose H_{t-1} and Z_t are held in LDS at once.
template <int V>
struct BwdSub {
  static constexpr int value = V <= 64 ? 8 : 2;
};

// Checkpoint interval of the backward: every sub-segment where that stays a modest multiple of
// the state (V <= 64: every 16 or 8 steps), so the backward needs no forward pass to find the
// sub-segments' entry states; every segment at V = 128 (sub-segments of 2 steps), where the
// backward runs that pass itself.
template <int V>
struct BwdCkpt {
  static constexpr bool sub = V <= 64;
  static constexpr int interval = sub ? BwdSub<V>::value : kBwdSeg;
};

// Loads steps [t0, t0 + n_steps) of one 16-row block into the stage; the records from n_steps up
// to `n_pad` get f = 1 and zero q, k, v, u.
template <int V, bool BF16IN>
__device__ __forceinline__ void bwd_stage_segment(const BwdArgs& a, int b, int nh, int row0, int t0, int n_steps,
                                                  int n_pad, float* stage, int tid, int nth, float uscale) {
  using St = BwdStage<V>;
  const int esz = BF16IN ? 2 : 4;
  constexpr int VEC = BF16IN ? 8 : 4;
  // q, k: 16 values per step, VEC per load.
  constexpr int QV = 16 / VEC;
  for (int i = tid; i < n_pad * QV * 2; i += nth) {
    const int which = i / (n_pad * QV);  // 0 = q, 1 = k
    const int r = i % (n_pad * QV);
    const int step = r / QV, cv = r % QV;
    float vals[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) vals[e] = 0.0f;
    if (step < n_steps) {
      const long off = ((((long)b * a.T + t0 + step) * a.Nqk + (a.Nqk == 1 ? 0 : nh)) * a.K + row0 + cv * VEC);
      const void* src = which == 0 ? a.q : a.k;
      const uint4 raw = *(const uint4*)((const char*)src + off * esz);
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
  for (int i = tid; i < n_pad * VV; i += nth) {
    const int step = i / VV, cv = i % VV;
    float* d = stage + step * St::STEP + St::OV + cv * VEC;
    if (step >= n_steps) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) d[e] = 0.0f;
      continue;
    }
    const long off = (((long)b * a.T + t0 + step) * a.N + nh) * V + cv * VEC;
    const uint4 raw = *(const uint4*)((const char*)a.v + off * esz);
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
  for (int i = tid; i < n_pad * UV; i += nth) {
    const int step = i / UV, cv = i % UV;
    float4 u4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (step < n_steps) u4 = *(const float4*)(a.dy + (((long)b * a.T + t0 + step) * a.N + nh) * V + cv * 4);
    *(float4*)(stage + step * St::STEP + St::OU + cv * 4) =
        make_float4(u4.x * uscale, u4.y * uscale, u4.z * uscale, u4.w * uscale);
  }
  for (int i = tid; i < n_pad; i += nth) {
    const float fv = i < n_steps ? a.f[((long)b * a.T + t0 + i) * a.N + nh] : 1.0f;
    *(float4*)(stage + i * St::STEP) = make_float4(fv, 0.0f, 0.0f, 0.0f);
  }
}

// One sub-segment's stage records (SUB steps of one 16-row block), loaded into registers ahead of
// use and written to LDS later, so that their HBM latency overlaps the walk of the sub-segment
// after them in time.  The loads go through buffer resources that end at the last step of the
// (b, n) pair: steps past T read zeros (and get f = 1), with no branch around any load.
template <int V, bool BF16IN, int SUB, int NTH>
struct BwdSubRegs {
  static constexpr int VEC = BF16IN ? 8 : 4;
  static constexpr int QV = 16 / VEC;          // loads per step of q (and of k)
  static constexpr int NQ = SUB * QV;
  static constexpr int NVV = SUB * (V / VEC);
  static constexpr int NU = SUB * (V / 4);
  static constexpr int PQ = (NQ + NTH - 1) / NTH, PVV = (NVV + NTH - 1) / NTH, PU = (NU + NTH - 1) / NTH;
  uint4 q[PQ], k[PQ], vv[PVV];
  float4 uu[PU];
  float f;

  static __device__ __forceinline__ uint4 ld128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
  }

  __device__ __forceinline__ void load(const BwdArgs& a, int b, int nh, int row0, int t0, int n_steps, int tid) {
    const int esz = BF16IN ? 2 : 4;
    const int nq = a.Nqk == 1 ? 0 : nh;
    const long bt = (long)b * a.T;
    const __amdgpu_buffer_rsrc_t qres = __builtin_amdgcn_make_buffer_rsrc(
        (char*)a.q + (bt * a.Nqk + nq) * a.K * esz, (short)0, (a.T * a.Nqk - nq) * a.K * esz, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t kres = __builtin_amdgcn_make_buffer_rsrc(
        (char*)a.k + (bt * a.Nqk + nq) * a.K * esz, (short)0, (a.T * a.Nqk - nq) * a.K * esz, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vres = __builtin_amdgcn_make_buffer_rsrc(
        (char*)a.v + (bt * a.N + nh) * V * esz, (short)0, (a.T * a.N - nh) * V * esz, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t ures = __builtin_amdgcn_make_buffer_rsrc(
        (float*)a.dy + (bt * a.N + nh) * V, (short)0, (a.T * a.N - nh) * V * 4, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t fres = __builtin_amdgcn_make_buffer_rsrc(
        (float*)a.f + bt * a.N + nh, (short)0, (a.T * a.N - nh) * 4, kBufferRsrcWord3);
#pragma unroll
    for (int p = 0; p < PQ; ++p) {
      const int i = tid + p * NTH;
      const int step = i / QV, cv = i % QV;
      const uint32_t off = i < NQ ? (uint32_t)(((t0 + step) * a.Nqk * a.K + row0 + cv * VEC) * esz) : kBufferDrop;
      q[p] = ld128(qres, off);
      k[p] = ld128(kres, off);
    }
#pragma unroll
    for (int p = 0; p < PVV; ++p) {
      const int i = tid + p * NTH;
      const int step = i / (V / VEC), cv = i % (V / VEC);
      vv[p] = ld128(vres, i < NVV ? (uint32_t)(((t0 + step) * a.N * V + cv * VEC) * esz) : kBufferDrop);
    }
#pragma unroll
    for (int p = 0; p < PU; ++p) {
      const int i = tid + p * NTH;
      const int step = i / (V / 4), cv = i % (V / 4);
      const uint4 x = ld128(ures, i < NU ? (uint32_t)(((t0 + step) * a.N * V + cv * 4) * 4) : kBufferDrop);
      uu[p] = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    }
    const float fl = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(fres, tid < SUB ? (uint32_t)((t0 + tid) * a.N * 4) : kBufferDrop, 0, 0));
    f = tid < n_steps ? fl : 1.0f;
  }

  __device__ __forceinline__ void store(float* stage, int tid, float uscale) const {
    using St = BwdStage<V>;
    auto widen = [](const uint4& raw, float (&x)[VEC]) {
      if constexpr (BF16IN) {
        const uint32_t wds[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[2 * e] = bf16_lo_to_f32(wds[e]);
          x[2 * e + 1] = bf16_hi_to_f32(wds[e]);
        }
      } else {
        x[0] = __uint_as_float(raw.x); x[1] = __uint_as_float(raw.y);
        x[2] = __uint_as_float(raw.z); x[3] = __uint_as_float(raw.w);
      }
    };
#pragma unroll
    for (int p = 0; p < PQ; ++p) {
      const int i = tid + p * NTH;
      if (i < NQ) {
        const int step = i / QV, cv = i % QV;
        float xq[VEC], xk[VEC];
        widen(q[p], xq);
        widen(k[p], xk);
        float* d = stage + step * St::STEP;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          d[St::OQ + cv * VEC + e] = xq[e];
          d[St::OCK + cv * VEC + e] = kTwoLog2e * xk[e];
          d[St::OK + cv * VEC + e] = xk[e];
        }
      }
    }
#pragma unroll
    for (int p = 0; p < PVV; ++p) {
      const int i = tid + p * NTH;
      if (i < NVV) {
        const int step = i / (V / VEC), cv = i % (V / VEC);
        float x[VEC];
        widen(vv[p], x);
        float* d = stage + step * St::STEP + St::OV + cv * VEC;
#pragma unroll
        for (int e = 0; e < VEC; ++e) d[e] = x[e];
      }
    }
#pragma unroll
    for (int p = 0; p < PU; ++p) {
      const int i = tid + p * NTH;
      if (i < NU) {
        const int step = i / (V / 4), cv = i % (V / 4);
        const float4 x = uu[p];
        *(float4*)(stage + step * St::STEP + St::OU + cv * 4) =
            make_float4(x.x * uscale, x.y * uscale, x.z * uscale, x.w * uscale);
      }
    }
    if (tid < SUB) *(float4*)(stage + tid * St::STEP) = make_float4(f, 0.0f, 0.0f, 0.0f);
  }
};

// Slot (8-byte unit) of columns [4gam, 4gam + 4) of row rho in a 16x16 fp16 tile stored as 64 slots
// (512 bytes).  The xor keeps three access patterns free of LDS bank conflicts: a lane (g, n)
// writing or reading its own record (row n, group g), and the transposing read in which the 16
// lanes of group g fetch rows 4g .. 4g+3 of all four column groups.
__device__ __forceinline__ int tile_slot(int rho, int gam) { return 16 * gam + (rho ^ (4 * gam)); }

// Transposing LDS read of a 16x16 fp16 tile stored with tile_slot: lane (g, i) supplies the slot of
// row 4g + (i >> 2), columns 4(i & 3) ..; the 16 lanes of a group then receive column i of rows
// 4g .. 4g+3, i.e. the 16x16x16 MFMA operand layout with the contraction index running over rows.
__device__ __forceinline__ uint2 lds_read_tr(const uint32_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  uint2 o;
  __builtin_memcpy(&o, &r, sizeof(o));
  return o;
}

// WS (V = 64 only): the interleaved walk with waves of their own.  Waves 0 .. NT-1 walk (exchange
// of D, the chain, R and D, dk, df, and dv, dw_r from the transposed D tiles), waves NT .. 2NT-1
// recompute (exchange of H, the forward step, dq) and form dW, so that each SIMD holds one wave of
// each and the two roles split the LDS reads, which one wave can only drain at a limited rate, and
// the issue of VALU and MFMA work.  Both roles meet at the same barriers; the arithmetic is the
// one-role kernel's, operation for operation.
// Waves per SIMD the compiler schedules for: one for the one-role kernel at V = 64 (its LDS holds
// one workgroup of four waves per CU), two otherwise.  (The one-wave hint on the one-wave
// workgroups of V = 16, of which two share each SIMD, took the paper shape's reverse scan from 2.9
// to 4.0 ms.)
template <int V, bool BF16IN, bool WS = false>
__global__ void __launch_bounds__(64 * (V / 16) * (WS ? 2 : 1))
__attribute__((amdgpu_waves_per_eu(!WS && V == 64 ? 1 : 2, !WS && V == 64 ? 1 : 2)))
m2rnn_scan_bwd_kernel(const BwdArgs a) {
  constexpr bool SUBCK = BwdCkpt<V>::sub;  // checkpoints at every sub-segment
  constexpr int NT = V / 16;
  constexpr int NTH = 64 * NT;
  constexpr int NCH = (NT + 1) / 2;
  constexpr int NOTH = NCH > 1 ? NCH - 1 : 1;
  constexpr int SUB = BwdSub<V>::value;
  constexpr int NSUB = kBwdSeg / SUB;
  constexpr bool GROUP4 = SUB % 4 == 0;  // dq, dk, df, dv reduced four steps at a time
  constexpr int ENTRY = NT * 256;        // dwords of one step's split tiles (all waves)
  // A single wave needs no parity buffers for D (its own LDS accesses complete in order) and
  // writes dq, dk, df straight from its lanes.
  constexpr bool ONE = NT == 1;
  // Interleaved walk (V = 64): sub-segment p is walked while sub-segment p - 1 is recomputed into
  // a second set of buffers, one barrier per pair of steps, so that each chain fills the other's
  // waits.  (A one-wave workgroup gets that from the other workgroups on its SIMD instead.)
  constexpr bool INTERLEAVE = SUBCK && V == 64;
  constexpr int NBUF = INTERLEAVE ? 2 : 1;
  static_assert(!WS || INTERLEAVE, "the roles split the interleaved walk");
  using St = BwdStage<V>;
  static_assert(kBwdSeg % SUB == 0 && SUB % 2 == 0, "sub-segments tile a segment");

  // Stage records: the whole segment (segment checkpoints: pass A runs over it), or only the
  // sub-segment being recomputed and walked (sub-segment checkpoints).
  __shared__ __attribute__((aligned(16))) float stage[NBUF * (SUBCK ? SUB : kBwdSeg) * St::STEP];
  // H_{t-1} of the sub-segment's steps, split fp16: [SUB][hi|lo][NT tiles][64 slots][2 dwords].
  // Pass A uses entries 0 and 1 as its exchange buffer.
  __shared__ __attribute__((aligned(16))) uint32_t hst[NBUF * SUB * ENTRY];
  // Z_t of the sub-segment's steps: [SUB][NT][64 lanes][4 floats].
  __shared__ __attribute__((aligned(16))) float zst[NBUF * SUB * NT * 64 * 4];
  // D_t exchange, by step parity (one buffer for a single wave): [2][hi|lo][NT tiles][64 slots][2 dwords].
  __shared__ __attribute__((aligned(16))) uint32_t dx[(ONE ? 1 : 2) * ENTRY];
  // Per-wave partial sums of dq, dk (per row) and df over the sub-segment's steps (several waves;
  // red_f holds 16 equal copies, one per lane of a row, so that every lane stores).
  constexpr int RED = ONE ? 1 : SUB;
  __shared__ float red[3][RED][NT][16];
  auto& red_q = red[0];
  auto& red_k = red[1];
  auto& red_f = red[2];

  const int tid = threadIdx.x;
  const int w = WS ? (tid >> 6) & (NT - 1) : tid >> 6;  // value tile of this wave
  const bool walker = !WS || (tid >> 6) < NT;           // (uniform in a wave)
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
  const int nck = (a.T + BwdCkpt<V>::interval - 1) / BwdCkpt<V>::interval;  // checkpoints per (b, n)
  const int wg = blockIdx.x;

  // ---- operands of W ----
  // forward contraction: A = (c W)^T, A[m][k] = c W[k][16w + m]   (as in the forward scan)
  // backward chain:      A = W,       A[m][k] = W[16w + m][k]
  // Chunk cc covers tiles 2cc (k-slots 0..3) and 2cc+1 (k-slots 4..7).  The chunk co = w/2 holding
  // this wave's own tile is listed first ("own"), with the own tile in k-slots 0..3 and its partner
  // w ^ 1 in 4..7 (so that the own halves come from registers); the others after it.
  const float* Wn = a.W + (long)nh * V * V;
  const int col = 16 * w + n;
  const int co = w >> 1;
  auto wchunk = [&](int t_lo, int t_hi, bool fwd, uint4& hi, uint4& lo) {
    float wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tile = (i >> 2) ? t_hi : t_lo;
      const int vin = 16 * tile + 4 * g + (i & 3);
      wv[i] = tile < NT ? (fwd ? opaque1(kTwoLog2e * Wn[vin * V + col]) : Wn[col * V + vin]) : 0.0f;
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = pack_f16(wv[2 * i], wv[2 * i + 1]);
      l[i] = pack_f16(wv[2 * i] - f16_lo_to_f32(h[i]), wv[2 * i + 1] - f16_hi_to_f32(h[i]));
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
  };
  uint4 fOwnHi, fOwnLo, bOwnHi, bOwnLo, fOthHi[NOTH], fOthLo[NOTH], bOthHi[NOTH], bOthLo[NOTH];
  auto load_w = [&](bool fwd, bool bwd) __attribute__((always_inline)) {
    if (fwd) wchunk(w, w ^ 1, true, fOwnHi, fOwnLo);
    if (bwd) wchunk(w, w ^ 1, false, bOwnHi, bOwnLo);
#pragma unroll
    for (int i = 0; i < NCH - 1; ++i) {
      const int cc = i < co ? i : i + 1;
      if (fwd) wchunk(2 * cc, 2 * cc + 1, true, fOthHi[i], fOthLo[i]);
      if (bwd) wchunk(2 * cc, 2 * cc + 1, false, bOthHi[i], bOthLo[i]);
    }
  };
  // (with roles each role loads its own operands, inside its own branch)
  if constexpr (!WS) load_w(true, true);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};

  // Lane-constant slots: own record (row n, group g) and the transposing-read slot.
  const int own_slot = tile_slot(n, g);
  const int tr_slot = tile_slot(4 * g + (n >> 2), n & 3);
  // Dword offset of (tile, hi|lo) within one entry of hst or dx: [hi|lo][tile][64 slots][2 dwords],
  // so that the two tiles of a chunk are one 512-byte stride apart (one paired read each).
  auto tile_off = [](int tile, int hl) { return (hl * NT + tile) * 128; };
  constexpr bool has_partner = NT > 1;  // (with an even tile count every wave has one)

  // Writes this wave's tile (split fp16) into `entry`; returns the split (own B-operand halves).
  auto put_tile = [&](uint32_t* entry, float (&x)[4], uint2& hi, uint2& lo) {
    uint32_t h01, h23, l01, l23;
    opaque4(x);  // the split is a function of the fp32 values alone
    split_pair<MATH_F16X3>(x[0], x[1], h01, l01);
    split_pair<MATH_F16X3>(x[2], x[3], h23, l23);
    hi = make_uint2(h01, h23);
    lo = make_uint2(l01, l23);
    *(uint2*)(entry + tile_off(w, 0) + 2 * own_slot) = hi;
    *(uint2*)(entry + tile_off(w, 1) + 2 * own_slot) = lo;
  };
  // B operands of one contraction from a step's entry: the partner half of the own chunk and every
  // other chunk read whole (the own tile's halves are in registers); a single tile (no partner)
  // gets zeros in k-slots 4..7.
  struct Ops {
    uint2 ph, pl;  // partner tile of the own chunk
    uint4 oh[NOTH], ol[NOTH];
  };
  // (the lo read's offset goes through an empty asm so that the two 8-byte partner reads are not
  // paired into one instruction, whose four destination registers would then need copies)
  int plo = tile_off(w ^ 1, 1) + 2 * own_slot;
  asm volatile("" : "+v"(plo));
  auto read_ops = [&](const uint32_t* entry) {
    Ops o;
    o.ph = o.pl = make_uint2(0, 0);
    if constexpr (has_partner) {
      o.ph = *(const uint2*)(entry + tile_off(w ^ 1, 0) + 2 * own_slot);
      o.pl = *(const uint2*)(entry + plo);
    }
#pragma unroll
    for (int i = 0; i < NCH - 1; ++i) {
      const int cc = i < co ? i : i + 1;
      const uint2 h0 = *(const uint2*)(entry + tile_off(2 * cc, 0) + 2 * own_slot);
      const uint2 h1 = *(const uint2*)(entry + tile_off(2 * cc + 1, 0) + 2 * own_slot);
      const uint2 l0 = *(const uint2*)(entry + tile_off(2 * cc, 1) + 2 * own_slot);
      const uint2 l1 = *(const uint2*)(entry + tile_off(2 * cc + 1, 1) + 2 * own_slot);
      o.oh[i] = make_uint4(h0.x, h0.y, h1.x, h1.y);
      o.ol[i] = make_uint4(l0.x, l0.y, l1.x, l1.y);
    }
    return o;
  };
  // acc += A B over all chunks (three split passes per chunk).  A single tile (V = 16) has no
  // partner: its low halves take the empty k-slots 4..7, and two MFMAs, against [A_hi | A_hi] and
  // [A_lo | 0] (A_lo's slots 4..7 are zero), form the three products.
  auto contract = [&](f32x4 acc, const uint4& AownHi, const uint4& AownLo, const uint4 (&AothHi)[NOTH],
                      const uint4 (&AothLo)[NOTH], const uint2& own_hi, const uint2& own_lo, const Ops& o) {
    if constexpr (!has_partner) {
      const uint4 b = make_uint4(own_hi.x, own_hi.y, own_lo.x, own_lo.y);
      acc = mfma_f16(make_uint4(AownHi.x, AownHi.y, AownHi.x, AownHi.y), b, acc);
      return mfma_f16(AownLo, b, acc);
    }
    const uint4 bh = make_uint4(own_hi.x, own_hi.y, o.ph.x, o.ph.y);
    const uint4 bl = make_uint4(own_lo.x, own_lo.y, o.pl.x, o.pl.y);
    acc = mfma_f16(AownHi, bh, acc);
    acc = mfma_f16(AownLo, bh, acc);
    acc = mfma_f16(AownHi, bl, acc);
#pragma unroll
    for (int i = 0; i < NCH - 1; ++i) {
      acc = mfma_f16(AothHi[i], o.oh[i], acc);
      acc = mfma_f16(AothLo[i], o.oh[i], acc);
      acc = mfma_f16(AothHi[i], o.ol[i], acc);
    }
    return acc;
  };

  // Rank-1 term (c k_t) v_t^T of the step whose stage record is `st`.
  auto rank1 = [&](const float* st) {
    return mfma_f32(st[g == 0 ? St::OV + 16 * w + n : 3], st[g == 0 ? St::OCK + n : 3], zero4);
  };
  // One recompute step: reads H_{t-1} from `src` (own halves in hh, hl), adds the contraction to
  // the rank-1 term kv, advances H, returns Z_t, and publishes H_t's split into `dst` (if
  // non-null), leaving its halves in hh, hl.  Ends with the next step's rank-1 MFMA (record
  // `st_next`, if non-null), issued before the caller's barrier.
  auto fwd_step = [&](const float* st, const float* st_next, const uint32_t* src, uint32_t* dst, f32x4& kv,
                      float (&H)[4], float (&Z)[4], uint2& hh, uint2& hl) {
    const Ops o = read_ops(src);
    float avn = 0.0f, bkn = 0.0f;
    if (st_next) {
      avn = st_next[g == 0 ? St::OV + 16 * w + n : 3];
      bkn = st_next[g == 0 ? St::OCK + n : 3];
    }
    __builtin_amdgcn_sched_barrier(0);
    const float f = st[0], g1 = 1.0f - f, m2g = -2.0f * g1;
    f32x4 acc = contract(kv, fOwnHi, fOwnLo, fOthHi, fOthLo, hh, hl, o);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float rr = tanh_recip(acc[r]);
      Z[r] = __builtin_fmaf(-2.0f, rr, 1.0f);
      H[r] = __builtin_fmaf(m2g, rr, __builtin_fmaf(f, H[r], g1));
    }
    if (dst) {
      put_tile(dst, H, hh, hl);
    } else {
      uint32_t h01, h23, l01, l23;
      opaque4(H);
      split_pair<MATH_F16X3>(H[0], H[1], h01, l01);
      split_pair<MATH_F16X3>(H[2], H[3], h23, l23);
      hh = make_uint2(h01, h23);
      hl = make_uint2(l01, l23);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (st_next) kv = mfma_f32(avn, bkn, zero4);
  };

  // Scale of this pair: us = 2^e puts the largest |dy|, |dH_T| of the pair in [1, 2); gradients
  // are stored times ug = 2^-e.  (Zero, infinite or NaN maxima keep the unit scale.)
  float us = 1.0f, ug = 1.0f;
  {
    float m = 0.0f;
    for (int i = lane; i < a.umax_parts; i += 64) m = fmaxf(m, a.umax[(long)u * a.umax_parts + i]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (m > 0.0f && m <= 3.0e38f) {
      // m = mant 2^ex with mant in [0.5, 1): us = 2^(1 - ex), kept well inside the normal range.
      const int e = min(max(1 - __builtin_amdgcn_frexp_expf(m), -100), 100);
      us = __builtin_amdgcn_ldexpf(1.0f, e);
      ug = __builtin_amdgcn_ldexpf(1.0f, -e);
    }
  }

  // State of the chain.
  float C[4];
  // Bounds of the chain state (infinite without clipping: the clamp is then the identity).
  const float clip_hi = a.clip > 0.0f ? a.clip * us : __builtin_inff();
  const float clip_lo = -clip_hi;
  const long own_off = ((long)b * a.N + nh) * KV + (long)(row0 + n) * V + 16 * w + 4 * g;
  auto init_C = [&]() __attribute__((always_inline)) {
    if (a.dH_T) {
      const float4 c4 = *(const float4*)(a.dH_T + own_off);
      C[0] = c4.x * us; C[1] = c4.y * us; C[2] = c4.z * us; C[3] = c4.w * us;
    } else {
      C[0] = C[1] = C[2] = C[3] = 0.0f;
    }
  };
  if constexpr (!WS) init_C();
  f32x4 dWacc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) dWacc[tt] = zero4;

  // Per-workgroup scratch of the states entering sub-segments 1 .. NSUB-1: [NSUB][16 rows][V].
  float* subck = a.subck + (long)wg * NSUB * 16 * V + (long)n * V + 16 * w + 4 * g;

  // dv goes through a buffer resource that ends at the last valid step of this (b, n), so the
  // stores of padded steps are dropped (see the forward's y stores).
  const long plane = (long)a.B * a.T * a.N * V;
  float* dv_base = a.dv + (a.S > 1 ? (long)s * plane : 0) + ((long)b * a.T * a.N + nh) * V;  // [b, 0, nh, 0]
  const __amdgpu_buffer_rsrc_t dvres =
      __builtin_amdgcn_make_buffer_rsrc(dv_base, (short)0, (a.T * a.N - nh) * V * 4, kBufferRsrcWord3);
  const int ystep = a.N * V;
  // Byte offset of this lane's dv element at step 0 (grouped: step g), column 16w + n.
  const uint32_t dv_lane = (uint32_t)(((GROUP4 ? g * ystep : 0) + 16 * w + n) * 4);
  const float wr_col = a.S == 1 ? a.w_r[(long)nh * V + 16 * w + n] : 0.0f;  // for dv's w_r (.) u term
  float* df_dst = a.df + (a.S > 1 ? (long)s * a.B * a.T * a.N : 0);
  // A one-wave workgroup stores dq, dk and df from its lanes, likewise through resources that end
  // at the last valid step of this (b, n).  Byte offsets of step 0 (grouped: step g), row row0 + n.
  const __amdgpu_buffer_rsrc_t dqres = __builtin_amdgcn_make_buffer_rsrc(
      a.dq + ((long)b * a.T * a.N + nh) * a.K, (short)0, (a.T * a.N - nh) * a.K * 4, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t dkres = __builtin_amdgcn_make_buffer_rsrc(
      a.dk + ((long)b * a.T * a.N + nh) * a.K, (short)0, (a.T * a.N - nh) * a.K * 4, kBufferRsrcWord3);
  const __amdgpu_buffer_rsrc_t dfres = __builtin_amdgcn_make_buffer_rsrc(
      df_dst + (long)b * a.T * a.N + nh, (short)0, (a.T * a.N - nh) * 4, kBufferRsrcWord3);
  const int qkstep = a.N * a.K;
  const uint32_t qk_lane = (uint32_t)(((GROUP4 ? g * qkstep : 0) + row0 + n) * 4);
  const uint32_t df_lane = (GROUP4 ? n == 0 : g == 0 && n == 0) ? (uint32_t)((GROUP4 ? g * a.N : 0) * 4) : kBufferDrop;
  // dw_r[16w + 4g + r] partial over this batch entry (every lane of a row group holds the same sums;
  // the workgroups with s == 0 write them).
  float dwr4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // (grouped steps: lane (g, n) sums the products of column 16w + n at the steps congruent to g mod 4
  // instead, and the four lane rows are added at the end)
  float dwr1 = 0.0f;

  // dq, dk, df of the sub-segment's steps [tb, tb + SUB) from the per-wave partials.
  // (tbq: first step of the sub-segment whose dq is pending, tbk: whose dk, df; < 0: none.)
  auto finalize2 = [&](int tbq, int tbk) {
    if constexpr (ONE) return;
    for (int i = tid; i < SUB * 16 * 2 + SUB; i += NTH) {
      if (i < SUB * 32) {
        const int which = i / (SUB * 16), j = (i / 16) % SUB, row = i % 16;
        const int tb = which == 0 ? tbq : tbk;
        if (tb < 0) continue;
        const int t = tb + j;
        float acc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) acc += which == 0 ? red_q[j][ww][row] : red_k[j][ww][row];
        if (t < a.T) (which == 0 ? a.dq : a.dk)[(((long)b * a.T + t) * a.N + nh) * a.K + row0 + row] = acc * ug;
      } else {
        const int j = i - SUB * 32;
        if (tbk < 0) continue;
        const int t = tbk + j;
        float acc = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) acc += red_f[j][ww][0];
        if (t < a.T) df_dst[((long)b * a.T + t) * a.N + nh] = acc * ug;
      }
    }
  };
  auto finalize = [&](int tb) { finalize2(tb, tb); };
  // The interleaved walk sums the four waves' partials of one group of four steps in the step
  // after they are written, one gradient per wave: wave 0 dq, wave 1 dk, wave 2 df (lane (g, n):
  // step t0 + g, row n), in the order of finalize2.  group_read issues the reads of groups jq (dq)
  // and jk (dk, df) of the partial arrays, group_store adds and stores them (first steps tq, tk;
  // a negative first step stores nothing).
  const int wv = __builtin_amdgcn_readfirstlane(w);
  auto group_read = [&](int jq, int jk, float (&x)[4]) __attribute__((always_inline)) {
    const float* src = &red[min(wv, 2)][(wv == 0 ? jq : jk) + g][0][n];
#pragma unroll
    for (int ww = 0; ww < NT; ++ww) x[ww] = src[ww * 16];
  };
  auto group_store = [&](const float (&x)[4], int tq, int tk) __attribute__((always_inline)) {
    float acc = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NT; ++ww) acc += x[ww];
    const uint32_t val = __float_as_uint(acc * ug);
    if (wv == 0) {
      if (tq >= 0) __builtin_amdgcn_raw_buffer_store_b32(val, dqres, qk_lane + (uint32_t)(tq * qkstep * 4), 0, 0);
    } else if (wv == 1) {
      if (tk >= 0) __builtin_amdgcn_raw_buffer_store_b32(val, dkres, qk_lane + (uint32_t)(tk * qkstep * 4), 0, 0);
    } else if (wv == 2) {
      if (tk >= 0)
        __builtin_amdgcn_raw_buffer_store_b32(
            val, dfres, df_lane == kBufferDrop ? kBufferDrop : df_lane + (uint32_t)(tk * a.N * 4), 0, 0);
    }
  };

  // Lane partials of the current group of four steps: dv, dk, df (walk) and dq (recompute).
  float xq[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xk[4] = {0.0f, 0.0f, 0.0f, 0.0f}, xf[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  float xh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  int pending_tb = -1;                     // sub-segment whose dq, dk, df await finalize

  // ---------------- walk helpers ----------------
  struct RevIn {
    float f, qn;
    float4 u4, v4, z4;
    uint2 h_hi, h_lo;
  };
  // Inputs of walk step j from a sub-segment's stage records (ss), H_{t-1} tiles (hs) and Z (zs).
  auto load_rev = [&](const float* ss, const uint32_t* hs, const float* zs, int j) __attribute__((always_inline)) {
    RevIn in;
    const float* st = ss + j * St::STEP;
    const uint32_t* hj = hs + j * ENTRY;
    in.f = st[0];
    in.qn = st[St::OQ + n];
    in.u4 = *(const float4*)(st + St::OU + 16 * w + 4 * g);
    in.v4 = *(const float4*)(st + St::OV + 16 * w + 4 * g);
    in.h_hi = *(const uint2*)(hj + tile_off(w, 0) + 2 * own_slot);
    in.h_lo = *(const uint2*)(hj + tile_off(w, 1) + 2 * own_slot);
    in.z4 = *(const float4*)(zs + ((j * NT + w) * 64 + lane) * 4);
    return in;
  };
  struct RevFront {
    uint2 dh, dl;   // own split D tile (own halves of the chain's B operand)
    f32x4 cinit;    // f R
    float dk_l, df_l;
  };
  // R, D of step j (the chain's critical path), published at once; then f R and the per-lane
  // partial sums of dk, df and dw_r in the shadow of that write.
  auto front = [&](int j, const RevIn& in) __attribute__((always_inline)) {
    RevFront fr;
    const float Z[4] = {in.z4.x, in.z4.y, in.z4.z, in.z4.w};
    const float uu[4] = {in.u4.x, in.u4.y, in.u4.z, in.u4.w};
    const float vv[4] = {in.v4.x, in.v4.y, in.v4.z, in.v4.w};
    const float g1 = 1.0f - in.f;
    float R[4], D[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      R[r] = __builtin_fmaf(in.qn, uu[r], C[r]);
      D[r] = (g1 * R[r]) * __builtin_fmaf(-Z[r], Z[r], 1.0f);
    }
    put_tile(dx + (ONE ? 0 : (j & 1) * ENTRY), D, fr.dh, fr.dl);
    __builtin_amdgcn_sched_barrier(0);
    // H_{t-1} - Z_t from the fp16 halves of H_{t-1}: (hi - Z) + lo, each a v_fma_mix_f32
    float HmZ[4];
    HmZ[0] = add_mix_f16<false>(in.h_lo.x, sub_mix_f16<false>(in.h_hi.x, Z[0]));
    HmZ[1] = add_mix_f16<true>(in.h_lo.x, sub_mix_f16<true>(in.h_hi.x, Z[1]));
    HmZ[2] = add_mix_f16<false>(in.h_lo.y, sub_mix_f16<false>(in.h_hi.y, Z[2]));
    HmZ[3] = add_mix_f16<true>(in.h_lo.y, sub_mix_f16<true>(in.h_hi.y, Z[3]));
    fr.dk_l = fr.df_l = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      fr.cinit[r] = in.f * R[r];
      fr.df_l = __builtin_fmaf(R[r], HmZ[r], fr.df_l);
      fr.dk_l = __builtin_fmaf(D[r], vv[r], fr.dk_l);
      if constexpr (!GROUP4) dwr4[r] = __builtin_fmaf(uu[r], vv[r], dwr4[r]);
    }
    return fr;
  };

  // dq of a recomputed step j of the sub-segment starting at step tb (H = H_t): grouped four steps
  // at a time (lane (g, n) ends with step j0 + g, j0 = j & ~3).
  // (u4: the step's u at this lane's four columns, read by the caller ahead of use)
  auto rec_u4 = [&](const float* st) { return *(const float4*)(st + St::OU + 16 * w + 4 * g); };
  auto rec_dq = [&](const float (&Hn)[4], const float4 u4, int j, int tb) __attribute__((always_inline)) {
    float dq_l = Hn[0] * u4.x;
    dq_l = __builtin_fmaf(Hn[1], u4.y, dq_l);
    dq_l = __builtin_fmaf(Hn[2], u4.z, dq_l);
    dq_l = __builtin_fmaf(Hn[3], u4.w, dq_l);
    if constexpr (GROUP4) {
      xh[j & 3] = dq_l;
      if ((j & 3) == 3) {
        const float dq4 = reduce_rows4(xh[0], xh[1], xh[2], xh[3]);
        if constexpr (ONE) {
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dq4 * ug), dqres,
                                                qk_lane + (uint32_t)((tb + j - 3) * qkstep * 4), 0, 0);
        } else {
          red_q[j - 3 + g][w][n] = dq4;
        }
      }
    } else {
      dq_l = sum_rows4(dq_l);
      if constexpr (ONE) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dq_l * ug), dqres,
                                              g == 0 ? qk_lane + (uint32_t)((tb + j) * qkstep * 4) : kBufferDrop, 0, 0);
      } else if (g == 0) {
        red_q[j][w][n] = dq_l;
      }
    }
  };

  RevIn nxt;
  RevFront fr;
  // dk, df of walk step j + 1 (the partials of the front carried in fr): sums over this wave's 16
  // columns (the four lane rows); df also over the 16 rows.  Grouped: steps j .. j+3 (j % 4 == 0)
  // reduced together, lane (g, n) ending with step j + g.
  auto walk_sums = [&](int j, int js) __attribute__((always_inline)) {
    if (!GROUP4 || (j & 3) == 0) {
      float dk_l, df_l;
      if constexpr (GROUP4) {
        xk[j & 3] = fr.dk_l;
        xf[j & 3] = fr.df_l;
        dk_l = reduce_rows4(xk[0], xk[1], xk[2], xk[3]);
        df_l = reduce_rows4(xf[0], xf[1], xf[2], xf[3]);
      } else {
        dk_l = sum_rows4(fr.dk_l);
        df_l = sum_rows4(fr.df_l);
      }
      df_l += dpp<kDppRowMirror>(df_l);
      df_l += dpp<kDppRowHalfMirror>(df_l);
      df_l += dpp<kDppQuadXor1>(df_l);
      df_l += dpp<kDppQuadXor2>(df_l);
      if constexpr (ONE) {
        const uint32_t tstep = (uint32_t)js;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dk_l * ug), dkres,
                                              GROUP4 || g == 0 ? qk_lane + tstep * qkstep * 4 : kBufferDrop, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(df_l * ug), dfres,
                                              df_lane == kBufferDrop ? kBufferDrop : df_lane + tstep * a.N * 4, 0, 0);
      } else if constexpr (GROUP4) {
        red_k[j + g][w][n] = dk_l;
        red_f[j + g][w][n] = df_l;
      } else if (g == 0) {
        red_k[j][w][n] = dk_l;
        red_f[j][w][n] = df_l;
      }
    } else {
      xk[j & 3] = fr.dk_l;
      xf[j & 3] = fr.df_l;
    }
  };
  // dv[col 16w + i] of walk step j = sum_rows D[row][col] k[row] (+ w_r u when this workgroup holds
  // all rows), from the transposed D tile's hi and lo halves on the MFMA (k in one fp16 pass: a
  // relative rounding of 2^-12 per term, as dW's); st is the step's record; ucol, vcol the grouped u,
  // v reads (step j + g, column 16w + n).
  auto dv_step = [&](int j, int js, const float* st, uint2 dThi, uint2 dTlo, float4 k4, float ucol, float vcol)
                     __attribute__((always_inline)) {
    // One 16x16x32 fp16 MFMA: B = D's transposed hi and lo halves stacked on the contraction index
    // (rows 4g .. 4g+3 of each), A = the rows' k (one fp16 pass) twice, the same in every output
    // row: every lane (g, i) ends with dv[16w + i] in all four registers.
    const uint32_t k01 = pack_f16(k4.x, k4.y), k23 = pack_f16(k4.z, k4.w);
    const f32x4 c = mfma_f16(make_uint4(k01, k23, k01, k23), make_uint4(dThi.x, dThi.y, dTlo.x, dTlo.y), zero4);
    if constexpr (GROUP4) {
      // lane (g, i) keeps step j0 + g of the group of four, stored once the group is complete
      if ((j & 3) == g) xq[0] = c[0];
      if ((j & 3) == 0) {
        dwr1 = __builtin_fmaf(ucol, vcol, dwr1);  // dw_r's product of step j + g, column 16w + n
        const float dvv = __builtin_fmaf(wr_col, ucol, xq[0]);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dvv * ug), dvres, dv_lane + (uint32_t)(js * ystep * 4), 0, 0);
      }
    } else {
      const float u1 = st[St::OU + 16 * w + n];
      const float dvv = __builtin_fmaf(wr_col, u1, c[0]);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(dvv * ug), dvres,
                                            g == 0 ? dv_lane + (uint32_t)(js * ystep * 4) : kBufferDrop, 0, 0);
    }
  };

  // Walk step j of the sub-segment starting at step tb (records ss, tiles hs, Z zs), software-
  // pipelined: the inputs of step j-1 are read right after step j's barrier together with step
  // j's exchange reads, and the step ends with step j-1's R, D and publish (which wait for step
  // j's chain MFMAs).  The hooks add independent work: reads (issued with the step's reads),
  // MFMAs (queued behind the chain's), and a tail (after the publish of D).
  // (fr: step j's front, nxt: step j-1's inputs, both carried from step to step.)
  auto walk_step = [&](int j, int tb, const float* ss, const uint32_t* hs, const float* zs, auto&& hook_reads,
                       auto&& hook_mfma, auto&& hook_tail) __attribute__((always_inline)) {
    const int js = tb + j;  // global step
    const float* st = ss + j * St::STEP;
    const uint32_t* hj = hs + j * ENTRY;
    const uint32_t* dxp = dx + (ONE ? 0 : (j & 1) * ENTRY);
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();

    // Step j's exchange reads (chain operands, transposed tiles for dW and dv), and step j-1's
    // inputs.
    const Ops o = read_ops(dxp);
    hook_reads();
    __builtin_amdgcn_sched_barrier(0);

    // Chain: C_{t-1} = f R + D W^T on the split-precision MFMA.
    const f32x4 acc =
        contract(fr.cinit, bOwnHi, bOwnLo, bOthHi, bOthLo, fr.dh, fr.dl, o);
    // The reads that the chains do not wait for, issued behind the chain's MFMAs: the transposed
    // tiles for dW and dv, and step j-1's inputs.
    const uint2 hT = lds_read_tr(hj + tile_off(w, 0) + 2 * tr_slot);
    // (dT[tt] is tile w + tt mod NT, so that the own tile, which dv also reads, is dT[0])
    uint2 dT[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) dT[tt] = lds_read_tr(dxp + tile_off((w + tt) & (NT - 1), 0) + 2 * tr_slot);
    const uint2 dThi = dT[0];
    const uint2 dTlo = lds_read_tr(dxp + tile_off(w, 1) + 2 * tr_slot);
    const float4 k4 = *(const float4*)(st + St::OK + 4 * g);
    if (j > 0) nxt = load_rev(ss, hs, zs, j - 1);
    // (grouped steps: u and v of step j + g at column 16w + n, for dv's w_r term and dw_r)
    float ucol = 0.0f, vcol = 0.0f;
    if constexpr (GROUP4) {
      if ((j & 3) == 0) {
        ucol = ss[(j + g) * St::STEP + St::OU + 16 * w + n];
        vcol = ss[(j + g) * St::STEP + St::OV + 16 * w + n];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    hook_mfma();
    // Off the chain, while the MFMAs run.
    walk_sums(j, js);

    // Step j-1's R, D and publish as soon as the chain has produced C.
    // (the padding steps of a ragged tail must leave the chain unchanged: no clamp there)
    const bool real = js < a.T;
    const float lo = real ? clip_lo : -__builtin_inff(), hi = real ? clip_hi : __builtin_inff();
#pragma unroll
    for (int r = 0; r < 4; ++r) C[r] = __builtin_amdgcn_fmed3f(acc[r], lo, hi);
    if (j > 0) fr = front(j - 1, nxt);
    __builtin_amdgcn_sched_barrier(0);
    // The cross-wave sums of one group of four steps (interleaved walk): at j = 3, dk and df of
    // steps tb + 4 .. 7 and the recompute's dq of steps tb - SUB .. tb - SUB + 3; at j = 7, dk and
    // df of steps tb + SUB .. tb + SUB + 3 (written at the last step of the previous pair) and the
    // recompute's dq of steps tb + 4 .. 7.
    float gx[4];
    if constexpr (INTERLEAVE) {
      if ((j & 3) == 3) group_read(j == 3 ? 0 : 4, j == 3 ? 4 : 0, gx);
    }
    dv_step(j, js, st, dThi, dTlo, k4, ucol, vcol);

    // dW[16w + m][16u + j] += sum_rows H_{t-1}[row][16w + m] D[row][16u + j], u = w + tt mod NT: one fp16 16x16x16
    // MFMA per D tile, both operands read transposed from LDS (rows on the contraction index).
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) dWacc[tt] = mfma16_f16(hT, dT[tt], dWacc[tt]);

    hook_tail();
    if constexpr (INTERLEAVE) {
      if ((j & 3) == 3) group_store(gx, j == 3 ? tb - SUB : tb + 4, j == 3 ? tb + 4 : tb + SUB);
    }

  };

  auto none = [] {};

  // Sub-segment checkpoints: the stage records of the next sub-segment to walk, in registers.
  BwdSubRegs<V, BF16IN, SUB, NTH> sub_regs;
  const long lane_off = (long)(row0 + n) * V + 16 * w + 4 * g;
  // The state entering the next sub-segment to walk (sub-segment checkpoints: prefetched one
  // sub-segment ahead; segment checkpoints: from this workgroup's scratch).
  float4 nextH = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  if constexpr (SUBCK && !WS) {
    const int tl = ((a.T - 1) / SUB) * SUB;  // the last sub-segment
    sub_regs.load(a, b, nh, row0, tl, min(SUB, a.T - tl), tid);
    nextH = *(const float4*)(a.ckpt + ((long)u * nck + nck - 1) * KV + lane_off);
  }
  // Prefetch of sub-segment p (clamped at 0) with sub-segment checkpoints.
  auto prefetch = [&](int p) __attribute__((always_inline)) {
    const int pp = max(p, 0);
    nextH = *(const float4*)(a.ckpt + ((long)u * nck + pp) * KV + lane_off);
    sub_regs.load(a, b, nh, row0, pp * SUB, min(SUB, a.T - pp * SUB), tid);
  };

  // Results held in registers, stored at the end (by the role that holds them).
  auto store_dH0 = [&]() __attribute__((always_inline)) {
    if (a.dH0) *(float4*)(a.dH0 + own_off) = make_float4(C[0] * ug, C[1] * ug, C[2] * ug, C[3] * ug);
  };
  auto store_dwr = [&]() __attribute__((always_inline)) {
    if constexpr (GROUP4) {
      const float dwr = sum_rows4(dwr1);
      if (s == 0 && g == 0) a.dwr_part[((long)b * a.N + nh) * V + 16 * w + n] = dwr * ug;
    } else if (s == 0 && n == 0) {
      *(float4*)(a.dwr_part + ((long)b * a.N + nh) * V + 16 * w + 4 * g) =
          make_float4(dwr4[0] * ug, dwr4[1] * ug, dwr4[2] * ug, dwr4[3] * ug);
    }
  };
  // dW partial of this workgroup: dWacc[tt] at lane (g, j) reg r = dW[16w + 4g + r][16((w + tt) mod NT) + j].
  auto store_dW = [&]() __attribute__((always_inline)) {
    float* dWp = a.dW_part + ((long)(b * a.S + s) * a.N + nh) * V * V;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dWp[(long)(16 * w + 4 * g + r) * V + 16 * ((w + tt) & (NT - 1)) + n] = dWacc[tt][r] * ug;
  };

  if constexpr (WS) {
    // Which role forms dW and which dv and dw_r: measured, dv and dw_r with the walk (2.19 -> 2.04 ms),
    // dW with the recompute (the same time with either role).
    constexpr bool DW_WALK = false, DV_WALK = true;
    // Buffers of sub-segment p (p >= -1), as in the one-role interleaved walk below.
    auto stg = [&](int p) { return stage + ((p + 2) & 1) * (SUB * St::STEP); };
    auto hsb = [&](int p) { return hst + ((p + 2) & 1) * (SUB * ENTRY); };
    auto zsb = [&](int p) { return zst + ((p + 2) & 1) * (SUB * NT * 64 * 4); };
    const int P = nck;  // sub-segments
    // Both roles pass the same barriers: one before the recompute of the last sub-segment, one per
    // step of it, then per pair two at its start and one per step, and one at the end.
    if (walker) {
      // ---------------- walk waves: the records, the chain, R and D, dk and df ----------------
      load_w(false, true);
      init_C();
      // (the walk waves stage every sub-segment's records: tid < NTH)
      auto load_records = [&](int p) __attribute__((always_inline)) {
        const int pp = max(p, 0);
        sub_regs.load(a, b, nh, row0, pp * SUB, min(SUB, a.T - pp * SUB), tid);
      };
      load_records(P - 1);
      sub_regs.store(stg(P - 1), tid, us);
      load_records(P - 2);
      lds_barrier();
      for (int j = 0; j < SUB; ++j) lds_barrier();  // the recompute waves' pass over sub-segment P - 1
      for (int p = P - 1; p >= 0; --p) {
        lds_barrier();                        // the previous pair is done with the buffers of p - 1
        sub_regs.store(stg(p - 1), tid, us);  // (at p = 0 a repeat of sub-segment 0, never used)
        load_records(p - 2);
        lds_barrier();
        const float* ws = stg(p);
        const uint32_t* wh = hsb(p);
        const float* wz = zsb(p);
        nxt = load_rev(ws, wh, wz, SUB - 1);
        fr = front(SUB - 1, nxt);
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int j = SUB - 1 - i;
          const int tb = p * SUB;
          const int js = tb + j;
          const uint32_t* dxp = dx + (j & 1) * ENTRY;
          __builtin_amdgcn_sched_barrier(0);
          lds_barrier();
          const Ops o = read_ops(dxp);
          if (j > 0) nxt = load_rev(ws, wh, wz, j - 1);
          // The cross-wave sums of dk (wave 0) and df (wave 1) of one group: at j = 3 steps
          // tb + 4 .. 7, at j = 7 steps tb + SUB .. tb + SUB + 3 (of the previous pair).
          const bool gsum = (j & 3) == 3 && w < 2;
          float gx[4];
          if (gsum) {
            const float* src = &red[1 + w][(j == 3 ? 4 : 0) + g][0][n];
#pragma unroll
            for (int ww = 0; ww < NT; ++ww) gx[ww] = src[ww * 16];
          }
          __builtin_amdgcn_sched_barrier(0);
          const f32x4 acc = contract(fr.cinit, bOwnHi, bOwnLo, bOthHi, bOthLo, fr.dh, fr.dl, o);
          uint2 hT = make_uint2(0, 0), dT[NT], dTlo = make_uint2(0, 0);
          float4 k4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          float ucol = 0.0f, vcol = 0.0f;
          if constexpr (DW_WALK) {
            hT = lds_read_tr(wh + j * ENTRY + tile_off(w, 0) + 2 * tr_slot);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) dT[tt] = lds_read_tr(dxp + tile_off((w + tt) & (NT - 1), 0) + 2 * tr_slot);
          } else if constexpr (DV_WALK) {
            dT[0] = lds_read_tr(dxp + tile_off(w, 0) + 2 * tr_slot);
          }
          if constexpr (DV_WALK) {
            dTlo = lds_read_tr(dxp + tile_off(w, 1) + 2 * tr_slot);
            k4 = *(const float4*)(ws + j * St::STEP + St::OK + 4 * g);
            if ((j & 3) == 0) {
              ucol = ws[(j + g) * St::STEP + St::OU + 16 * w + n];
              vcol = ws[(j + g) * St::STEP + St::OV + 16 * w + n];
            }
          }
          walk_sums(j, js);
          // Step j-1's R, D and publish as soon as the chain has produced C (no clamp on the
          // padding steps of a ragged tail, which must leave the chain unchanged).
          const bool real = js < a.T;
          const float lo = real ? clip_lo : -__builtin_inff(), hi = real ? clip_hi : __builtin_inff();
#pragma unroll
          for (int r = 0; r < 4; ++r) C[r] = __builtin_amdgcn_fmed3f(acc[r], lo, hi);
          if (j > 0) fr = front(j - 1, nxt);
          if constexpr (DW_WALK) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) dWacc[tt] = mfma16_f16(hT, dT[tt], dWacc[tt]);
          }
          if constexpr (DV_WALK) dv_step(j, js, ws + j * St::STEP, dT[0], dTlo, k4, ucol, vcol);
          if (gsum) {
            float acc_s = 0.0f;
#pragma unroll
            for (int ww = 0; ww < NT; ++ww) acc_s += gx[ww];
            const int tk = j == 3 ? tb + 4 : tb + SUB;
            const uint32_t val = __float_as_uint(acc_s * ug);
            if (w == 0) {
              __builtin_amdgcn_raw_buffer_store_b32(val, dkres, qk_lane + (uint32_t)(tk * qkstep * 4), 0, 0);
            } else {
              __builtin_amdgcn_raw_buffer_store_b32(
                  val, dfres, df_lane == kBufferDrop ? kBufferDrop : df_lane + (uint32_t)(tk * a.N * 4), 0, 0);
            }
          }
        }
      }
      lds_barrier();
      if (w < 2) {  // dk, df of steps 0 .. 3
        float acc_s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) acc_s += red[1 + w][g][ww][n];
        const uint32_t val = __float_as_uint(acc_s * ug);
        if (w == 0) {
          __builtin_amdgcn_raw_buffer_store_b32(val, dkres, qk_lane, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b32(val, dfres, df_lane, 0, 0);
        }
      }
      store_dH0();
      if constexpr (DW_WALK) store_dW();
      if constexpr (DV_WALK) store_dwr();
    } else {
      // ---------------- recompute waves: the forward step, dq, and dW, dv, dw_r of the walk ----------------
      load_w(true, false);
      float Hr[4];
      uint2 hh, hl;
      auto load_entry = [&](int p) __attribute__((always_inline)) {
        return *(const float4*)(a.ckpt + ((long)u * nck + max(p, 0)) * KV + lane_off);
      };
      auto take_entry = [&](int p, float4 h) __attribute__((always_inline)) {
        Hr[0] = h.x; Hr[1] = h.y; Hr[2] = h.z; Hr[3] = h.w;
        put_tile(hsb(p), Hr, hh, hl);
      };
      // the cross-wave dq sum of one group (wave 0): reads of red_q rows jq .. jq + 3, then the store
      auto dq_read = [&](int jq, float (&x)[4]) __attribute__((always_inline)) {
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) x[ww] = red_q[jq + g][ww][n];
      };
      auto dq_store = [&](const float (&x)[4], int tq) __attribute__((always_inline)) {
        float acc_s = 0.0f;
#pragma unroll
        for (int ww = 0; ww < NT; ++ww) acc_s += x[ww];
        if (tq >= 0)
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc_s * ug), dqres, qk_lane + (uint32_t)(tq * qkstep * 4),
                                                0, 0);
      };
      take_entry(P - 1, load_entry(P - 1));
      float4 nextE = load_entry(P - 2);
      lds_barrier();
      {
        const float* ss = stg(P - 1);
        f32x4 kv = rank1(ss);
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
          float Z[4];
          const float* st = ss + j * St::STEP;
          float gq[4];
          if (j == 4 && w == 0) dq_read(0, gq);  // dq of steps 0 .. 3 of this sub-segment
          fwd_step(st, j + 1 < SUB ? st + St::STEP : nullptr, hsb(P - 1) + j * ENTRY,
                   j + 1 < SUB ? hsb(P - 1) + (j + 1) * ENTRY : nullptr, kv, Hr, Z, hh, hl);
          *(float4*)(zsb(P - 1) + ((j * NT + w) * 64 + lane) * 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
          __builtin_amdgcn_sched_barrier(0);
          rec_dq(Hr, rec_u4(st), j, (P - 1) * SUB);
          if (j == 4 && w == 0) dq_store(gq, (P - 1) * SUB);
          lds_barrier();
        }
      }
      for (int p = P - 1; p >= 0; --p) {
        lds_barrier();  // the previous pair is done with the buffers of p - 1
        take_entry(p - 1, nextE);
        nextE = load_entry(p - 2);
        lds_barrier();
        const float* ws = stg(p);
        const uint32_t* wh = hsb(p);
        const float* rs = stg(p - 1);
        uint32_t* rh = hsb(p - 1);
        float* rz = zsb(p - 1);
        f32x4 kv = rank1(rs);
#pragma unroll
        for (int i = 0; i < SUB; ++i) {
          const int j = SUB - 1 - i;  // the walk step of this barrier
          const int js = p * SUB + j;
          const float* st = rs + i * St::STEP;
          const float* sw = ws + j * St::STEP;
          const uint32_t* hj = wh + j * ENTRY;
          const uint32_t* dxp = dx + (j & 1) * ENTRY;
          __builtin_amdgcn_sched_barrier(0);
          lds_barrier();
          // Recompute step i's operands and inputs first; the dq sum of one group (wave 0): at
          // j = 3 steps (p - 1) SUB .. + 3 of the recompute, at j = 7 steps p SUB + 4 .. 7.
          const Ops ro = read_ops(rh + i * ENTRY);
          float avn = 0.0f, bkn = 0.0f;
          if (i + 1 < SUB) {
            avn = st[St::STEP + (g == 0 ? St::OV + 16 * w + n : 3)];
            bkn = st[St::STEP + (g == 0 ? St::OCK + n : 3)];
          }
          const float f = st[0];
          const float4 uq4 = rec_u4(st);
          const bool gsum = (j & 3) == 3 && w == 0;
          float gq[4];
          if (gsum) dq_read(j == 3 ? 0 : 4, gq);
          __builtin_amdgcn_sched_barrier(0);
          const f32x4 racc = contract(kv, fOwnHi, fOwnLo, fOthHi, fOthLo, hh, hl, ro);
          // Walk step j's transposed tiles (H_{t-1} and D) and k for dW and dv, behind the MFMAs.
          uint2 hT = make_uint2(0, 0), dT[NT], dTlo = make_uint2(0, 0);
          float4 k4 = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
          float ucol = 0.0f, vcol = 0.0f;
          if constexpr (!DW_WALK) {
            hT = lds_read_tr(hj + tile_off(w, 0) + 2 * tr_slot);
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) dT[tt] = lds_read_tr(dxp + tile_off((w + tt) & (NT - 1), 0) + 2 * tr_slot);
          } else if constexpr (!DV_WALK) {
            dT[0] = lds_read_tr(dxp + tile_off(w, 0) + 2 * tr_slot);
          }
          if constexpr (!DV_WALK) {
            dTlo = lds_read_tr(dxp + tile_off(w, 1) + 2 * tr_slot);
            k4 = *(const float4*)(sw + St::OK + 4 * g);
            if ((j & 3) == 0) {
              ucol = ws[(j + g) * St::STEP + St::OU + 16 * w + n];
              vcol = ws[(j + g) * St::STEP + St::OV + 16 * w + n];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (!DW_WALK) {
#pragma unroll
            for (int tt = 0; tt < NT; ++tt) dWacc[tt] = mfma16_f16(hT, dT[tt], dWacc[tt]);
          }
          {
            const float g1 = 1.0f - f, m2g = -2.0f * g1;
            float Z[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float rr = tanh_recip(racc[r]);
              Z[r] = __builtin_fmaf(-2.0f, rr, 1.0f);
              Hr[r] = __builtin_fmaf(m2g, rr, __builtin_fmaf(f, Hr[r], g1));
            }
            if (i + 1 < SUB) put_tile(rh + (i + 1) * ENTRY, Hr, hh, hl);
            *(float4*)(rz + ((i * NT + w) * 64 + lane) * 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
            rec_dq(Hr, uq4, i, (p - 1) * SUB);
            if (i + 1 < SUB) kv = mfma_f32(avn, bkn, zero4);
          }
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (!DV_WALK) dv_step(j, js, sw, dT[0], dTlo, k4, ucol, vcol);
          if (gsum) dq_store(gq, j == 3 ? (p - 1) * SUB : p * SUB + 4);
        }
      }
      lds_barrier();
      if constexpr (!DV_WALK) store_dwr();
      if constexpr (!DW_WALK) store_dW();
    }
  } else if constexpr (INTERLEAVE) {
    // Buffers of sub-segment p (p >= -1).
    auto stg = [&](int p) { return stage + ((p + 2) & 1) * (SUB * St::STEP); };
    auto hsb = [&](int p) { return hst + ((p + 2) & 1) * (SUB * ENTRY); };
    auto zsb = [&](int p) { return zst + ((p + 2) & 1) * (SUB * NT * 64 * 4); };
    const int P = nck;  // sub-segments
    float Hr[4];        // state of the sub-segment being recomputed
    uint2 hh, hl;
    // Writes the prefetched records and entry state of sub-segment p into its buffers.
    auto take = [&](int p) __attribute__((always_inline)) {
      Hr[0] = nextH.x; Hr[1] = nextH.y; Hr[2] = nextH.z; Hr[3] = nextH.w;
      sub_regs.store(stg(p), tid, us);
      put_tile(hsb(p), Hr, hh, hl);
    };

    // Prologue: the last sub-segment is recomputed alone.
    take(P - 1);
    prefetch(P - 2);
    lds_barrier();
    {
      const float* ss = stg(P - 1);
      f32x4 kv = rank1(ss);
#pragma unroll
      for (int j = 0; j < SUB; ++j) {
        float Z[4];
        const float* st = ss + j * St::STEP;
        float gx[4];
        if (j == 4) group_read(0, 0, gx);  // dq of steps 0 .. 3 of this sub-segment
        fwd_step(st, j + 1 < SUB ? st + St::STEP : nullptr, hsb(P - 1) + j * ENTRY,
                 j + 1 < SUB ? hsb(P - 1) + (j + 1) * ENTRY : nullptr, kv, Hr, Z, hh, hl);
        *(float4*)(zsb(P - 1) + ((j * NT + w) * 64 + lane) * 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
        __builtin_amdgcn_sched_barrier(0);
        rec_dq(Hr, rec_u4(st), j, (P - 1) * SUB);
        if (j == 4) group_store(gx, (P - 1) * SUB, -1);
        lds_barrier();
      }
    }

    for (int p = P - 1; p >= 0; --p) {
      lds_barrier();  // the previous pair of sub-segments is done with the buffers of p - 1
      take(p - 1);    // (at p = 0 a repeat of sub-segment 0, recomputed and never used)
      prefetch(p - 2);
      lds_barrier();

      const float* ws = stg(p);
      const uint32_t* wh = hsb(p);
      const float* wz = zsb(p);
      const float* rs = stg(p - 1);
      uint32_t* rh = hsb(p - 1);
      float* rz = zsb(p - 1);
      nxt = load_rev(ws, wh, wz, SUB - 1);
      fr = front(SUB - 1, nxt);
      f32x4 kv = rank1(rs);
#pragma unroll
      for (int i = 0; i < SUB; ++i) {
        const int j = SUB - 1 - i;
        // Recompute step i of sub-segment p - 1 (as fwd_step, split around the walk step's phases).
        const float* st = rs + i * St::STEP;
        Ops ro;
        float4 uq4;
        float avn = 0.0f, bkn = 0.0f, f = 0.0f;
        f32x4 racc;
        walk_step(
            j, p * SUB, ws, wh, wz,
            [&]() __attribute__((always_inline)) {
              ro = read_ops(rh + i * ENTRY);
              if (i + 1 < SUB) {
                avn = st[St::STEP + (g == 0 ? St::OV + 16 * w + n : 3)];
                bkn = st[St::STEP + (g == 0 ? St::OCK + n : 3)];
              }
              f = st[0];
              uq4 = rec_u4(st);
            },
            [&]() __attribute__((always_inline)) { racc = contract(kv, fOwnHi, fOwnLo, fOthHi, fOthLo, hh, hl, ro); },
            [&]() __attribute__((always_inline)) {
              const float g1 = 1.0f - f, m2g = -2.0f * g1;
              float Z[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float rr = tanh_recip(racc[r]);
                Z[r] = __builtin_fmaf(-2.0f, rr, 1.0f);
                Hr[r] = __builtin_fmaf(m2g, rr, __builtin_fmaf(f, Hr[r], g1));
              }
              if (i + 1 < SUB) {
                put_tile(rh + (i + 1) * ENTRY, Hr, hh, hl);
              }
              *(float4*)(rz + ((i * NT + w) * 64 + lane) * 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
              rec_dq(Hr, uq4, i, (p - 1) * SUB);
              if (i + 1 < SUB) kv = mfma_f32(avn, bkn, zero4);
            });
      }
    }
    lds_barrier();
    {
      float x[4];
      group_read(0, 0, x);
      group_store(x, -1, 0);  // dk, df of steps 0 .. 3
    }
  } else {
    for (int seg = nseg - 1; seg >= 0; --seg) {
      const int t0 = seg * kBwdSeg;
      const int nst = min(kBwdSeg, a.T - t0);
      const int nsub = (nst + SUB - 1) / SUB;
      if constexpr (!SUBCK) {
        lds_barrier();  // the previous segment's readers are done with the stage
        if (pending_tb >= 0) finalize(pending_tb);
        pending_tb = -1;
        bwd_stage_segment<V, BF16IN>(a, b, nh, row0, t0, nst, nsub * SUB, stage, tid, NTH, us);
      }

      // The checkpoint entering this segment (segment checkpoints).
      const float* ck = a.ckpt + ((long)u * nck + seg) * KV + lane_off;
      float H[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      if constexpr (!SUBCK) {
        const float4 h4 = *(const float4*)ck;
        H[0] = h4.x; H[1] = h4.y; H[2] = h4.z; H[3] = h4.w;
      }

      // ---------------- pass A: forward up to the last sub-segment (segment checkpoints only) ----------------
      if (!SUBCK && nsub > 1) {
        uint2 hh, hl;
        put_tile(hst, H, hh, hl);
        lds_barrier();  // (also makes the stage written above visible)
        f32x4 kv = rank1(stage);
        for (int m = 0; m < nsub - 1; ++m) {
          if (m > 0) *(float4*)(subck + (long)m * 16 * V) = make_float4(H[0], H[1], H[2], H[3]);
#pragma unroll
          for (int j = 0; j < SUB; ++j) {
            float Z[4];
            const float* st = stage + (m * SUB + j) * St::STEP;
            fwd_step(st, st + St::STEP, hst + (j & 1) * ENTRY, hst + ((j + 1) & 1) * ENTRY, kv, H, Z, hh, hl);
            lds_barrier();
          }
        }
        __threadfence_block();  // the scratch states are read back by the same lanes below
      }

      // ---------------- sub-segments, last to first ----------------
      for (int m = nsub - 1; m >= 0; --m) {
        const int jb = m * SUB;
        if constexpr (!SUBCK) {
          if (m < nsub - 1) {
            H[0] = nextH.x; H[1] = nextH.y; H[2] = nextH.z; H[3] = nextH.w;
          }
          if (m > 0) nextH = *(const float4*)(m - 1 > 0 ? subck + (long)(m - 1) * 16 * V : ck);
        }

        // 1. Recompute the sub-segment: hst[j] = H_{t-1} (split), zst[j] = Z_t.
        lds_barrier();  // the previous walk is done with hst, zst, the partial sums (and the stage)
        // Records of this sub-segment: in the segment's stage, or (sub-segment checkpoints) written
        // now from the registers prefetched during the previous walk.
        const float* sstage = SUBCK ? stage : stage + jb * St::STEP;
        uint2 hh, hl;
        if constexpr (SUBCK) {
          // Everything prefetched for this sub-segment is used before the next prefetch is issued,
          // so that waiting for it never waits for the new loads.
          H[0] = nextH.x; H[1] = nextH.y; H[2] = nextH.z; H[3] = nextH.w;
          sub_regs.store(stage, tid, us);
          put_tile(hst, H, hh, hl);
          if (pending_tb >= 0) finalize(pending_tb);
          pending_tb = t0 + jb;
          // Prefetch the sub-segment before this one in time (at the first one: itself again).
          prefetch(seg * NSUB + m - 1);
        } else {
          if (pending_tb >= 0) finalize(pending_tb);
          pending_tb = t0 + jb;
          put_tile(hst, H, hh, hl);
        }
        lds_barrier();  // hst, and the stage records written above by every wave, are complete
        f32x4 kv = rank1(sstage);
#pragma unroll
        for (int j = 0; j < SUB; ++j) {
          float Z[4];
          const float* st = sstage + j * St::STEP;
          fwd_step(st, j + 1 < SUB ? st + St::STEP : nullptr, hst + j * ENTRY,
                   j + 1 < SUB ? hst + (j + 1) * ENTRY : nullptr, kv, H, Z, hh, hl);
          *(float4*)(zst + ((j * NT + w) * 64 + lane) * 4) = make_float4(Z[0], Z[1], Z[2], Z[3]);
          __builtin_amdgcn_sched_barrier(0);
          // dq_t = H_t u_t (row sums over this wave's 16 columns) needs no backward quantity: it
          // is formed here, in the shadow of the writes above.
          rec_dq(H, rec_u4(st), j, t0 + jb);
          lds_barrier();
        }

        // 2. Walk the sub-segment backwards.
        nxt = load_rev(sstage, hst, zst, SUB - 1);
        fr = front(SUB - 1, nxt);
#pragma unroll
        for (int j = SUB - 1; j >= 0; --j) walk_step(j, t0 + jb, sstage, hst, zst, none, none, none);
      }
    }
    lds_barrier();
    if (pending_tb >= 0) finalize(pending_tb);
  }

  if constexpr (!WS) {
    store_dH0();
    store_dwr();
    store_dW();
  }
}

// Partial maxima of |dy| and |dH_T| per (b, n) pair, for the pair's power-of-two scale in the
// reverse kernel.  Block (b P + p, w) covers time part p of batch entry b and the 1024-float window w of
// the N V features of a step (1024 / V whole heads; a thread keeps one float4 column): each step's
// window is one contiguous 4 KiB read.  The blocks with p == 0 add the pair's |dH_T|.  Every entry
// part[(b N + n) P + p] is written by exactly one thread (zero for an empty part).
__global__ void __launch_bounds__(256) m2rnn_bwd_absmax_kernel(const float* __restrict__ dy,
                                                                const float* __restrict__ dH_T, int T, int N, int K,
                                                                int V, int P, float* __restrict__ part) {
  const int p = blockIdx.x % P, b = blockIdx.x / P;
  const long NV = (long)N * V;
  const long c = (long)blockIdx.y * 1024 + 4 * threadIdx.x;  // first feature of this thread
  const bool live = c < NV;
  const int len = (T + P - 1) / P;
  const int t0 = p * len, t1 = min(T, t0 + len);
  float m = 0.0f;
  if (live) {
    // (eight steps' loads in flight per thread: the read is latency-bound otherwise)
    const float* src = dy + (long)b * T * NV + c;
    int t = t0;
    for (; t + 8 <= t1; t += 8) {
      f32x4 x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_nontemporal_load((const f32x4*)(src + (long)(t + i) * NV));
#pragma unroll
      for (int i = 0; i < 8; ++i)
        m = fmaxf(m, fmaxf(fmaxf(fabsf(x[i][0]), fabsf(x[i][1])), fmaxf(fabsf(x[i][2]), fabsf(x[i][3]))));
    }
    for (; t < t1; ++t) {
      const float4 x = *(const float4*)(src + (long)t * NV);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  }
  const int nh = (int)(c / V);
  const int sub = (int)((c % V) / 4);  // this thread's float4 within the head (V / 4 per head)
  if (live && p == 0 && dH_T) {
    const float* h = dH_T + ((long)b * N + nh) * K * V;
    for (long i = sub; i < (long)K * V / 4; i += V / 4) {
      const float4 x = *(const float4*)(h + 4 * i);
      m = fmaxf(m, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  }
  // Maximum over the V / 4 consecutive threads of a head (within one wave: V / 4 <= 32).
  for (int o = 1; o < V / 4; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (live && sub == 0) part[((long)b * N + nh) * P + p] = m;
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

// Gradient of a query/key shared by all heads (§2.7: summed over the heads): out[bt][k] =
// sum over n (in order) of the per-head gradients part[bt][n][k].  A thread takes 4 consecutive k
// (K is a multiple of 16); the loads do not depend on the running sum, so they go out eight heads
// ahead of the additions, and as non-temporal loads (each partial is read once).
__global__ void __launch_bounds__(256) m2rnn_bwd_sum_heads_kernel(const float* __restrict__ part, int N, long rows,
                                                                   int K, float* __restrict__ out) {
  const int K4 = K / 4;
  const long i4 = (long)blockIdx.x * blockDim.x + threadIdx.x;  // index into [rows][K / 4]
  if (i4 >= rows * K4) return;
  const long bt = i4 / K4;
  const f32x4* p = (const f32x4*)(part + bt * N * K) + (i4 - bt * K4);
  f32x4 acc = __builtin_nontemporal_load(p);
  int n = 1;
  for (; n + 8 <= N; n += 8) {
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + (long)(n + u) * K4);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += v[u];
  }
  for (; n < N; ++n) acc += __builtin_nontemporal_load(p + (long)n * K4);
  *(f32x4*)(out + 4 * i4) = acc;
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
