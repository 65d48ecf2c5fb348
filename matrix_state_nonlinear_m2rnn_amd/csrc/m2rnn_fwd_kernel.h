// Forward scan of the M²RNN recurrence (M²RNN notes §2.1, Eq. 10-12) for gfx950.
//
// Work decomposition
//   One workgroup carries ROWS = 16*RB consecutive rows of the K x V state of one (b, n) pair;
//   the rows of a state never mix (W acts on the value side only, §1.2), so a pair's K rows may
//   be spread over S = K/ROWS workgroups.  Inside a workgroup, wave w (of V/16) owns the 16
//   value columns [16w, 16w+16) of every row block: it computes those columns of
//   P = H_{t-1} W + k v^T, applies tanh and the gate, and keeps the result in registers.
//
// Register layout (16x16 MFMA tiles, transposed)
//   The kernel computes P^T = W^T H^T so that the accumulator of lane (g = lane/16, n = lane%16),
//   register r holds P[row n][col 16w + 4g + r].  That is exactly the B-operand layout of the
//   next step's MFMA (B[k][n] at lane (k-group, n)) once the contraction index k is permuted to
//   v = 16*tile + 4g + r; the A operand W^T uses the same permutation.  So the state never needs
//   a transpose: each step every wave publishes its 16-column tile to LDS (16 B per lane), one
//   barrier, and every wave reads the other tiles back as B operands (its own stays in registers).
//
// Per step, per wave: acc = (c k) v^T (MFMA) ; acc += W'^T H^T (MFMA, c = 2 log2 e folded into W')
//   ; r = 1/(1 + 2^acc) ; H = fma(-2(1-f), r, fma(f, H, 1-f))      [= f H + (1-f) tanh(P)]
//   ; y partial = sum over the block's rows of H[row][col] q[row] (transposing MFMA + cross-lane
//   reduction; DPP row reduction in the fp32 mode).
// q, k, v, f are staged through LDS in chunks of TC steps, double-buffered: chunk c+1 is read
// from HBM into registers while chunk c is consumed.
#pragma once

#include "m2rnn_device.h"

namespace m2rnn {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* f;
  const float* W;
  const float* w_r;
  const float* H0;
  float* y;       // final readout (S == 1) or partial readouts [S][B*T*N*V] (S > 1)
  float* H_T;     // may be null
  float* ckpt;    // states entering each seg-step segment [B][N][nck][K][V] (checkpoint mode;
                  // optional in the forward mode, null = none)
  int B, T, N, K;
  int Nqk;        // heads of q and k: N, or 1 when one query/key is shared by all heads
  int S;          // workgroups per (b, n)
  int seg;        // checkpoint interval, a multiple of 8 (when ckpt is set)
  int nck;        // checkpoints per (b, n) in ckpt
  int ck0;        // index of the checkpoint entering this launch's first step (a time segment of a
                  // longer sequence starts at a multiple of seg)
  int Ts;         // steps between batch entries in q, k, v and f: T, or more when the launch covers
                  // a time segment of a longer sequence (the pointers then start at the segment's
                  // first step)
  int Tp;         // steps between batch entries in y (S == 1) or the readout planes (S > 1): Ts
                  // when they cover the whole sequence, or the segment's length for planes that
                  // hold one segment only
};

// RW: row waves, independent groups of NT waves in one workgroup, each carrying its own row
// blocks (used when V/16 < 4, so that a workgroup still has a wave on each SIMD of its CU).
template <int V, int RW = 1>
struct FwdShape {
  static constexpr int NT = V / 16;          // value tiles = waves per row group
  static constexpr int NTH = 64 * NT * RW;   // threads per workgroup
  // Steps per staged chunk (the step loop is unrolled per chunk): 32 where the state is narrow
  // (V <= 32: the step is short, so the staging step and its barriers weigh more), else 16.
  static constexpr int TC = V <= 32 ? 32 : 16;
  // Steps per chunk of the readout-waves kernel: its readout waves stage a chunk while the chain
  // runs, and fewer, longer chunks mean fewer staging steps (64 against 16: 2% faster at 16K steps).
  // At V = 128 a chunk of 32 keeps the staging registers within the 128 VGPRs of a 16-wave group.
  static constexpr int TC_RO = V <= 64 ? 64 : 32;
};

// Per-step stage record (fp32): [f, 1-f, -2(1-f), 0 | q rows | c*k rows | v (V)] (slot 3 is the
// zero that the lanes without a rank-1 operand read).
template <int V, int RB>
struct Stage {
  static constexpr int ROWS = 16 * RB;
  static constexpr int OQ = 4;
  static constexpr int OK = 4 + ROWS;
  static constexpr int OV = 4 + 2 * ROWS;
  static constexpr int STEP = 4 + 2 * ROWS + V;  // floats, multiple of 4
};

// Copies of a TC x COLS tile of a [.., T, N, COLS_total] tensor into registers, 16 B at a time.
template <int TC, int COLS, int NTH, bool BF16>
struct TileLoader {
  static constexpr int VEC = BF16 ? 8 : 4;  // elements per 16-byte load
  static constexpr int PER_ROW = COLS / VEC;
  static constexpr int NVEC = TC * PER_ROW;
  static constexpr int PER = (NVEC + NTH - 1) / NTH;
  uint4 r[PER];

  __device__ __forceinline__ void load(const void* base, long row_stride_elems, int valid_rows, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NTH;
      const int row = idx / PER_ROW, cv = idx % PER_ROW;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (idx < NVEC && row < valid_rows) {
        const char* p = (const char*)base + ((long)row * row_stride_elems + cv * VEC) * (BF16 ? 2 : 4);
        val = *(const uint4*)p;
      }
      r[i] = val;
    }
  }
  // Writes the tile as fp32 into LDS rows of `row_pitch` floats starting at column `col0`,
  // multiplied by `scale`.
  __device__ __forceinline__ void store(float* lds, int row_pitch, int col0, float scale, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * NTH;
      if (idx < NVEC) {
        const int row = idx / PER_ROW, cv = idx % PER_ROW;
        float* d = lds + row * row_pitch + col0 + cv * VEC;
        if constexpr (BF16) {
          const uint32_t w[4] = {r[i].x, r[i].y, r[i].z, r[i].w};
          float4 a = make_float4(bf16_lo_to_f32(w[0]) * scale, bf16_hi_to_f32(w[0]) * scale,
                                 bf16_lo_to_f32(w[1]) * scale, bf16_hi_to_f32(w[1]) * scale);
          float4 b = make_float4(bf16_lo_to_f32(w[2]) * scale, bf16_hi_to_f32(w[2]) * scale,
                                 bf16_lo_to_f32(w[3]) * scale, bf16_hi_to_f32(w[3]) * scale);
          *(float4*)d = a;
          *(float4*)(d + 4) = b;
        } else {
          *(float4*)d = make_float4(__uint_as_float(r[i].x) * scale, __uint_as_float(r[i].y) * scale,
                                    __uint_as_float(r[i].z) * scale, __uint_as_float(r[i].w) * scale);
        }
      }
    }
  }
};

// Prefetch registers for one chunk of q, k, v, f.
template <int V, int RB, bool BF16, int RW = 1, int TC = FwdShape<V, RW>::TC>
struct ChunkRegs {
  using S = FwdShape<V, RW>;
  static constexpr int ROWS = 16 * RB * RW;  // rows staged for the whole workgroup
  TileLoader<TC, ROWS, S::NTH, BF16> q, k;
  TileLoader<TC, V, S::NTH, BF16> v;
  float f;

  // The pieces of q, k, v and f start at different waves (thread indices rotated by 64 per
  // tensor), so that no single wave carries the whole staging while the others wait for it at
  // the next barrier.
  static __device__ __forceinline__ int rot(int tid, int r) { return (tid + S::NTH - r % S::NTH) % S::NTH; }

  __device__ __forceinline__ void load(const FwdArgs& a, int b, int nh, int row0, int t0, int tid) {
    const int valid = min(TC, a.T - t0);
    const long qk_off = (((long)b * a.Ts + t0) * a.Nqk + (a.Nqk == 1 ? 0 : nh)) * a.K + row0;
    const long v_off = (((long)b * a.Ts + t0) * a.N + nh) * V;
    const int esz = BF16 ? 2 : 4;
    q.load((const char*)a.q + qk_off * esz, (long)a.Nqk * a.K, valid, tid);
    k.load((const char*)a.k + qk_off * esz, (long)a.Nqk * a.K, valid, rot(tid, 64));
    v.load((const char*)a.v + v_off * esz, (long)a.N * V, valid, rot(tid, 128));
    const int tf = rot(tid, 192);
    f = 1.0f;
    if (tf < valid) f = a.f[((long)b * a.Ts + t0 + tf) * a.N + nh];
  }
  __device__ __forceinline__ void store(float* stage, int tid) const {
    using St = Stage<V, RB * RW>;
    q.store(stage, St::STEP, St::OQ, 1.0f, tid);
    k.store(stage, St::STEP, St::OK, kTwoLog2e, rot(tid, 64));
    v.store(stage, St::STEP, St::OV, 1.0f, rot(tid, 128));
    const int tf = rot(tid, 192);
    if (tf < TC) {
      const float gf = 1.0f - f;
      *(float4*)(stage + tf * St::STEP) = make_float4(f, gf, -2.0f * gf, 0.0f);
    }
  }
};

// Per-step inputs a lane needs, read from the stage ring one step ahead.
template <int RB, bool SPLIT>
struct StepIn {
  float f, gf, m2g;            // the gate f, 1 - f and -2(1 - f)
  float av;                    // A operand of the rank-1 MFMA: v[16w + n] on lanes with g == 0, else 0
  float bk[RB];                // B operand of the rank-1 MFMA: c*k[row] on lanes with g == 0, else 0
  // q for the readout.  Split modes with one row block: q of rows 4g .. 4g+3 (q4).  Split modes
  // with several row blocks, where registers are scarce: q of row 16rb + 4g + (n & 3) (qn; a quad of
  // lanes holds rows 4g .. 4g+3, broadcast by DPP).  f32 mode: q of row 16rb + n (qn).
  static constexpr bool Q4 = SPLIT && RB == 1;
  float4 q4[Q4 ? RB : 1];
  float qn[Q4 ? 1 : RB];
  float vcol;                  // f32 mode: v[ycol] for the w_r (.) v readout term
};

// Lane-constant offsets (in floats) into one stage record.
template <int RB>
struct StepOffsets {
  int av;
  int bk[RB];
  int q;
  int vcol;
};

template <int V, int RB, bool SPLIT>
__device__ __forceinline__ StepIn<RB, SPLIT> read_step(const float* st, const StepOffsets<RB>& o) {
  using Sg = Stage<V, RB>;
  StepIn<RB, SPLIT> s;
  const float4 gate = *(const float4*)st;
  s.f = gate.x;
  s.gf = gate.y;
  s.m2g = gate.z;
  s.av = st[o.av];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) s.bk[rb] = st[o.bk[rb]];
  if constexpr (StepIn<RB, SPLIT>::Q4) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s.q4[rb] = *(const float4*)(st + o.q + 16 * rb);
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s.qn[rb] = st[o.q + 16 * rb];
  }
  s.vcol = SPLIT ? 0.0f : st[o.vcol];
  return s;
}

// Splits (a, b) into packed 16-bit high parts and the packed 16-bit rounding remainders.
//   F16X3:  hi = fp16(x) (RNE), lo = fp16(x - hi) computed by v_fma_mix in fp32 (x - hi is exact).
//   BF16X3: hi = bf16(x), lo = bf16(x - hi).
//   BF16:   hi = bf16(x), lo = 0.
template <int MATH>
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  if constexpr (MATH == MATH_F16X3) {
    hi = pack_f16(a, b);
    uint32_t l;
    // Both halves in one asm block (the output is written before b is read: early clobber).  The
    // trailing s_nop gives the two wait states that a VALU write needs before an MFMA may read the
    // register; the compiler inserts them for its own instructions but not after inline asm.
    asm("v_fma_mixlo_f16 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]\n\t"
        "v_fma_mixhi_f16 %0, %1, -1.0, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]\n\ts_nop 1"
        : "=&v"(l)
        : "v"(hi), "v"(a), "v"(b));
    lo = l;
  } else if constexpr (MATH == MATH_BF16X3) {
    hi = pack_bf16(a, b);
    // The fp32 values of hi's halves, each one byte permute of the packed word (a shift or a mask
    // written plainly, the compiler converts a once more to form the first, or copies hi).
    const float ha = __uint_as_float(__builtin_amdgcn_perm(0u, hi, 0x01000c0cu));
    const float hb = __uint_as_float(__builtin_amdgcn_perm(0u, hi, 0x03020c0cu));
    lo = pack_bf16(a - ha, b - hb);
  } else {
    hi = pack_bf16(a, b);
    lo = 0;
  }
}

// Sum over the four 16-lane rows of the wave (lanes j, j+16, j+32, j+48) with the gfx950
// row-swap permutes; every lane ends with the total of its column j.
__device__ __forceinline__ float sum_rows4(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float s = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto p2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(p2[0]) + __uint_as_float(p2[1]);
}

// Sums of four values over the four 16-lane rows at once: lane (g, j) returns
// x_g(j) + x_g(16 + j) + x_g(32 + j) + x_g(48 + j).  The 32-lane swap pairs x0 with x2 and x1
// with x3 (each half of the wave keeps the value it will return), the 16-lane swap then pairs the
// two partial sums: three swaps and three adds for four reductions.
__device__ __forceinline__ float reduce_rows4(float x0, float x1, float x2, float x3) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x0), __float_as_uint(x2), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x1), __float_as_uint(x3), false, false);
  const float s02 = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const float s13 = __uint_as_float(b[0]) + __uint_as_float(b[1]);
  const auto c = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}

// MODE_FWD: full forward with readout.  MODE_CKPT: state only, storing the state that enters
// every `seg`-step segment (used by the backward pass).
enum { MODE_FWD = 0, MODE_CKPT = 1 };
// MODE_FWD_RO: the forward with readout waves of its own (m2rnn_scan_fwd_ro_kernel), where built.
constexpr int MODE_FWD_RO = 2;

template <int V, int RB, int MATH, bool BF16IN, int MODE, int RW = 1>
__global__ void __launch_bounds__(64 * (V / 16) * RW) m2rnn_scan_fwd_kernel(const FwdArgs a) {
  using Sh = FwdShape<V, RW>;
  using St = Stage<V, RB * RW>;
  constexpr int NT = Sh::NT;
  constexpr int TC = Sh::TC;
  constexpr int ROWS = 16 * RB;  // rows of one wave (of one row group)
  constexpr bool SPLIT = MATH != MATH_F32;
  constexpr int NCH = (NT + 1) / 2;  // 32-wide contraction chunks of the split modes
  static_assert(TC % 2 == 0, "the exchange-buffer parity is derived from the step index within a chunk");

  __shared__ __attribute__((aligned(16))) float stage[2][TC * St::STEP];
  // Exchange buffer of the state tiles, double-buffered by step parity.
  //   F32:   [2][RB][NT][64 lanes][4 floats]
  //   split: [2][RB][NCH][hi|lo][half][64 lanes][2 dwords]; wave w fills half w&1 of chunk w/2.
  //          Every access is 8 contiguous bytes per lane (no LDS bank conflicts); the two halves
  //          of a chunk, 512 bytes apart, are read by one 2 x 8-byte instruction.
  constexpr int XWORDS = SPLIT ? (RB * NCH * 2 * 64 * 4) : (RB * NT * 64 * 4);
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2][RW][XWORDS];
  // Several row groups (split modes): their readout partials meet here, [3 chunks][TC / 4 groups of
  // four steps][RW][NT][64 lanes], and are summed in the workgroup (a ring of three chunks: a
  // chunk's groups are summed one chunk later, and its slot is reused two chunks after that, so
  // barriers at every chunk keep writers and readers apart).
  constexpr bool YRED = MODE == MODE_FWD && SPLIT && RW > 1;
  constexpr int GPC = TC / 4;  // groups of four steps per chunk
  __shared__ float ybuf[YRED ? 3 * GPC * RW * NT * 64 : 1];

  const int tid = threadIdx.x;
  const int w = (tid >> 6) % NT;   // value tile of this wave
  const int wr = (tid >> 6) / NT;  // row group of this wave
  const int lane = tid & 63;
  const int g = lane >> 4;
  const int n = lane & 15;

  // Block -> (pair u, row group s).  When the pair count is a multiple of 8, the S workgroups
  // of one pair get block ids congruent mod 8, which the dispatcher places on the same XCD, so
  // they share that XCD's L2 for q, k, v, f.
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
  const int row0_wg = s * ROWS * RW;       // first row of the workgroup
  const int row0 = row0_wg + wr * ROWS;    // first row of this wave
  const long KV = (long)a.K * V;

  // ---- W operands (A = W'^T with the permuted contraction index), W' = c W ----
  const float* Wn = a.W + (long)nh * V * V;
  const int col = 16 * w + n;  // output column of A-operand row m = n
  float wA[SPLIT ? 1 : NT * 4];
  // Split modes: the 32-wide chunk holding this wave's own tile is contracted with the own tile's
  // values taken from registers (k-slots 0..3 of each lane group) and only the partner tile's read
  // from LDS (k-slots 4..7); the other chunks are read whole.  The A operands follow that order.
  constexpr int NOTH = NCH > 1 ? NCH - 1 : 1;
  const int co = w >> 1;  // own chunk
  // A single tile (V = 16) leaves k-slots 4..7 of its chunk empty; the split modes put the state's
  // low halves there (hq = [hi | lo]), so that one MFMA against [W_hi | W_hi] forms
  // W_hi H_hi + W_hi H_lo and a second against [W_lo | 0] adds W_lo H_hi: two MFMAs a step instead
  // of three (paper head shape 1.10 -> 1.02 ms), and the readout transposes [hi | lo] with one.
  constexpr bool PACK1 = SPLIT && NT == 1 && MATH != MATH_BF16;
  uint4 wOwnHi, wOwnLo, wOthHi[NOTH], wOthLo[NOTH];
  auto wchunk = [&](int t_lo, int t_hi, uint4& hi, uint4& lo) {
    float wv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int tile = (i >> 2) ? t_hi : t_lo;
      const int vin = 16 * tile + 4 * g + (i & 3);
      wv[i] = tile < NT ? opaque1(kTwoLog2e * Wn[vin * V + col]) : 0.0f;
    }
    uint32_t h[4], l[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float x0 = wv[2 * i], x1 = wv[2 * i + 1];
      if constexpr (MATH == MATH_F16X3) {
        h[i] = pack_f16(x0, x1);
        l[i] = pack_f16(x0 - f16_lo_to_f32(h[i]), x1 - f16_hi_to_f32(h[i]));
      } else {
        h[i] = pack_bf16(x0, x1);
        l[i] = pack_bf16(x0 - bf16_lo_to_f32(h[i]), x1 - bf16_hi_to_f32(h[i]));
      }
    }
    hi = make_uint4(h[0], h[1], h[2], h[3]);
    lo = make_uint4(l[0], l[1], l[2], l[3]);
  };
  if constexpr (!SPLIT) {
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) wA[tt * 4 + r] = kTwoLog2e * Wn[(16 * tt + 4 * g + r) * V + col];
  } else {
    wchunk(w, w ^ 1, wOwnHi, wOwnLo);
#pragma unroll
    for (int i = 0; i < NCH - 1; ++i) {
      const int cc = i < co ? i : i + 1;
      wchunk(2 * cc, 2 * cc + 1, wOthHi[i], wOthLo[i]);
    }
  }
  // B operand of the readout's transposing MFMAs (16x16x16, contraction over the tile's 16
  // columns): the identity, k-slot (g, e) = column 4g + e selected for output column j = 4g + e.
  uint2 bsel = make_uint2(0, 0);
  if constexpr (SPLIT) {
    const uint32_t one = MATH == MATH_F16X3 ? 0x3C00u : 0x3F80u;
    uint32_t e16[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) e16[e] = (n == 4 * g + e) ? one : 0u;
    bsel = make_uint2(e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16));
  }

  // ---- initial state ----
  float H[RB][4];
  const long state_base = ((long)b * a.N + nh) * KV;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const long off = state_base + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g;
    if (a.H0) {
      const float4 h = *(const float4*)(a.H0 + off);
      H[rb][0] = h.x; H[rb][1] = h.y; H[rb][2] = h.z; H[rb][3] = h.w;
    } else {
      H[rb][0] = H[rb][1] = H[rb][2] = H[rb][3] = 0.0f;
    }
  }

  // This wave's tile of H_{t-1} as B operands of its own 32-wide chunk (split modes): hq holds the
  // high halves [own tile, k-slots 0..3 | partner tile, k-slots 4..7], lq the low halves.  The own
  // halves are written when the tile is published (and are also the A operands of the readout's
  // transposing MFMAs); the partner halves are read from LDS straight into the upper two dwords.
  uint4 hq[RB], lq[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) hq[rb] = lq[rb] = make_uint4(0, 0, 0, 0);
  // Publishes this wave's tile of H into exchange buffer `buf`.
  auto publish = [&](int buf) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if constexpr (!SPLIT) {
        if constexpr (NT > 1)
          *(float4*)&xbuf[buf][wr][((rb * NT + w) * 64 + lane) * 4] = make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
      } else {
        uint32_t h0, h1, l0, l1;
        opaque4(H[rb]);  // the split is a function of the fp32 state alone
        split_pair<MATH>(H[rb][0], H[rb][1], h0, l0);
        split_pair<MATH>(H[rb][2], H[rb][3], h1, l1);
        hq[rb].x = h0;
        hq[rb].y = h1;
        lq[rb].x = l0;
        lq[rb].y = l1;
        if constexpr (PACK1) {
          hq[rb].z = l0;
          hq[rb].w = l1;
        }
        if constexpr (NT > 1) {
          const int base = ((rb * NCH + (w >> 1)) * 4 + (w & 1)) * 128 + lane * 2;
          *(uint2*)&xbuf[buf][wr][base] = make_uint2(h0, h1);
          if constexpr (MATH != MATH_BF16) *(uint2*)&xbuf[buf][wr][base + 256] = make_uint2(l0, l1);
        }
      }
    }
  };

  // Odd tile counts leave half of the last chunk unwritten: zero both buffers once.
  if constexpr (SPLIT && (NT & 1) && NT > 1) {
    for (int i = tid; i < 2 * RW * XWORDS; i += Sh::NTH) (&xbuf[0][0][0])[i] = 0u;
    lds_barrier();
  }

  // Readout.
  //   split modes: the transposing MFMAs (issued after H_t is published, before the barrier) leave
  //                lane (g, j) with rows 4g..4g+3 of column 16w + j; after the barrier, while the
  //                exchange reads are in flight, each lane forms its q-weighted sum of those rows;
  //                the lane's q-weighted sum over them is kept for four consecutive steps, and one
  //                cross-row reduction of the four leaves lane (g, j) with y[t0 + g][16w + j], so
  //                every lane stores, once per four steps.
  //   f32 mode:    after the DPP row reduction lane (g, n) holds column 16w + 4g + n/4; lanes with
  //                n % 4 == 0 store, every step.
  // Stores go through a buffer resource whose size ends at the last valid step of this (b, n):
  // the (padded) steps past T and the lanes that do not store get offsets past that end, which
  // the buffer unit drops, so the step loop carries no branches for them.
  // (w_r is read before chunk 0 so that the wait for chunk 0 covers it and no wait is left inside
  // the step loop.)
  const int ycol = SPLIT ? 16 * w + n : 16 * w + 4 * g + (n >> 2);
  const bool ystore = SPLIT || ((n & 3) == 0);
  // Readout planes: one per workgroup (the row groups' partials are summed in the workgroup);
  // with one plane y is final here, and row group 0 adds the w_r (.) v term.
  const int planes = a.S;
  const float wrv = (MODE == MODE_FWD && planes == 1 && wr == 0) ? a.w_r[(long)nh * V + ycol] : 0.0f;
  const int ystep = a.N * V;  // floats between consecutive steps of y
  float* ybase = nullptr;  // y (S == 1) or this row group's partial plane, at [b, 0, nh, 0]
  int ybytes = 0;
  if constexpr (MODE == MODE_FWD) {
    const long plane = (long)a.B * a.Tp * a.N * V;
    ybase = a.y + (planes > 1 ? (long)s * plane : 0) + ((long)b * a.Tp * a.N + nh) * V;
    // Element (t, nh, c) is valid iff t < T, i.e. iff it lies below (T N V - nh V) floats from ybase.
    ybytes = (a.T * a.N - nh) * V * 4;
  }
  const __amdgpu_buffer_rsrc_t yres = __builtin_amdgcn_make_buffer_rsrc(ybase, (short)0, ybytes, kBufferRsrcWord3);
  // Byte offset of this lane's element at step 0 (split: step g), or kBufferDrop.
  const uint32_t ylane = ystore ? (uint32_t)(((SPLIT ? g * ystep : 0) + ycol) * 4) : kBufferDrop;
  // Stage-record offset of v[ycol] for the readout of step t0 + g (split modes).
  const int vlane = (SPLIT ? g * St::STEP : 0) + St::OV + ycol;

  StepOffsets<RB> so;
  so.av = g == 0 ? St::OV + 16 * w + n : 3;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) so.bk[rb] = g == 0 ? St::OK + wr * ROWS + 16 * rb + n : 3;
  so.q = wr * ROWS + (!SPLIT ? St::OQ + n : (StepIn<RB, SPLIT>::Q4 ? St::OQ + 4 * g : St::OQ + 4 * g + (n & 3)));
  so.vcol = St::OV + ycol;

  // Row groups' readouts of the group of four steps starting at tg: kept in ybuf ...
  auto ykeep = [&](int tg, float yv) {
    if constexpr (YRED) {
      const int slot = (tg / TC) % 3, k = (tg % TC) / 4;
      ybuf[(((slot * GPC + k) * RW + wr) * NT + w) * 64 + lane] = yv;
    }
  };
  // ... and summed, for the chunk starting at tc: wave (w, wr) stores the groups k = wr, wr + RW, ...
  // of its value tile.
  auto ysum = [&](int tc) {
    if constexpr (YRED) {
      const int slot = (tc / TC) % 3;
#pragma unroll
      for (int k = wr; k < GPC; k += RW) {
        float yv = 0.0f;
#pragma unroll
        for (int r = 0; r < RW; ++r) yv += ybuf[(((slot * GPC + k) * RW + r) * NT + w) * 64 + lane];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yres, ylane + (uint32_t)((tc + 4 * k) * ystep * 4), 0,
                                              0);
      }
    }
  };

  // ---- stage chunk 0, prefetch chunk 1 ----
  ChunkRegs<V, RB, BF16IN, RW> pre;
  pre.load(a, b, nh, row0_wg, 0, tid);
  pre.store(stage[0], tid);
  if (a.T > TC) pre.load(a, b, nh, row0_wg, TC, tid);
  publish(0);

  lds_barrier();

  // Software pipeline of the step loop.  Step t:
  //   1. the LDS reads of the B operands (the state tiles published at step t-1), and, while they
  //      are in flight, the readout sums of step t-1;
  //   2. the MFMA contraction acc = (c k_t) v_t^T + W'^T H_{t-1}^T (the rank-1 term was issued at
  //      the end of step t-1), and step t+1's staged inputs read while the MFMAs run;
  //   3. tanh + gate blend -> H_t, publish H_t's tile;
  //   4. while that write completes: the readout store of a finished group of four steps, the
  //      transposing MFMAs of H_t's tile and the rank-1 MFMA of step t+1; one barrier.
  // Chunk c+1 is written to the stage ring at step TC-2 of chunk c, so every step's inputs are in
  // LDS one barrier before step 2 of the previous step reads them.  Two chunks are unrolled per
  // loop trip, which makes the stage offsets and the exchange-buffer parity compile-time.  The
  // last chunk runs whole: its steps past T are staged with f = 1 and k = v = q = 0, which leaves
  // H bit-for-bit unchanged (H = fma(-0, r, fma(1, H, 0)) = H), and their y stores are dropped.
  StepIn<RB, SPLIT> cur = read_step<V, RB, SPLIT>(stage[0], so);
  const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
  float xq[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // split readout: partial sums of the last four steps
  f32x4 yT[RB];                            // split readout: transposed tile of H_{t-1}
  float4 qprev[RB];                        // and q_{t-1} of rows 4g .. 4g+3 (x only: see StepIn::qn)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    yT[rb] = zero4;
    qprev[rb] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // q of rows 4g .. 4g+3 for the readout: read whole (one row block) or quad-broadcast by DPP.
  auto q_rows = [](const float4& qp) -> float4 {
    if constexpr (StepIn<RB, SPLIT>::Q4) return qp;
    return make_float4(dpp_all<kDppQuadBcast0>(qp.x), dpp_all<kDppQuadBcast1>(qp.x), dpp_all<kDppQuadBcast2>(qp.x),
                       dpp_all<kDppQuadBcast3>(qp.x));
  };
  f32x4 kv[RB];                            // rank-1 term (c k_t) v_t^T of the coming step
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) kv[rb] = mfma_f32(cur.av, cur.bk[rb], zero4);
  // Offsets (in 8-byte units) of the partner half of the own chunk, high and low parts.  The low
  // offset goes through an empty asm so that the compiler keeps the two 8-byte reads apart
  // (fused into one 16-byte read, the halves would need copies into their operand registers).
  int phi_off[RB], plo_off[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    phi_off[rb] = ((rb * NCH + co) * 4 + ((w & 1) ^ 1)) * 64 + lane;
    plo_off[rb] = phi_off[rb] + 128;
    asm volatile("" : "+v"(plo_off[rb]));
  }

  auto run_chunk = [&](auto CB, int c0) __attribute__((always_inline)) {
    constexpr int cb = decltype(CB)::value;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const int t = c0 + j;
      // The state entering every seg-step segment (checkpoint mode, or a forward asked to keep
      // checkpoints for the backward).  seg is a multiple of 8, so only steps 0 and 8 of a chunk
      // can start a segment.
      if ((j % 8) == 0 && (MODE == MODE_CKPT || a.ckpt != nullptr)) {
        if (t % a.seg == 0 && t < a.T) {
          float* dst = a.ckpt + ((long)(b * a.N + nh) * a.nck + a.ck0 + t / a.seg) * KV;
#pragma unroll
          for (int rb = 0; rb < RB; ++rb)
            *(float4*)(dst + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g) =
                make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
        }
      }
      const uint32_t* xr = xbuf[j & 1][wr];

      // (1) B operands of this step.
      float4 hb[SPLIT ? 1 : RB * NT];
      uint4 bh[SPLIT ? RB * NOTH : 1], bl[SPLIT ? RB * NOTH : 1];
      if constexpr (!SPLIT) {
        if constexpr (NT == 1) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) hb[rb] = make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
        } else {
#pragma unroll
          for (int i = 0; i < RB * NT; ++i) hb[i] = *(const float4*)&xr[(i * 64 + lane) * 4];
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          // partner half of the own chunk (a single tile has none: those k-slots stay zero)
          if constexpr (NT > 1) {
            const uint2 ph = ((const uint2*)xr)[phi_off[rb]];
            hq[rb].z = ph.x;
            hq[rb].w = ph.y;
            if constexpr (MATH != MATH_BF16) {
              const uint2 pl = ((const uint2*)xbuf[j & 1][wr])[plo_off[rb]];
              lq[rb].z = pl.x;
              lq[rb].w = pl.y;
            }
          }
#pragma unroll
          for (int i = 0; i < NCH - 1; ++i) {
            const int cc = i < co ? i : i + 1;
            const int base = (rb * NCH + cc) * 4 * 128 + lane * 2;
            const uint2 h0 = *(const uint2*)&xr[base], h1 = *(const uint2*)&xr[base + 128];
            bh[rb * NOTH + i] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            if constexpr (MATH != MATH_BF16) {
              const uint2 l0 = *(const uint2*)&xr[base + 256], l1 = *(const uint2*)&xr[base + 384];
              bl[rb * NOTH + i] = make_uint4(l0.x, l0.y, l1.x, l1.y);
            }
          }
        }
      }
      float vterm = 0.0f, ygrp = 0.0f;
      if constexpr (MODE == MODE_FWD && SPLIT) {
        // v of steps t-4 .. t-1 for the readout finished at this step (j % 4 == 0); at j == 0 they
        // are the last four of the previous chunk.
        if (j % 4 == 0)
          vterm = (j == 0 ? stage[cb ^ 1] + (TC - 4) * St::STEP : stage[cb] + (j - 4) * St::STEP)[vlane];
      }
      // Keep every LDS read above issued before the work below, so that their latencies overlap.
      __builtin_amdgcn_sched_barrier(0);

      // Readout of step t-1 (split modes) while those reads are in flight: the q-weighted sum of the
      // transposed tile (broadcast of q within each quad of lanes), and every fourth step the
      // cross-row reduction and store of four steps.  Nothing is stored for t = 0: its offsets are
      // moved past the end.
      if constexpr (MODE == MODE_FWD && SPLIT) {
        float x = 0.0f;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const float4 qq = q_rows(qprev[rb]);
          x = rb == 0 ? qq.x * yT[rb][0] : __builtin_fmaf(qq.x, yT[rb][0], x);
          x = __builtin_fmaf(qq.y, yT[rb][1], x);
          x = __builtin_fmaf(qq.z, yT[rb][2], x);
          x = __builtin_fmaf(qq.w, yT[rb][3], x);
        }
        xq[(j + 3) & 3] = x;
        if (j % 4 == 0) ygrp = reduce_rows4(xq[0], xq[1], xq[2], xq[3]);  // finished after the publish
      }
      __builtin_amdgcn_sched_barrier(0);

      // (2) Contraction acc = (c k_t) v_t^T + W'^T H^T.
      f32x4 acc[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc[rb] = kv[rb];
      if constexpr (!SPLIT) {
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const float4 h4 = hb[rb * NT + tt];
            acc[rb] = mfma_f32(wA[tt * 4 + 0], h4.x, acc[rb]);
            acc[rb] = mfma_f32(wA[tt * 4 + 1], h4.y, acc[rb]);
            acc[rb] = mfma_f32(wA[tt * 4 + 2], h4.z, acc[rb]);
            acc[rb] = mfma_f32(wA[tt * 4 + 3], h4.w, acc[rb]);
          }
        }
      } else {
        auto contract = [&](int rb, const uint4& Ahi, const uint4& Alo, const uint4& h, const uint4& l) {
          if constexpr (MATH == MATH_F16X3) {
            acc[rb] = mfma_f16(Ahi, h, acc[rb]);
            acc[rb] = mfma_f16(Alo, h, acc[rb]);
            acc[rb] = mfma_f16(Ahi, l, acc[rb]);
          } else if constexpr (MATH == MATH_BF16X3) {
            acc[rb] = mfma_bf16(Ahi, h, acc[rb]);
            acc[rb] = mfma_bf16(Alo, h, acc[rb]);
            acc[rb] = mfma_bf16(Ahi, l, acc[rb]);
          } else {
            acc[rb] = mfma_bf16(Ahi, h, acc[rb]);
          }
        };
        if constexpr (PACK1) {
          const uint4 a1 = make_uint4(wOwnHi.x, wOwnHi.y, wOwnHi.x, wOwnHi.y);  // [W_hi | W_hi]
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            if constexpr (MATH == MATH_F16X3) {
              acc[rb] = mfma_f16(a1, hq[rb], acc[rb]);
              acc[rb] = mfma_f16(wOwnLo, hq[rb], acc[rb]);  // [W_lo | 0]
            } else {
              acc[rb] = mfma_bf16(a1, hq[rb], acc[rb]);
              acc[rb] = mfma_bf16(wOwnLo, hq[rb], acc[rb]);
            }
          }
        } else {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) contract(rb, wOwnHi, wOwnLo, hq[rb], lq[rb]);
#pragma unroll
          for (int i = 0; i < NCH - 1; ++i)
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) contract(rb, wOthHi[i], wOthLo[i], bh[rb * NOTH + i], bl[rb * NOTH + i]);
        }
      }

      // Next step's inputs (the stage record of step t+1 is complete, see above; past the last
      // step this reads a stale record that is never used).
      const StepIn<RB, SPLIT> nxt =
          read_step<V, RB, SPLIT>(j + 1 == TC ? stage[cb ^ 1] : stage[cb] + (j + 1) * St::STEP, so);

      // (3) tanh + gate blend: H = f H + (1-f)(1 - 2r) = fma(-2(1-f), r, fma(f, H, 1-f)).
      const float gf = cur.gf, m2g = cur.m2g;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float keep = __builtin_fmaf(cur.f, H[rb][r], gf);
          H[rb][r] = __builtin_fmaf(m2g, tanh_recip(acc[rb][r]), keep);
        }
      }
      publish((j + 1) & 1);
      // The work below fills the wait for that write; keep it after the write and before the barrier.
      __builtin_amdgcn_sched_barrier(0);

      // (4) Readout of step t and the rank-1 term of step t+1, in the shadow of the write.
      if constexpr (MODE == MODE_FWD) {
        if constexpr (SPLIT) {
          if (j % 4 == 0) {
            const float yv = __builtin_fmaf(wrv, vterm, ygrp);
            if constexpr (YRED) {
              if (j > 0 || c0 > 0) ykeep(t - 4, yv);
            } else {
              const uint32_t off = (j > 0 || c0 > 0) ? ylane + (uint32_t)((t - 4) * ystep * 4) : kBufferDrop;
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yres, off, 0, 0);
            }
          }
          // Transposing MFMAs: yT at lane (g, j) = H_t[row 16rb + 4g + r][col 16w + j] (hi + lo),
          // used by the next step.
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            const uint2 oh = make_uint2(hq[rb].x, hq[rb].y), ol = make_uint2(lq[rb].x, lq[rb].y);
            if constexpr (PACK1) {
              // [hi | lo] against the identity twice (hi + lo is exact in fp32)
              const uint4 bs2 = make_uint4(bsel.x, bsel.y, bsel.x, bsel.y);
              if constexpr (MATH == MATH_F16X3) yT[rb] = mfma_f16(hq[rb], bs2, zero4);
              else yT[rb] = mfma_bf16(hq[rb], bs2, zero4);
            } else if constexpr (MATH == MATH_F16X3) {
              yT[rb] = mfma16_f16(ol, bsel, mfma16_f16(oh, bsel, zero4));
            } else if constexpr (MATH == MATH_BF16X3) {
              yT[rb] = mfma16_bf16(ol, bsel, mfma16_bf16(oh, bsel, zero4));
            } else {
              yT[rb] = mfma16_bf16(oh, bsel, zero4);
            }
            if constexpr (StepIn<RB, SPLIT>::Q4) qprev[rb] = cur.q4[rb];
            else qprev[rb].x = cur.qn[rb];
          }
        } else {
          float x[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float sacc = H[0][r] * cur.qn[0];
#pragma unroll
            for (int rb = 1; rb < RB; ++rb) sacc = __builtin_fmaf(H[rb][r], cur.qn[rb], sacc);
            x[r] = sacc;
          }
          float yv = row16_sum4(x[0], x[1], x[2], x[3], lane);
          yv = __builtin_fmaf(wrv, cur.vcol, yv);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yres, ylane + (uint32_t)(t * ystep * 4), 0, 0);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) kv[rb] = mfma_f32(nxt.av, nxt.bk[rb], zero4);
      __builtin_amdgcn_sched_barrier(0);

      // With one 16-column tile per row group nothing is exchanged, so the only barriers are the
      // two around the stage-ring write (every wave has finished the previous chunk's reads of that
      // buffer before it is overwritten, and sees the new records after); a single-wave workgroup's
      // own LDS writes and reads are ordered and need none.
      if (j == TC - 2) {
        if constexpr (NT == 1 && RW > 1) lds_barrier();
        pre.store(stage[cb ^ 1], tid);
      }
      if constexpr (NT > 1) {
        lds_barrier();
      } else if constexpr (RW > 1) {
        if (j == TC - 2) lds_barrier();
      }
      if (j == TC - 2) {
        const int t_next = c0 + 2 * TC;  // first step of the chunk after the one just staged
        if (t_next < a.T) pre.load(a, b, nh, row0_wg, t_next, tid);
        // The previous chunk's readout groups are all kept (its last one at this chunk's step 0).
        if (c0 > 0) ysum(c0 - TC);
      }
      cur = nxt;
    }
  };

  for (int c0 = 0; c0 < a.T; c0 += 2 * TC) {
    run_chunk(std::integral_constant<int, 0>{}, c0);
    if (c0 + TC < a.T) run_chunk(std::integral_constant<int, 1>{}, c0 + TC);
  }

  // Readout of the last group of four steps (split modes).
  if constexpr (MODE == MODE_FWD && SPLIT) {
    const int tp = (a.T + TC - 1) / TC * TC;  // steps run, a multiple of TC
    if (tp > 0) {
      const int cbl = (tp / TC - 1) & 1;      // stage buffer of the last chunk
      float x = 0.0f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float4 qq = q_rows(qprev[rb]);
        x = __builtin_fmaf(qq.x, yT[rb][0], x);
        x = __builtin_fmaf(qq.y, yT[rb][1], x);
        x = __builtin_fmaf(qq.z, yT[rb][2], x);
        x = __builtin_fmaf(qq.w, yT[rb][3], x);
      }
      xq[3] = x;
      float yv = reduce_rows4(xq[0], xq[1], xq[2], xq[3]);
      yv = __builtin_fmaf(wrv, stage[cbl][(TC - 4) * St::STEP + vlane], yv);
      if constexpr (YRED) {
        ykeep(tp - 4, yv);
        lds_barrier();
        ysum(tp - TC);
      } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yres, ylane + (uint32_t)((tp - 4) * ystep * 4), 0,
                                              0);
      }
    }
  }

  if (a.H_T) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      *(float4*)(a.H_T + state_base + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g) =
          make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
  }
}

// Forward scan with its readout and input staging in waves of their own (MODE_FWD of the split
// contractions, one row group).  The workgroup has NT chain waves, which carry the recurrence exactly
// as m2rnn_scan_fwd_kernel does (exchange reads, contraction, tanh and gate blend, publish of the
// split state, the next step's rank-1 term), and NT readout waves, one per value tile, which
//   - read the published split tile of H_{t-1} at step t (from the same exchange buffer the chain
//     reads at that step), transpose it with one MFMA against the identity, form its q-weighted
//     row sums, and every four steps reduce across rows and store y (or the partial plane), and
//   - stage the next chunk of q, k, v, f from HBM into the LDS ring.
// Both roles meet at the one LDS barrier per step.  With two waves on every SIMD, the scheduler
// fills one wave's waits (barrier, LDS round trip, MFMA latency) with the other's instructions, and
// the chain waves no longer issue the readout and staging work at all.  The arithmetic is
// m2rnn_scan_fwd_kernel's, operation for operation, except that the readout's transpose is one MFMA
// where that kernel issues two (hi, then lo); hi + lo is exact in fp32, so the two give the same bits.
template <int V, int RB, int MATH, bool BF16IN>
__global__ void __launch_bounds__(2 * 64 * (V / 16)) m2rnn_scan_fwd_ro_kernel(const FwdArgs a) {
  using Sh = FwdShape<V, 1>;
  using St = Stage<V, RB>;
  constexpr int NT = Sh::NT;
  constexpr int TC = Sh::TC_RO;
  constexpr int ROWS = 16 * RB;
  constexpr int NCH = NT / 2;  // 32-wide contraction chunks
  constexpr int NOTH = NCH > 1 ? NCH - 1 : 1;
  static_assert(MATH != MATH_F32 && NT >= 2 && NT % 2 == 0, "split contractions with an even tile count");
  static_assert(TC % 4 == 0, "readout groups of four steps do not straddle chunks");

  __shared__ __attribute__((aligned(16))) float stage[2][TC * St::STEP];
  // Exchange buffer by step parity: [2][RB][NCH][hi|lo][half][64 lanes][2 dwords], as in
  // m2rnn_scan_fwd_kernel.
  constexpr int XWORDS = RB * NCH * 2 * 64 * 4;
  __shared__ __attribute__((aligned(16))) uint32_t xbuf[2][XWORDS];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const bool chain = wave < NT;  // uniform in a wave
  const int w = chain ? wave : wave - NT;  // value tile of this wave
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
  const int row0 = s * ROWS;
  const long KV = (long)a.K * V;
  const long state_base = ((long)b * a.N + nh) * KV;

  if (chain) {
    // ---------------- chain waves: the recurrence ----------------
    const float* Wn = a.W + (long)nh * V * V;
    const int col = 16 * w + n;
    const int co = w >> 1;  // own chunk
    uint4 wOwnHi, wOwnLo, wOthHi[NOTH], wOthLo[NOTH];
    auto wchunk = [&](int t_lo, int t_hi, uint4& hi, uint4& lo) {
      float wv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tile = (i >> 2) ? t_hi : t_lo;
        wv[i] = opaque1(kTwoLog2e * Wn[(16 * tile + 4 * g + (i & 3)) * V + col]);
      }
      uint32_t h[4], l[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float x0 = wv[2 * i], x1 = wv[2 * i + 1];
        if constexpr (MATH == MATH_F16X3) {
          h[i] = pack_f16(x0, x1);
          l[i] = pack_f16(x0 - f16_lo_to_f32(h[i]), x1 - f16_hi_to_f32(h[i]));
        } else {
          h[i] = pack_bf16(x0, x1);
          l[i] = pack_bf16(x0 - bf16_lo_to_f32(h[i]), x1 - bf16_hi_to_f32(h[i]));
        }
      }
      hi = make_uint4(h[0], h[1], h[2], h[3]);
      lo = make_uint4(l[0], l[1], l[2], l[3]);
    };
    wchunk(w, w ^ 1, wOwnHi, wOwnLo);
#pragma unroll
    for (int i = 0; i < NCH - 1; ++i) {
      const int cc = i < co ? i : i + 1;
      wchunk(2 * cc, 2 * cc + 1, wOthHi[i], wOthLo[i]);
    }

    float H[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const long off = state_base + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g;
      if (a.H0) {
        const float4 h = *(const float4*)(a.H0 + off);
        H[rb][0] = h.x; H[rb][1] = h.y; H[rb][2] = h.z; H[rb][3] = h.w;
      } else {
        H[rb][0] = H[rb][1] = H[rb][2] = H[rb][3] = 0.0f;
      }
    }
    uint4 hq[RB], lq[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) hq[rb] = lq[rb] = make_uint4(0, 0, 0, 0);
    auto publish = [&](int buf) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        uint32_t h0, h1, l0, l1;
        opaque4(H[rb]);  // the split is a function of the fp32 state alone
        split_pair<MATH>(H[rb][0], H[rb][1], h0, l0);
        split_pair<MATH>(H[rb][2], H[rb][3], h1, l1);
        hq[rb].x = h0;
        hq[rb].y = h1;
        lq[rb].x = l0;
        lq[rb].y = l1;
        const int base = ((rb * NCH + (w >> 1)) * 4 + (w & 1)) * 128 + lane * 2;
        *(uint2*)&xbuf[buf][base] = make_uint2(h0, h1);
        if constexpr (MATH != MATH_BF16) *(uint2*)&xbuf[buf][base + 256] = make_uint2(l0, l1);
      }
    };
    // Per-step inputs of the chain: the gate scalars and the rank-1 operands.
    const int o_av = g == 0 ? St::OV + 16 * w + n : 3;
    int o_bk[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o_bk[rb] = g == 0 ? St::OK + 16 * rb + n : 3;
    struct In {
      float f, gf, m2g, av;
      float bk[RB];
    };
    auto read_in = [&](const float* st) {
      In r;
      const float4 gate = *(const float4*)st;
      r.f = gate.x;
      r.gf = gate.y;
      r.m2g = gate.z;
      r.av = st[o_av];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) r.bk[rb] = st[o_bk[rb]];
      return r;
    };
    int phi_off[RB], plo_off[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      phi_off[rb] = ((rb * NCH + co) * 4 + ((w & 1) ^ 1)) * 64 + lane;
      plo_off[rb] = phi_off[rb] + 128;
      asm volatile("" : "+v"(plo_off[rb]));
    }

    publish(0);
    lds_barrier();  // the readout waves have staged chunk 0; every wave's H0 tile is published

    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    In cur = read_in(stage[0]);
    f32x4 kv[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) kv[rb] = mfma_f32(cur.av, cur.bk[rb], zero4);

    auto run_chunk = [&](auto CB, int c0) __attribute__((always_inline)) {
      constexpr int cb = decltype(CB)::value;
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        const int t = c0 + j;
        if ((j % 8) == 0 && a.ckpt != nullptr) {
          if (t % a.seg == 0 && t < a.T) {
            float* dst = a.ckpt + ((long)(b * a.N + nh) * a.nck + a.ck0 + t / a.seg) * KV;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb)
              *(float4*)(dst + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g) =
                  make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
          }
        }
        const uint32_t* xr = xbuf[j & 1];
        // (1) B operands: the partner half of the own chunk and the other chunks.
        uint4 bh[RB * NOTH], bl[RB * NOTH];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const uint2 ph = ((const uint2*)xr)[phi_off[rb]];
          hq[rb].z = ph.x;
          hq[rb].w = ph.y;
          if constexpr (MATH != MATH_BF16) {
            const uint2 pl = ((const uint2*)xbuf[j & 1])[plo_off[rb]];
            lq[rb].z = pl.x;
            lq[rb].w = pl.y;
          }
#pragma unroll
          for (int i = 0; i < NCH - 1; ++i) {
            const int cc = i < co ? i : i + 1;
            const int base = (rb * NCH + cc) * 4 * 128 + lane * 2;
            const uint2 h0 = *(const uint2*)&xr[base], h1 = *(const uint2*)&xr[base + 128];
            bh[rb * NOTH + i] = make_uint4(h0.x, h0.y, h1.x, h1.y);
            if constexpr (MATH != MATH_BF16) {
              const uint2 l0 = *(const uint2*)&xr[base + 256], l1 = *(const uint2*)&xr[base + 384];
              bl[rb * NOTH + i] = make_uint4(l0.x, l0.y, l1.x, l1.y);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        // (2) contraction acc = (c k_t) v_t^T + W'^T H^T
        f32x4 acc[RB];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) acc[rb] = kv[rb];
        auto contract = [&](int rb, const uint4& Ahi, const uint4& Alo, const uint4& h, const uint4& l) {
          if constexpr (MATH == MATH_F16X3) {
            acc[rb] = mfma_f16(Ahi, h, acc[rb]);
            acc[rb] = mfma_f16(Alo, h, acc[rb]);
            acc[rb] = mfma_f16(Ahi, l, acc[rb]);
          } else if constexpr (MATH == MATH_BF16X3) {
            acc[rb] = mfma_bf16(Ahi, h, acc[rb]);
            acc[rb] = mfma_bf16(Alo, h, acc[rb]);
            acc[rb] = mfma_bf16(Ahi, l, acc[rb]);
          } else {
            acc[rb] = mfma_bf16(Ahi, h, acc[rb]);
          }
        };
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) contract(rb, wOwnHi, wOwnLo, hq[rb], lq[rb]);
#pragma unroll
        for (int i = 0; i < NCH - 1; ++i)
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) contract(rb, wOthHi[i], wOthLo[i], bh[rb * NOTH + i], bl[rb * NOTH + i]);
        // the next step's inputs (complete one barrier before this step; past the last step a stale
        // record that is never used)
        const In nxt = read_in(j + 1 == TC ? stage[cb ^ 1] : stage[cb] + (j + 1) * St::STEP);
        // (3) tanh + gate blend, publish
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float keep = __builtin_fmaf(cur.f, H[rb][r], cur.gf);
            H[rb][r] = __builtin_fmaf(cur.m2g, tanh_recip(acc[rb][r]), keep);
          }
        }
        publish((j + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
        // (4) the rank-1 term of step t+1 in the shadow of the write
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) kv[rb] = mfma_f32(nxt.av, nxt.bk[rb], zero4);
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        cur = nxt;
      }
    };
    for (int c0 = 0; c0 < a.T; c0 += 2 * TC) {
      run_chunk(std::integral_constant<int, 0>{}, c0);
      if (c0 + TC < a.T) run_chunk(std::integral_constant<int, 1>{}, c0 + TC);
    }
    if (a.H_T) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        *(float4*)(a.H_T + state_base + (long)(row0 + 16 * rb + n) * V + 16 * w + 4 * g) =
            make_float4(H[rb][0], H[rb][1], H[rb][2], H[rb][3]);
    }
  } else {
    // ---------------- readout waves: y and the staging of the inputs ----------------
    const int rtid = tid - Sh::NTH;  // thread index among the readout waves
    const int ycol = 16 * w + n;
    const float wrv = a.S == 1 ? a.w_r[(long)nh * V + ycol] : 0.0f;
    const int ystep = a.N * V;
    const long plane = (long)a.B * a.Tp * a.N * V;
    float* ybase = a.y + (a.S > 1 ? (long)s * plane : 0) + ((long)b * a.Tp * a.N + nh) * V;
    const __amdgpu_buffer_rsrc_t yres =
        __builtin_amdgcn_make_buffer_rsrc(ybase, (short)0, (a.T * a.N - nh) * V * 4, kBufferRsrcWord3);
    const uint32_t ylane = (uint32_t)((g * ystep + ycol) * 4);
    const int vlane = g * St::STEP + St::OV + ycol;  // v[ycol] of step g of a group, in the stage
    const int qlane = St::OQ + 4 * g;                // q of rows 4g .. 4g+3 (+ 16 rb)
    uint2 bsel;
    {
      const uint32_t one = MATH == MATH_F16X3 ? 0x3C00u : 0x3F80u;
      uint32_t e16[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) e16[e] = (n == 4 * g + e) ? one : 0u;
      bsel = make_uint2(e16[0] | (e16[1] << 16), e16[2] | (e16[3] << 16));
    }
    const uint4 bsel2 = make_uint4(bsel.x, bsel.y, bsel.x, bsel.y);
    int tile_off[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) tile_off[rb] = ((rb * NCH + (w >> 1)) * 4 + (w & 1)) * 128 + lane * 2;
    const f32x4 zero4 = {0.0f, 0.0f, 0.0f, 0.0f};
    float xq[4] = {0.0f, 0.0f, 0.0f, 0.0f};

    // Readout of step tr (state H_tr in exchange buffer xb, q_tr in record `st`): the q-weighted sum of
    // the transposed tile over this lane's rows, kept for the group of four steps.
    auto readout = [&](const uint32_t* xb, const float* st, int slot) __attribute__((always_inline)) {
      f32x4 yT[RB];
      float4 q4[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const uint2 oh = *(const uint2*)&xb[tile_off[rb]];
        uint2 ol = make_uint2(0, 0);
        if constexpr (MATH != MATH_BF16) ol = *(const uint2*)&xb[tile_off[rb] + 256];
        q4[rb] = *(const float4*)(st + qlane + 16 * rb);
        // One 16x16x32 MFMA with hi and lo side by side on the contraction index and the identity
        // twice: hi + lo is exact in fp32, so this gives the bits of the two 16x16x16 transposes
        // (hi, then + lo) for one MFMA issue instead of two.
        const uint4 hl4 = make_uint4(oh.x, oh.y, ol.x, ol.y);
        if constexpr (MATH == MATH_F16X3) {
          yT[rb] = mfma_f16(hl4, bsel2, zero4);
        } else if constexpr (MATH == MATH_BF16X3) {
          yT[rb] = mfma_bf16(hl4, bsel2, zero4);
        } else {
          yT[rb] = mfma16_bf16(oh, bsel, zero4);
        }
      }
      float x = 0.0f;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        x = rb == 0 ? q4[rb].x * yT[rb][0] : __builtin_fmaf(q4[rb].x, yT[rb][0], x);
        x = __builtin_fmaf(q4[rb].y, yT[rb][1], x);
        x = __builtin_fmaf(q4[rb].z, yT[rb][2], x);
        x = __builtin_fmaf(q4[rb].w, yT[rb][3], x);
      }
      xq[slot] = x;
    };
    // The group of four steps starting at step tg, its v records starting at `vst`: one cross-row
    // reduction leaves lane (g, j) with y[tg + g][16w + j].
    auto store_group = [&](int tg, const float* vst) __attribute__((always_inline)) {
      float yv = reduce_rows4(xq[0], xq[1], xq[2], xq[3]);
      yv = __builtin_fmaf(wrv, vst[vlane], yv);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(yv), yres, ylane + (uint32_t)(tg * ystep * 4), 0, 0);
    };

    ChunkRegs<V, RB, BF16IN, 1, TC> pre;
    pre.load(a, b, nh, row0, 0, rtid);
    pre.store(stage[0], rtid);
    if (a.T > TC) pre.load(a, b, nh, row0, TC, rtid);
    lds_barrier();

    auto run_chunk = [&](auto CB, int c0) __attribute__((always_inline)) {
      constexpr int cb = decltype(CB)::value;
#pragma unroll
      for (int j = 0; j < TC; ++j) {
        const int t = c0 + j;
        // readout of step t-1 (published at step t-1 into the buffer the chain reads now)
        if (j > 0 || c0 > 0) {
          const float* st = j == 0 ? stage[cb ^ 1] + (TC - 1) * St::STEP : stage[cb] + (j - 1) * St::STEP;
          readout(xbuf[j & 1], st, (j + 3) & 3);
          if (j % 4 == 0) store_group(t - 4, j == 0 ? stage[cb ^ 1] + (TC - 4) * St::STEP : stage[cb] + (j - 4) * St::STEP);
        }
        if (j == TC - 2) pre.store(stage[cb ^ 1], rtid);
        lds_barrier();
        if (j == TC - 2) {
          const int t_next = c0 + 2 * TC;  // first step of the chunk after the one just staged
          if (t_next < a.T) pre.load(a, b, nh, row0, t_next, rtid);
        }
      }
    };
    for (int c0 = 0; c0 < a.T; c0 += 2 * TC) {
      run_chunk(std::integral_constant<int, 0>{}, c0);
      if (c0 + TC < a.T) run_chunk(std::integral_constant<int, 1>{}, c0 + TC);
    }
    // the last step of the last chunk, and its group
    const int tp = (a.T + TC - 1) / TC * TC;
    if (tp > 0) {
      const int cbl = (tp / TC - 1) & 1;
      readout(xbuf[tp & 1], stage[cbl] + (TC - 1) * St::STEP, 3);
      store_group(tp - 4, stage[cbl] + (TC - 4) * St::STEP);
    }
  }
}

// y = sum_s partial_s + w_r (.) v, elementwise over [B,T,N,V] (4 elements per thread): for batch
// entry blockIdx.y, the `count` elements from off0 + blockIdx.y * bstride of y and v, and from
// poff0 + blockIdx.y * pbstride of each plane (the whole tensor: one row of blocks, zero offsets
// and strides; a time segment of every batch entry: planes laid out like y, or holding that
// segment only).  The planes are read once and y written once: non-temporal accesses keep them
// from displacing each other in the caches (258 -> 224 us at B2 N32 T16384 K=V=64, S = 4).
template <bool BF16IN>
__global__ void __launch_bounds__(256) m2rnn_fwd_finish_kernel(const float* __restrict__ part, int S,
                                                                long plane, long poff0, long pbstride,
                                                                const void* __restrict__ v,
                                                                const float* __restrict__ w_r, int N, int V,
                                                                float* __restrict__ y, long count, long bstride,
                                                                long off0) {
  const long i4 = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i4 * 4 >= count) return;
  const long i = off0 + (long)blockIdx.y * bstride + i4 * 4;
  const long pi = poff0 + (long)blockIdx.y * pbstride + i4 * 4;
  f32x4 acc = __builtin_nontemporal_load((const f32x4*)(part + pi));
  for (int s = 1; s < S; ++s) acc += __builtin_nontemporal_load((const f32x4*)(part + (long)s * plane + pi));
  const int colv = (int)(i % V);
  const int nh = (int)((i / V) % N);
  const float4 wr = *(const float4*)(w_r + (long)nh * V + colv);
  float4 vv;
  if constexpr (BF16IN) {
    const uint2 raw = *(const uint2*)((const char*)v + i * 2);
    vv = make_float4(bf16_lo_to_f32(raw.x), bf16_hi_to_f32(raw.x), bf16_lo_to_f32(raw.y), bf16_hi_to_f32(raw.y));
  } else {
    vv = *(const float4*)((const float*)v + i);
  }
  acc[0] = __builtin_fmaf(wr.x, vv.x, acc[0]);
  acc[1] = __builtin_fmaf(wr.y, vv.y, acc[1]);
  acc[2] = __builtin_fmaf(wr.z, vv.z, acc[2]);
  acc[3] = __builtin_fmaf(wr.w, vv.w, acc[3]);
  __builtin_nontemporal_store(acc, (f32x4*)(y + i));
}

}  // namespace m2rnn
