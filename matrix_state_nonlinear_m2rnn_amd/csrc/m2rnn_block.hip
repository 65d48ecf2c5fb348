// C entry points for the steps on either side of the recurrence (gate, output gate + RMSNorm,
// causal conv4 + SiLU), declared in include/m2rnn.h.
#include <hip/hip_runtime.h>

#include "../../include/m2rnn.h"
#include "m2rnn_block_kernels.h"
#include "m2rnn_block_launch.h"

using namespace m2rnn;

namespace m2rnn {
// Status of a HIP call, recording a failure for m2rnn_last_hip_error() (defined with it).
int record_hip_status(hipError_t e);
}  // namespace m2rnn

namespace {

int status(hipError_t e) { return record_hip_status(e); }

bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

size_t round_up256(size_t x) { return (x + 255) & ~(size_t)255; }

unsigned grid_for(long count) {
  long blocks = (count + kBlkThreads - 1) / kBlkThreads;
  if (blocks > 65536) blocks = 65536;  // grid-stride beyond that
  return (unsigned)(blocks > 0 ? blocks : 1);
}

constexpr int kNormRowsPer = 16;      // rows per workgroup of the RMSNorm backward
constexpr long kGateMaxParts = 1024;  // workgroups (partial sums) of the gate backward
constexpr int kSlice = 64;            // rows per slice of the partial-sum reduction tree
// features per row of the RMSNorm: 8 groups of 4 per thread
constexpr int kNormMaxD = 4 * kBlkThreads * 8;
static_assert(kNormMaxD == kNormMaxFeatures, "the recurrence's entry points check rows against kNormMaxFeatures");

long ceil_div(long a, long b) { return (a + b - 1) / b; }

// Floats of scratch that reduce_rows needs for `parts` rows of M columns.
size_t reduce_scratch(long parts, long M) { return (size_t)2 * ceil_div(parts, kSlice) * M; }

// Sums `parts` rows of M floats (row p at part + p * stride) into one row by a fixed tree of
// kSlice-row slices; the last level writes columns j < M0 to out0[j] and the others to
// out1[j - M0] (dropped when out1 is null).  `scratch` holds reduce_scratch(parts, M) floats.
void reduce_rows(const float* part, long parts, long M, long stride, float* out0, long M0, float* out1, float* scratch,
                 hipStream_t s) {
  float* bufs[2] = {scratch, scratch + ceil_div(parts, kSlice) * M};
  const float* src = part;
  long n = parts, src_stride = stride;
  int which = 0;
  const unsigned gx = (unsigned)ceil_div(M, kBlkThreads);
  while (n > kSlice) {
    const long m = ceil_div(n, kSlice);
    hipLaunchKernelGGL(m2rnn_sum_slices_kernel, dim3(gx, (unsigned)m), dim3(kBlkThreads), 0, s, src, (int)n, M,
                       src_stride, kSlice, bufs[which], M, (float*)nullptr);
    src = bufs[which];
    src_stride = M;
    n = m;
    which ^= 1;
  }
  hipLaunchKernelGGL(m2rnn_sum_slices_kernel, dim3(gx, 1), dim3(kBlkThreads), 0, s, src, (int)n, M, src_stride,
                     (int)(n > 0 ? n : 1), out0, M0, out1);
}

int check_gate(int64_t B, int64_t T, int64_t N) {
  if (B < 0 || T < 0 || N < 0) return M2RNN_EINVAL;
  if ((double)B * T * N > 2147483647.0 * 64.0) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

int check_norm(int64_t rows, int64_t D, int gz_dtype, float eps) {
  if (rows < 0 || D <= 0) return M2RNN_EINVAL;
  if (gz_dtype != M2RNN_DTYPE_F32 && gz_dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (!(eps >= 0.0f) || eps > 1e30f) return M2RNN_EINVAL;
  if (D % 4 != 0 || D > kNormMaxD) return M2RNN_EUNSUPPORTED;
  if (rows > 2147483647) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

int check_conv(int64_t B, int64_t T, int64_t C, int dtype) {
  if (B < 0 || T < 0 || C <= 0) return M2RNN_EINVAL;
  if (dtype != M2RNN_DTYPE_F32 && dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (C % 4 != 0) return M2RNN_EUNSUPPORTED;
  if (B > 2147483647 || T > 2147483647 || C > 2147483647) return M2RNN_EUNSUPPORTED;
  // the kernels number their waves with an int
  if ((double)B * ceil_div(T, kConvChunkMin) * ceil_div(C / 4, 64) > 2147483647.0) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

// Gate backward workspace: the partials [parts][2N] and their reduction scratch, or (more than
// kBlkThreads heads) the per-element dalpha terms.
size_t gate_ws_bytes(int64_t B, int64_t T, int64_t N) {
  if (N <= kBlkThreads)
    return round_up256((size_t)2 * N * kGateMaxParts * sizeof(float)) +
           round_up256(reduce_scratch(kGateMaxParts, 2 * N) * sizeof(float));
  return round_up256((size_t)B * T * N * sizeof(float));
}

size_t norm_ws_bytes(int64_t rows, int64_t D) {
  const long parts = ceil_div(rows, kNormRowsPer);
  return round_up256((size_t)parts * D * sizeof(float)) + round_up256(reduce_scratch(parts, D) * sizeof(float));
}

// Steps per thread of the conv kernels: `base`, halved down to kConvChunkMin while the grid (one
// wave per batch entry, chunk and 64 channel groups) would hold fewer than kConvMinWaves waves.
int conv_chunk(int64_t B, int64_t T, int64_t C, int base) {
  int chunk = base;
  while (chunk > kConvChunkMin && B * ceil_div(T, chunk) * ceil_div(C / 4, 64) < kConvMinWaves) chunk /= 2;
  return chunk;
}

size_t conv_ws_bytes(int64_t B, int64_t T, int64_t C) {
  const long parts = (long)B * ceil_div(T, conv_chunk(B, T, C, kConvChunkBwd));
  return round_up256((size_t)parts * 5 * C * sizeof(float)) + round_up256(reduce_scratch(parts, 5 * C) * sizeof(float));
}

// Workgroups of the conv kernels: one wave per (b, chunk of `chunk` steps, 64 groups of 4 channels).
long conv_blocks(int64_t B, int64_t T, int64_t C, int chunk) {
  return ceil_div(B * ceil_div(T, chunk) * ceil_div(C / 4, 64), kBlkThreads / 64);
}

}  // namespace

extern "C" {

int m2rnn_gate_fwd(int64_t B, int64_t T, int64_t N, const float* a, const float* alpha, const float* beta, float* f,
                   void* stream) {
  int st = check_gate(B, T, N);
  if (st) return st;
  const long count = (long)B * T * N;
  if (count == 0) return M2RNN_OK;
  if (!a || !alpha || !beta || !f || !al4(a) || !al4(alpha) || !al4(beta) || !al4(f)) return M2RNN_EINVAL;
  hipLaunchKernelGGL(m2rnn_gate_fwd_kernel, dim3(grid_for(count)), dim3(kBlkThreads), 0, (hipStream_t)stream, a,
                     alpha, beta, count, (int)N, f);
  return status(hipGetLastError());
}

int m2rnn_gate_bwd_workspace_size(int64_t B, int64_t T, int64_t N, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_gate(B, T, N);
  if (st) return st;
  *bytes = gate_ws_bytes(B, T, N);
  return M2RNN_OK;
}

int m2rnn_gate_bwd(int64_t B, int64_t T, int64_t N, const float* a, const float* alpha, const float* beta,
                   const float* df, float* da, float* dalpha, float* dbeta, void* workspace, size_t workspace_bytes,
                   void* stream) {
  int st = check_gate(B, T, N);
  if (st) return st;
  if (N == 0) return M2RNN_OK;
  if (!alpha || !beta || !dalpha || !dbeta) return M2RNN_EINVAL;
  const long count = (long)B * T * N;
  if (count > 0 && (!a || !df || !da)) return M2RNN_EINVAL;
  const void* ps[] = {a, alpha, beta, df, da, dalpha, dbeta};
  for (const void* p : ps)
    if (p && !al4(p)) return M2RNN_EINVAL;
  const size_t need = gate_ws_bytes(B, T, N);
  if (count > 0 && (!workspace || workspace_bytes < need || !al16(workspace))) return M2RNN_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (N <= kBlkThreads && count > 0) {
    // Workgroups of a multiple of N threads, each summing a contiguous range of (b, t) rows.
    const int tb = (int)(kBlkThreads / N * N);
    const long per_block = ceil_div(ceil_div(count, kGateMaxParts), tb) * tb;
    const long parts = ceil_div(count, per_block);
    float* part = (float*)workspace;
    float* scratch = (float*)((char*)workspace + round_up256((size_t)2 * N * kGateMaxParts * sizeof(float)));
    hipLaunchKernelGGL(m2rnn_gate_bwd_part_kernel, dim3((unsigned)parts), dim3(tb), 0, s, a, alpha, beta, df, count,
                       (int)N, per_block, da, part);
    reduce_rows(part, parts, 2 * N, 2 * N, dbeta, N, dalpha, scratch, s);
    return status(hipGetLastError());
  }
  float* ga = (float*)workspace;
  if (count > 0)
    hipLaunchKernelGGL(m2rnn_gate_bwd_kernel, dim3(grid_for(count)), dim3(kBlkThreads), 0, s, a, alpha, beta, df,
                       count, (int)N, da, ga);
  hipLaunchKernelGGL(m2rnn_col_sum2_kernel, dim3((unsigned)N), dim3(kBlkThreads), 0, s, (const float*)da,
                     (const float*)ga, (long)B * T, (int)N, dbeta, dalpha);
  return status(hipGetLastError());
}

int m2rnn_out_norm_fwd(int64_t rows, int64_t D, const float* y, const void* gz, int gz_dtype, const float* gamma,
                       float eps, float* out, void* stream) {
  int st = check_norm(rows, D, gz_dtype, eps);
  if (st) return st;
  if (rows == 0) return M2RNN_OK;
  if (!y || !gz || !gamma || !out) return M2RNN_EINVAL;
  const void* ps[] = {y, gz, gamma, out};
  for (const void* p : ps)
    if (!al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  // groups of 4 features per thread: 2 up to 2048 features, else 8 (kNormMaxD)
  static_assert(kNormMaxD <= 4 * kBlkThreads * 8, "RMSNorm forward: row wider than its registers");
  const bool bf = gz_dtype == M2RNN_DTYPE_BF16;
  const auto kern = D <= 4 * kBlkThreads * 2
                        ? (bf ? &m2rnn_out_norm_fwd_kernel<true, 2> : &m2rnn_out_norm_fwd_kernel<false, 2>)
                        : (bf ? &m2rnn_out_norm_fwd_kernel<true, 8> : &m2rnn_out_norm_fwd_kernel<false, 8>);
  hipLaunchKernelGGL(kern, dim3((unsigned)rows), dim3(kBlkThreads), 0, s, y, gz, gamma, (int)D, eps, out);
  return status(hipGetLastError());
}

int m2rnn_out_norm_bwd_workspace_size(int64_t rows, int64_t D, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_norm(rows, D, M2RNN_DTYPE_F32, 0.0f);
  if (st) return st;
  *bytes = norm_ws_bytes(rows, D);
  return M2RNN_OK;
}

int m2rnn_out_norm_bwd(int64_t rows, int64_t D, const float* y, const void* gz, int gz_dtype, const float* gamma,
                       float eps, const float* dout, float* dy, float* dgz, float* dgamma, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int st = check_norm(rows, D, gz_dtype, eps);
  if (st) return st;
  if (!gamma || !dgamma) return M2RNN_EINVAL;
  if (rows > 0 && (!y || !gz || !dout || !dy || !dgz)) return M2RNN_EINVAL;
  const void* ps[] = {y, gz, gamma, dout, dy, dgz, dgamma};
  for (const void* p : ps)
    if (p && !al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const long parts = ceil_div(rows, kNormRowsPer);  // one workgroup per kNormRowsPer rows
  if (parts == 0) {
    reduce_rows(nullptr, 0, D, D, dgamma, D, nullptr, nullptr, s);
    return status(hipGetLastError());
  }
  if (!workspace || workspace_bytes < norm_ws_bytes(rows, D) || !al16(workspace)) return M2RNN_EWORKSPACE;
  float* part = (float*)workspace;
  float* scratch = (float*)((char*)workspace + round_up256((size_t)parts * D * sizeof(float)));
  const dim3 grid((unsigned)parts);
  const bool bf = gz_dtype == M2RNN_DTYPE_BF16;
  // groups of 4 features per thread, as in the forward
  const auto kern = D <= 4 * kBlkThreads * 2
                        ? (bf ? &m2rnn_out_norm_bwd_kernel<true, 2> : &m2rnn_out_norm_bwd_kernel<false, 2>)
                        : (bf ? &m2rnn_out_norm_bwd_kernel<true, 8> : &m2rnn_out_norm_bwd_kernel<false, 8>);
  hipLaunchKernelGGL(kern, grid, dim3(kBlkThreads), 0, s, y, gz, gamma, (int)D, eps, dout, (long)rows, kNormRowsPer,
                     dy, dgz, part);
  reduce_rows(part, parts, D, D, dgamma, D, nullptr, scratch, s);
  return status(hipGetLastError());
}

int m2rnn_conv4_silu_fwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w, const float* bias,
                         void* u, void* stream) {
  int st = check_conv(B, T, C, dtype);
  if (st) return st;
  const int chunk = conv_chunk(B, T, C, kConvChunkFwd);
  const long blocks = conv_blocks(B, T, C, chunk);
  if (blocks == 0) return M2RNN_OK;
  if (!x || !w || !u) return M2RNN_EINVAL;
  const void* ps[] = {x, w, bias, u};
  for (const void* p : ps)
    if (p && !al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  if (dtype == M2RNN_DTYPE_BF16)
    hipLaunchKernelGGL(m2rnn_conv4_silu_fwd_kernel<true>, dim3((unsigned)blocks), dim3(kBlkThreads), 0, s, x, w, bias,
                       (int)B, (int)T, (int)C, chunk, u);
  else
    hipLaunchKernelGGL(m2rnn_conv4_silu_fwd_kernel<false>, dim3((unsigned)blocks), dim3(kBlkThreads), 0, s, x, w, bias,
                       (int)B, (int)T, (int)C, chunk, u);
  return status(hipGetLastError());
}

int m2rnn_conv4_silu_bwd_workspace_size(int64_t B, int64_t T, int64_t C, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_conv(B, T, C, M2RNN_DTYPE_F32);
  if (st) return st;
  *bytes = conv_ws_bytes(B, T, C);
  return M2RNN_OK;
}

int m2rnn_conv4_silu_bwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w, const float* bias,
                         const float* du, float* dx, float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_conv(B, T, C, dtype);
  if (st) return st;
  if (!w || !dw) return M2RNN_EINVAL;
  const int chunk = conv_chunk(B, T, C, kConvChunkBwd);
  const long blocks = conv_blocks(B, T, C, chunk);
  if (blocks > 0 && (!x || !du || !dx)) return M2RNN_EINVAL;
  const void* ps[] = {x, w, bias, du, dx, dw, dbias};
  for (const void* p : ps)
    if (p && !al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const long parts = (long)B * ceil_div(T, chunk);
  if (parts > 0 && (!workspace || workspace_bytes < conv_ws_bytes(B, T, C) || !al16(workspace)))
    return M2RNN_EWORKSPACE;
  float* part = (float*)workspace;
  float* scratch = parts > 0 ? (float*)((char*)workspace + round_up256((size_t)parts * 5 * C * sizeof(float))) : nullptr;
  if (blocks > 0) {
    if (dtype == M2RNN_DTYPE_BF16)
      hipLaunchKernelGGL(m2rnn_conv4_silu_bwd_kernel<true>, dim3((unsigned)blocks), dim3(kBlkThreads), 0, s, x, w, bias,
                         du, (int)B, (int)T, (int)C, chunk, dx, part);
    else
      hipLaunchKernelGGL(m2rnn_conv4_silu_bwd_kernel<false>, dim3((unsigned)blocks), dim3(kBlkThreads), 0, s, x, w, bias,
                         du, (int)B, (int)T, (int)C, chunk, dx, part);
  }
  reduce_rows(part, parts, 5 * C, 5 * C, dw, 4 * C, dbias, scratch, s);
  return status(hipGetLastError());
}

}  // extern "C"

namespace m2rnn {

int launch_fwd_finish_norm(const float* part, int S, const void* v, bool v_bf16, const float* w_r, const void* gz,
                           bool gz_bf16, const float* gamma, long B, long T, long t0, long len, int D, float eps,
                           float* out, hipStream_t stream) {
  if (B == 0 || len == 0) return hipSuccess;
  const long plane = B * T * D;
  const bool wide = D > 4 * kBlkThreads * 2;
  using Kern = void (*)(const float*, int, long, const void*, const float*, const void*, const float*, int, float,
                        float*, long, long);
  static const Kern kerns[2][2][2] = {
      {{m2rnn_fwd_finish_norm_kernel<false, false, 2>, m2rnn_fwd_finish_norm_kernel<false, true, 2>},
       {m2rnn_fwd_finish_norm_kernel<true, false, 2>, m2rnn_fwd_finish_norm_kernel<true, true, 2>}},
      {{m2rnn_fwd_finish_norm_kernel<false, false, 8>, m2rnn_fwd_finish_norm_kernel<false, true, 8>},
       {m2rnn_fwd_finish_norm_kernel<true, false, 8>, m2rnn_fwd_finish_norm_kernel<true, true, 8>}}};
  hipLaunchKernelGGL(kerns[wide][v_bf16][gz_bf16], dim3((unsigned)len, (unsigned)B), dim3(kBlkThreads), 0, stream,
                     part, S, plane, v, w_r, gz, gamma, D, eps, out, T, t0);
  return hipGetLastError();
}

}  // namespace m2rnn
