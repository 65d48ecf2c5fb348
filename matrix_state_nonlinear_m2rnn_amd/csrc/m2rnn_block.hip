// C entry points for the steps on either side of the recurrence (gate, output gate + RMSNorm,
// causal conv4 + SiLU), declared in include/m2rnn.h.
#include <hip/hip_runtime.h>

#include "../../include/m2rnn.h"
#include "m2rnn_block_kernels.h"

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

constexpr int kNormRowsPer = 64;  // rows per workgroup of the RMSNorm backward

int check_gate(int64_t B, int64_t T, int64_t N) {
  if (B < 0 || T < 0 || N < 0) return M2RNN_EINVAL;
  if ((double)B * T * N > 2147483647.0 * 64.0) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

int check_norm(int64_t rows, int64_t D, int gz_dtype, float eps) {
  if (rows < 0 || D <= 0) return M2RNN_EINVAL;
  if (gz_dtype != M2RNN_DTYPE_F32 && gz_dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (!(eps >= 0.0f) || eps > 1e30f) return M2RNN_EINVAL;
  if (D % 4 != 0 || D > 4 * kBlkThreads * kNormMaxGroups) return M2RNN_EUNSUPPORTED;
  if (rows > 2147483647) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

int check_conv(int64_t B, int64_t T, int64_t C, int dtype) {
  if (B < 0 || T < 0 || C <= 0) return M2RNN_EINVAL;
  if (dtype != M2RNN_DTYPE_F32 && dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (C % 4 != 0) return M2RNN_EUNSUPPORTED;
  if (B > 2147483647 || T > 2147483647 || C > 2147483647) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

long conv_threads(int64_t B, int64_t T, int64_t C) {
  return (long)B * ((T + kConvChunk - 1) / kConvChunk) * (C / 4);
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
  *bytes = round_up256((size_t)B * T * N * sizeof(float));
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
  const size_t need = round_up256((size_t)count * sizeof(float));
  if (count > 0 && (!workspace || workspace_bytes < need || !al4(workspace))) return M2RNN_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
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
  if (gz_dtype == M2RNN_DTYPE_BF16)
    hipLaunchKernelGGL(m2rnn_out_norm_fwd_kernel<true>, dim3((unsigned)rows), dim3(kBlkThreads), 0, s, y, gz, gamma,
                       (int)D, eps, out);
  else
    hipLaunchKernelGGL(m2rnn_out_norm_fwd_kernel<false>, dim3((unsigned)rows), dim3(kBlkThreads), 0, s, y, gz, gamma,
                       (int)D, eps, out);
  return status(hipGetLastError());
}

int m2rnn_out_norm_bwd_workspace_size(int64_t rows, int64_t D, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_norm(rows, D, M2RNN_DTYPE_F32, 0.0f);
  if (st) return st;
  const long parts = (rows + kNormRowsPer - 1) / kNormRowsPer;
  *bytes = round_up256((size_t)parts * D * sizeof(float));
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
  const long parts = (rows + kNormRowsPer - 1) / kNormRowsPer;
  if (parts == 0) {
    hipLaunchKernelGGL(m2rnn_sum_parts_kernel, dim3((unsigned)((D + kBlkThreads - 1) / kBlkThreads)),
                       dim3(kBlkThreads), 0, s, (const float*)nullptr, 0, (long)D, dgamma);
    return status(hipGetLastError());
  }
  const size_t need = round_up256((size_t)parts * D * sizeof(float));
  if (!workspace || workspace_bytes < need || !al16(workspace)) return M2RNN_EWORKSPACE;
  float* part = (float*)workspace;
  if (gz_dtype == M2RNN_DTYPE_BF16)
    hipLaunchKernelGGL(m2rnn_out_norm_bwd_kernel<true>, dim3((unsigned)parts), dim3(kBlkThreads), 0, s, y, gz, gamma,
                       (int)D, eps, dout, (long)rows, kNormRowsPer, dy, dgz, part);
  else
    hipLaunchKernelGGL(m2rnn_out_norm_bwd_kernel<false>, dim3((unsigned)parts), dim3(kBlkThreads), 0, s, y, gz, gamma,
                       (int)D, eps, dout, (long)rows, kNormRowsPer, dy, dgz, part);
  hipLaunchKernelGGL(m2rnn_sum_parts_kernel, dim3((unsigned)((D + kBlkThreads - 1) / kBlkThreads)), dim3(kBlkThreads),
                     0, s, (const float*)part, (int)parts, (long)D, dgamma);
  return status(hipGetLastError());
}

int m2rnn_conv4_silu_fwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w, const float* bias,
                         void* u, void* stream) {
  int st = check_conv(B, T, C, dtype);
  if (st) return st;
  const long nth = conv_threads(B, T, C);
  if (nth == 0) return M2RNN_OK;
  if (!x || !w || !u) return M2RNN_EINVAL;
  const void* ps[] = {x, w, bias, u};
  for (const void* p : ps)
    if (p && !al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const unsigned blocks = (unsigned)((nth + kBlkThreads - 1) / kBlkThreads);
  if (dtype == M2RNN_DTYPE_BF16)
    hipLaunchKernelGGL(m2rnn_conv4_silu_fwd_kernel<true>, dim3(blocks), dim3(kBlkThreads), 0, s, x, w, bias, (int)B,
                       (int)T, (int)C, u);
  else
    hipLaunchKernelGGL(m2rnn_conv4_silu_fwd_kernel<false>, dim3(blocks), dim3(kBlkThreads), 0, s, x, w, bias, (int)B,
                       (int)T, (int)C, u);
  return status(hipGetLastError());
}

int m2rnn_conv4_silu_bwd_workspace_size(int64_t B, int64_t T, int64_t C, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_conv(B, T, C, M2RNN_DTYPE_F32);
  if (st) return st;
  const long parts = (long)B * ((T + kConvChunk - 1) / kConvChunk);
  *bytes = round_up256((size_t)parts * C * 5 * sizeof(float));
  return M2RNN_OK;
}

int m2rnn_conv4_silu_bwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w, const float* bias,
                         const float* du, float* dx, float* dw, float* dbias, void* workspace, size_t workspace_bytes,
                         void* stream) {
  int st = check_conv(B, T, C, dtype);
  if (st) return st;
  if (!w || !dw) return M2RNN_EINVAL;
  const long nth = conv_threads(B, T, C);
  if (nth > 0 && (!x || !du || !dx)) return M2RNN_EINVAL;
  const void* ps[] = {x, w, bias, du, dx, dw, dbias};
  for (const void* p : ps)
    if (p && !al16(p)) return M2RNN_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  const long parts = (long)B * ((T + kConvChunk - 1) / kConvChunk);
  const size_t need = round_up256((size_t)parts * C * 5 * sizeof(float));
  if (parts > 0 && (!workspace || workspace_bytes < need || !al16(workspace))) return M2RNN_EWORKSPACE;
  float* part = (float*)workspace;
  if (nth > 0) {
    const unsigned blocks = (unsigned)((nth + kBlkThreads - 1) / kBlkThreads);
    if (dtype == M2RNN_DTYPE_BF16)
      hipLaunchKernelGGL(m2rnn_conv4_silu_bwd_kernel<true>, dim3(blocks), dim3(kBlkThreads), 0, s, x, w, bias, du,
                         (int)B, (int)T, (int)C, dx, part);
    else
      hipLaunchKernelGGL(m2rnn_conv4_silu_bwd_kernel<false>, dim3(blocks), dim3(kBlkThreads), 0, s, x, w, bias, du,
                         (int)B, (int)T, (int)C, dx, part);
  }
  hipLaunchKernelGGL(m2rnn_conv4_sum_kernel, dim3((unsigned)((C * 5 + kBlkThreads - 1) / kBlkThreads)),
                     dim3(kBlkThreads), 0, s, (const float*)part, (int)parts, (int)C, dw, dbias);
  return status(hipGetLastError());
}

}  // extern "C"
