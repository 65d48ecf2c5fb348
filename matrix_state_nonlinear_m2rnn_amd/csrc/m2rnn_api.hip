// Host side of libm2rnn.so: argument validation, launch planning and the C entry points
// declared in include/m2rnn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <mutex>
#include <new>
#include <unordered_map>

#include "../../include/m2rnn.h"
#include "m2rnn_block_launch.h"
#include "m2rnn_bwd_kernel.h"
#include "m2rnn_decode_kernel.h"
#include "m2rnn_select.h"

using namespace m2rnn;

namespace {

thread_local int g_last_hip_error = 0;

int hip_status(hipError_t e) {
  if (e == hipSuccess) return M2RNN_OK;
  g_last_hip_error = (int)e;
  return M2RNN_EHIP;
}

}  // namespace

namespace m2rnn {
int record_hip_status(hipError_t e) { return hip_status(e); }
}  // namespace m2rnn

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_dims(const m2rnn_dims* d, int qkv_dtype) {
  if (!d) return M2RNN_EINVAL;
  if (d->B < 0 || d->T < 0 || d->N < 0 || d->K < 0 || d->V < 0) return M2RNN_EINVAL;
  if (qkv_dtype != M2RNN_DTYPE_F32 && qkv_dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (d->Nqk != 0 && d->Nqk != 1 && d->Nqk != d->N) return M2RNN_EINVAL;
  if (d->V != 16 && d->V != 32 && d->V != 64 && d->V != 128) return M2RNN_EUNSUPPORTED;
  if (d->K <= 0 || d->K % 16 != 0) return M2RNN_EUNSUPPORTED;
  // Offsets from a tensor's start are 64-bit; inside the kernels, offsets within the slice of one
  // batch entry (the buffer resources that end at a pair's last step) are 32-bit, so that slice,
  // T N max(K, V) fp32 values, must stay below 2 GiB.  Grids hold B N K / 16 workgroups at most.
  const double slice = (double)d->T * d->N * (d->K > d->V ? d->K : d->V);
  if (slice * 4.0 > 2147483647.0 || (double)d->B * d->N * d->K / 16 > 2147483647.0) return M2RNN_EUNSUPPORTED;
  return M2RNN_OK;
}

// Heads of q and k: N (one query/key per head) or 1 (shared by all heads).
int qk_heads(const m2rnn_dims* d) { return d->Nqk == 1 ? 1 : (int)d->N; }

int resolve_math(int math) {
  if (math == M2RNN_MATH_AUTO) return M2RNN_MATH_BF16X3;
  if (math < M2RNN_MATH_F32 || math > M2RNN_MATH_BF16) return -1;
  return math;
}

const void* fwd_kernel(int math, int V, int rb, int rw, bool bf16, int mode) {
  switch (math) {
    case M2RNN_MATH_F32: return fwd_kernel_f32(V, rb, rw, bf16, mode);
    case M2RNN_MATH_F16X3: return fwd_kernel_f16x3(V, rb, rw, bf16, mode);
    case M2RNN_MATH_BF16X3: return fwd_kernel_bf16x3(V, rb, rw, bf16, mode);
    case M2RNN_MATH_BF16: return fwd_kernel_bf16(V, rb, rw, bf16, mode);
    default: return nullptr;
  }
}

// Row groups per workgroup of the forward scan: with fewer than four 16-column tiles (V < 64) and
// one row block per wave, a workgroup carries 4 / (V/16) row blocks side by side, one group of
// V/16 waves each, so that it has one wave on every SIMD of its CU (single-wave workgroups were
// spread unevenly over the SIMDs), and sums their readouts itself.  The row blocks of a state must
// divide evenly; built for the split-precision contractions.
int row_groups(const m2rnn_dims* d, int rb, int math) {
  if (rb != 1 || d->V >= 64 || math == M2RNN_MATH_F32) return 1;
  const long kb = d->K / 16;
  for (int rw = (int)(64 / d->V); rw > 1; rw /= 2)
    if (kb % rw == 0) return rw;
  return 1;
}

struct DeviceInfo {
  int cus = 0;
};

DeviceInfo device_info() {
  static std::mutex mu;
  static std::unordered_map<int, DeviceInfo> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DeviceInfo{};
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  DeviceInfo info;
  if (hipDeviceGetAttribute(&info.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) info.cus = 0;
  cache[dev] = info;
  return info;
}

int occupancy(const void* kernel, int threads) {
  static std::mutex mu;
  static std::unordered_map<const void*, int> cache;
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = cache.find(kernel);
    if (it != cache.end()) return it->second;
  }
  int blocks = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, threads, 0) != hipSuccess) blocks = 0;
  std::lock_guard<std::mutex> lock(mu);
  cache[kernel] = blocks;
  return blocks;
}

// Whether a kernel spills registers to scratch memory (its per-lane private segment is not empty).
bool spills(const void* kernel) {
  static std::mutex mu;
  static std::unordered_map<const void*, bool> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(kernel);
  if (it != cache.end()) return it->second;
  hipFuncAttributes attr{};
  const bool s = hipFuncGetAttributes(&attr, kernel) == hipSuccess && attr.localSizeBytes > 0;
  cache[kernel] = s;
  return s;
}

// Whether the forward runs its readout in waves of their own where that kernel is built (the
// default).  M2RNN_FWD_READOUT_WAVES=0 in the environment selects the single-role kernel, which
// gives the same bits (for comparison).
bool readout_waves() {
  const char* e = getenv("M2RNN_FWD_READOUT_WAVES");
  return !(e && e[0] == '0');
}

// The forward kernel of a launch (MODE_FWD: with readout waves where built and kept in registers)
// and its threads.
const void* fwd_launch_kernel(const m2rnn_dims* d, int math, int rb, bool bf16, int mode, int* threads) {
  const int rw = row_groups(d, rb, math);
  if (mode == MODE_FWD && readout_waves()) {
    const void* k = fwd_kernel(math, (int)d->V, rb, rw, bf16, MODE_FWD_RO);
    if (k && !(device_info().cus > 0 && spills(k))) {
      *threads = (int)(8 * d->V * rw);
      return k;
    }
  }
  *threads = (int)(4 * d->V * rw);
  return fwd_kernel(math, (int)d->V, rb, rw, bf16, mode);
}

// Row blocks per wave: the fewest whose kernel keeps everything in registers.  A wave's work per
// step grows with its row blocks, so once a CU holds enough waves, packing more row blocks into a
// wave saves nothing, and smaller workgroups fill the last round of resident workgroups better.
// Measured with bf16x3 at T = 2048 over 512 to 8192 row blocks and V = 16..128, one row block was
// the fastest or tied in every case, also where it needs more rounds of workgroups (K = V = 64,
// B12 N32: 2.25 ms against 3.20 ms with four row blocks and half the rounds; K = V = 128, B6 N16:
// 2.99 against 4.19 ms with two).  A kernel that spills runs far slower still, so it is taken only
// when nothing else is built.
int plan_row_blocks(const m2rnn_dims* d, int math, bool bf16, int mode, int requested) {
  const int kb = (int)(d->K / 16);
  if (requested > 0)
    return (kb % requested == 0 && fwd_kernel(math, (int)d->V, requested, row_groups(d, requested, math), bf16, mode))
               ? requested
               : -1;
  const bool on_device = device_info().cus > 0;
  int spilling = -1;
  for (int rb : {1, 2, 4}) {
    if (kb % rb != 0) continue;
    int threads = 0;
    const void* kern = fwd_launch_kernel(d, math, rb, bf16, mode, &threads);
    if (!kern) continue;
    if (on_device && spills(kern)) {
      if (spilling < 0) spilling = rb;
      continue;
    }
    return rb;
  }
  return spilling;
}

size_t round_up(size_t x) { return (x + 255) & ~(size_t)255; }

// dst = src (or zeros when src is null), as a kernel: no memset or copy nodes, so the calls stay
// capturable in a HIP graph.
__global__ void m2rnn_fill_kernel(float* __restrict__ dst, const float* __restrict__ src, long count) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) dst[i] = src ? src[i] : 0.0f;
}

int fill(float* dst, const float* src, long count, hipStream_t stream) {
  if (!dst || count <= 0) return M2RNN_OK;
  hipLaunchKernelGGL(m2rnn_fill_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, stream, dst, src, count);
  return hip_status(hipGetLastError());
}

// Readout planes of the scan: one per workgroup of a (b, n) pair; more than one go to the workspace
// and are summed by the finish pass.
long readout_planes(const m2rnn_dims* d, int rb, int math) { return d->K / (16 * rb * row_groups(d, rb, math)); }

size_t fwd_partial_bytes(const m2rnn_dims* d, int rb, int math) {
  const long S = readout_planes(d, rb, math);
  if (S <= 1) return 0;
  return round_up((size_t)S * d->B * d->T * d->N * d->V * sizeof(float));
}

// Steps between the backward's checkpoints for value size V (see BwdCkpt).
int ckpt_interval(int V) {
  switch (V) {
    case 16: return BwdCkpt<16>::interval;
    case 32: return BwdCkpt<32>::interval;
    case 64: return BwdCkpt<64>::interval;
    default: return BwdCkpt<128>::interval;
  }
}

struct FwdCall {
  const m2rnn_dims* d;
  int qkv_dtype, math, row_blocks;
  const void *q, *k, *v;
  const float *f, *W, *w_r, *H0;
  float *y, *H_T;
  void* ws;
  size_t ws_bytes;
  hipStream_t stream;
  float* ckpt = nullptr;  // optional: the backward's checkpoints (every ckpt_interval(V) steps)
};

// Validates a forward call and fills the resolved math mode and row blocks (also when the only
// fault is the workspace, M2RNN_EWORKSPACE, the last check).  need_ws = false: the caller brings
// the partial planes' memory itself.
int check_fwd(const FwdCall& c, int* math_out, int* rb_out, bool need_ws = true) {
  int st = check_dims(c.d, c.qkv_dtype);
  if (st) return st;
  const int math = resolve_math(c.math);
  if (math < 0 || c.row_blocks < 0) return M2RNN_EINVAL;
  const m2rnn_dims* d = c.d;
  const bool empty = d->B == 0 || d->N == 0;
  const bool bf16 = c.qkv_dtype == M2RNN_DTYPE_BF16;
  if (!empty) {
    if (!c.W || !c.w_r) return M2RNN_EINVAL;
    if (d->T > 0 && (!c.q || !c.k || !c.v || !c.f || !c.y)) return M2RNN_EINVAL;
    const void* ptrs[] = {c.q, c.k, c.v, c.W, c.w_r, c.H0, c.y, c.H_T, c.ckpt};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return M2RNN_EINVAL;
    if (c.f && ((uintptr_t)c.f & 3u)) return M2RNN_EINVAL;
  }
  const int rb = plan_row_blocks(d, math, bf16, MODE_FWD, c.row_blocks);
  if (rb < 0) return c.row_blocks > 0 && (d->K / 16) % c.row_blocks != 0 ? M2RNN_EINVAL : M2RNN_EUNSUPPORTED;
  *math_out = math;
  *rb_out = rb;
  const size_t need = empty || !need_ws ? 0 : fwd_partial_bytes(d, rb, math);
  if (need > 0 && (!c.ws || c.ws_bytes < need || !aligned16(c.ws))) return M2RNN_EWORKSPACE;
  return M2RNN_OK;
}

// Where a launch's partial readouts go (S > 1): planes [S][B][Tp][N][V] from `base`, the launch's
// first step at step t0 of them.  The whole sequence: the workspace, Tp = T, t0 = the launch's own
// first step; planes that hold one time segment only: Tp = its length, t0 = 0.
struct Planes {
  float* base;
  long Tp, t0;
};
Planes whole_planes(const FwdCall& c, long t0) { return Planes{(float*)c.ws, c.d->T, t0}; }

// The scan over steps [t0, t0 + len) of the sequence, from state H0 (null: zeros) to H_T (null:
// not kept).  The whole sequence is t0 = 0, len = T with the call's own H0 and H_T.  The call's
// checkpoints (if any) of the steps in the range are kept: t0 is then a multiple of the interval.
int launch_scan_seg(const FwdCall& c, int math, int rb, long t0, long len, const float* H0, float* H_T,
                    const Planes& pl) {
  const m2rnn_dims* d = c.d;
  const bool bf16 = c.qkv_dtype == M2RNN_DTYPE_BF16;
  const int rw = row_groups(d, rb, math);
  const int S = (int)readout_planes(d, rb, math);  // workgroups per (b, n), one readout plane each
  const long qk_row = qk_heads(d) * d->K, v_row = d->N * d->V;
  const size_t esz = bf16 ? 2 : 4;
  FwdArgs a{};
  a.q = (const char*)c.q + t0 * qk_row * esz;
  a.k = (const char*)c.k + t0 * qk_row * esz;
  a.v = (const char*)c.v + t0 * v_row * esz;
  a.f = c.f + t0 * d->N;
  a.W = c.W; a.w_r = c.w_r; a.H0 = H0;
  if (S > 1) {
    a.y = pl.base + pl.t0 * v_row;
    a.Tp = (int)pl.Tp;
  } else {
    a.y = c.y + t0 * v_row;
    a.Tp = (int)d->T;
  }
  a.H_T = H_T;
  a.ckpt = c.ckpt;
  a.B = (int)d->B; a.T = (int)len; a.N = (int)d->N; a.K = (int)d->K;
  a.Nqk = qk_heads(d);
  a.S = S;
  if (a.ckpt) {
    a.seg = ckpt_interval((int)d->V);
    a.nck = (int)((d->T + a.seg - 1) / a.seg);
    a.ck0 = (int)(t0 / a.seg);
  }
  a.Ts = (int)d->T;
  int threads = 0;
  const void* kern = fwd_launch_kernel(d, math, rb, bf16, MODE_FWD, &threads);
  if (!kern) return M2RNN_EUNSUPPORTED;
  void* args[] = {&a};
  const dim3 grid((unsigned)(d->B * d->N * S)), block((unsigned)threads);
  return hip_status(hipLaunchKernel(kern, grid, block, args, 0, c.stream));
}

int launch_scan(const FwdCall& c, int math, int rb) {
  const m2rnn_dims* d = c.d;
  if (d->B == 0 || d->N == 0) return M2RNN_OK;
  if (d->T == 0) {
    // Nothing to scan: H_T = H0 (or zeros); there are no segments to checkpoint.
    return fill(c.H_T, c.H0, d->B * d->N * d->K * d->V, c.stream);
  }
  return launch_scan_seg(c, math, rb, 0, d->T, c.H0, c.H_T, whole_planes(c, 0));
}

// The finish pass over steps [t0, t0 + len) of every batch entry (the whole tensor: t0 = 0, len = T),
// from the planes `pl` of that range.
int launch_finish_seg(const FwdCall& c, int math, int rb, long t0, long len, hipStream_t stream, const Planes& pl) {
  const m2rnn_dims* d = c.d;
  const int S = (int)readout_planes(d, rb, math);
  const long row = d->N * d->V, plane = d->B * pl.Tp * row;
  const bool whole = t0 == 0 && len == d->T && pl.Tp == d->T;
  const long count = whole ? d->B * d->T * row : len * row;  // elements per row of blocks
  const dim3 grid((unsigned)((count / 4 + 255) / 256), whole ? 1u : (unsigned)d->B);
  const long bstride = whole ? 0 : d->T * row, pbstride = whole ? 0 : pl.Tp * row;
  if (c.qkv_dtype == M2RNN_DTYPE_BF16)
    hipLaunchKernelGGL(m2rnn_fwd_finish_kernel<true>, grid, dim3(256), 0, stream, (const float*)pl.base, S, plane,
                       pl.t0 * row, pbstride, c.v, c.w_r, (int)d->N, (int)d->V, c.y, count, bstride, t0 * row);
  else
    hipLaunchKernelGGL(m2rnn_fwd_finish_kernel<false>, grid, dim3(256), 0, stream, (const float*)pl.base, S, plane,
                       pl.t0 * row, pbstride, c.v, c.w_r, (int)d->N, (int)d->V, c.y, count, bstride, t0 * row);
  return hip_status(hipGetLastError());
}

int launch_finish(const FwdCall& c, int math, int rb) {
  const m2rnn_dims* d = c.d;
  if (d->B == 0 || d->N == 0 || d->T == 0) return M2RNN_OK;
  if (readout_planes(d, rb, math) <= 1) return M2RNN_OK;
  return launch_finish_seg(c, math, rb, 0, d->T, c.stream, whole_planes(c, 0));
}

// Time segments of m2rnn_fwd for long sequences with split rows: each segment's finish pass runs
// on the caller's side stream while the next segment is scanned (the scan keeps one wave per SIMD,
// so the finish pass's waves use the free slots), instead of the whole finish pass after the whole
// scan.  The state goes from one segment to the next through two buffers after the partial planes.
constexpr int kFwdSegs = 2;
constexpr long kFwdSegMinT = 4096;

bool fwd_segmentable(const m2rnn_dims* d, int rb, int math) {
  return d->T >= kFwdSegMinT && d->B * d->N > 0 && d->B <= 65535 && readout_planes(d, rb, math) > 1;
}

size_t fwd_seg_state_bytes(const m2rnn_dims* d) {
  return round_up((size_t)d->B * d->N * d->K * d->V * sizeof(float));
}

// m2rnn_fwd's workspace: the partial planes, and the state between the time segments when it
// segments.
size_t fwd_ws_bytes(const m2rnn_dims* d, int rb, int math) {
  if (d->B == 0 || d->N == 0) return 0;
  return fwd_partial_bytes(d, rb, math) + (fwd_segmentable(d, rb, math) ? fwd_seg_state_bytes(d) : 0);
}

}  // namespace

// A caller's side stream and the events that fork the finish passes off the call's stream and join
// them back (include/m2rnn.h: m2rnn_overlap).
struct m2rnn_overlap_s {
  int device = -1;
  hipStream_t side = nullptr;
  hipEvent_t ev[kFwdSegs + 1] = {};
};

namespace {

// Estimated time of the second pass per step over the scan's time per step, for the segment plan.
// The second pass streams the S partial planes and v in and the output out, B N V (4 S + 8) bytes
// per step, taken at 5.5 TB/s; the scan takes at least 220 ns per step and round of resident
// workgroups on MI355X (228 ns at K = V = 64 with one round; more at larger V and in the fp32
// contraction), so the ratio is an upper estimate except for the one-pass bf16 contraction.
double second_pass_ratio(const FwdCall& c, int math, int rb) {
  const m2rnn_dims* d = c.d;
  const DeviceInfo info = device_info();
  int threads = 0;
  const void* kern = fwd_launch_kernel(d, math, rb, c.qkv_dtype == M2RNN_DTYPE_BF16, MODE_FWD, &threads);
  const int occ = kern && info.cus > 0 ? occupancy(kern, threads) : 0;
  if (occ <= 0) return 1e30;
  const long S = readout_planes(d, rb, math);
  const long blocks = d->B * d->N * S;
  const long cap = (long)occ * info.cus;
  const double rounds = (double)((blocks + cap - 1) / cap);
  const double second = (double)d->B * d->N * d->V * (4.0 * S + 8.0) / 5.5e12;
  return second / (220e-9 * rounds);
}

// The segmented forward: the scan of each time segment on the call's stream, then
// second(t0, len, side stream) for that segment.  Returns 1 when it does not apply (no overlap
// object, or a stream under graph capture); the caller then runs the single pass.  Segment ends
// are multiples of 64 steps, so that they fall on checkpoints.
template <class Second>
int fwd_segmented(const FwdCall& c, m2rnn_overlap_s* ov, int math, int rb, Second second) {
  if (!ov) return 1;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(c.stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return 1;
  const m2rnn_dims* d = c.d;
  // Two segments: the first segment's second pass runs under the second segment's scan, and only
  // the second segment's own second pass is left over, so the second segment is made just long
  // enough to cover the first's: a fraction r / (1 + r) of T, with r the estimated ratio above
  // times a margin of 1.5 (at 16K steps and K = V = 64, r = 0.12 and 1792 steps), at most half.
  // Every launch boundary costs about 15 us, so more segments do not pay where r is small (as at
  // every split-row shape the kernels are built for, r <= 0.25).
  const double r = 1.5 * second_pass_ratio(c, math, rb);
  const long tail = std::min(((long)(d->T * std::min(r / (1.0 + r), 0.5)) + 63) / 64 * 64, d->T / 2);
  const long ends[kFwdSegs] = {(d->T - std::max(tail, 64L)) / 64 * 64, d->T};
  float* hmid = (float*)((char*)c.ws + fwd_partial_bytes(d, rb, math));  // the state between them
  const float* H0 = c.H0;
  int st = M2RNN_OK, i = 0;
  bool forked = false;
  for (long t0 = 0; i < kFwdSegs && st == M2RNN_OK; t0 = ends[i++]) {
    const long len = ends[i] - t0;
    float* HT = i == kFwdSegs - 1 ? c.H_T : hmid;
    st = launch_scan_seg(c, math, rb, t0, len, H0, HT, whole_planes(c, t0));
    if (st) break;
    st = record_hip_status(hipEventRecord(ov->ev[i], c.stream));
    if (!st) st = record_hip_status(hipStreamWaitEvent(ov->side, ov->ev[i], 0));
    if (st) break;
    forked = true;
    st = second(t0, len, ov->side);
    H0 = HT;
  }
  if (forked) {  // the call's stream waits for every finish pass, also after an error
    const int j = record_hip_status(hipEventRecord(ov->ev[kFwdSegs], ov->side));
    const int k = j ? j : record_hip_status(hipStreamWaitEvent(c.stream, ov->ev[kFwdSegs], 0));
    if (!st) st = k;
  }
  return st;
}

// An overlap object is usable on the current device only.
int check_overlap(const m2rnn_overlap_s* ov) {
  if (!ov) return M2RNN_OK;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return M2RNN_EHIP;
  return dev == ov->device ? M2RNN_OK : M2RNN_EINVAL;
}

// ---------------------------------------------------------------- backward

struct BwdLayout {
  size_t ckpt = 0, seg = 0, dv = 0, df = 0, dW = 0, dwr = 0, dq = 0, dk = 0, umax = 0, total = 0;
  size_t total_no_ckpt = 0;  // the workspace when the caller supplies the checkpoints
};

static_assert(BwdCkpt<16>::interval % 8 == 0 && BwdCkpt<64>::interval % 8 == 0 && BwdCkpt<128>::interval % 8 == 0,
              "the forward takes checkpoints at steps 0 and 8 of a chunk");

// Checkpoints: [B][N][ceil(T / ckpt_interval(V))][K][V] fp32.
size_t ckpt_bytes(const m2rnn_dims* d) {
  const long I = ckpt_interval((int)d->V);
  const long nck = (d->T + I - 1) / I;
  return (size_t)d->B * d->N * nck * d->K * d->V * sizeof(float);
}

// Time parts of the |dy| maxima per (b, n) (m2rnn_bwd_absmax_kernel): about 1024 blocks over the
// read of dy, at most 64 parts (one per lane of the wave that combines them), at least 16 steps each.
int absmax_parts(const m2rnn_dims* d) {
  const long win = (d->N * d->V + 1023) / 1024;
  long P = (1024 + d->B * win - 1) / (d->B * win);
  P = std::min(P, 64L);
  P = std::min(P, std::max(1L, (long)(d->T / 16)));
  return (int)std::max(P, 1L);
}

// A shared query/key (Nqk = 1) with several heads: per-head dq, dk go to the workspace and are
// summed over the heads afterwards.
bool shared_qk_sum(const m2rnn_dims* d) { return qk_heads(d) == 1 && d->N > 1; }

BwdLayout bwd_layout(const m2rnn_dims* d) {
  BwdLayout L;
  const long S = d->K / 16;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += round_up(bytes);
    return at;
  };
  // Per-workgroup states entering the sub-segments, when the checkpoints are per segment only.
  const long nsub = kBwdSeg / (d->V <= 32 ? BwdSub<32>::value : d->V == 64 ? BwdSub<64>::value : BwdSub<128>::value);
  const bool sub_ckpt = ckpt_interval((int)d->V) < kBwdSeg;
  L.seg = take(sub_ckpt ? 0 : (size_t)d->B * d->N * S * nsub * 16 * d->V * sizeof(float));
  L.dv = take(S > 1 ? (size_t)S * d->B * d->T * d->N * d->V * sizeof(float) : 0);
  L.df = take(S > 1 ? (size_t)S * d->B * d->T * d->N * sizeof(float) : 0);
  L.dW = take((size_t)d->B * S * d->N * d->V * d->V * sizeof(float));
  L.dwr = take((size_t)d->B * d->N * d->V * sizeof(float));
  const size_t qk_part = shared_qk_sum(d) ? (size_t)d->B * d->T * d->N * d->K * sizeof(float) : 0;
  L.dq = take(qk_part);
  L.dk = take(qk_part);
  L.umax = take((size_t)d->B * d->N * absmax_parts(d) * sizeof(float));
  L.total_no_ckpt = off;
  L.ckpt = take(ckpt_bytes(d));
  L.total = off;
  return L;
}

// The reverse kernel at V = 64 with the walk and the recompute in waves of their own (8 waves per
// workgroup); M2RNN_BWD_ROLES=0 selects the one-role kernel (4 waves), which gives the same bits.
bool bwd_roles() {
  const char* e = getenv("M2RNN_BWD_ROLES");
  return !(e && e[0] == '0');
}

const void* bwd_kernel(int V, bool bf16, bool roles) {
  if (V == 64 && roles)
    return bf16 ? (const void*)&m2rnn_scan_bwd_kernel<64, true, true> : (const void*)&m2rnn_scan_bwd_kernel<64, false, true>;
  switch (V) {
    case 16: return bf16 ? (const void*)&m2rnn_scan_bwd_kernel<16, true> : (const void*)&m2rnn_scan_bwd_kernel<16, false>;
    case 32: return bf16 ? (const void*)&m2rnn_scan_bwd_kernel<32, true> : (const void*)&m2rnn_scan_bwd_kernel<32, false>;
    case 64: return bf16 ? (const void*)&m2rnn_scan_bwd_kernel<64, true> : (const void*)&m2rnn_scan_bwd_kernel<64, false>;
    case 128: return bf16 ? (const void*)&m2rnn_scan_bwd_kernel<128, true> : (const void*)&m2rnn_scan_bwd_kernel<128, false>;
    default: return nullptr;
  }
}

int resolve_bwd_math(int math) {
  if (math == M2RNN_MATH_AUTO || math == M2RNN_MATH_F16X3) return M2RNN_MATH_F16X3;
  if (math >= M2RNN_MATH_F32 && math <= M2RNN_MATH_BF16) return -2;  // valid enum, not built
  return -1;
}

}  // namespace

extern "C" {

int m2rnn_version(void) { return M2RNN_VERSION; }

const char* m2rnn_status_string(int status) {
  switch (status) {
    case M2RNN_OK: return "ok";
    case M2RNN_EINVAL: return "invalid argument";
    case M2RNN_EUNSUPPORTED: return "unsupported size or mode";
    case M2RNN_EWORKSPACE: return "workspace missing or too small";
    case M2RNN_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int m2rnn_last_hip_error(void) { return g_last_hip_error; }

int m2rnn_overlap_create(m2rnn_overlap* out) {
  if (!out) return M2RNN_EINVAL;
  *out = nullptr;
  m2rnn_overlap_s* ov = new (std::nothrow) m2rnn_overlap_s;
  if (!ov) return M2RNN_EINVAL;
  int st = hip_status(hipGetDevice(&ov->device));
  // default priority: streams of other priorities are not used by this library
  if (!st) st = hip_status(hipStreamCreateWithFlags(&ov->side, hipStreamNonBlocking));
  for (int i = 0; !st && i <= kFwdSegs; ++i) st = hip_status(hipEventCreateWithFlags(&ov->ev[i], hipEventDisableTiming));
  if (st) {
    m2rnn_overlap_destroy(ov);
    return st;
  }
  *out = ov;
  return M2RNN_OK;
}

int m2rnn_overlap_destroy(m2rnn_overlap ov) {
  if (!ov) return M2RNN_OK;
  int st = M2RNN_OK;
  for (hipEvent_t& e : ov->ev)
    if (e && hipEventDestroy(e) != hipSuccess && !st) st = M2RNN_EHIP;
  if (ov->side && hipStreamDestroy(ov->side) != hipSuccess && !st) st = M2RNN_EHIP;
  delete ov;
  return st;
}

int m2rnn_fwd_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  const int m = resolve_math(math);
  if (m < 0 || row_blocks < 0) return M2RNN_EINVAL;
  const int rb = plan_row_blocks(dims, m, qkv_dtype == M2RNN_DTYPE_BF16, MODE_FWD, row_blocks);
  if (rb < 0) return row_blocks > 0 && (dims->K / 16) % row_blocks != 0 ? M2RNN_EINVAL : M2RNN_EUNSUPPORTED;
  *bytes = fwd_ws_bytes(dims, rb, m);
  return M2RNN_OK;
}

#define FWD_CALL                                                                                          \
  FwdCall c{dims, qkv_dtype, math, row_blocks, q, k, v, f, W, w_r, H0, y, H_T, workspace, workspace_bytes, \
            (hipStream_t)stream};                                                                         \
  int m = 0, rb = 0;                                                                                      \
  int st = check_fwd(c, &m, &rb);                                                                         \
  if (st) return st;

int m2rnn_scan_fwd(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q, const void* k,
                   const void* v, const float* f, const float* W, const float* w_r, const float* H0, float* y,
                   float* H_T, void* workspace, size_t workspace_bytes, void* stream) {
  FWD_CALL
  return launch_scan(c, m, rb);
}

int m2rnn_scan_fwd_finish(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
                          const void* k, const void* v, const float* f, const float* W, const float* w_r,
                          const float* H0, float* y, float* H_T, void* workspace, size_t workspace_bytes,
                          void* stream) {
  FWD_CALL
  return launch_finish(c, m, rb);
}

int m2rnn_fwd(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q, const void* k,
              const void* v, const float* f, const float* W, const float* w_r, const float* H0, float* y, float* H_T,
              void* workspace, size_t workspace_bytes, void* stream, m2rnn_overlap overlap) {
  FWD_CALL
  if ((st = check_overlap(overlap))) return st;
  if (overlap && fwd_segmentable(dims, rb, m) && workspace_bytes >= fwd_ws_bytes(dims, rb, m)) {
    st = fwd_segmented(c, overlap, m, rb, [&](long t0, long len, hipStream_t s2) {
      return launch_finish_seg(c, m, rb, t0, len, s2, whole_planes(c, t0));
    });
    if (st != 1) return st;
  }
  st = launch_scan(c, m, rb);
  if (st) return st;
  return launch_finish(c, m, rb);
}

// The block forward's workspace: the gate f [B,T,N], then the scan's readout planes (S > 1) or y
// (S = 1), which the epilogue reads once.
size_t fwd_block_f_bytes(const m2rnn_dims* d) { return round_up((size_t)d->B * d->T * d->N * sizeof(float)); }

size_t fwd_block_ws_bytes(const m2rnn_dims* d, int rb, int math) {
  if (d->B == 0 || d->N == 0 || d->T == 0) return 0;
  const size_t planes = fwd_partial_bytes(d, rb, math);
  // planes, or y; then the state between the time segments (as m2rnn_fwd's workspace after the planes)
  return fwd_block_f_bytes(d) + (planes > 0 ? planes : round_up((size_t)d->B * d->T * d->N * d->V * sizeof(float))) +
         (fwd_segmentable(d, rb, math) ? fwd_seg_state_bytes(d) : 0);
}

int m2rnn_fwd_block_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks,
                                   size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  const int m = resolve_math(math);
  if (m < 0 || row_blocks < 0) return M2RNN_EINVAL;
  const int rb = plan_row_blocks(dims, m, qkv_dtype == M2RNN_DTYPE_BF16, MODE_FWD, row_blocks);
  if (rb < 0) return row_blocks > 0 && (dims->K / 16) % row_blocks != 0 ? M2RNN_EINVAL : M2RNN_EUNSUPPORTED;
  *bytes = fwd_block_ws_bytes(dims, rb, m);
  return M2RNN_OK;
}

int m2rnn_fwd_block(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q, const void* k,
                    const void* v, const float* a, const float* alpha, const float* beta, const float* W,
                    const float* w_r, const float* H0, const void* gz, int gz_dtype, const float* gamma, float eps,
                    float* out, float* H_T, void* workspace, size_t workspace_bytes, void* stream,
                    m2rnn_overlap overlap) {
  // Validated as m2rnn_fwd with f = a; the workspace is checked below (the gate comes first in it).
  FwdCall c{dims, qkv_dtype, math, row_blocks, q, k, v, a, W, w_r, H0, out, H_T, nullptr, 0,
            (hipStream_t)stream};
  int m = 0, rb = 0;
  int st = check_fwd(c, &m, &rb);
  if (st == M2RNN_EWORKSPACE) st = M2RNN_OK;  // the partial planes live after the gate
  if (st) return st;
  if ((st = check_overlap(overlap))) return st;
  if (gz_dtype != M2RNN_DTYPE_F32 && gz_dtype != M2RNN_DTYPE_BF16) return M2RNN_EINVAL;
  if (!(eps >= 0.0f) || eps > 1e30f) return M2RNN_EINVAL;
  if (dims->N * dims->V > kNormMaxFeatures || dims->B > 65535) return M2RNN_EUNSUPPORTED;
  const bool work = dims->B > 0 && dims->N > 0 && dims->T > 0;
  if (work) {
    if (!alpha || !beta || !gz || !gamma) return M2RNN_EINVAL;
    if (((uintptr_t)alpha | (uintptr_t)beta) & 3u) return M2RNN_EINVAL;
    if (!aligned16(gz) || !aligned16(gamma)) return M2RNN_EINVAL;
    const size_t need = fwd_block_ws_bytes(dims, rb, m);
    if (!workspace || workspace_bytes < need || !aligned16(workspace)) return M2RNN_EWORKSPACE;
  }
  if (!work) return launch_scan(c, m, rb);  // T = 0: H_T = H0; B N = 0: nothing
  // 1. the gate into the workspace.  A pass of its own: forming it in the scan's staging would put
  //    three dependent transcendentals before every chunk's barrier.
  float* f = (float*)workspace;
  st = m2rnn_gate_fwd(dims->B, dims->T, dims->N, a, alpha, beta, f, stream);
  if (st) return st;
  // 2. the scan: partial readouts (S > 1) or y (S = 1) into the workspace after f
  const int S = (int)readout_planes(dims, rb, m);
  float* planes = (float*)((char*)workspace + fwd_block_f_bytes(dims));
  c.f = f;
  c.ws = planes;
  c.ws_bytes = workspace_bytes - fwd_block_f_bytes(dims);
  if (S <= 1) c.y = planes;
  // 3. the epilogue: y, the output gate and the norm, token by token (over a time segment, or all)
  const int D = (int)(dims->N * dims->V);
  auto epilogue = [&](long t0, long len, hipStream_t s2) {
    return hip_status((hipError_t)launch_fwd_finish_norm(planes, S, v, qkv_dtype == M2RNN_DTYPE_BF16,
                                                         S > 1 ? w_r : nullptr, gz, gz_dtype == M2RNN_DTYPE_BF16,
                                                         gamma, dims->B, dims->T, t0, len, D, eps, out, s2));
  };
  if (overlap && fwd_segmentable(dims, rb, m)) {  // the workspace holds the segment state (checked above)
    st = fwd_segmented(c, overlap, m, rb, epilogue);
    if (st != 1) return st;
  }
  st = launch_scan(c, m, rb);
  if (st) return st;
  return epilogue(0, dims->T, (hipStream_t)stream);
}

int m2rnn_bwd_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  const int m = resolve_bwd_math(math);
  if (m == -1) return M2RNN_EINVAL;
  if (m == -2) return M2RNN_EUNSUPPORTED;
  *bytes = (dims->B == 0 || dims->N == 0 || dims->T == 0) ? 0 : bwd_layout(dims).total;
  return M2RNN_OK;
}

}  // extern "C"

namespace {

// Parts of the backward: the checkpoint pass, the scale pass and the reverse scan, and the sums of
// the per-workgroup partials.
enum { BWD_SCAN = 1, BWD_SUMS = 2, BWD_ALL = 3 };

// The backward; ckpt_in = the checkpoints of a forward that kept them (then no forward re-run), or
// null (then the checkpoints are computed here, into the workspace).  `parts` selects what runs.
int bwd_impl(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k, const void* v,
             const float* f, const float* W, const float* w_r, const float* H0, const float* ckpt_in,
             const float* dy, const float* dH_T, float grad_clip, float* dq, float* dk, float* dv, float* df,
             float* dW, float* dw_r, float* dH0, void* workspace, size_t workspace_bytes, void* stream_,
             int parts = BWD_ALL) {
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  if (!(grad_clip >= 0.0f)) return M2RNN_EINVAL;  // negative or NaN
  const int m = resolve_bwd_math(math);
  if (m == -1) return M2RNN_EINVAL;
  if (m == -2) return M2RNN_EUNSUPPORTED;
  const m2rnn_dims* d = dims;
  hipStream_t stream = (hipStream_t)stream_;
  const bool bf16 = qkv_dtype == M2RNN_DTYPE_BF16;
  if (d->B == 0 || d->N == 0) return M2RNN_OK;
  if (!W || !w_r || !dW || !dw_r) return M2RNN_EINVAL;
  if (d->T > 0 && (!q || !k || !v || !f || !dy || !dq || !dk || !dv || !df)) return M2RNN_EINVAL;
  {
    const void* ptrs[] = {q, k, v, W, w_r, H0, ckpt_in, dy, dH_T, dq, dk, dv, dW, dw_r, dH0};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return M2RNN_EINVAL;
    if ((f && ((uintptr_t)f & 3u)) || (df && ((uintptr_t)df & 3u))) return M2RNN_EINVAL;
  }
  const long N = d->N, V = d->V, K = d->K, B = d->B, T = d->T;
  if (T == 0) {
    // No steps: every gradient is zero except dH0 = dH_T.
    if (!(parts & BWD_SUMS)) return M2RNN_OK;
    if ((st = fill(dW, nullptr, N * V * V, stream))) return st;
    if ((st = fill(dw_r, nullptr, N * V, stream))) return st;
    return fill(dH0, dH_T, B * N * K * V, stream);
  }
  const BwdLayout L = bwd_layout(d);
  const size_t need = ckpt_in ? L.total_no_ckpt : L.total;
  if (!workspace || workspace_bytes < need || !aligned16(workspace)) return M2RNN_EWORKSPACE;
  char* ws = (char*)workspace;
  const int S = (int)(K / 16);

  // 1. Checkpoints: the state entering every I-th step, I = ckpt_interval (unless the forward kept
  //    them).
  const float* ckpt = ckpt_in ? ckpt_in : (const float*)(ws + L.ckpt);
  if (parts & BWD_SCAN) {
    if (!ckpt_in) {
      FwdArgs a{};
      a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.w_r = w_r; a.H0 = H0;
      a.y = nullptr; a.H_T = nullptr; a.ckpt = (float*)(ws + L.ckpt);
      a.B = (int)B; a.T = (int)T; a.N = (int)N; a.K = (int)K; a.S = S; a.seg = ckpt_interval((int)V);
      a.nck = (int)((T + a.seg - 1) / a.seg);
      a.ck0 = 0;
      a.Ts = (int)T;
      a.Tp = (int)T;
      a.Nqk = qk_heads(d);
      // (the forwards' contraction: the default's unless F16X3 was asked for)
      const void* kern = fwd_kernel(math == M2RNN_MATH_F16X3 ? M2RNN_MATH_F16X3 : resolve_math(M2RNN_MATH_AUTO),
                                    (int)V, 1, 1, bf16, MODE_CKPT);
      if (!kern) return M2RNN_EUNSUPPORTED;
      void* args[] = {&a};
      st = hip_status(hipLaunchKernel(kern, dim3((unsigned)(B * N * S)), dim3((unsigned)(4 * V)), args, 0, stream));
      if (st) return st;
    }
    // 2. The scale of every (b, n) pair: partial maxima of |dy| and |dH_T|.
    const int P = absmax_parts(d);
    {
      const dim3 grid((unsigned)(B * P), (unsigned)((N * V + 1023) / 1024));
      hipLaunchKernelGGL(m2rnn_bwd_absmax_kernel, grid, dim3(256), 0, stream, dy, dH_T, (int)T, (int)N, (int)K,
                         (int)V, P, (float*)(ws + L.umax));
      st = hip_status(hipGetLastError());
      if (st) return st;
    }
    // 3. Reverse scan.
    {
      BwdArgs a{};
      a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.w_r = w_r; a.dy = dy; a.dH_T = dH_T;
      a.ckpt = ckpt;
      a.subck = (float*)(ws + L.seg);
      const bool sum_qk = shared_qk_sum(d);
      a.dq = sum_qk ? (float*)(ws + L.dq) : dq;
      a.dk = sum_qk ? (float*)(ws + L.dk) : dk;
      a.dv = S > 1 ? (float*)(ws + L.dv) : dv;
      a.df = S > 1 ? (float*)(ws + L.df) : df;
      a.dW_part = (float*)(ws + L.dW);
      a.dwr_part = (float*)(ws + L.dwr);
      a.dH0 = dH0;
      a.umax = (const float*)(ws + L.umax);
      a.umax_parts = P;
      a.B = (int)B; a.T = (int)T; a.N = (int)N; a.K = (int)K; a.S = S;
      a.Nqk = qk_heads(d);
      a.clip = grad_clip;
      const bool roles = V == 64 && bwd_roles();
      const void* kern = bwd_kernel((int)V, bf16, roles);
      if (!kern) return M2RNN_EUNSUPPORTED;
      void* args[] = {&a};
      st = hip_status(
          hipLaunchKernel(kern, dim3((unsigned)(B * N * S)), dim3((unsigned)(roles ? 8 * V : 4 * V)), args, 0, stream));
      if (st) return st;
    }
  }
  if (!(parts & BWD_SUMS)) return M2RNN_OK;
  // 4. Deterministic sums of the per-workgroup partials, and dw_r.
  if (S > 1) {
    const long plane = B * T * N * V;
    hipLaunchKernelGGL(m2rnn_fwd_finish_kernel<false>, dim3((unsigned)((plane / 4 + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(ws + L.dv), S, plane, 0L, 0L, (const void*)dy, w_r, (int)N, (int)V, dv, plane, 0L,
                       0L);
    const long cnt = B * T * N;
    hipLaunchKernelGGL(m2rnn_bwd_sum_df_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(ws + L.df), S, cnt, df);
  }
  if (shared_qk_sum(d)) {
    const long cnt = B * T * K / 4;  // one thread per 4 consecutive k
    hipLaunchKernelGGL(m2rnn_bwd_sum_heads_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(ws + L.dq), (int)N, B * T, (int)K, dq);
    hipLaunchKernelGGL(m2rnn_bwd_sum_heads_kernel, dim3((unsigned)((cnt + 255) / 256)), dim3(256), 0, stream,
                       (const float*)(ws + L.dk), (int)N, B * T, (int)K, dk);
  }
  hipLaunchKernelGGL(m2rnn_bwd_sum_dW_kernel, dim3((unsigned)((N * V * V + 255) / 256)), dim3(256), 0, stream,
                     (const float*)(ws + L.dW), (int)(B * S), (int)N, (int)(V * V), dW);
  hipLaunchKernelGGL(m2rnn_bwd_sum_dwr_kernel, dim3((unsigned)((N * V + 255) / 256)), dim3(256), 0, stream,
                     (const float*)(ws + L.dwr), (int)B, (int)(N * V), dw_r);
  return hip_status(hipGetLastError());
}

}  // namespace

extern "C" {

int m2rnn_bwd(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k, const void* v,
              const float* f, const float* W, const float* w_r, const float* H0, const float* dy,
              const float* dH_T, float grad_clip, float* dq, float* dk, float* dv, float* df, float* dW,
              float* dw_r, float* dH0, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_impl(dims, qkv_dtype, math, q, k, v, f, W, w_r, H0, nullptr, dy, dH_T, grad_clip, dq, dk, dv, df, dW,
                  dw_r, dH0, workspace, workspace_bytes, stream);
}

int m2rnn_checkpoint_interval(const m2rnn_dims* dims, int64_t* steps) {
  if (!steps) return M2RNN_EINVAL;
  int st = check_dims(dims, M2RNN_DTYPE_F32);
  if (st) return st;
  *steps = ckpt_interval((int)dims->V);
  return M2RNN_OK;
}

int m2rnn_bwd_ckpt_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  const int m = resolve_bwd_math(math);
  if (m == -1) return M2RNN_EINVAL;
  if (m == -2) return M2RNN_EUNSUPPORTED;
  *bytes = (dims->B == 0 || dims->N == 0 || dims->T == 0) ? 0 : bwd_layout(dims).total_no_ckpt;
  return M2RNN_OK;
}

int m2rnn_bwd_ckpt(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k, const void* v,
                   const float* f, const float* W, const float* w_r, const float* ckpt, const float* dy,
                   const float* dH_T, float grad_clip, float* dq, float* dk, float* dv, float* df, float* dW,
                   float* dw_r, float* dH0, void* workspace, size_t workspace_bytes, void* stream) {
  if (dims && dims->T > 0 && dims->B > 0 && dims->N > 0 && !ckpt) return M2RNN_EINVAL;
  return bwd_impl(dims, qkv_dtype, math, q, k, v, f, W, w_r, nullptr, ckpt, dy, dH_T, grad_clip, dq, dk, dv, df, dW,
                  dw_r, dH0, workspace, workspace_bytes, stream);
}

int m2rnn_scan_bwd(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k, const void* v,
                   const float* f, const float* W, const float* w_r, const float* ckpt, const float* dy,
                   const float* dH_T, float grad_clip, float* dq, float* dk, float* dv, float* df, float* dW,
                   float* dw_r, float* dH0, void* workspace, size_t workspace_bytes, void* stream) {
  if (dims && dims->T > 0 && dims->B > 0 && dims->N > 0 && !ckpt) return M2RNN_EINVAL;
  return bwd_impl(dims, qkv_dtype, math, q, k, v, f, W, w_r, nullptr, ckpt, dy, dH_T, grad_clip, dq, dk, dv, df, dW,
                  dw_r, dH0, workspace, workspace_bytes, stream, BWD_SCAN);
}

int m2rnn_scan_bwd_finish(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                          const void* v, const float* f, const float* W, const float* w_r, const float* ckpt,
                          const float* dy, const float* dH_T, float grad_clip, float* dq, float* dk, float* dv,
                          float* df, float* dW, float* dw_r, float* dH0, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (dims && dims->T > 0 && dims->B > 0 && dims->N > 0 && !ckpt) return M2RNN_EINVAL;
  return bwd_impl(dims, qkv_dtype, math, q, k, v, f, W, w_r, nullptr, ckpt, dy, dH_T, grad_clip, dq, dk, dv, df, dW,
                  dw_r, dH0, workspace, workspace_bytes, stream, BWD_SUMS);
}

int m2rnn_fwd_ckpt(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q, const void* k,
                   const void* v, const float* f, const float* W, const float* w_r, const float* H0, float* y,
                   float* H_T, float* ckpt, void* workspace, size_t workspace_bytes, void* stream,
                   m2rnn_overlap overlap) {
  FwdCall c{dims, qkv_dtype, math, row_blocks, q, k, v, f, W, w_r, H0, y, H_T, workspace, workspace_bytes,
            (hipStream_t)stream, ckpt};
  int m = 0, rb = 0;
  int st = check_fwd(c, &m, &rb);
  if (st) return st;
  if ((st = check_overlap(overlap))) return st;
  if (dims->T > 0 && dims->B > 0 && dims->N > 0 && !ckpt) return M2RNN_EINVAL;
  if (overlap && fwd_segmentable(dims, rb, m) && workspace_bytes >= fwd_ws_bytes(dims, rb, m)) {
    st = fwd_segmented(c, overlap, m, rb, [&](long t0, long len, hipStream_t s2) {
      return launch_finish_seg(c, m, rb, t0, len, s2, whole_planes(c, t0));
    });
    if (st != 1) return st;
  }
  st = launch_scan(c, m, rb);
  if (st) return st;
  return launch_finish(c, m, rb);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free forward

namespace {

// Device memory of m2rnn_fwd_noalloc: the partial readout planes of one time segment, then the two
// states that carry the recurrence from one segment to the next.  Every device that runs the
// library holds one copy until the process ends.  In host code `scratch` names a host-side stand-in,
// not device memory: its address on a device comes from hipGetSymbolAddress (scratch_on_device).
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;  // device -> address of `scratch` on it

// The address of `scratch` on the current device, looked up once per device with that device current.
int scratch_on_device(void** out) {
  int dev = 0;
  int st = hip_status(hipGetDevice(&dev));
  if (st) return st;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    st = hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (st) return st;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *out = it->second;
  return M2RNN_OK;
}

}  // namespace

extern "C" {

int m2rnn_fwd_noalloc_max_bytes(size_t* bytes) {
  if (!bytes) return M2RNN_EINVAL;
  *bytes = kNoAllocScratchBytes;
  return M2RNN_OK;
}

int m2rnn_fwd_noalloc(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q, const void* k,
                      const void* v, const float* f, const float* W, const float* w_r, const float* H0, float* y,
                      float* H_T, void* stream) {
  FwdCall c{dims, qkv_dtype, math, row_blocks, q, k, v, f, W, w_r, H0, y, H_T, nullptr, 0, (hipStream_t)stream};
  int m = 0, rb = 0;
  int st = check_fwd(c, &m, &rb, /*need_ws=*/false);
  if (st) return st;
  const m2rnn_dims* d = dims;
  if (d->B == 0 || d->N == 0 || d->T == 0) return launch_scan(c, m, rb);
  const long S = readout_planes(d, rb, m);
  if (S <= 1) return launch_scan(c, m, rb);  // one workgroup per pair: the scan writes y itself
  // Segments of L steps (a multiple of 16) whose planes fit beside the two states.
  const size_t state = fwd_seg_state_bytes(d);
  const size_t per_step = (size_t)S * d->B * d->N * d->V * sizeof(float);
  if (d->B > 65535 || 2 * state + 256 + 16 * per_step > kNoAllocScratchBytes) return M2RNN_EUNSUPPORTED;
  const long L = (long)((kNoAllocScratchBytes - 2 * state - 256) / per_step) / 16 * 16;
  void* base = nullptr;
  if ((st = scratch_on_device(&base))) return st;
  float* planes = (float*)base;
  char* hb = (char*)base + round_up((size_t)L * per_step);
  float* hbuf[2] = {(float*)hb, (float*)(hb + state)};
  // Every plane element of a segment is written by its scan before the finish pass reads it, and
  // every state before the next segment reads it: nothing needs clearing between calls.
  const float* Hin = c.H0;
  long i = 0;
  for (long t0 = 0; t0 < d->T; t0 += L, ++i) {
    const long len = std::min(L, d->T - t0);
    float* Hout = t0 + len == d->T ? c.H_T : hbuf[i & 1];
    const Planes pl{planes, len, 0};
    if ((st = launch_scan_seg(c, m, rb, t0, len, Hin, Hout, pl))) return st;
    if ((st = launch_finish_seg(c, m, rb, t0, len, c.stream, pl))) return st;
    Hin = Hout;
  }
  return M2RNN_OK;
}

int m2rnn_decode_step(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                      const void* v, const float* f, const float* W, const float* w_r, const float* H_in,
                      float* H_out, float* y, void* stream) {
  int st = check_dims(dims, qkv_dtype);
  if (st) return st;
  if (dims->T != 1) return M2RNN_EINVAL;
  const int m = resolve_bwd_math(math);  // the decode kernel is built for F16X3 (= AUTO) only
  if (m == -1) return M2RNN_EINVAL;
  if (m == -2) return M2RNN_EUNSUPPORTED;
  const m2rnn_dims* d = dims;
  if (d->B == 0 || d->N == 0) return M2RNN_OK;
  if (!q || !k || !v || !f || !W || !w_r || !H_out || !y) return M2RNN_EINVAL;
  {
    const void* ptrs[] = {q, k, v, W, w_r, H_in, H_out, y};
    for (const void* p : ptrs)
      if (p && !aligned16(p)) return M2RNN_EINVAL;
    if ((uintptr_t)f & 3u) return M2RNN_EINVAL;
  }
  // H_out may be H_in itself (in-place update), but must not overlap it partially.
  const size_t sbytes = (size_t)d->B * d->N * d->K * d->V * sizeof(float);
  if (H_in && H_in != H_out) {
    const char *a0 = (const char*)H_in, *b0 = (const char*)H_out;
    if (a0 < b0 + sbytes && b0 < a0 + sbytes) return M2RNN_EINVAL;
  }
  const void* kern = decode_kernel((int)d->V, qkv_dtype == M2RNN_DTYPE_BF16);
  if (!kern) return M2RNN_EUNSUPPORTED;
  const long groups = (d->B + kDecWaves - 1) / kDecWaves;
  if ((double)groups * d->N > 2147483647.0) return M2RNN_EUNSUPPORTED;
  DecArgs a{};
  a.q = q; a.k = k; a.v = v; a.f = f; a.W = W; a.w_r = w_r; a.H_in = H_in; a.H_out = H_out; a.y = y;
  a.B = (int)d->B; a.N = (int)d->N; a.K = (int)d->K;
  a.Nqk = qk_heads(d);
  void* args[] = {&a};
  return hip_status(hipLaunchKernel(kern, dim3((unsigned)(groups * d->N)), dim3(64 * kDecWaves), args, 0,
                                    (hipStream_t)stream));
}

}  // extern "C"
