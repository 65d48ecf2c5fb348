/*
 * m2rnn.h — C ABI of the MI355X (gfx950) M²RNN recurrence library (libm2rnn.so).
 *
 * The operation is the M²RNN matrix-state nonlinear recurrence of the reading notes
 * "M²RNN：矩阵状态非线性 RNN 的容量、表达力与系统代价" on arXiv:2603.14360v2 ("M²RNN notes"):
 * for every batch entry b and head n, independently, starting from H_0 (zeros, or a given state),
 *
 *     Z_t = tanh(H_{t-1} W_n + k_t v_t^T)          (§2.1, Eq. 10)
 *     H_t = f_t H_{t-1} + (1 - f_t) Z_t             (§2.1, Eq. 11)
 *     y_t = H_t^T q_t + w_r,n (.) v_t               (§2.1, Eq. 12)
 *
 * with H_t a K x V state, W_n a V x V matrix per head (right-multiplied, so it mixes the value
 * dimension only: (H W)[i][j] = sum_l H[i][l] W[l][j]), f_t a scalar per (batch, step, head),
 * and w_r,n a V-vector per head.  The backward is the chain-rule BPTT of §2.7.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Tensor layouts are contiguous row-major:
 *        q, k      [B, T, Nqk, K]   (dtype given by qkv_dtype; Nqk = N, or 1 when all value heads
 *                                    share one query/key, the notes' multi-value layout §2.4)
 *        v         [B, T, N, V]     (dtype given by qkv_dtype)
 *        f         [B, T, N]        fp32, expected in [0, 1] (not checked, computed as given)
 *        W         [N, V, V]        fp32
 *        w_r       [N, V]           fp32
 *        H0, H_T   [B, N, K, V]     fp32
 *        y, dy     [B, T, N, V]     fp32
 *    Gradients have the shape of their input and are fp32.
 *  - Every array pointer is a DEVICE pointer on the current HIP device, 16-byte aligned.  The
 *    caller owns all memory, including the workspace, and every stream: the library allocates no
 *    device memory and keeps no state that one call leaves for another (bar m2rnn_fwd_noalloc's
 *    fixed array, below; the host side caches only device and kernel attributes, under a lock),
 *    so calls on different streams may run concurrently.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *    without synchronising.  Outputs are valid once the stream reaches that point.
 *  - Outputs are overwritten, never accumulated.  Outputs must not alias inputs or each other.
 *  - Arguments are validated on the host before anything is enqueued; an invalid call returns
 *    an error status and touches no memory.  M2RNN_EHIP reports a launch failure
 *    (m2rnn_last_hip_error() gives the hipError_t of the most recent one on this thread).
 *  - Supported sizes: V in {16, 32, 64, 128}; K a positive multiple of 16; B, T, N >= 0;
 *    Nqk in {0, 1, N}; one batch entry's slice of a tensor below 2 GiB (T N max(K, V) fp32 values),
 *    whatever the batch (whole tensors may exceed 4 GiB); B N K / 16 below 2^31.
 *    T = 0 is legal: y is empty and H_T = H0 (or zeros).
 */
#ifndef M2RNN_H_
#define M2RNN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct m2rnn_dims {
  int64_t B; /* batch */
  int64_t T; /* steps */
  int64_t N; /* heads */
  int64_t K; /* key size: rows of the state */
  int64_t V; /* value size: columns of the state, side of W */
  int64_t Nqk; /* heads of q and k: N (one query/key per head) or 1 (one query/key shared by all
                  N value heads, §2.4: N_q = N_k = 1); 0 means N.  With Nqk = 1, dq and dk are
                  the gradients of the shared q and k, summed over the heads (§2.7). */
} m2rnn_dims;

/* dtype of q, k, v. */
enum { M2RNN_DTYPE_F32 = 0, M2RNN_DTYPE_BF16 = 1 };

/* How the per-step contraction H_{t-1} W runs on the matrix cores.  The state, the
 * accumulation and everything outside the contraction are fp32 in every mode.
 *   F32     fp32 MFMA (v_mfma_f32_16x16x4_f32).
 *   F16X3   split precision: H = H_hi + H_lo and W = W_hi + W_lo, all four fp16 (H_lo, W_lo the
 *           fp16 rounding remainders); H W ~ W_hi H_hi + W_lo H_hi + W_hi H_lo on fp16 MFMA with
 *           fp32 accumulation (about 22 significant bits per product).
 *   BF16X3  split precision with bf16 halves: W_hi H_hi + W_lo H_hi + W_hi H_lo.
 *   BF16    one bf16 pass: bf16(W) bf16(H) (coarse; meant for a 2e-2 error budget).
 *   AUTO    the forwards' default: BF16X3 (measured as fast as F16X3 at the 16K-token
 *           workload, with the full fp32 exponent range; about 3e-6 max-abs error on the state
 *           where F16X3 gives 3e-7, both far inside a 5e-4 budget).  The backward's own
 *           contraction is F16X3 (below).
 * Range of the split modes: the contraction takes 2 log2(e) W (so that tanh is one exp2) and the
 * state as 16-bit halves.  F16X3 needs |W| < 65504 / (2 log2 e) ~ 22700 elementwise and a state
 * below 65504 (with f in [0, 1] the state stays within max(|H0|, 1), Eq. 11); the fp16 remainder is
 * subnormal below about 6e-5, so its absolute rounding is about 3e-8 whatever the value's size,
 * which the state's [-1, 1] range makes small.  Outside these bounds the results are undefined
 * (inf or NaN); they are not checked. */
enum { M2RNN_MATH_AUTO = -1, M2RNN_MATH_F32 = 0, M2RNN_MATH_F16X3 = 1, M2RNN_MATH_BF16X3 = 2, M2RNN_MATH_BF16 = 3 };

/* Status codes. */
enum {
  M2RNN_OK = 0,
  M2RNN_EINVAL = -1,      /* null required pointer, negative size, misaligned pointer, bad enum */
  M2RNN_EUNSUPPORTED = -2, /* K or V outside the supported set, or a mode not built */
  M2RNN_EWORKSPACE = -3,   /* workspace missing or smaller than the *_workspace_size answer */
  M2RNN_EHIP = -4          /* a HIP launch or runtime call failed */
};

/* Library version, as MAJOR*10000 + MINOR*100 + PATCH.  The minor number changes with every
 * change of an entry point's arguments; a caller built against this header should check that
 * m2rnn_version() == M2RNN_VERSION before calling anything else. */
#define M2RNN_VERSION 400
int m2rnn_version(void);

/* Human-readable text for a status code (static storage). */
const char* m2rnn_status_string(int status);

/* hipError_t of the last HIP failure seen by this thread (0 if none). */
int m2rnn_last_hip_error(void);

/*
 * Overlap object: a side stream (default priority) and the events that fork work onto it from a
 * call's stream and join it back, on the device current at creation.  The forward calls below take
 * one to overlap the second pass of a long sequence with its scan (see m2rnn_fwd); NULL runs
 * everything on the call's stream.  The caller owns it: one object serves one call at a time, so
 * give each stream (or thread) that issues calls its own, and destroy it once its work is done.
 * Returns M2RNN_EHIP if the stream or an event cannot be made.
 */
typedef struct m2rnn_overlap_s* m2rnn_overlap;
int m2rnn_overlap_create(m2rnn_overlap* out);
int m2rnn_overlap_destroy(m2rnn_overlap overlap);

/*
 * Forward pass, Eq. (10)-(12).  One pass over all T steps for every (b, n).
 *
 *   row_blocks   0 = automatic (one, wherever that kernel keeps its state in registers);
 *                otherwise the number of 16-row blocks of the state that one workgroup carries
 *                (must divide K/16).  The K rows of a state evolve
 *                independently (W mixes only the value dimension, §1.2), so a (b, n) pair may be
 *                split over S = K/(16*row_blocks) workgroups; when S > 1 their partial readouts are
 *                summed by a second, deterministic pass.
 *   H0           initial state, or NULL for zeros.
 *   y            output [B,T,N,V] (may be NULL only when T == 0 or B*N == 0).
 *   H_T          final state [B,N,K,V], or NULL to skip it.
 *   workspace    device scratch of at least m2rnn_fwd_workspace_size() bytes (NULL if that is 0).
 *
 *   overlap      NULL, or an overlap object of the current device (see above).
 *
 * With split rows, T >= 4096 and an overlap object, m2rnn_fwd runs the sequence in two time
 * segments, the second starting from the state the first ended in, and the first segment's second
 * pass runs on the object's side stream while the second segment is scanned (the second segment is
 * sized to cover it); the call's stream waits for all of it before any later work.  This needs the
 * state buffer that m2rnn_fwd_workspace_size() adds for such shapes; with a smaller workspace (the
 * partial planes only), without an overlap object, or on a stream under graph capture, the single
 * pass runs instead.  The two ways of running give the same bits: H_t is a function of H_{t-1} and the
 * step's inputs only, and a scan started from a stored state computes exactly what a continuous
 * scan does.
 */
int m2rnn_fwd_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks,
                             size_t* bytes);
int m2rnn_fwd(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
              const void* k, const void* v, const float* f, const float* W, const float* w_r,
              const float* H0, float* y, float* H_T, void* workspace, size_t workspace_bytes,
              void* stream, m2rnn_overlap overlap);

/*
 * m2rnn_fwd for callers that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments as m2rnn_fwd without the workspace and the
 * overlap object; the same bits as m2rnn_fwd.  It allocates nothing: the partial readouts of split
 * rows and the states between time segments live in a fixed device array of the library
 * (m2rnn_fwd_noalloc_max_bytes() = 64 MiB; every device that runs the library holds one copy until
 * the process ends).  Long sequences run in time segments whose partial planes fit in it (each
 * segment's second pass on the call's stream).  Sizes whose two states and 16 steps of partial
 * planes do not fit return M2RNN_EUNSUPPORTED: 2 B N K V + 16 S B N V floats (S = partial planes,
 * K / 16 / row_blocks when the rows are split) at most.  When one workgroup carries all rows the
 * array is not used.  All calls on one device share the array: calls that overlap in time on one
 * device (on different streams, or from several threads) race, and must be ordered by the caller.
 */
int m2rnn_fwd_noalloc_max_bytes(size_t* bytes);
int m2rnn_fwd_noalloc(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
                      const void* k, const void* v, const float* f, const float* W, const float* w_r,
                      const float* H0, float* y, float* H_T, void* stream);

/*
 * The two launches of m2rnn_fwd's single pass, exposed so that a caller can time them apart.
 * Same arguments as m2rnn_fwd.  m2rnn_scan_fwd runs the recurrence over the whole sequence (it
 * writes y directly when one workgroup carries all K rows, else per-workgroup partial readouts
 * into the workspace); m2rnn_scan_fwd_finish then forms y = sum of partials + w_r (.) v, and is a
 * no-op when the scan already wrote y.  Calling both, in order, on one stream is exactly
 * m2rnn_fwd's single pass (see above for the time segments of long sequences).
 */
int m2rnn_scan_fwd(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
                   const void* k, const void* v, const float* f, const float* W, const float* w_r,
                   const float* H0, float* y, float* H_T, void* workspace, size_t workspace_bytes,
                   void* stream);
int m2rnn_scan_fwd_finish(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks,
                          const void* q, const void* k, const void* v, const float* f,
                          const float* W, const float* w_r, const float* H0, float* y, float* H_T,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass (BPTT of §2.7) for the loss L = sum_t <dy_t, y_t> + <dH_T, H_T>.
 *
 * The forward states are not taken from the caller: the library re-runs the recurrence and keeps
 * the state every I = m2rnn_checkpoint_interval() steps, then walks the `M2RNN_BWD_CHECKPOINT`-step
 * segments from last to first, recomputing each sub-segment's states from its checkpoint in
 * on-chip memory (the notes' §2.6 re-runs the recurrence at the start of the backward; here only
 * checkpoints are stored, not every state).
 *
 *   dH_T   upstream gradient of the final state, or NULL for zeros.
 *   grad_clip  0 for the exact gradient; > 0 clamps every element of the gradient that each step
 *          sends back to its input state, C_{t-1} = f_t R_t + D_t W^T, to [-grad_clip, grad_clip]
 *          before it is used (the per-step recurrent-gradient clipping of the notes' §2.3, read as
 *          an elementwise bound; dH0 is then the clamped C_0).  The readout gradient q_t u_t^T and
 *          dH_T enter unclamped.  Negative or NaN: M2RNN_EINVAL.
 *   dq, dk [B,T,Nqk,K]; dv [B,T,N,V]; df [B,T,N]; dW [N,V,V] and dw_r [N,V] summed over batch and
 *   time; dH0 [B,N,K,V] or NULL to skip it.  All fp32.
 *   math   M2RNN_MATH_F16X3 or M2RNN_MATH_AUTO (the other modes return M2RNN_EUNSUPPORTED).  The
 *          reverse scan recomputes the forward with F16X3 either way; the checkpoint pass that
 *          m2rnn_bwd runs first uses the forwards' default for AUTO and F16X3 for F16X3.
 *
 * Scale of dy.  Every gradient is linear in (dy, dH_T) jointly, and the walk holds the chain's
 * D_t = ((1 - f_t) R_t) (.) (1 - Z_t^2) in split fp16, whose accurate range is narrow.  So each
 * (b, n) pair runs at its own power-of-two scale: a first pass finds the largest |dy| and |dH_T|
 * of the pair, the walk takes 2^e dy and 2^e dH_T with the largest in [1, 2) (and the clip bound
 * 2^e grad_clip), and every gradient is multiplied by 2^-e before it is stored.  Both products
 * are exact, so the result for 2^k dy is exactly 2^k times the result for dy (over the whole
 * fp32 range of dy, bar fp32 underflow or overflow of the gradients themselves): training without
 * loss scaling, whose activation gradients are far below unit size, keeps the same accuracy.
 * W must satisfy |W| < 65504 elementwise (the chain multiplies by W^T in split fp16), and k
 * |k| < 65504 (dv = D^T k is formed on fp16 MFMA with k in one fp16 pass, a relative rounding of
 * 2^-12 per term, as dW's operands).
 */
#define M2RNN_BWD_CHECKPOINT 64
int m2rnn_bwd_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, size_t* bytes);
int m2rnn_bwd(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
              const void* v, const float* f, const float* W, const float* w_r, const float* H0,
              const float* dy, const float* dH_T, float grad_clip, float* dq, float* dk, float* dv,
              float* df, float* dW, float* dw_r, float* dH0, void* workspace, size_t workspace_bytes,
              void* stream);

/*
 * Training pair: a forward that keeps the backward's checkpoints, and a backward that takes them
 * instead of re-running the recurrence.  The notes' §2.6 re-runs the recurrence at the start of the
 * backward so that the forward keeps no history; when a training step runs the forward anyway,
 * keeping only the states that enter every I-th step (an eighth to a sixty-fourth of the states)
 * lets the backward skip that re-run.
 *
 * m2rnn_fwd_ckpt     m2rnn_fwd (time segments included, with the same overlap argument and the
 *                    same bits) plus `ckpt` [B,N,ceil(T/I),K,V] fp32 with I = m2rnn_checkpoint_interval():
 *                    ckpt[b][n][s] is the state entering step I s (ckpt[b][n][0] = H0, or zeros).
 *                    Required when T > 0.
 * m2rnn_bwd_ckpt     m2rnn_bwd with `ckpt` from m2rnn_fwd_ckpt on the same inputs in place of H0
 *                    (H0 is ckpt[., ., 0]); its workspace (m2rnn_bwd_ckpt_workspace_size) excludes
 *                    the checkpoints.  Gradients equal m2rnn_bwd's when the forward used the
 *                    contraction of m2rnn_bwd's own checkpoint pass: the forwards' default for
 *                    math = AUTO, F16X3 for math = F16X3.  Checkpoints from another mode give
 *                    gradients that differ within that mode's error.
 */
/* Steps between checkpoints (I above): 8 for V <= 64, 64 for V = 128.  Smaller
 * intervals let the backward skip a forward pass over every segment; at V = 128 the state is large
 * and the backward runs that pass itself. */
int m2rnn_checkpoint_interval(const m2rnn_dims* dims, int64_t* steps);
int m2rnn_fwd_ckpt(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
                   const void* k, const void* v, const float* f, const float* W, const float* w_r,
                   const float* H0, float* y, float* H_T, float* ckpt, void* workspace,
                   size_t workspace_bytes, void* stream, m2rnn_overlap overlap);
int m2rnn_bwd_ckpt_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, size_t* bytes);
int m2rnn_bwd_ckpt(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                   const void* v, const float* f, const float* W, const float* w_r, const float* ckpt,
                   const float* dy, const float* dH_T, float grad_clip, float* dq, float* dk, float* dv,
                   float* df, float* dW, float* dw_r, float* dH0, void* workspace, size_t workspace_bytes,
                   void* stream);

/*
 * The launches of m2rnn_bwd_ckpt apart, so that a caller can time the reverse scan alone.  Same
 * arguments as m2rnn_bwd_ckpt.  m2rnn_scan_bwd runs the pass that finds each pair's scale (the
 * largest |dy|, |dH_T|) and the reverse scan, which writes dq, dk and dH0 (or per-head partials of
 * a shared q/k), and dv, df (or per-workgroup partials when a pair's rows are split) and per-
 * workgroup partials of dW, dw_r into the workspace; m2rnn_scan_bwd_finish sums those partials in a
 * fixed order.  Calling both, in order, on one stream with the same workspace is m2rnn_bwd_ckpt.
 */
int m2rnn_scan_bwd(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                   const void* v, const float* f, const float* W, const float* w_r, const float* ckpt,
                   const float* dy, const float* dH_T, float grad_clip, float* dq, float* dk, float* dv,
                   float* df, float* dW, float* dw_r, float* dH0, void* workspace, size_t workspace_bytes,
                   void* stream);
int m2rnn_scan_bwd_finish(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                          const void* v, const float* f, const float* W, const float* w_r,
                          const float* ckpt, const float* dy, const float* dH_T, float grad_clip, float* dq,
                          float* dk, float* dv, float* df, float* dW, float* dw_r, float* dH0,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * One step of Eq. (10)-(12) for every (b, n), with the state kept in device memory: the decode
 * (token-by-token inference) form of the layer.  The notes point out that inference carries a
 * fixed-size recurrent state (§2.6); this call reads it, advances it by one token and writes it
 * back, so its cost is the state traffic (about 8 K V bytes per (b, n)), not the contraction.
 *
 *   dims         T must be 1.  Layouts are those of m2rnn_fwd with T = 1:
 *                q, k [B,1,N,K]; v [B,1,N,V] (dtype qkv_dtype); f [B,1,N]; W [N,V,V]; w_r [N,V].
 *   H_in         the state before the step [B,N,K,V], or NULL for zeros.
 *   H_out        the state after the step [B,N,K,V].  H_out == H_in updates the state in place;
 *                any other overlap of the two is rejected (M2RNN_EINVAL).
 *   y            the readout of the step [B,1,N,V].
 *   math         M2RNN_MATH_F16X3 or M2RNN_MATH_AUTO (the other modes return M2RNN_EUNSUPPORTED).
 * No workspace.  Results equal m2rnn_fwd over one step with H0 = H_in, up to rounding order.
 */
int m2rnn_decode_step(const m2rnn_dims* dims, int qkv_dtype, int math, const void* q, const void* k,
                      const void* v, const float* f, const float* W, const float* w_r,
                      const float* H_in, float* H_out, float* y, void* stream);

/*
 * The steps on either side of the recurrence in the M²RNN block (§2.2, §2.3).  Each is an
 * HBM-bound stream with its backward; reductions over batch and time run in a fixed order.
 * Sizes are passed directly; every call enqueues on `stream` and validates arguments on the host
 * like the calls above.
 *
 * Gate (§2.2, Eq. 13/17): f = (1 + e^{a + beta})^{-alpha} = exp(-alpha softplus(a + beta)), with
 * a the gate pre-activation [B,T,N] (fp32) and alpha, beta [N] per head (alpha >= 0 keeps f in
 * [0, 1]; not checked).  f [B,T,N] fp32 is the recurrence's f.  The backward takes df (the
 * recurrence backward's gradient of f) and gives da [B,T,N] and dalpha, dbeta [N] (summed over
 * batch and time); its workspace holds B T N floats.  Pointers 4-byte aligned.
 */
int m2rnn_gate_fwd(int64_t B, int64_t T, int64_t N, const float* a, const float* alpha,
                   const float* beta, float* f, void* stream);
int m2rnn_gate_bwd_workspace_size(int64_t B, int64_t T, int64_t N, size_t* bytes);
int m2rnn_gate_bwd(int64_t B, int64_t T, int64_t N, const float* a, const float* alpha,
                   const float* beta, const float* df, float* da, float* dalpha, float* dbeta,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * Output gate + RMSNorm (§2.3, step 4; the norm's statistic and gradient as in Appendix C):
 *     x = y (.) SiLU(gz),   out = gamma (.) x / sqrt(mean_j x_j^2 + eps)
 * normalised over the D features of each of `rows` rows: y, out [rows, D] fp32 (for the layer's
 * y [B,T,N,V], rows = B T and D = N V, so the statistic spans all heads), gz the output gate's
 * pre-activation [rows, D] (gz_dtype fp32 or bf16), gamma [D] fp32.  The gate multiplies before
 * the norm.  eps >= 0 is the caller's (the notes leave it out).  D a multiple of 4, at most 8192.
 * The backward gives dy, dgz [rows, D] fp32 and dgamma [D] (summed over rows).  Pointers 16-byte
 * aligned.
 */
int m2rnn_out_norm_fwd(int64_t rows, int64_t D, const float* y, const void* gz, int gz_dtype,
                       const float* gamma, float eps, float* out, void* stream);
int m2rnn_out_norm_bwd_workspace_size(int64_t rows, int64_t D, size_t* bytes);
int m2rnn_out_norm_bwd(int64_t rows, int64_t D, const float* y, const void* gz, int gz_dtype,
                       const float* gamma, float eps, const float* dout, float* dy, float* dgz,
                       float* dgamma, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The block's forward from the gate pre-activation to the normalised output, for inference and
 * prefill (§2.2, §2.3 steps 2-4, Appendix C):
 *     f = exp(-alpha softplus(a + beta)),   y = M2RNN(q, k, v, f; W, w_r, H0)  (as m2rnn_fwd),
 *     out = gamma (.) x / sqrt(mean_j x_j^2 + eps),   x = y (.) SiLU(gz)  over the N V features of a token.
 * The gate goes into the workspace ([B,T,N], 1/V of y's size); then the scan, and one epilogue
 * pass per token that sums the scan's partial readouts, adds w_r (.) v and applies the output
 * gate and the norm, so y is never written to HBM (when one workgroup carries all K rows the scan
 * writes y to the workspace and the epilogue reads it once).  Long sequences run in time segments
 * as in m2rnn_fwd, each segment's epilogue on the overlap object's side stream (NULL: one pass).
 * out is bit-identical to
 * m2rnn_gate_fwd, m2rnn_fwd and m2rnn_out_norm_fwd in turn.  The backward needs y: a training
 * step takes those three calls instead.
 *   a            gate pre-activation [B,T,N] fp32; alpha, beta [N] fp32 (4-byte aligned).
 *   gz           output gate pre-activation [B,T,N,V] (gz_dtype fp32 or bf16); gamma [N V] fp32;
 *                eps >= 0.  N V at most 8192.
 *   out          [B,T,N,V] fp32.  The other arguments are m2rnn_fwd's.
 *   workspace    at least m2rnn_fwd_block_workspace_size() bytes.
 */
int m2rnn_fwd_block_workspace_size(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks,
                                   size_t* bytes);
int m2rnn_fwd_block(const m2rnn_dims* dims, int qkv_dtype, int math, int row_blocks, const void* q,
                    const void* k, const void* v, const float* a, const float* alpha,
                    const float* beta, const float* W, const float* w_r, const float* H0,
                    const void* gz, int gz_dtype, const float* gamma, float eps, float* out,
                    float* H_T, void* workspace, size_t workspace_bytes, void* stream,
                    m2rnn_overlap overlap);

/*
 * Causal depthwise Conv1D of kernel size 4 + SiLU (§2.3, step 1), applied to each of q, k, v:
 *     u_t[c] = SiLU(sum_{i<4} w[c][i] x_{t-3+i}[c] + bias[c]),   x_t = 0 for t < 0
 * x, u [B,T,C] in `dtype` (fp32 or bf16; u is rounded to nearest even for bf16), w [C,4] fp32,
 * bias [C] fp32 or NULL (none).  C a multiple of 4.  The backward takes du [B,T,C] fp32 and gives
 * dx [B,T,C], dw [C,4] and dbias [C] (NULL to skip) fp32, summed over batch and time.  Pointers
 * 16-byte aligned.
 */
int m2rnn_conv4_silu_fwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w,
                         const float* bias, void* u, void* stream);
int m2rnn_conv4_silu_bwd_workspace_size(int64_t B, int64_t T, int64_t C, size_t* bytes);
int m2rnn_conv4_silu_bwd(int64_t B, int64_t T, int64_t C, int dtype, const void* x, const float* w,
                         const float* bias, const float* du, float* dx, float* dw, float* dbias,
                         void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* M2RNN_H_ */
