/*
 * retention.h -- C ABI of libretention.so, the MI355X (gfx950) hot path of
 * RetNet multi-scale retention.
 *
 * Sources (page title, section):
 *   [notes]  RetNet reading notes, mzeromiko.github.io ("阅读笔记：RetNet"):
 *            §2.2 recurrent mode, §2.3 parallel mode (xPos Theta, decay mask D),
 *            §2.4 chunkwise recurrent mode (R_i, zeta, xi), §三.2 MSR module
 *            (per-head gamma, GroupNorm_h, swish gate), §三.3 normalisation.
 *   [zyxy]   zyxy.net lecture on RetNet, §5 multi-scale grouping (the
 *            (batch, heads, seq, d_head) head layout).
 *
 * Conventions shared by every entry point
 *   - All device buffers belong to the caller.  The library never allocates,
 *     frees or synchronises; work is enqueued on `stream` (NULL = the null
 *     stream) and completes asynchronously.
 *   - gamma and theta are HOST float64 arrays, read during the call only.
 *   - Every call validates its arguments before any HIP call and returns a
 *     ret_status; it never aborts or prints.  retention_last_error() returns a
 *     thread-local message describing the last non-OK return.  Device faults
 *     surface at the caller's next synchronisation, as usual in HIP.
 *   - Tensors are row-major; the innermost (feature) axis is contiguous.
 *     ret_strides gives the element strides of the batch, head and sequence
 *     axes of a [b, h, L, d] view.
 *   - bf16 values are stored as raw 16-bit patterns; every conversion to
 *     bf16 inside the library rounds to nearest even.
 *   - Calls on different streams are independent when their output buffers
 *     (and workspaces) are distinct.
 */
#ifndef RETENTION_H
#define RETENTION_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RETENTION_ABI_VERSION 2

typedef enum {
  RET_OK = 0,
  RET_E_INVAL = 1,        /* null pointer, non-positive size, gamma outside (0,1), ... */
  RET_E_UNSUPPORTED = 2,  /* a shape or dtype combination without a compiled kernel */
  RET_E_ALIGN = 3,        /* a pointer or stride breaks the required alignment */
  RET_E_WORKSPACE = 4,    /* workspace missing or too small */
  RET_E_HIP = 5,          /* a HIP launch failed; the message names the HIP error */
  RET_E_RANGE = 6         /* retention_range_status: a call wrote non-finite results */
} ret_status;

typedef enum { RET_F32 = 0, RET_BF16 = 1, RET_F16 = 2 } ret_dtype;

/* Flag bits selecting the steps of [notes] §2.3 and §三.3. */
enum {
  RET_XPOS = 1u,        /* rotate q and k: pair (2j, 2j+1) times e^{i p theta_j} ([notes] §2.3) */
  RET_SCALE_QK = 2u,    /* QK^T -> QK^T / sqrt(d_k)                                ([notes] §三.3) */
  RET_NORM_DROW = 4u,   /* D_nm -> D_nm / sqrt(sum_{i<=n} D_ni)                       ([notes] §三.3) */
  RET_NORM_SCORE = 8u   /* R_nm -> R_nm / max(|sum_i R_ni|, 1), R = QK^T (.) D        ([notes] §三.3) */
};
#define RET_NORM_ALL (RET_SCALE_QK | RET_NORM_DROW | RET_NORM_SCORE)

typedef struct { int64_t b, h, l; } ret_strides;   /* element strides of a [b,h,L,d] view */

/*
 * retention_chunkwise_fwd -- chunkwise recurrent retention forward ([notes]
 * §2.4), with the xPos rotation of §2.3 and the normalisations of §三.3.
 *
 * For each (batch, head) and chunk i of B consecutive tokens (the last chunk
 * may be shorter, B_i = min(B, L - iB)):
 *   O_[i] = (Q_[i] K_[i]^T (.) D) V_[i] + (Q_[i] R_{i-1}) (.) xi,  xi_j = gamma^(j+1)
 *   R_i   = K_[i]^T (V_[i] (.) zeta) + gamma^(B_i) R_{i-1},        zeta_j = gamma^(B_i-j-1)
 * Q and K are rotated by their absolute position pos0 + t when RET_XPOS is set.
 * The normalisations are those of the parallel form over the whole sequence
 * (including the n_prev tokens summarised by state_in/z_in): row t has seen
 * n = n_prev + t + 1 tokens, its score row sum is carried across chunks by
 * the key-sum z_i = K_[i]^T zeta + gamma^(B_i) z_{i-1}, and
 *   o_t = s_t num_t / max(|s_t den_t|, 1)   (the division only with RET_NORM_SCORE)
 * with s_t = d_k^{-1/2} (RET_SCALE_QK) * sqrt((1-gamma)/(1-gamma^n)) (RET_NORM_DROW).
 *
 *   q, k   [b,h,L,d_k] of in_dt, strides sq / sk (d axis contiguous)
 *   v      [b,h,L,d_v] of in_dt, strides sv
 *   o      [b,h,L,d_v] of out_dt, strides so; must not overlap q, k, v
 *   gamma  host float64 [h], each in (0, 1) ([notes] §三.2 uses 1 - 2^(-5-i))
 *   theta  host float64 [d_k/2]; required with RET_XPOS, ignored otherwise
 *   chunk_B  the chunk size B >= 1 (the interval at which R is carried)
 *   pos0   absolute position of token 0 (xPos phase); n_prev tokens already
 *          summarised by state_in / z_in (0 for a fresh sequence)
 *   state_in / state_out  device float32 [b,h,d_k,d_v] or NULL (= zero / not
 *          written); state_out may equal state_in
 *   z_in / z_out  device float32 [b,h,d_k] key-sums or NULL (same rules);
 *          a continued sequence with RET_NORM_SCORE needs z_in
 *   workspace  device scratch of retention_chunkwise_workspace_bytes() bytes,
 *          256-byte aligned, overlapping none of q, k, v, o and the state /
 *          key-sum buffers; its contents on entry do not matter.  It may be
 *          NULL when that size is 0, and for shapes served by the fused kernel
 *          (those the large-chunk kernels do not take) unless z_out overlaps
 *          z_in, where it holds a snapshot of z_in.  Calls sharing a
 *          workspace must be ordered (one stream, or events).
 * Supported: in_dt bf16 with (d_k, d_v) in {(32,32), (64,64), (128,128),
 * (128,256), (256,256), (256,512)}; in_dt f16 with (d_k, d_v) in
 * {(128,256), (256,512)}; in_dt f32 with (d_k, d_v) in {(32,32), (64,64)};
 * out_dt f32, bf16 or f16; q/k/v/o 16-byte aligned with strides that keep
 * every row 16-byte aligned; L >= 1, b*h >= 1, h <= 64.
 * Numerics: f32 inputs are contracted in fp32 MFMA.  bf16 and f16 inputs are
 * contracted with fp16 MFMA operands and fp32 accumulation; the operands
 * require |q|, |k| < 2^15, |v| < 2^16 and normalised scores
 * s_t |q'_t . k'_m| < 2^16 (the state copy used as an operand is rescaled by
 * a power of two per chunk, so the state itself has no such limit).  An
 * operand that overflows anyway makes the outputs it feeds non-finite (with
 * d_k = 256, d_v = 512 and B a multiple of 64, also a returned state_out);
 * that is recorded and reported by retention_range_status() (the call itself
 * returns RET_OK).
 */
int retention_chunkwise_fwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                            const void* v, ret_strides sv, void* o, ret_strides so,
                            int b, int h, int L, int d_k, int d_v, int chunk_B,
                            const double* gamma, const double* theta,
                            int64_t pos0, int64_t n_prev, unsigned flags,
                            ret_dtype in_dt, ret_dtype out_dt,
                            const float* state_in, float* state_out,
                            const float* z_in, float* z_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace retention_chunkwise_fwd needs for this problem. */
size_t retention_chunkwise_workspace_bytes(int b, int h, int L, int d_k, int d_v, int chunk_B,
                                           unsigned flags);

/*
 * retention_parallel_fwd -- the parallel form of a fresh sequence ([notes]
 * §2.3 with §三.3): O = (Q'K'^T (.) D) V, row-normalised as in
 * retention_chunkwise_fwd, for short sequences where the whole L x L causal
 * score matrix is one chunk.  It is retention_chunkwise_fwd with chunk_B = L
 * (rounded up to a multiple of 64 for the bf16 / f16 (256, 512) kernels), no
 * state in or out and n_prev = 0: every query tile takes every key tile up to
 * its diagonal, and no state is carried.  Arguments as in
 * retention_chunkwise_fwd; the workspace comes from
 * retention_parallel_workspace_bytes() (may be 0).  The work grows as L^2:
 * for long sequences the chunkwise call is the one to use.
 */
int retention_parallel_fwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                           const void* v, ret_strides sv, void* o, ret_strides so,
                           int b, int h, int L, int d_k, int d_v,
                           const double* gamma, const double* theta, int64_t pos0, unsigned flags,
                           ret_dtype in_dt, ret_dtype out_dt,
                           void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace retention_parallel_fwd needs for this problem. */
size_t retention_parallel_workspace_bytes(int b, int h, int L, int d_k, int d_v, ret_dtype in_dt, unsigned flags);

/*
 * retention_chunkwise_bwd -- gradients of retention_chunkwise_fwd for a fresh
 * sequence (the training path of [notes] §三.5 and §四.3, chunkwise as in §2.4):
 * given g = dL/dO, writes dq = dL/dq, dk = dL/dk, dv = dL/dv of
 *   o_p = s_p num_p / n_p,  num_p = sum_{m<=p} A_pm v_m,
 *   A_pm = (q'_p . k'_m) gamma^(p-m),  n_p = max(|s_p sum_m A_pm|, 1)
 * (n_p = 1 without RET_NORM_SCORE; q', k' rotated as in the forward).  The
 * normalisers are differentiated, not detached; where |s_p den_p| = 1 the
 * clamp's constant branch is used.
 *   q, k, v, dout   [b,h,L,d] views of in_dt (bf16 or f16), as in the forward
 *   dq, dk          [b,h,L,d_k] views of grad_dt (f32 or bf16); dv [b,h,L,d_v]
 *                   (written, not accumulated; must not overlap the inputs)
 *   chunk_B         the backward's own chunk size, a multiple of 64 (any
 *                   value gives the same result up to rounding)
 *   gamma, theta, pos0, flags  as in the forward (n_prev = 0, no state_in)
 *   workspace       device scratch of retention_chunkwise_bwd_workspace_bytes()
 *                   bytes, 256-byte aligned
 * Products are fp16 MFMA with fp32 accumulation.  g is scaled per (batch,
 * head) by a power of two that brings its largest magnitude near 1 (undone
 * exactly on the results), so g has no range precondition; q, k, v have the
 * forward's (|q|, |k| < 2^15, |v| < 2^16, s_p |q'_p . k'_m| < 2^16), and
 * |a_p (g_p . v_m) + c_p| < 2^15 must hold for the scaled g (a_p = s_p / n_p,
 * c_p the clamp term), with the score normalisation also s_p |g_p . v_m| < 2^15.
 * Supported (d_k, d_v): (64,64), (128,128), (128,256),
 * (256,512).
 */
int retention_chunkwise_bwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                            const void* v, ret_strides sv, const void* dout, ret_strides sdo,
                            void* dq, ret_strides sdq, void* dk, ret_strides sdk, void* dv, ret_strides sdv,
                            int b, int h, int L, int d_k, int d_v, int chunk_B,
                            const double* gamma, const double* theta, int64_t pos0, unsigned flags,
                            ret_dtype in_dt, ret_dtype grad_dt,
                            void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Bytes of device workspace retention_chunkwise_bwd needs for this problem. */
size_t retention_chunkwise_bwd_workspace_bytes(int b, int h, int L, int d_k, int d_v, int chunk_B);

/*
 * retention_recurrent_step -- one decode step of the recurrent form
 * ([notes] §2.2): S <- gamma S + k'^T v, o = q' S, the current token included.
 *
 *   q, k   [b,h,d_k] of in_dt (contiguous); v [b,h,d_v] of in_dt
 *   S      device float32 [b,h,d_k,d_v], updated in place
 *   z      device float32 [b,h,d_k] key-sum, updated in place (z <- gamma z + k'),
 *          or NULL; required with RET_NORM_SCORE
 *   o      [b,h,d_v] of out_dt (contiguous); must not overlap the inputs
 *   pos    absolute position of this token (xPos phase)
 *   n_tokens  tokens seen including this one (the D-row count n >= 1)
 * The row scalings of §三.3 apply as in retention_chunkwise_fwd, so a
 * chunkwise prefill handing (state_out, z_out) to this call continues the
 * same sequence.  Supported: d_k even, 2 <= d_k <= 512; d_v a multiple of 4,
 * 4 <= d_v <= 1024; S 16-byte aligned.
 */
int retention_recurrent_step(const void* q, const void* k, const void* v, float* S, float* z,
                             void* o, int b, int h, int d_k, int d_v,
                             const double* gamma, const double* theta,
                             int64_t pos, int64_t n_tokens, unsigned flags,
                             ret_dtype in_dt, ret_dtype out_dt, hipStream_t stream);

/*
 * msr_gate_norm -- the MSR epilogue before W_O ([notes] §三.2):
 *   Z = swish(G) (.) GroupNorm_h(Concat(head_1 .. head_h))
 * GroupNorm_h normalises each head's d_v outputs of one token by their mean
 * and biased variance (eps added to the variance), then applies the optional
 * per-channel affine; swish(x) = x / (1 + e^{-x}).
 *
 *   y    [b,h,L,d_v] head outputs of y_dt (f32, bf16 or f16), strides sy
 *   g    [b,L,h*d_v] gate pre-activation X W_G of g_dt (contiguous)
 *   out  [b,L,h*d_v] of out_dt (contiguous)
 *   gn_weight, gn_bias  device float32 [h*d_v] or NULL (= 1 and 0)
 * Supported: d_v a multiple of 8, 8 <= d_v <= 4096; 16-byte aligned rows.
 */
int msr_gate_norm(const void* y, ret_strides sy, const void* g, void* out,
                  int b, int L, int h, int d_v,
                  const float* gn_weight, const float* gn_bias, float eps,
                  ret_dtype y_dt, ret_dtype g_dt, ret_dtype out_dt, hipStream_t stream);

/*
 * msr_gemm -- the projections of the gated MSR block ([notes] §三.2 and
 * §2.1: Q = X W_Q, K = X W_K, V = X W_V, G = X W_G, Out = Z W_O):
 *   C[M][N] = A[M][K] . B[N][K]^T, fp32 accumulation
 *   A  device [M][K] row-major activations of a_dt (bf16 or f16)
 *   B  device bf16 [N][K] row-major: the weight as [out_features][in_features],
 *      i.e. the transpose of the X W layout
 *   C  device [M][N] row-major of c_dt (f32, bf16 or f16); must not overlap A, B
 * bf16 A is contracted with B on bf16 MFMA as given; f16 A is contracted on
 * fp16 MFMA with B converted to fp16 (exact for |w| < 2^16).
 * Supported: K a multiple of 32; 16-byte aligned pointers.
 */
int msr_gemm(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
             hipStream_t stream);

/*
 * msr_gemm_bf16 -- msr_gemm for bf16 activations: C = A . B^T with A and B
 * both bf16 ([notes] §三.2 and §2.1, the block's projections).  A thin call
 * of msr_gemm with a_dt = RET_BF16; arguments, layouts (B is the weight as
 * [N][K] = [out_features][in_features]) and errors as msr_gemm.
 */
int msr_gemm_bf16(const void* A, const void* B, void* C, int M, int N, int K, ret_dtype c_dt, hipStream_t stream);

/*
 * msr_gemm_ex -- msr_gemm with an epilogue, for the RetNet layer ([notes]
 * §三.4: Y = MSR(LN(X)) + X, X' = FFN(LN(Y)) + Y, FFN(X) = gelu(X W_1) W_2):
 *   C = act(A . B^T) (+ residual)
 *   epilogue   MSR_GEMM_GELU applies the exact gelu x Phi(x) = x (1 +
 *              erf(x / sqrt 2)) / 2 to each fp32 output (FFN's first
 *              projection); 0 applies none
 *   residual   device [M][N] row-major of r_dt (f32, bf16 or f16, which
 *              need not be c_dt) added in fp32 after act (the layer's
 *              residual connections), or NULL (r_dt is then ignored); it may
 *              be C itself when r_dt == c_dt (each element is read, then
 *              written, by one thread) but must not overlap A or B
 * Everything else as msr_gemm.  Supported: K a multiple of 32; 16-byte
 * aligned pointers.
 */
#define MSR_GEMM_GELU 1u
int msr_gemm_ex(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                const void* residual, ret_dtype r_dt, unsigned epilogue, hipStream_t stream);

/*
 * msr_gemm_ws -- msr_gemm_ex with a caller-provided workspace, for the
 * projections of a decode step (one token per sequence, M <= 128 rows; the
 * same products as msr_gemm_ex, [notes] §三.2 and §三.4).  With M <= 128 and
 * K a multiple of 128 the columns are taken 128 per workgroup and K is split
 * into up to 8 slices whose fp32 partial products go to the workspace; a
 * second kernel sums them in slice order (the result does not depend on
 * scheduling) and applies the epilogue.  Otherwise msr_gemm_ex runs and the
 * workspace is not touched.
 *   workspace   device memory of msr_gemm_workspace_bytes(M, N, K) bytes,
 *               256-byte aligned, overlapping none of A, B, C and residual;
 *               may be NULL when that size is 0; its contents on entry do
 *               not matter and are overwritten
 * Calls that share a workspace must be ordered (one stream, or events).
 * Everything else, including the errors, as msr_gemm_ex; RET_E_WORKSPACE when
 * the workspace is missing or too small, RET_E_ALIGN when it is misaligned.
 */
size_t msr_gemm_workspace_bytes(int M, int N, int K);
int msr_gemm_ws(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                const void* residual, ret_dtype r_dt, unsigned epilogue, void* workspace, size_t workspace_bytes,
                hipStream_t stream);

/*
 * msr_gemm_scratch -- msr_gemm_ws without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  The split-K partial
 * products go to a scratch array inside the library: MSR_GEMM_SCRATCH_BYTES
 * per GPU, a static device array that each GPU the library runs on holds
 * until the process ends.  Its address is looked up once per device (on the
 * first call with that device current); the call itself allocates and frees
 * nothing.  Every partial element is written before it is read, so the
 * scratch needs no clearing, and it keeps the last call's contents.
 * All calls on one GPU share its scratch array: calls that may overlap (on
 * different streams without ordering) race; order them (one stream, or events).
 * Arguments, results and errors as msr_gemm_ws; RET_E_WORKSPACE when
 * msr_gemm_workspace_bytes(M, N, K) exceeds MSR_GEMM_SCRATCH_BYTES (which
 * covers every M <= 128 with N <= 65536).
 */
#define MSR_GEMM_SCRATCH_BYTES ((size_t)32 << 20)
int msr_gemm_scratch(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                     const void* residual, ret_dtype r_dt, unsigned epilogue, hipStream_t stream);

/*
 * ret_layer_norm -- the LayerNorm of the RetNet layer ([notes] §三.4):
 *   y = (x - mean) / sqrt(biased variance + eps) over each row, then the
 *   optional per-channel affine
 *   x  device [rows][d] row-major of x_dt (f32, bf16 or f16)
 *   y  device [rows][d] row-major of y_dt; must not overlap x
 *   weight, bias  device float32 [d] or NULL (= 1 and 0)
 * The page names LN without its variant; this biased-variance form with eps
 * under the square root is the reading taken.  Supported: d a multiple of 8,
 * 8 <= d <= 8192; 16-byte aligned pointers.
 */
int ret_layer_norm(const void* x, void* y, int rows, int d, const float* weight, const float* bias, float eps,
                   ret_dtype x_dt, ret_dtype y_dt, hipStream_t stream);

/*
 * retention_range_status -- reports whether retention_chunkwise_fwd,
 * retention_parallel_fwd or retention_chunkwise_bwd wrote any non-finite
 * value (NaN, inf, or a value beyond the output type's range) since the
 * previous query on this device, and clears that record.
 *
 * The fp16 operands of the bf16 / f16 paths ([notes] §2.3, §2.4: every
 * product of the rotated q', k' with each other and with v) hold at most
 * 65504; an operand beyond that (for instance |v| >= 65520) becomes inf, and
 * inf reaches every output it feeds, as inf or NaN.  The kernels test every
 * value they store and set a per-device record when one is not finite, so an
 * out-of-range input surfaces here instead of passing silently.  Non-finite
 * inputs are reported the same way.
 *
 * Returns RET_OK when nothing non-finite was written, RET_E_RANGE when
 * something was (retention_last_error() says whether by a forward or a
 * backward call), RET_E_HIP on a HIP failure.  The query enqueues a one-thread
 * kernel and a 4-byte copy on `stream` and waits for `stream`: calls enqueued
 * on `stream` before it are covered; calls on other streams are covered once
 * they have completed (order them before the query with events).  The record
 * is one word per device, shared by all callers: concurrent queries on one
 * device split the record between them.  It allocates nothing.
 */
int retention_range_status(hipStream_t stream);

/* Message for the last non-OK return on the calling thread ("" if none). */
const char* retention_last_error(void);

/* RETENTION_ABI_VERSION of the loaded library. */
int retention_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RETENTION_H */
