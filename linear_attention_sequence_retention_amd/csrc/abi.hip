// C ABI of libretention.so: argument validation (before any HIP call),
// launch configuration and error reporting.  The operations are specified in
// include/retention.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "internal.h"
#include "retention_calib.h"

namespace {

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return RET_OK;
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool valid_dt(ret_dtype d) { return d == RET_F32 || d == RET_BF16 || d == RET_F16; }
size_t dt_size(ret_dtype d) { return d == RET_F32 ? 4 : 2; }

int check_gamma(const double* gamma, int h) {
  if (!gamma) return fail(RET_E_INVAL, "gamma is NULL");
  for (int i = 0; i < h; ++i)
    if (!(gamma[i] > 0.0 && gamma[i] < 1.0)) return fail(RET_E_INVAL, "gamma[%d] = %g is not in (0, 1)", i, gamma[i]);
  return RET_OK;
}

int check_theta(const double* theta, int dk, unsigned flags) {
  if (!(flags & RET_XPOS)) return RET_OK;
  if (!theta) return fail(RET_E_INVAL, "RET_XPOS needs theta");
  if (dk % 2) return fail(RET_E_INVAL, "RET_XPOS needs an even d_k (got %d)", dk);
  for (int j = 0; j < dk / 2; ++j)
    if (!isfinite(theta[j])) return fail(RET_E_INVAL, "theta[%d] is not finite", j);
  return RET_OK;
}

// a [b,h,L,d] view whose rows are 16-byte aligned
int check_view(const char* name, const void* p, ret_strides s, size_t esz) {
  if (!p) return fail(RET_E_INVAL, "%s is NULL", name);
  if (!aligned(p, 16)) return fail(RET_E_ALIGN, "%s is not 16-byte aligned", name);
  const int64_t a = 16 / (int64_t)esz;
  if (s.b % a || s.h % a || s.l % a)
    return fail(RET_E_ALIGN, "%s strides (%lld, %lld, %lld) break 16-byte row alignment", name, (long long)s.b,
                (long long)s.h, (long long)s.l);
  if (s.b < 0 || s.h < 0 || s.l < 0) return fail(RET_E_INVAL, "%s has a negative stride", name);
  return RET_OK;
}

// bytes from the first to one past the last element of a [b,h,L,d] view
size_t view_span(ret_strides s, int b, int h, int L, int d, size_t esz) {
  return ((size_t)(b - 1) * s.b + (size_t)(h - 1) * s.h + (size_t)(L - 1) * s.l + d) * esz;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return a && b && x < y + nb && y < x + na;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(RET_E_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

void fill_params(ret::HeadParams& hp, const double* gamma, int h, const double* theta, int dk, unsigned flags) {
  memset(&hp, 0, sizeof(hp));
  for (int i = 0; i < h; ++i) {
    hp.gamma[i] = gamma[i];
    hp.lg2[i] = (float)log2(gamma[i]);
    hp.omg[i] = (float)(1.0 - gamma[i]);
    hp.lng[i] = (float)log1p(-(1.0 - gamma[i]));
  }
  if ((flags & RET_XPOS) && theta)
    for (int j = 0; j < dk / 2; ++j) hp.theta[j] = theta[j];
}

}  // namespace

// ---------------------------------------------------------------- non-finite flag
// word 0: bits OR-ed in by kernels that wrote a non-finite output; word 1: the
// value taken by the last retention_range_status() (read back by the host)
namespace {
__device__ __align__(16) unsigned g_nf[4];
std::mutex g_nf_mu;
unsigned* g_nf_ptr[64];

__global__ void take_nonfinite_kernel(unsigned* w) { w[1] = atomicExch(&w[0], 0u); }
}  // namespace

namespace ret {
hipError_t nonfinite_flag_ptr(unsigned** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_nf_mu);
  if (!g_nf_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_nf));
    if (e != hipSuccess) return e;
    g_nf_ptr[dev] = static_cast<unsigned*>(p);
  }
  *out = g_nf_ptr[dev];
  return hipSuccess;
}
}  // namespace ret

extern "C" {

int retention_abi_version(void) { return RETENTION_ABI_VERSION; }

const char* retention_last_error(void) { return g_err; }

size_t retention_chunkwise_workspace_bytes(int b, int h, int L, int d_k, int d_v, int chunk_B, unsigned flags) {
  if (b <= 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0 || chunk_B <= 0) return 0;
  return ret::chunkwise_workspace(b, h, L, d_k, d_v, chunk_B, flags);
}

int retention_chunkwise_fwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                            const void* v, ret_strides sv, void* o, ret_strides so,
                            int b, int h, int L, int d_k, int d_v, int chunk_B,
                            const double* gamma, const double* theta,
                            int64_t pos0, int64_t n_prev, unsigned flags,
                            ret_dtype in_dt, ret_dtype out_dt,
                            const float* state_in, float* state_out,
                            const float* z_in, float* z_out,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (b <= 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0)
    return fail(RET_E_INVAL, "sizes must be positive (b=%d h=%d L=%d d_k=%d d_v=%d)", b, h, L, d_k, d_v);
  if (h > ret::kMaxHeads) return fail(RET_E_UNSUPPORTED, "h = %d exceeds %d heads", h, ret::kMaxHeads);
  if (d_k > 2 * ret::kMaxPairs) return fail(RET_E_UNSUPPORTED, "d_k = %d exceeds %d", d_k, 2 * ret::kMaxPairs);
  if (chunk_B <= 0) return fail(RET_E_INVAL, "chunk_B must be >= 1 (got %d)", chunk_B);
  if (pos0 < 0 || n_prev < 0) return fail(RET_E_INVAL, "pos0 and n_prev must be >= 0");
  if (flags & ~15u) return fail(RET_E_INVAL, "unknown flag bits 0x%x", flags & ~15u);
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return fail(RET_E_INVAL, "unknown dtype");
  int r;
  if ((r = check_gamma(gamma, h))) return r;
  if ((r = check_theta(theta, d_k, flags))) return r;
  const size_t ie = dt_size(in_dt), oe = dt_size(out_dt);
  if ((r = check_view("q", q, sq, ie))) return r;
  if ((r = check_view("k", k, sk, ie))) return r;
  if ((r = check_view("v", v, sv, ie))) return r;
  if ((r = check_view("o", o, so, oe))) return r;
  if (o == q || o == k || o == v) return fail(RET_E_INVAL, "o must not alias q, k or v");
  if (sq.l >= (1 << 25) || sk.l >= (1 << 25) || sv.l >= (1 << 25))
    return fail(RET_E_UNSUPPORTED, "sequence strides must be below 2^25 elements");
  if ((state_in && !aligned(state_in, 16)) || (state_out && !aligned(state_out, 16)))
    return fail(RET_E_ALIGN, "state buffers must be 16-byte aligned");
  if ((flags & RET_NORM_SCORE) && n_prev > 0 && state_in && !z_in)
    return fail(RET_E_INVAL, "a continued sequence with RET_NORM_SCORE needs z_in");
  if (!ret::chunkwise_supported(in_dt, d_k, d_v))
    return fail(RET_E_UNSUPPORTED, "no chunkwise kernel for in_dt=%s d_k=%d d_v=%d",
                in_dt == RET_BF16 ? "bf16" : (in_dt == RET_F16 ? "f16" : "f32"), d_k, d_v);
  size_t need = ret::chunkwise_workspace(b, h, L, d_k, d_v, chunk_B, flags);
  const size_t zb = (size_t)b * h * d_k * sizeof(float), sb = zb * d_v;
  if (!ret::three_phase_applies(in_dt, d_k, d_v, chunk_B) && !overlaps(z_in, zb, z_out, zb))
    need = 0;   // the fused kernel uses its workspace only for a key-sum snapshot
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(RET_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(RET_E_ALIGN, "workspace must be 256-byte aligned");
    if (overlaps(workspace, need, q, view_span(sq, b, h, L, d_k, ie)) ||
        overlaps(workspace, need, k, view_span(sk, b, h, L, d_k, ie)) ||
        overlaps(workspace, need, v, view_span(sv, b, h, L, d_v, ie)) ||
        overlaps(workspace, need, o, view_span(so, b, h, L, d_v, oe)) || overlaps(workspace, need, state_in, sb) ||
        overlaps(workspace, need, state_out, sb) || overlaps(workspace, need, z_in, zb) ||
        overlaps(workspace, need, z_out, zb))
      return fail(RET_E_INVAL, "workspace must not overlap q, k, v, o or the state buffers");
  }

  ret::HeadParams hp;
  fill_params(hp, gamma, h, theta, d_k, flags);
  ret::ChunkArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o;
  a.sq = sq; a.sk = sk; a.sv = sv; a.so = so;
  a.b = b; a.h = h; a.L = L; a.dk = d_k; a.dv = d_v; a.B = chunk_B;
  a.pos0 = pos0; a.n_prev = n_prev; a.flags = flags; a.in_dt = in_dt; a.out_dt = out_dt;
  a.state_in = state_in; a.z_in = z_in; a.state_out = state_out; a.z_out = z_out;
  a.ws = workspace; a.ws_bytes = workspace_bytes; a.hp = &hp;
  hipError_t fe = ret::nonfinite_flag_ptr(&a.nf);
  if (fe != hipSuccess) return hip_status(fe, "retention_chunkwise_fwd flag lookup");
  bool sup = true;
  hipError_t e = ret::launch_chunkwise(a, stream, &sup);
  if (!sup) return fail(RET_E_UNSUPPORTED, "no chunkwise kernel for this shape");
  return hip_status(e, "retention_chunkwise_fwd launch");
}

// the chunk that makes the chunkwise kernels compute the parallel form: one
// chunk covering the sequence (rounded up to a multiple of 64 where the
// large-chunk kernels serve the shape; a ragged chunk is the same form)
static int parallel_chunk(ret_dtype in_dt, int L, int d_k, int d_v) {
  const int B64 = (L + 63) / 64 * 64;
  return ret::three_phase_applies(in_dt, d_k, d_v, B64) ? B64 : L;
}

size_t retention_parallel_workspace_bytes(int b, int h, int L, int d_k, int d_v, ret_dtype in_dt, unsigned flags) {
  if (b <= 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0 || !valid_dt(in_dt)) return 0;
  const int B = parallel_chunk(in_dt, L, d_k, d_v);
  return ret::three_phase_applies(in_dt, d_k, d_v, B) ? ret::three_phase_workspace(b, h, L, B) : 0;
}

int retention_parallel_fwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                           const void* v, ret_strides sv, void* o, ret_strides so,
                           int b, int h, int L, int d_k, int d_v,
                           const double* gamma, const double* theta, int64_t pos0, unsigned flags,
                           ret_dtype in_dt, ret_dtype out_dt,
                           void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (L <= 0) return fail(RET_E_INVAL, "sizes must be positive (L=%d)", L);
  if (!valid_dt(in_dt)) return fail(RET_E_INVAL, "unknown dtype");
  const int B = parallel_chunk(in_dt, L, d_k, d_v);
  const size_t need = retention_parallel_workspace_bytes(b, h, L, d_k, d_v, in_dt, flags);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(RET_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : 0);
  return retention_chunkwise_fwd(q, sq, k, sk, v, sv, o, so, b, h, L, d_k, d_v, B, gamma, theta, pos0, 0, flags,
                                 in_dt, out_dt, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes,
                                 stream);
}

size_t retention_chunkwise_bwd_workspace_bytes(int b, int h, int L, int d_k, int d_v, int chunk_B) {
  if (b <= 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0 || chunk_B <= 0) return 0;
  return ret::chunkwise_bwd_workspace(b, h, L, d_k, d_v, chunk_B);
}

int retention_chunkwise_bwd(const void* q, ret_strides sq, const void* k, ret_strides sk,
                            const void* v, ret_strides sv, const void* dout, ret_strides sdo,
                            void* dq, ret_strides sdq, void* dk, ret_strides sdk, void* dv, ret_strides sdv,
                            int b, int h, int L, int d_k, int d_v, int chunk_B,
                            const double* gamma, const double* theta, int64_t pos0, unsigned flags,
                            ret_dtype in_dt, ret_dtype grad_dt,
                            void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (b <= 0 || h <= 0 || L <= 0 || d_k <= 0 || d_v <= 0)
    return fail(RET_E_INVAL, "sizes must be positive (b=%d h=%d L=%d d_k=%d d_v=%d)", b, h, L, d_k, d_v);
  if (h > ret::kMaxHeads) return fail(RET_E_UNSUPPORTED, "h = %d exceeds %d heads", h, ret::kMaxHeads);
  if (chunk_B < 64 || chunk_B % 64) return fail(RET_E_UNSUPPORTED, "chunk_B must be a multiple of 64 (got %d)", chunk_B);
  if (pos0 < 0) return fail(RET_E_INVAL, "pos0 must be >= 0");
  if (flags & ~15u) return fail(RET_E_INVAL, "unknown flag bits 0x%x", flags & ~15u);
  if (!valid_dt(in_dt) || !valid_dt(grad_dt)) return fail(RET_E_INVAL, "unknown dtype");
  if (in_dt == RET_F32) return fail(RET_E_UNSUPPORTED, "the backward takes bf16 or f16 inputs");
  if (grad_dt == RET_F16) return fail(RET_E_UNSUPPORTED, "gradients are written as f32 or bf16");
  if (!ret::chunkwise_bwd_supported(d_k, d_v))
    return fail(RET_E_UNSUPPORTED, "no backward kernel for d_k=%d d_v=%d", d_k, d_v);
  int r;
  if ((r = check_gamma(gamma, h))) return r;
  if ((r = check_theta(theta, d_k, flags))) return r;
  const size_t ie = dt_size(in_dt), ge = dt_size(grad_dt);
  if ((r = check_view("q", q, sq, ie))) return r;
  if ((r = check_view("k", k, sk, ie))) return r;
  if ((r = check_view("v", v, sv, ie))) return r;
  if ((r = check_view("dout", dout, sdo, ie))) return r;
  if ((r = check_view("dq", dq, sdq, ge))) return r;
  if ((r = check_view("dk", dk, sdk, ge))) return r;
  if ((r = check_view("dv", dv, sdv, ge))) return r;
  const void* ins[4] = {q, k, v, dout};
  const void* outs[3] = {dq, dk, dv};
  for (const void* o : outs)
    for (const void* i : ins)
      if (o == i) return fail(RET_E_INVAL, "gradient buffers must not alias the inputs");
  if (dq == dk || dq == dv || dk == dv) return fail(RET_E_INVAL, "dq, dk and dv must be distinct");
  const size_t need = ret::chunkwise_bwd_workspace(b, h, L, d_k, d_v, chunk_B);
  if (!workspace || workspace_bytes < need)
    return fail(RET_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : 0);
  if (!aligned(workspace, 256)) return fail(RET_E_ALIGN, "workspace must be 256-byte aligned");

  ret::HeadParams hp;
  fill_params(hp, gamma, h, theta, d_k, flags);
  ret::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.dout = dout;
  a.gq = dq; a.gk = dk; a.gv = dv;
  a.sq = sq; a.sk = sk; a.sv = sv; a.sdo = sdo; a.sgq = sdq; a.sgk = sdk; a.sgv = sdv;
  a.b = b; a.h = h; a.L = L; a.d_k = d_k; a.d_v = d_v; a.B = chunk_B;
  a.pos0 = pos0; a.flags = flags; a.in_dt = in_dt; a.grad_dt = grad_dt;
  a.ws = workspace; a.hp = &hp;
  const hipError_t fe = ret::nonfinite_flag_ptr(&a.nf);
  if (fe != hipSuccess) return hip_status(fe, "retention_chunkwise_bwd flag lookup");
  return hip_status(ret::launch_chunkwise_bwd(a, stream), "retention_chunkwise_bwd launch");
}

int retention_recurrent_step(const void* q, const void* k, const void* v, float* S, float* z,
                             void* o, int b, int h, int d_k, int d_v,
                             const double* gamma, const double* theta,
                             int64_t pos, int64_t n_tokens, unsigned flags,
                             ret_dtype in_dt, ret_dtype out_dt, hipStream_t stream) {
  if (b <= 0 || h <= 0 || d_k <= 0 || d_v <= 0)
    return fail(RET_E_INVAL, "sizes must be positive (b=%d h=%d d_k=%d d_v=%d)", b, h, d_k, d_v);
  if (h > ret::kMaxHeads) return fail(RET_E_UNSUPPORTED, "h = %d exceeds %d heads", h, ret::kMaxHeads);
  if (d_k % 2 || d_k > 2 * ret::kMaxPairs) return fail(RET_E_UNSUPPORTED, "d_k must be even and <= 512 (got %d)", d_k);
  if (d_v % 4 || d_v > 1024) return fail(RET_E_UNSUPPORTED, "d_v must be a multiple of 4 and <= 1024 (got %d)", d_v);
  if (pos < 0 || n_tokens < 1) return fail(RET_E_INVAL, "pos must be >= 0 and n_tokens >= 1");
  if (flags & ~15u) return fail(RET_E_INVAL, "unknown flag bits 0x%x", flags & ~15u);
  if (!valid_dt(in_dt) || !valid_dt(out_dt)) return fail(RET_E_INVAL, "unknown dtype");
  if (!q || !k || !v || !S || !o) return fail(RET_E_INVAL, "q, k, v, S and o must be non-NULL");
  if (!aligned(S, 16)) return fail(RET_E_ALIGN, "S must be 16-byte aligned");
  if (!aligned(q, 4) || !aligned(k, 4) || !aligned(v, 4) || !aligned(o, 4) || (z && !aligned(z, 4)))
    return fail(RET_E_ALIGN, "q, k, v, z and o must be 4-byte aligned");
  if ((flags & RET_NORM_SCORE) && !z) return fail(RET_E_INVAL, "RET_NORM_SCORE needs the key-sum z");
  if (o == (void*)S || o == q || o == k || o == v) return fail(RET_E_INVAL, "o must not alias the inputs");
  int r;
  if ((r = check_gamma(gamma, h))) return r;
  if ((r = check_theta(theta, d_k, flags))) return r;

  ret::HeadParams hp;
  fill_params(hp, gamma, h, theta, d_k, flags);
  ret::StepArgs a;
  a.q = q; a.k = k; a.v = v; a.S = S; a.z = z; a.o = o;
  a.b = b; a.h = h; a.dk = d_k; a.dv = d_v; a.pos = pos; a.n_tokens = n_tokens; a.flags = flags;
  a.in_dt = in_dt; a.out_dt = out_dt; a.hp = &hp;
  return hip_status(ret::launch_recurrent_step(a, stream), "retention_recurrent_step launch");
}

int msr_gate_norm(const void* y, ret_strides sy, const void* g, void* out,
                  int b, int L, int h, int d_v,
                  const float* gn_weight, const float* gn_bias, float eps,
                  ret_dtype y_dt, ret_dtype g_dt, ret_dtype out_dt, hipStream_t stream) {
  if (b <= 0 || L <= 0 || h <= 0 || d_v <= 0)
    return fail(RET_E_INVAL, "sizes must be positive (b=%d L=%d h=%d d_v=%d)", b, L, h, d_v);
  if (d_v % 8 || d_v > 4096) return fail(RET_E_UNSUPPORTED, "d_v must be a multiple of 8 and <= 4096 (got %d)", d_v);
  if (!valid_dt(y_dt) || !valid_dt(g_dt) || !valid_dt(out_dt)) return fail(RET_E_INVAL, "unknown dtype");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(RET_E_INVAL, "eps must be finite and >= 0");
  int r;
  if ((r = check_view("y", y, sy, dt_size(y_dt)))) return r;
  if (!g || !out) return fail(RET_E_INVAL, "g and out must be non-NULL");
  if (!aligned(g, 16) || !aligned(out, 16)) return fail(RET_E_ALIGN, "g and out must be 16-byte aligned");
  if (out == y || out == g) return fail(RET_E_INVAL, "out must not alias y or g");
  ret::GateArgs a;
  a.y = y; a.sy = sy; a.g = g; a.out = out; a.b = b; a.L = L; a.h = h; a.dv = d_v;
  a.w = gn_weight; a.bias = gn_bias; a.eps = eps; a.y_dt = y_dt; a.g_dt = g_dt; a.out_dt = out_dt;
  return hip_status(ret::launch_gate_norm(a, stream), "msr_gate_norm launch");
}

static int gemm_checks(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                       const void* residual, ret_dtype r_dt, unsigned epilogue) {
  if (M <= 0 || N <= 0 || K <= 0) return fail(RET_E_INVAL, "sizes must be positive (M=%d N=%d K=%d)", M, N, K);
  if (K % 32) return fail(RET_E_UNSUPPORTED, "K must be a multiple of 32 (got %d)", K);
  if (!valid_dt(c_dt) || !valid_dt(a_dt) || (residual && !valid_dt(r_dt))) return fail(RET_E_INVAL, "unknown dtype");
  if (a_dt == RET_F32) return fail(RET_E_UNSUPPORTED, "A must be bf16 or f16");
  if (epilogue & ~(unsigned)MSR_GEMM_GELU) return fail(RET_E_INVAL, "unknown epilogue bits 0x%x", epilogue);
  if (!A || !B || !C) return fail(RET_E_INVAL, "A, B and C must be non-NULL");
  if (!aligned(A, 16) || !aligned(B, 16) || !aligned(C, 16) || (residual && !aligned(residual, 16)))
    return fail(RET_E_ALIGN, "A, B, C and residual must be 16-byte aligned");
  if (C == A || C == B) return fail(RET_E_INVAL, "C must not alias A or B");
  if (residual && (residual == A || residual == B)) return fail(RET_E_INVAL, "residual must not alias A or B");
  if (residual == C && r_dt != c_dt) return fail(RET_E_INVAL, "a residual that is C must have C's dtype");
  return RET_OK;
}

int msr_gemm_ex(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                const void* residual, ret_dtype r_dt, unsigned epilogue, hipStream_t stream) {
  const int st = gemm_checks(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt, epilogue);
  if (st != RET_OK) return st;
  return hip_status(ret::launch_gemm(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt, (epilogue & MSR_GEMM_GELU) ? 1 : 0,
                                     stream),
                    "msr_gemm launch");
}

size_t msr_gemm_workspace_bytes(int M, int N, int K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return ret::gemm_workspace_bytes(M, N, K);
}

int msr_gemm_ws(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                const void* residual, ret_dtype r_dt, unsigned epilogue, void* workspace, size_t workspace_bytes,
                hipStream_t stream) {
  const int st = gemm_checks(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt, epilogue);
  if (st != RET_OK) return st;
  const size_t need = ret::gemm_workspace_bytes(M, N, K);
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(RET_E_WORKSPACE, "workspace of %zu bytes needed (got %zu)", need, workspace ? workspace_bytes : 0);
    if (!aligned(workspace, 256)) return fail(RET_E_ALIGN, "workspace must be 256-byte aligned");
    const size_t ea = 2, ec = c_dt == RET_F32 ? 4 : 2, er = r_dt == RET_F32 ? 4 : 2;
    if (overlaps(workspace, need, A, ea * M * K) || overlaps(workspace, need, B, (size_t)2 * N * K) ||
        overlaps(workspace, need, C, ec * M * N) || (residual && overlaps(workspace, need, residual, er * M * N)))
      return fail(RET_E_INVAL, "workspace must not overlap A, B, C or residual");
  }
  return hip_status(ret::launch_gemm_ws(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt,
                                        (epilogue & MSR_GEMM_GELU) ? 1 : 0, workspace, stream),
                    "msr_gemm_ws launch");
}

int msr_gemm_scratch(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                     const void* residual, ret_dtype r_dt, unsigned epilogue, hipStream_t stream) {
  const int st = gemm_checks(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt, epilogue);
  if (st != RET_OK) return st;
  const size_t need = ret::gemm_workspace_bytes(M, N, K);
  if (need > MSR_GEMM_SCRATCH_BYTES)
    return fail(RET_E_WORKSPACE, "split-K partials of %zu bytes exceed the %zu-byte scratch", need,
                (size_t)MSR_GEMM_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0) {
    const hipError_t e = ret::gemm_scratch_ptr(&ws);
    if (e != hipSuccess) return hip_status(e, "msr_gemm_scratch scratch lookup");
  }
  return hip_status(ret::launch_gemm_ws(A, a_dt, B, C, c_dt, M, N, K, residual, r_dt,
                                        (epilogue & MSR_GEMM_GELU) ? 1 : 0, ws, stream),
                    "msr_gemm_scratch launch");
}

int msr_gemm(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
             hipStream_t stream) {
  return msr_gemm_ex(A, a_dt, B, C, c_dt, M, N, K, nullptr, c_dt, 0u, stream);
}

int msr_gemm_bf16(const void* A, const void* B, void* C, int M, int N, int K, ret_dtype c_dt, hipStream_t stream) {
  return msr_gemm(A, RET_BF16, B, C, c_dt, M, N, K, stream);
}

int ret_layer_norm(const void* x, void* y, int rows, int d, const float* weight, const float* bias, float eps,
                   ret_dtype x_dt, ret_dtype y_dt, hipStream_t stream) {
  if (rows <= 0 || d <= 0) return fail(RET_E_INVAL, "sizes must be positive (rows=%d d=%d)", rows, d);
  if (d % 8 || d > 8192) return fail(RET_E_UNSUPPORTED, "d must be a multiple of 8 and <= 8192 (got %d)", d);
  if (!valid_dt(x_dt) || !valid_dt(y_dt)) return fail(RET_E_INVAL, "unknown dtype");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(RET_E_INVAL, "eps must be finite and >= 0");
  if (!x || !y) return fail(RET_E_INVAL, "x and y must be non-NULL");
  if (!aligned(x, 16) || !aligned(y, 16) || (weight && !aligned(weight, 16)) || (bias && !aligned(bias, 16)))
    return fail(RET_E_ALIGN, "x, y, weight and bias must be 16-byte aligned");
  if (x == y) return fail(RET_E_INVAL, "y must not alias x");
  return hip_status(ret::launch_layer_norm(x, y, rows, d, weight, bias, eps, x_dt, y_dt, stream),
                    "ret_layer_norm launch");
}

int retention_range_status(hipStream_t stream) {
  unsigned* w = nullptr;
  hipError_t e = ret::nonfinite_flag_ptr(&w);
  if (e != hipSuccess) return hip_status(e, "retention_range_status flag lookup");
  hipLaunchKernelGGL(take_nonfinite_kernel, dim3(1), dim3(1), 0, stream, w);
  if ((e = hipGetLastError()) != hipSuccess) return hip_status(e, "retention_range_status launch");
  unsigned taken = 0;
  if ((e = hipMemcpyAsync(&taken, w + 1, sizeof(taken), hipMemcpyDeviceToHost, stream)) != hipSuccess)
    return hip_status(e, "retention_range_status copy");
  if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_status(e, "retention_range_status sync");
  if (taken == 0) return ok();
  return fail(RET_E_RANGE, "non-finite values were written by %s%s%s", (taken & ret::kNonFiniteFwd) ? "a forward call" : "",
              (taken & ret::kNonFiniteFwd) && (taken & ret::kNonFiniteBwd) ? " and " : "",
              (taken & ret::kNonFiniteBwd) ? "a backward call" : "");
}

int ret_calib_copy(const void* src, void* dst, size_t n16, hipStream_t stream) {
  if (!src || !dst || n16 == 0) return fail(RET_E_INVAL, "src, dst must be non-NULL and n16 >= 1");
  if (!aligned(src, 16) || !aligned(dst, 16)) return fail(RET_E_ALIGN, "src and dst must be 16-byte aligned");
  if (overlaps(src, n16 * 16, dst, n16 * 16)) return fail(RET_E_INVAL, "src and dst must not overlap");
  return hip_status(ret::launch_calib_copy(src, dst, n16, stream), "ret_calib_copy launch");
}

int ret_calib_mfma(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks < 1 || iters < 1) return fail(RET_E_INVAL, "out must be non-NULL, blocks and iters >= 1");
  if (!aligned(out, 4)) return fail(RET_E_ALIGN, "out must be 4-byte aligned");
  return hip_status(ret::launch_calib_mfma(out, blocks, iters, stream), "ret_calib_mfma launch");
}

}  // extern "C"
