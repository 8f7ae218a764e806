// Internal launch interface between the C ABI (abi.hip) and the kernels.
#pragma once
#include "common.h"

namespace ret {

// kLim: the smallest magnitude that is no longer finite once converted to TO
// with round-to-nearest-even (half: 65504 + half an ulp; bf16 likewise)
template <typename TO> struct Store;
template <> struct Store<float> {
  static constexpr float kLim = __builtin_huge_valf();
  __device__ __forceinline__ static float cvt(float x) { return x; }
};
template <> struct Store<bf16> {
  static constexpr float kLim = 0x1.ffp127f;
  __device__ __forceinline__ static bf16 cvt(float x) { return bf16{f2bf(x)}; }
};
template <> struct Store<half> {
  static constexpr float kLim = 65520.f;
  __device__ __forceinline__ static half cvt(float x) { return (half)x; }
};
// true when x, written as TO, is not a finite number (NaN, inf or beyond TO's range)
template <typename TO> __device__ __forceinline__ bool nonfinite_as(float x) { return !(fabsf(x) < Store<TO>::kLim); }

// Non-finite output flag: kernels that write a non-finite result OR their bit
// into a per-device word (nf), which retention_range_status() reads and clears.
// An fp16 operand that overflowed its range becomes inf and reaches every
// output it feeds, so this is how such an overflow surfaces.
enum : unsigned { kNonFiniteFwd = 1u, kNonFiniteBwd = 2u };
__device__ __forceinline__ void flag_nonfinite(unsigned* nf, bool bad, unsigned bit) {
  if (bad && nf) atomicOr(nf, bit);
}
// the per-device flag word (device address, looked up once per device)
hipError_t nonfinite_flag_ptr(unsigned** out);

// four consecutive outputs (8-byte aligned for 16-bit types, 16 for float)
__device__ __forceinline__ void store4(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void store4(bf16* p, const float* x) {
  uint2 u;
  u.x = pack_bf2(x[0], x[1]);
  u.y = pack_bf2(x[2], x[3]);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(half* p, const float* x) {
  typedef __attribute__((ext_vector_type(4))) _Float16 h4;
  h4 v;
  v[0] = (half)x[0]; v[1] = (half)x[1]; v[2] = (half)x[2]; v[3] = (half)x[3];
  *reinterpret_cast<h4*>(p) = v;
}

struct StepArgs {
  const void *q, *k, *v;
  float *S, *z;
  void* o;
  int b, h, dk, dv;
  int64_t pos, n_tokens;
  unsigned flags;
  ret_dtype in_dt, out_dt;
  const HeadParams* hp;
};
hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t st);

struct GateArgs {
  const void* y;
  ret_strides sy;
  const void* g;
  void* out;
  int b, L, h, dv;
  const float *w, *bias;
  float eps;
  ret_dtype y_dt, g_dt, out_dt;
};
hipError_t launch_gate_norm(const GateArgs& a, hipStream_t st);

struct ChunkArgs {
  const void *q, *k, *v;
  void* o;
  ret_strides sq, sk, sv, so;
  int b, h, L, dk, dv, B;
  int64_t pos0, n_prev;
  unsigned flags;
  ret_dtype in_dt, out_dt;
  const float *state_in, *z_in;
  float *state_out, *z_out;
  void* ws;
  size_t ws_bytes;
  const HeadParams* hp;
  unsigned* nf;     // non-finite output flag word
};
// returns false in *supported when no kernel is compiled for the shape
hipError_t launch_chunkwise(const ChunkArgs& a, hipStream_t st, bool* supported);
bool chunkwise_supported(ret_dtype in_dt, int dk, int dv);
size_t chunkwise_workspace(int b, int h, int L, int dk, int dv, int B, unsigned flags);
// true when the call takes the fused kernel with z_out overlapping z_in: the
// key-sums are then read from a snapshot in the workspace
bool fused_z_snapshot(const ChunkArgs& a);
// large-chunk path (delta / scan / output kernels)
bool three_phase_applies(ret_dtype in_dt, int dk, int dv, int B);
size_t three_phase_workspace(int b, int h, int L, int B);
hipError_t launch_three_phase(const ChunkArgs& a, hipStream_t st);

// chunkwise backward of a fresh sequence: dq, dk, dv (gq, gk, gv) from dO
struct BwdArgs {
  const void *q, *k, *v, *dout;
  void *gq, *gk, *gv;
  ret_strides sq, sk, sv, sdo, sgq, sgk, sgv;
  int b, h, L, d_k, d_v, B;
  int64_t pos0;
  unsigned flags;
  ret_dtype in_dt, grad_dt;
  void* ws;
  const HeadParams* hp;
  unsigned* nf;     // non-finite output flag word
};
bool chunkwise_bwd_supported(int dk, int dv);
size_t chunkwise_bwd_workspace(int b, int h, int L, int dk, int dv, int B);
hipError_t launch_chunkwise_bwd(const BwdArgs& a, hipStream_t st);

// R: optional residual [M][N] of c_dt added after the optional exact gelu (act != 0)
hipError_t launch_gemm(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                       const void* R, ret_dtype r_dt, int act, hipStream_t st);
// M <= 128 with K a multiple of 128: split-K through a workspace of
// gemm_workspace_bytes() bytes (0: no workspace is needed and launch_gemm runs)
size_t gemm_workspace_bytes(int M, int N, int K);
hipError_t launch_gemm_ws(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                          const void* R, ret_dtype r_dt, int act, void* ws, hipStream_t st);
// device address of the static split-K scratch of the current device
// (MSR_GEMM_SCRATCH_BYTES, looked up once per device)
hipError_t gemm_scratch_ptr(void** out);
hipError_t launch_layer_norm(const void* x, void* y, int rows, int d, const float* w, const float* bias, float eps,
                             ret_dtype x_dt, ret_dtype y_dt, hipStream_t st);

// measured ceilings (calib.hip)
hipError_t launch_calib_copy(const void* src, void* dst, size_t n16, hipStream_t st);
hipError_t launch_calib_mfma(float* out, int blocks, int iters, hipStream_t st);

}  // namespace ret
