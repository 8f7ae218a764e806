// Shared device helpers for the gfx950 retention kernels: storage types,
// bf16 conversion, MFMA fragment conventions, wave reductions, and the
// per-head scalars derived from the decay gamma.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "retention.h"

namespace ret {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;   // 16-byte raw piece (a native vector, so arrays of it stay in registers)
typedef __attribute__((ext_vector_type(8))) float f32x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef _Float16 half;

struct bf16 { uint16_t bits; };   // storage-only bf16

constexpr int kMaxHeads = 64;
constexpr int kMaxPairs = 256;    // d_k <= 512

// Host-side constants copied into kernel arguments.  gamma and theta are the
// caller's float64 values; everything else is derived on the device.
struct HeadParams {
  double gamma[kMaxHeads];
  double theta[kMaxPairs];
  // per-head decay scalars, from gamma in float64 on the host, rounded once:
  // lg2 = log2(gamma), omg = 1 - gamma, lng = ln(gamma) (see Decay)
  float lg2[kMaxHeads], omg[kMaxHeads], lng[kMaxHeads];
};

__device__ __forceinline__ float bf2f(uint16_t u) { return __uint_as_float((uint32_t)u << 16); }
__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint16_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);   // v_cvt_pk_bf16_f32: round to nearest even
}
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  bf16x2 v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Element loaders for the two input storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float ld(const float* p) { return *p; }
  // two consecutive elements (an xPos pair)
  __device__ __forceinline__ static float2 ld2(const float* p) { return *reinterpret_cast<const float2*>(p); }
};
template <> struct Elem<bf16> {
  __device__ __forceinline__ static float ld(const bf16* p) { return bf2f(p->bits); }
  __device__ __forceinline__ static float2 ld2(const bf16* p) {
    uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    return make_float2(lo_bf(u), hi_bf(u));
  }
};
template <> struct Elem<_Float16> {
  __device__ __forceinline__ static float ld(const _Float16* p) { return (float)*p; }
  __device__ __forceinline__ static float2 ld2(const _Float16* p) {
    typedef __attribute__((ext_vector_type(2))) _Float16 h2;
    h2 v = *reinterpret_cast<const h2*>(p);
    return make_float2((float)v.x, (float)v.y);
  }
};

// ---------------------------------------------------------------------------
// Per-head scalars.  All of them come from gamma in float64 (on the host,
// in HeadParams) and are rounded to float32 once.  lg2 = log2(gamma) feeds gamma^k = exp2(k * lg2); omg = 1 -
// gamma (exact for the 1 - 2^-k ladder); lng = ln(gamma) feeds
// 1 - gamma^n = -expm1(n * lng), which keeps full relative accuracy when
// gamma^n is close to 1 (gamma = 1 - 2^-20 at n = 1).
// ---------------------------------------------------------------------------
struct Decay {
  float lg2, omg, lng;
  __device__ __forceinline__ void init(const HeadParams& hp, int head) {
    lg2 = hp.lg2[head];
    omg = hp.omg[head];
    lng = hp.lng[head];
  }
  __device__ __forceinline__ float pow(float k) const { return exp2f(k * lg2); }
  // D-row factor sqrt((1-gamma)/(1-gamma^n)) for a row that has seen n tokens
  // (the D row sum is the geometric series (1-gamma^n)/(1-gamma)).
  __device__ __forceinline__ float drow(float n) const { return sqrtf(omg / (-expm1f(n * lng))); }
};

// xPos phase e^{i p theta}: range-reduce p*theta in float64, then an fp32
// sincos of the reduced angle (|r| <= pi, error ~1e-7 rad).
__device__ __forceinline__ void phase(int64_t p, double theta, float& c, float& s) {
  const double two_pi = 6.283185307179586476925286766559;
  double a = (double)p * theta;
  double k = rint(a * (1.0 / two_pi));
  double r = fma(-k, two_pi, a);
  r = fma(-k, 2.4492935982947064e-16, r);   // low part of 2*pi
  sincosf((float)r, &s, &c);
}

// Rotate a pair (x0, x1) by (c, s): the real form of (x0 + i x1) e^{i phi}.
__device__ __forceinline__ void rot(float& x0, float& x1, float c, float s) {
  float y0 = x0 * c - x1 * s;
  float y1 = x0 * s + x1 * c;
  x0 = y0;
  x1 = y1;
}
// Advance a phase by a fixed step: (c + i s) * (c1 + i s1).
__device__ __forceinline__ void advance(float& c, float& s, float c1, float s1) {
  float nc = c * c1 - s * s1;
  float ns = c * s1 + s * c1;
  c = nc;
  s = ns;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// ---------------------------------------------------------------------------
// MFMA 32x32 with a 16-deep k block.  Fragment convention shared by A and B:
// lane l supplies row (A) / column (B) l%32 and the 8 consecutive k values
// 8*(l/32) .. 8*(l/32)+7 of the block.  The accumulator lane l, register r
// holds C[8*(r/4) + 4*(l/32) + r%4][l%32].
// bf16 operands use one v_mfma_f32_32x32x16_bf16; float operands use eight
// v_mfma_f32_32x32x2_f32, the e-th taking element e of each lane (so lane
// half h supplies k = 8h + e), which covers the same 16-deep block.
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  typedef bf16x8 frag;
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16* p) {   // 16-byte aligned
    return *reinterpret_cast<const frag*>(p);
  }
};
template <> struct Mfma<half> {
  typedef f16x8 frag;
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const half* p) {   // 16-byte aligned
    return *reinterpret_cast<const frag*>(p);
  }
};
template <> struct Mfma<float> {
  typedef f32x8 frag;
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b[e], c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const float* p) {  // 32-byte aligned
    f32x4 lo = *reinterpret_cast<const f32x4*>(p);
    f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
    frag f;
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    return f;
  }
};

// MFMA operand type used for an input storage type: float inputs stay
// float (v_mfma_f32_32x32x2_f32); bf16 inputs are contracted as fp16
// (v_mfma_f32_32x32x16_f16, the same rate as bf16), whose 11-bit significand
// keeps the roundings of the rotated q/k, of the scores and of the state copy
// 8x smaller than bf16 operands would.  Every bf16 input value inside the
// fp16 range converts exactly.
template <typename T> struct OpOf { typedef float type; };
template <> struct OpOf<bf16> { typedef half type; };
template <> struct OpOf<half> { typedef half type; };

// conversions between the compute float and the LDS operand type (RNE)
template <typename T> __device__ __forceinline__ T to_op(float x);
template <> __device__ __forceinline__ float to_op<float>(float x) { return x; }
template <> __device__ __forceinline__ half to_op<half>(float x) { return (half)x; }
template <typename T> __device__ __forceinline__ float from_op(T x);
template <> __device__ __forceinline__ float from_op<float>(float x) { return x; }
template <> __device__ __forceinline__ float from_op<half>(half x) { return (float)x; }

// store two consecutive operands
__device__ __forceinline__ void st2(float* p, float a, float b) { *reinterpret_cast<float2*>(p) = make_float2(a, b); }
__device__ __forceinline__ void st2(half* p, float a, float b) {
  f16x2 v;
  v.x = (half)a;
  v.y = (half)b;
  *reinterpret_cast<f16x2*>(p) = v;
}
// store eight consecutive operands (16-byte aligned)
__device__ __forceinline__ void st8(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  *reinterpret_cast<f32x4*>(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}
__device__ __forceinline__ void st8(half* p, const float* x) {
  f16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (half)x[e];
  *reinterpret_cast<f16x8*>(p) = v;
}
// store four consecutive operands (8-byte aligned for half, 16 for float)
__device__ __forceinline__ void st4(float* p, const float* x) {
  *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
}
__device__ __forceinline__ void st4(half* p, const float* x) {
  f16x4 v;
  v[0] = (half)x[0]; v[1] = (half)x[1]; v[2] = (half)x[2]; v[3] = (half)x[3];
  *reinterpret_cast<f16x4*>(p) = v;
}

__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

}  // namespace ret
