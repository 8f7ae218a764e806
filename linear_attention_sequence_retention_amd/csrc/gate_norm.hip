// MSR epilogue before W_O (RetNet reading notes, §三.2):
//   Z = swish(G) (.) GroupNorm_h(Concat(head_1 .. head_h))
// One wave per GP (batch, token, head) groups of d_v channels: each group is
// held in registers (8 channels per lane per 512-wide slab), its mean and biased
// variance come from two wave reductions (centred second pass), and the
// normalised, gated result is written once.  HBM-bound: Y and G are read
// once and Z written once.
#include "internal.h"

namespace ret {

template <typename T> struct Vec8;
// Every byte is touched once, so the 16-bit types load and store non-temporally
// (no reuse to keep in the caches).
template <> struct Vec8<bf16> {
  __device__ __forceinline__ static void ld(const bf16* p, float* x) {
    u32x4 u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    x[0] = lo_bf(u.x); x[1] = hi_bf(u.x); x[2] = lo_bf(u.y); x[3] = hi_bf(u.y);
    x[4] = lo_bf(u.z); x[5] = hi_bf(u.z); x[6] = lo_bf(u.w); x[7] = hi_bf(u.w);
  }
  __device__ __forceinline__ static void st(bf16* p, const float* x) {
    u32x4 u;
    u.x = pack_bf2(x[0], x[1]); u.y = pack_bf2(x[2], x[3]);
    u.z = pack_bf2(x[4], x[5]); u.w = pack_bf2(x[6], x[7]);
    __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
  }
};
template <> struct Vec8<half> {
  __device__ __forceinline__ static void ld(const half* p, float* x) {
    f16x8 v = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(p));
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)v[j];
  }
  __device__ __forceinline__ static void st(half* p, const float* x) {
    f16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (half)x[j];
    __builtin_nontemporal_store(v, reinterpret_cast<f16x8*>(p));
  }
};
template <> struct Vec8<float> {
  __device__ __forceinline__ static void ld(const float* p, float* x) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w; x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
  __device__ __forceinline__ static void st(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
};

template <typename TY, typename TG, typename TO, int NI, int GP>
__global__ void __launch_bounds__(256)
gate_norm_kernel(const TY* __restrict__ y, ret_strides sy, const TG* __restrict__ g, TO* __restrict__ out,
                 int L, int h, int dv, int64_t ngroups, const float* __restrict__ w,
                 const float* __restrict__ bias, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t g0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * GP;
  if (g0 >= ngroups) return;
  // every load of the wave's GP groups is issued before the first reduction,
  // so GP * NI * 2 16-byte requests per lane are in flight together (two
  // groups of 512 measured best: more cost occupancy, 8 waves per SIMD)
  float x[GP][NI][8], gg[GP][NI][8];
  float sum[GP];
#pragma unroll
  for (int k = 0; k < GP; ++k) {
    const int64_t gi = g0 + k;
    sum[k] = 0.f;
    if (gi < ngroups) {
      const int hh = (int)(gi % h);
      const int64_t bt = gi / h;
      const TY* yp = y + (bt / L) * sy.b + hh * sy.h + (bt % L) * sy.l;
#pragma unroll
      for (int it = 0; it < NI; ++it) {
        const int e = 8 * lane + 512 * it;
        if (e < dv) {
          Vec8<TY>::ld(yp + e, x[k][it]);
          Vec8<TG>::ld(g + gi * dv + e, gg[k][it]);
        }
      }
    }
  }
  const float inv_n = 1.f / (float)dv;
  float mean[GP], rstd[GP];
#pragma unroll
  for (int k = 0; k < GP; ++k) {
#pragma unroll
    for (int it = 0; it < NI; ++it)
      if (8 * lane + 512 * it < dv) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sum[k] += x[k][it][j];
      }
    mean[k] = wave_sum(sum[k]) * inv_n;
  }
#pragma unroll
  for (int k = 0; k < GP; ++k) {
    float sq = 0.f;
#pragma unroll
    for (int it = 0; it < NI; ++it)
      if (8 * lane + 512 * it < dv) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float d = x[k][it][j] - mean[k];
          sq += d * d;
        }
      }
    rstd[k] = rsqrtf(wave_sum(sq) * inv_n + eps);
  }
#pragma unroll
  for (int k = 0; k < GP; ++k) {
    const int64_t gi = g0 + k;
    if (gi >= ngroups) break;
    const int hh = (int)(gi % h);
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      const int e = 8 * lane + 512 * it;
      if (e < dv) {
        float r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float yn = (x[k][it][j] - mean[k]) * rstd[k];
          const int c = hh * dv + e + j;
          if (w) yn *= w[c];
          if (bias) yn += bias[c];
          const float sw = gg[k][it][j] / (1.f + __expf(-gg[k][it][j]));
          r[j] = sw * yn;
        }
        Vec8<TO>::st(out + gi * dv + e, r);
      }
    }
  }
}

template <typename TY, typename TG, typename TO>
static hipError_t launch_gn_t(const GateArgs& a, hipStream_t st) {
  const int64_t ng = (int64_t)a.b * a.L * a.h;
  const int ni = (a.dv + 511) / 512;
#define RET_GN(NI, GP)                                                                               \
  hipLaunchKernelGGL((gate_norm_kernel<TY, TG, TO, NI, GP>), dim3((unsigned)((ng + 4 * GP - 1) / (4 * GP))), \
                     dim3(256), 0, st, (const TY*)a.y, a.sy, (const TG*)a.g, (TO*)a.out, a.L, a.h, a.dv, ng, \
                     a.w, a.bias, a.eps)
  if (ni <= 1) RET_GN(1, 2);
  else if (ni <= 2) RET_GN(2, 1);
  else if (ni <= 4) RET_GN(4, 1);
  else RET_GN(8, 1);
#undef RET_GN
  return hipGetLastError();
}

template <typename TY, typename TG>
static hipError_t launch_gn_o(const GateArgs& a, hipStream_t st) {
  if (a.out_dt == RET_BF16) return launch_gn_t<TY, TG, bf16>(a, st);
  if (a.out_dt == RET_F16) return launch_gn_t<TY, TG, half>(a, st);
  return launch_gn_t<TY, TG, float>(a, st);
}
template <typename TY>
static hipError_t launch_gn_g(const GateArgs& a, hipStream_t st) {
  if (a.g_dt == RET_BF16) return launch_gn_o<TY, bf16>(a, st);
  if (a.g_dt == RET_F16) return launch_gn_o<TY, half>(a, st);
  return launch_gn_o<TY, float>(a, st);
}
// ---------------------------------------------------------------- LayerNorm
// The two LayerNorms of the RetNet layer (reading notes §三.4: Y = MSR(LN(X))
// + X, X' = FFN(LN(Y)) + Y): each row of d values (one token) is normalised by
// its mean and biased variance (eps added to the variance), then the optional
// per-channel affine.  One wave per row, the row in registers (8 values per
// lane per 512-wide slab); HBM-bound: x read once, y written once.
template <typename TX, typename TY, int NI>
__global__ void __launch_bounds__(256)
layer_norm_kernel(const TX* __restrict__ x, TY* __restrict__ y, int rows, int d, const float* __restrict__ w,
                  const float* __restrict__ bias, float eps) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const TX* xp = x + row * d;
  float v[NI][8];
  float sum = 0.f;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = 8 * lane + 512 * it;
    if (e < d) {
      Vec8<TX>::ld(xp + e, v[it]);
#pragma unroll
      for (int j = 0; j < 8; ++j) sum += v[it][j];
    }
  }
  const float inv_n = 1.f / (float)d;
  const float mean = wave_sum(sum) * inv_n;
  float sq = 0.f;
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = 8 * lane + 512 * it;
    if (e < d) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float t = v[it][j] - mean;
        sq += t * t;
      }
    }
  }
  const float rstd = rsqrtf(wave_sum(sq) * inv_n + eps);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int e = 8 * lane + 512 * it;
    if (e < d) {
      float r[8], wv[8], bv[8];
      if (w) Vec8<float>::ld(w + e, wv);
      if (bias) Vec8<float>::ld(bias + e, bv);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float t = (v[it][j] - mean) * rstd;
        if (w) t *= wv[j];
        if (bias) t += bv[j];
        r[j] = t;
      }
      Vec8<TY>::st(y + row * d + e, r);
    }
  }
}

template <typename TX, typename TY>
static hipError_t launch_ln_t(const void* x, void* y, int rows, int d, const float* w, const float* bias, float eps,
                              hipStream_t st) {
  dim3 grid((unsigned)((rows + 3) / 4));
  const int ni = (d + 511) / 512;
#define RET_LN(NI)                                                                                         \
  hipLaunchKernelGGL((layer_norm_kernel<TX, TY, NI>), grid, dim3(256), 0, st, (const TX*)x, (TY*)y, rows, d, \
                     w, bias, eps)
  if (ni <= 1) RET_LN(1);
  else if (ni <= 2) RET_LN(2);
  else if (ni <= 4) RET_LN(4);
  else if (ni <= 8) RET_LN(8);
  else RET_LN(16);
#undef RET_LN
  return hipGetLastError();
}

template <typename TX>
static hipError_t launch_ln_o(const void* x, void* y, int rows, int d, const float* w, const float* bias, float eps,
                              ret_dtype y_dt, hipStream_t st) {
  if (y_dt == RET_BF16) return launch_ln_t<TX, bf16>(x, y, rows, d, w, bias, eps, st);
  if (y_dt == RET_F16) return launch_ln_t<TX, half>(x, y, rows, d, w, bias, eps, st);
  return launch_ln_t<TX, float>(x, y, rows, d, w, bias, eps, st);
}

hipError_t launch_layer_norm(const void* x, void* y, int rows, int d, const float* w, const float* bias, float eps,
                             ret_dtype x_dt, ret_dtype y_dt, hipStream_t st) {
  if (x_dt == RET_BF16) return launch_ln_o<bf16>(x, y, rows, d, w, bias, eps, y_dt, st);
  if (x_dt == RET_F16) return launch_ln_o<half>(x, y, rows, d, w, bias, eps, y_dt, st);
  return launch_ln_o<float>(x, y, rows, d, w, bias, eps, y_dt, st);
}

hipError_t launch_gate_norm(const GateArgs& a, hipStream_t st) {
  if (a.y_dt == RET_BF16) return launch_gn_g<bf16>(a, st);
  if (a.y_dt == RET_F16) return launch_gn_g<half>(a, st);
  return launch_gn_g<float>(a, st);
}

}  // namespace ret
