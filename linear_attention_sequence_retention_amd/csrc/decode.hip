// One decode step of the recurrent form (RetNet reading notes, §2.2):
//   S <- gamma S + k'^T v,  o = q' S      (the current token included)
// with the xPos rotation of §2.3 and the row scalings of §三.3.
//
// The step is a pure HBM stream: S (d_k x d_v float32 per head) is read and
// written once, 8 bytes of traffic for 4 flops per element.  One workgroup
// owns one (batch, head); each thread owns 4 consecutive columns (one 16-byte
// vector per row) and a strided set of rows, so every wave reads and writes
// contiguous 1 KiB row segments.  q' S is reduced over the rows in registers,
// then across the row groups through LDS.
#include "internal.h"

namespace ret {

template <typename TI, typename TO, int TPB>
__global__ void __launch_bounds__(TPB)
recurrent_step_kernel(const TI* __restrict__ q, const TI* __restrict__ k, const TI* __restrict__ v,
                      float* __restrict__ S, float* __restrict__ z, TO* __restrict__ o,
                      int h, int dk, int dv, int64_t pos, int64_t n_tokens, unsigned flags,
                      HeadParams hp) {
  extern __shared__ float smem[];
  float* qs = smem;             // rotated q [dk]
  float* ks = smem + dk;        // rotated k [dk]
  float* red = smem + 2 * dk;   // [row groups][dv] partial sums, then the den scalar
  const int bh = blockIdx.x;
  const int head = bh % h;
  const int tid = threadIdx.x;
  const double g64 = hp.gamma[head];
  const float gam = (float)g64;

  const TI* qp = q + (int64_t)bh * dk;
  const TI* kp = k + (int64_t)bh * dk;
  for (int j = tid; j < dk / 2; j += TPB) {
    float2 qq = Elem<TI>::ld2(qp + 2 * j);
    float2 kk = Elem<TI>::ld2(kp + 2 * j);
    if (flags & RET_XPOS) {
      float c, s;
      phase(pos, hp.theta[j], c, s);
      rot(qq.x, qq.y, c, s);
      rot(kk.x, kk.y, c, s);
    }
    qs[2 * j] = qq.x; qs[2 * j + 1] = qq.y;
    ks[2 * j] = kk.x; ks[2 * j + 1] = kk.y;
  }
  __syncthreads();

  // key-sum z <- gamma z + k' and den = q' . z (the unscaled score row sum)
  float den = 0.f;
  if (z != nullptr) {
    float part = 0.f;
    float* zp = z + (int64_t)bh * dk;
    for (int d = tid; d < dk; d += TPB) {
      float zn = gam * zp[d] + ks[d];
      zp[d] = zn;
      part += qs[d] * zn;
    }
    part = wave_sum(part);
    __shared__ float wpart[TPB / 64];
    if ((tid & 63) == 0) wpart[tid >> 6] = part;
    __syncthreads();
    for (int w = 0; w < TPB / 64; ++w) den += wpart[w];
  }

  // state stream: thread -> 4 columns, rows rg, rg + RG, ...
  const int tpr = dv / 4;                 // threads per row
  const int RG = TPB / tpr;               // row groups (>= 1)
  const int rg = tid / tpr;
  const int c4 = tid % tpr;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  if (rg < RG) {
    const TI* vp = v + (int64_t)bh * dv + 4 * c4;
    f32x4 vv = {Elem<TI>::ld(vp), Elem<TI>::ld(vp + 1), Elem<TI>::ld(vp + 2), Elem<TI>::ld(vp + 3)};
    f32x4* Sp = reinterpret_cast<f32x4*>(S + (int64_t)bh * dk * dv) + c4;
    const int stride4 = dv / 4;
    constexpr int U = 8;
    int i = rg;
    for (; i + (U - 1) * RG < dk; i += U * RG) {
      f32x4 s[U];
#pragma unroll
      for (int u = 0; u < U; ++u) s[u] = __builtin_nontemporal_load(Sp + (int64_t)(i + u * RG) * stride4);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = i + u * RG;
        const float kr = ks[row], qr = qs[row];
        s[u] = gam * s[u] + kr * vv;
        acc += qr * s[u];
        __builtin_nontemporal_store(s[u], Sp + (int64_t)row * stride4);
      }
    }
    for (; i < dk; i += RG) {
      f32x4 s = Sp[(int64_t)i * stride4];
      const float kr = ks[i], qr = qs[i];
      s = gam * s + kr * vv;
      acc += qr * s;
      Sp[(int64_t)i * stride4] = s;
    }
  }
  // reduce over row groups
  if (RG > 1) {
    if (rg < RG) *reinterpret_cast<f32x4*>(red + rg * dv + 4 * c4) = acc;
    __syncthreads();
    if (rg == 0) {
      for (int r = 1; r < RG; ++r) {
        acc += *reinterpret_cast<const f32x4*>(red + r * dv + 4 * c4);
      }
    }
  }
  if (rg == 0) {
    Decay dec;
    dec.init(hp, head);
    float sc = 1.f;
    if (flags & RET_SCALE_QK) sc *= rsqrtf((float)dk);
    if (flags & RET_NORM_DROW) sc *= dec.drow((float)n_tokens);
    float mul = sc;
    if (flags & RET_NORM_SCORE) mul = sc / fmaxf(fabsf(sc * den), 1.f);
    TO* op = o + (int64_t)bh * dv + 4 * c4;
    op[0] = Store<TO>::cvt(acc[0] * mul);
    op[1] = Store<TO>::cvt(acc[1] * mul);
    op[2] = Store<TO>::cvt(acc[2] * mul);
    op[3] = Store<TO>::cvt(acc[3] * mul);
  }
}

template <typename TI, typename TO>
static hipError_t launch_step_t(const StepArgs& a, hipStream_t st) {
  // 512 threads: at d_v = 512 four row groups of 64 rows, eight 16-byte
  // loads in flight per thread (measured best of 128 / 256 / 512 / 1024)
  constexpr int TPB = 512;
  const int tpr = a.dv / 4;
  const int RG = tpr >= TPB ? 1 : TPB / tpr;
  size_t sh = sizeof(float) * (2 * (size_t)a.dk + (size_t)RG * a.dv);
  dim3 grid(a.b * a.h);
  hipLaunchKernelGGL((recurrent_step_kernel<TI, TO, TPB>), grid, dim3(TPB), sh, st,
                     (const TI*)a.q, (const TI*)a.k, (const TI*)a.v, a.S, a.z, (TO*)a.o,
                     a.h, a.dk, a.dv, a.pos, a.n_tokens, a.flags, *a.hp);
  return hipGetLastError();
}

template <typename TI>
static hipError_t launch_step_i(const StepArgs& a, hipStream_t st) {
  if (a.out_dt == RET_BF16) return launch_step_t<TI, bf16>(a, st);
  if (a.out_dt == RET_F16) return launch_step_t<TI, half>(a, st);
  return launch_step_t<TI, float>(a, st);
}

hipError_t launch_recurrent_step(const StepArgs& a, hipStream_t st) {
  if (a.in_dt == RET_BF16) return launch_step_i<bf16>(a, st);
  if (a.in_dt == RET_F16) return launch_step_i<half>(a, st);
  return launch_step_i<float>(a, st);
}

}  // namespace ret
