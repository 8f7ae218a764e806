// Chunkwise backward of the normalised retention (RetNet reading notes §2.4,
// with the xPos rotation of §2.3 and the normalisations of §三.3): dq, dk and
// dv of a fresh sequence from dL/dO.  Nothing is detached; on the clamp's
// boundary |s den| = 1 its constant branch is taken.
//
// With q', k' the rotated inputs, g_p = dL/do_p and, for m <= p,
//   A_pm = (q'_p . k'_m) gamma^(p-m),  num_p = sum_m A_pm v_m,  den_p = sum_m A_pm,
//   o_p  = s_p num_p / n_p,  n_p = max(|s_p den_p|, 1) (1 without the score normalisation),
// the chain rule reads
//   a_p  = s_p / n_p,  c_p = -s_p^2 sign(den_p) (g_p . num_p) / n_p^2 where |s_p den_p| > 1, else 0,
//   E_pm = gamma^(p-m) (a_p g_p . v_m + c_p)                (dL / d(q'_p . k'_m)),
//   dq'_p = sum_m E_pm k'_m,  dk'_m = sum_p E_pm q'_p,  dv_m = sum_p a_p A_pm g_p.
// Chunk c covers rows [c0, c1).  Terms reaching into earlier chunks go
// through the forward state R_c = sum_{m<c0} gamma^(c0-1-m) k'_m v_m^T (and
// the key-sum z_c); terms reaching into later chunks through the reverse
// state U_c = sum_{p>=c1} gamma^(p-c1) q'_p (a_p g_p)^T (and u_c, weighted by c_p):
//   dq'_p += gamma^(p-c0+1) (a_p R_c g_p + c_p z_c)
//   dk'_m += gamma^(c1-m) (U_c v_m + u_c),   dv_m += gamma^(c1-m) U_c^T k'_m
//   den_p += gamma^(p-c0+1) q'_p . z_c,      g_p . num_p += gamma^(p-c0+1) (q'_p R_c) . g_p
// and dq, dk are dq', dk' rotated back by -p theta.
//
// Kernels, in order: prep (rotated q', k' and fp16 copies of v, dO, once),
// fstate (R_c, z_c: a scan over the chunks), dq (with the score normalisation
// it also finds a_p, c_p), rstate (U_c, u_c: a scan over the chunks from the
// end), then dk and dv, one 64-row tile per workgroup.  Every product is
// an fp16 v_mfma_f32_32x32x16 with fp32 accumulation on 64-row tiles staged in
// LDS (fp16's 11-bit significand: bf16 operands would make the roundings of
// q', k' and of the E / a A tiles 8x larger).  Range: every gradient is linear
// in dO, so dO is scaled per (batch, head) by a power of two that brings its
// largest magnitude into [1/2, 1) (gmax + prep) and the results are scaled
// back exactly; each 64 x 64 slab of a state copied to fp16 gets its own
// power of two, undone when its product is added to the fp32 accumulator.
// The remaining preconditions are the forward's (|q|, |k| < 2^15, |v| < 2^16,
// s_p |q'_p . k'_m| < 2^16) and |a_p (g_p . v_m) + c_p|, s_p |g_p . v_m| < 2^15
// for the scaled dO.
// A workgroup is 4 waves; wave w owns the 32 x 32 block (w / 2, w % 2) of
// each 64 x 64 output tile.
#include "internal.h"

namespace ret {

namespace {

constexpr int BT = 256;        // threads per workgroup
constexpr int TL = 64;         // rows per tile
constexpr int SP = TL + 8;     // pitch (elements) of a 64-column LDS slab
constexpr int SCAN_DVB = 128; // widest column block of the state scans (128 measured ahead of 64 and 256)

typedef short s16x4 __attribute__((__vector_size__(8)));
typedef short s16x8 __attribute__((__vector_size__(16)));

struct BwdP {
  const void *q, *k, *v, *dout;
  void *dq, *dk, *dv;
  ret_strides sq, sk, sv, sdo, sdq, sdk, sdv;
  int h, L, B, nc, nt;           // nt: 64-row tiles of the sequence
  int64_t pos0;
  unsigned flags;
  uint16_t *Qr, *Kr, *Vb, *Gb;   // fp16 [bh][L][d]: q', k', v, 2^-e dO
  float *tmax, *gsc;             // [bh][nt] tile maxima of |dO|; [bh] the 2^e of each head
  float *rmax, *umax;            // [bh][nc][partial maxima] of |R_c| and |U_c|
  float *Rin, *zin, *Ust, *ust;  // [bh][nc][DK][DV] and [bh][nc][DK]
  float *ra, *rc;                // [bh][L]: a_p and c_p (with the score normalisation)
  unsigned* nf;                  // non-finite output flag word
};

// ------------------------------------------------------------ fp16 packing
__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  f16x2 v;
  v.x = (half)lo;
  v.y = (half)hi;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float h_lo(uint32_t u) { return (float)__builtin_bit_cast(f16x2, u).x; }
__device__ __forceinline__ float h_hi(uint32_t u) { return (float)__builtin_bit_cast(f16x2, u).y; }
__device__ __forceinline__ float h2f(uint16_t u) { return (float)__builtin_bit_cast(half, u); }
__device__ __forceinline__ uint16_t f2h(float x) { return __builtin_bit_cast(uint16_t, (half)x); }

// ------------------------------------------------------------ fragments
// A/B operand of v_mfma_f32_32x32x16_f16: lane l supplies row (A) or column
// (B) l % 32 and the 8 consecutive k values 8 (l / 32) .. 8 (l / 32) + 7.
// "nt": the LDS tile is stored [x][k] (k contiguous): one 16-byte read.
__device__ __forceinline__ f16x8 fr_nt(const uint16_t* t, int pitch, int x0, int k0, int lane) {
  return *reinterpret_cast<const f16x8*>(t + (x0 + (lane & 31)) * pitch + k0 + 8 * (lane >> 5));
}
// "tr": the LDS tile is stored [k][x].  ds_read_b64_tr_b16: within each group
// of 16 lanes, lane i returns element (i & 3) of the 8-byte rows addressed by
// lanes (i >> 2) + 4t, t = 0..3.  Lane j of group g addresses row
// k0 + 8 (g / 2) + (j >> 2) at column x0 + 16 (g % 2) + 4 (j & 3), so lane i
// receives rows k .. k + 3 at column x0 + 16 (g % 2) + i = x0 + l % 32; a
// second read 4 rows further gives k + 4 .. k + 7.
__device__ __forceinline__ f16x8 fr_tr(const uint16_t* t, int pitch, int x0, int k0, int lane) {
  const int g = lane >> 4, j = lane & 15;
  const uint16_t* p = t + (k0 + 8 * (g >> 1) + (j >> 2)) * pitch + x0 + 16 * (g & 1) + 4 * (j & 3);
  s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p + 4 * pitch));
  s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(f16x8, r);
}

// acc += A B^T over a 64-deep k range: A rows xa .. xa + 31, B columns
// xb .. xb + 31; ATR / BTR select the stored orientation of each operand
template <bool ATR, bool BTR>
__device__ __forceinline__ void mm64(f32x16& acc, const uint16_t* A, int pa, int xa, const uint16_t* B, int pb,
                                     int xb, int lane) {
#pragma unroll
  for (int k0 = 0; k0 < 64; k0 += 16) {
    const f16x8 a = ATR ? fr_tr(A, pa, xa, k0, lane) : fr_nt(A, pa, xa, k0, lane);
    const f16x8 b = BTR ? fr_tr(B, pb, xb, k0, lane) : fr_nt(B, pb, xb, k0, lane);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc, 0, 0, 0);
  }
}

// ------------------------------------------------------------ staging
// rows [0, 64) x columns [0, NC) of an fp16 array (row length ld) -> LDS
// [64][pitch]; rows >= nvalid are zero; scale (LDS, per row) multiplies a
// row.  The loads are issued in batches of up to 8 per thread before their
// stores, unconditionally (rows clamped, then selected), so they overlap.
template <int NC>
__device__ __forceinline__ void stage(uint16_t* dst, int pitch, const uint16_t* src, int ld, int nvalid,
                                      const float* scale) {
  constexpr int PR = NC / 8, NPC = TL * PR / BT, NBAT = NPC < 8 ? NPC : 8;
  static_assert(NPC % NBAT == 0, "pieces per thread");
#pragma unroll
  for (int b0 = 0; b0 < NPC; b0 += NBAT) {
    u32x4 v[NBAT];
#pragma unroll
    for (int u = 0; u < NBAT; ++u) {
      const int i = threadIdx.x + (b0 + u) * BT, r = i / PR, c8 = i - r * PR;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)min(r, nvalid - 1) * ld + 8 * c8);
      v[u] = r < nvalid ? x : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NBAT; ++u) {
      const int i = threadIdx.x + (b0 + u) * BT, r = i / PR, c8 = i - r * PR;
      u32x4 x = v[u];
      if (scale) {
        const float f = scale[r];
        x.x = pack_h2(h_lo(x.x) * f, h_hi(x.x) * f);
        x.y = pack_h2(h_lo(x.y) * f, h_hi(x.y) * f);
        x.z = pack_h2(h_lo(x.z) * f, h_hi(x.z) * f);
        x.w = pack_h2(h_lo(x.w) * f, h_hi(x.w) * f);
      }
      *reinterpret_cast<u32x4*>(dst + r * pitch + 8 * c8) = x;
    }
  }
}

// the positive row scale s_p of a row that has seen n tokens (§三.3, first two factors)
__device__ __forceinline__ float row_scale(const Decay& dec, unsigned flags, float qk, int64_t n) {
  float s = qk;
  if (flags & RET_NORM_DROW) s *= dec.drow((float)n);
  return s;
}

// a_p and c_p of row p (p < L)
__device__ __forceinline__ void row_ac(const BwdP& p, const Decay& dec, float qk, int bh, int row, float& a,
                                       float& c) {
  // the loads are unconditional (a select follows) so that the wait counts of
  // the loads in flight around them stay exact
  const float la = p.ra[(int64_t)bh * p.L + row], lc = p.rc[(int64_t)bh * p.L + row];
  const bool sn = (p.flags & RET_NORM_SCORE) != 0;
  a = sn ? la : row_scale(dec, p.flags, qk, row + 1);
  c = sn ? lc : 0.f;
}

template <typename TG> struct Out2;
template <> struct Out2<float> {
  __device__ __forceinline__ static void st(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
  }
};
template <> struct Out2<bf16> {
  __device__ __forceinline__ static void st(bf16* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = pack_bf2(a, b);
  }
};

// eight 16-bit values of T (bf16 or fp16) packed in 16 bytes, as floats
template <typename T> __device__ __forceinline__ float2 un2(uint32_t u);
template <> __device__ __forceinline__ float2 un2<bf16>(uint32_t u) { return make_float2(lo_bf(u), hi_bf(u)); }
template <> __device__ __forceinline__ float2 un2<half>(uint32_t u) { return make_float2(h_lo(u), h_hi(u)); }

// ------------------------------------------------------------ gmax
// the largest |dO| of each 64-row tile (16-byte loads: rows are 16-byte
// aligned and d_v is a multiple of 8)
template <typename T, int DV>
__global__ void __launch_bounds__(BT) bwd_gmax_kernel(BwdP p) {
  const int bh = blockIdx.x / p.nt, tile = blockIdx.x % p.nt;
  const int bb = bh / p.h, hh = bh % p.h;
  const int r0 = tile * TL, nv = min(TL, p.L - r0);
  const T* g = reinterpret_cast<const T*>(p.dout) + bb * p.sdo.b + hh * p.sdo.h + r0 * p.sdo.l;
  constexpr int V8 = DV / 8;
  float m = 0.f;
  for (int i = threadIdx.x; i < nv * V8; i += BT) {
    const int r = i / V8, c8 = i - r * V8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(g + (int64_t)r * p.sdo.l + 8 * c8);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 y = un2<T>(w[u]);
      m = fmaxf(m, fmaxf(fabsf(y.x), fabsf(y.y)));
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  __shared__ float red[BT / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) p.tmax[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// ------------------------------------------------------------ prep
// q', k' (rotated), v and 2^-e dO as contiguous fp16 rows, and 2^e of the head
template <typename T, int DK, int DV>
__global__ void __launch_bounds__(BT) bwd_prep_kernel(BwdP p, HeadParams hp) {
  const int bh = blockIdx.x / p.nt, tile = blockIdx.x % p.nt;
  const int bb = bh / p.h, hh = bh % p.h;
  const int r0 = tile * TL, nv = min(TL, p.L - r0);
  const T* q = reinterpret_cast<const T*>(p.q) + bb * p.sq.b + hh * p.sq.h + r0 * p.sq.l;
  const T* k = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + hh * p.sk.h + r0 * p.sk.l;
  const T* v = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + hh * p.sv.h + r0 * p.sv.l;
  const T* g = reinterpret_cast<const T*>(p.dout) + bb * p.sdo.b + hh * p.sdo.h + r0 * p.sdo.l;
  const int64_t ro = (int64_t)bh * p.L + r0;
  constexpr int PAIRS = DK / 2, RPP = BT / PAIRS;
  const int j = threadIdx.x % PAIRS, i0 = threadIdx.x / PAIRS;
  const bool xpos = (p.flags & RET_XPOS) != 0;
  float c = 1.f, s = 0.f, c1 = 1.f, s1 = 0.f;
  if (xpos) {
    phase(p.pos0 + r0 + i0, hp.theta[j], c, s);
    phase(RPP, hp.theta[j], c1, s1);
  }
  for (int i = i0; i < nv; i += RPP) {
    float2 x = Elem<T>::ld2(q + (int64_t)i * p.sq.l + 2 * j);
    float2 y = Elem<T>::ld2(k + (int64_t)i * p.sk.l + 2 * j);
    if (xpos) {
      rot(x.x, x.y, c, s);
      rot(y.x, y.y, c, s);
      advance(c, s, c1, s1);
    }
    *reinterpret_cast<uint32_t*>(p.Qr + (ro + i) * DK + 2 * j) = pack_h2(x.x, x.y);
    *reinterpret_cast<uint32_t*>(p.Kr + (ro + i) * DK + 2 * j) = pack_h2(y.x, y.y);
  }
  // the head's power of two: 2^-e puts max |dO| in [1/2, 1)
  __shared__ float red[BT / 64];
  float m = 0.f;
  for (int t = threadIdx.x; t < p.nt; t += BT) m = fmaxf(m, p.tmax[(int64_t)bh * p.nt + t]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int ex = 0;
  if (m > 0.f && m < 3.0e38f) {
    frexpf(m, &ex);
    ex = min(max(ex, -120), 120);
  }
  const float down = ldexpf(1.f, -ex);
  if (tile == 0 && threadIdx.x == 0) p.gsc[bh] = ldexpf(1.f, ex);
  constexpr int V8 = DV / 8;
  for (int i = threadIdx.x; i < nv * V8; i += BT) {
    const int r = i / V8, c8 = i - r * V8;
    const u32x4 x = *reinterpret_cast<const u32x4*>(v + (int64_t)r * p.sv.l + 8 * c8);
    const u32x4 y = *reinterpret_cast<const u32x4*>(g + (int64_t)r * p.sdo.l + 8 * c8);
    const uint32_t xw[4] = {x.x, x.y, x.z, x.w}, yw[4] = {y.x, y.y, y.z, y.w};
    uint32_t xo[4], yo[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float2 a = un2<T>(xw[u]), b = un2<T>(yw[u]);
      xo[u] = pack_h2(a.x, a.y);
      yo[u] = pack_h2(b.x * down, b.y * down);
    }
    *reinterpret_cast<u32x4*>(p.Vb + (ro + r) * DV + 8 * c8) = u32x4{xo[0], xo[1], xo[2], xo[3]};
    *reinterpret_cast<u32x4*>(p.Gb + (ro + r) * DV + 8 * c8) = u32x4{yo[0], yo[1], yo[2], yo[3]};
  }
}

// ------------------------------------------------------------ slab pipeline
// Operand slabs of 64 rows x 64 columns move global -> registers -> LDS with
// one slab in flight: slab i + 1 is loaded into registers while slab i is
// multiplied, and two LDS buffers alternate by a running slab count, so one
// barrier per slab separates a buffer's writes from its reads two slabs
// earlier.
struct H16 {          // an fp16 slab: 2 x 16 bytes per thread; rows >= nvalid read as zero
  u32x4 v[2];
  __device__ __forceinline__ void load(const uint16_t* src, int ld, int nvalid) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * BT, r = i >> 3, c8 = i & 7;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)min(r, nvalid - 1) * ld + 8 * c8);
      v[u] = r < nvalid ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst) const {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + u * BT, r = i >> 3, c8 = i & 7;
      *reinterpret_cast<u32x4*>(dst + r * SP + 8 * c8) = v[u];
    }
  }
};
struct F32 {          // a 64 x 64 slab of an fp32 state: 4 x 16 bytes per thread, scaled to fp16 on store
  f32x4 v[4];
  __device__ __forceinline__ void load(const float* src, int ld) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = threadIdx.x + u * BT, r = i >> 4, c4 = i & 15;
      v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)r * ld + 4 * c4);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, float down) const {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = threadIdx.x + u * BT, r = i >> 4, c4 = i & 15;
      uint2 w;
      w.x = pack_h2(v[u][0] * down, v[u][1] * down);
      w.y = pack_h2(v[u][2] * down, v[u][3] * down);
      *reinterpret_cast<uint2*>(dst + r * SP + 4 * c4) = w;
    }
  }
};

// a wide slab: 64 rows x NC columns of fp16 (NC <= 256), NC / 32 pieces of
// 16 bytes per thread; rows >= nvalid read as zero (loads clamped, not skipped)
template <int NC>
struct HW {
  static constexpr int PR = NC / 8, NP = TL * PR / BT;
  u32x4 v[NP];
  __device__ __forceinline__ void load(const uint16_t* src, int ld, int nvalid) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + u * BT, r = i / PR, c8 = i % PR;
      const u32x4 x = *reinterpret_cast<const u32x4*>(src + (int64_t)min(r, nvalid - 1) * ld + 8 * c8);
      v[u] = r < nvalid ? x : u32x4{0u, 0u, 0u, 0u};
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int pitch) const {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + u * BT, r = i / PR, c8 = i % PR;
      *reinterpret_cast<u32x4*>(dst + r * pitch + 8 * c8) = v[u];
    }
  }
};
// a wide slab of an fp32 state: 64 rows x NC columns, NC / 16 pieces of 16
// bytes per thread, scaled to fp16 on store
template <int NC>
struct FW {
  static constexpr int PR = NC / 4, NP = TL * PR / BT;
  f32x4 v[NP];
  __device__ __forceinline__ void load(const float* src, int ld) {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + u * BT, r = i / PR, c4 = i % PR;
      v[u] = *reinterpret_cast<const f32x4*>(src + (int64_t)r * ld + 4 * c4);
    }
  }
  __device__ __forceinline__ void store(uint16_t* dst, int pitch, float down) const {
#pragma unroll
    for (int u = 0; u < NP; ++u) {
      const int i = threadIdx.x + u * BT, r = i / PR, c4 = i % PR;
      uint2 w;
      w.x = pack_h2(v[u][0] * down, v[u][1] * down);
      w.y = pack_h2(v[u][2] * down, v[u][3] * down);
      *reinterpret_cast<uint2*>(dst + r * pitch + 4 * c4) = w;
    }
  }
};

template <int D, int WM = 256> struct Wide {   // the wide slabs (at most WM columns) of a D-column operand
  static constexpr int N = D < WM ? D : WM, W = D / N;
};

// the power of two of one (bh, chunk) state: 2^-e brings its largest
// magnitude (the maximum of the scan's NM partial maxima) into [2^14, 2^15);
// returns 2^e
template <int NM>
__device__ __forceinline__ float state_up(const float* smax) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < NM; ++i) m = fmaxf(m, smax[i]);
  int ex = 0;
  if (m > 0.f && m < 3.0e38f) {
    frexpf(m, &ex);
    ex = min(max(ex - 15, -120), 120);
  }
  return ldexpf(1.f, ex);
}

// ------------------------------------------------------------ state scans
// REV = false: R_c, z_c for every chunk (R <- gamma^(B_c) R + K'^T (zeta V),
// zeta_m = gamma^(c1-1-m)), walking the chunks forwards.
// REV = true: U_c, u_c (U <- gamma^(B_c) U + Q'^T (w G), w_p = gamma^(p-c0) a_p,
// and c_p in place of a_p for u), walking the chunks backwards.  The value
// stored for chunk c is the state before that chunk is folded in, with the
// largest magnitude of each wave's part (for the consumers' power of two).
// A workgroup owns rows [64 db, 64 db + 64) and columns [DVB eb, DVB eb +
// DVB) of the state; the next two 64-row tiles are in registers while the
// current one is multiplied.  DVB = scan_dvb(d_v) columns per workgroup; each
// of its 4 waves records one partial maximum per chunk, so a chunk's state
// has state_nm(d_k, d_v) of them.
__host__ __device__ constexpr int scan_dvb(int dv) { return dv < SCAN_DVB ? dv : SCAN_DVB; }
__host__ __device__ constexpr int state_nm(int dk, int dv) { return (dk / 64) * (dv / scan_dvb(dv)) * 4; }
template <int DVB>
struct StateSmem {
  uint16_t As[2][TL * SP];         // weighted k' (q') rows [row][d of the block]
  uint16_t Bs[2][TL * (DVB + 8)];  // v (dO) rows [row][e of the block]
  float zr[2][TL];                 // key-sum weight / row weight of As
  float zred[4][64];               // partial key-sums of the four row quarters
};

template <int DVB>
struct TileRegs {                  // one tile in flight: A and B pieces, weights of the A pieces
  static constexpr int BPC = TL * DVB / 8 / BT;
  H16 a;
  u32x4 b[BPC];
  float aw[2], az[2];
};

template <int DK, int DV, int DVB, bool REV>
__global__ void __launch_bounds__(BT) bwd_state_kernel(BwdP p, HeadParams hp) {
  typedef StateSmem<DVB> SM;
  typedef TileRegs<DVB> TR;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int NDB = DK / 64, NEB = DV / DVB, NB = DVB / 64;   // NB column blocks of 32 per wave
  constexpr int BP = DVB + 8;
  constexpr int BPC = TR::BPC;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bi = wave >> 1, bj = wave & 1;
  const int eb = blockIdx.x % NEB;
  const int db = (blockIdx.x / NEB) % NDB;
  const int bh = blockIdx.x / (NEB * NDB);
  const int head = bh % p.h;
  Decay dec;
  dec.init(hp, head);
  const float qk = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;
  const uint16_t* X = (REV ? p.Qr : p.Kr) + (int64_t)bh * p.L * DK + 64 * db;
  const uint16_t* Y = (REV ? p.Gb : p.Vb) + (int64_t)bh * p.L * DV + DVB * eb;
  float* dst = (REV ? p.Ust : p.Rin) + (int64_t)bh * p.nc * DK * DV;
  float* zdst = (REV ? p.ust : p.zin) + (int64_t)bh * p.nc * DK;
  float* mdst = (REV ? p.umax : p.rmax) + (int64_t)bh * p.nc * (NDB * NEB * 4) + (db * NEB + eb) * 4;

  // tile t of the walk -> (chunk, first row)
  const int tpc = p.B / TL;
  const int tl = p.nt - (p.nc - 1) * tpc;           // tiles of the last chunk
  auto tile_of = [&](int t, int& c, int& m0) {
    int tile;
    if (!REV) {
      tile = t;
      c = t / tpc;
    } else if (t < tl) {
      c = p.nc - 1;
      tile = c * tpc + t;
    } else {
      const int u = t - tl;
      c = p.nc - 2 - u / tpc;
      tile = c * tpc + u % tpc;
    }
    m0 = tile * TL;
  };

  auto load_tile = [&](int t, TR& g) {
    t = min(t, p.nt - 1);               // past the end: reload the last tile (every step issues the same loads)
    int c, m0;
    tile_of(t, c, m0);
    const int c0 = c * p.B, c1 = min(c0 + p.B, p.L), nv = min(TL, c1 - m0);
    g.a.load(X + (int64_t)m0 * DK, DK, nv);
#pragma unroll
    for (int u = 0; u < BPC; ++u) {
      const int i = tid + u * BT, r = i / (DVB / 8), c8 = i % (DVB / 8);
      const u32x4 x = *reinterpret_cast<const u32x4*>(Y + (int64_t)(m0 + min(r, nv - 1)) * DV + 8 * c8);
      g.b[u] = r < nv ? x : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = (tid + u * BT) >> 3, row = m0 + min(r, nv - 1);
      float w, z;
      if (REV) {
        float a, cc;
        row_ac(p, dec, qk, bh, row, a, cc);
        w = dec.pow((float)(row - c0)) * a;
        z = a > 0.f ? cc / a : 0.f;
      } else {
        w = dec.pow((float)(c1 - 1 - row));
        z = 1.f;
      }
      g.aw[u] = r < nv ? w : 0.f;
      g.az[u] = r < nv ? z : 0.f;
    }
  };

  f32x16 acc[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) acc[n] = f32x16{};
  // partial key-sum of d = 64 db + (tid & 63) over rows 16 (tid / 64) .. + 15 of each tile (eb == 0)
  float zpart = 0.f;
  const int zd = tid & 63, zq = tid >> 6;

  auto body = [&](int t, TR& g) {
    int c, m0;
    tile_of(t, c, m0);
    const int c0 = c * p.B, c1 = min(c0 + p.B, p.L), nv = min(TL, c1 - m0);
    if (m0 == c0) {
      // the state entering chunk c, then its decay over the chunk
      float* Sd = dst + (int64_t)c * DK * DV;
      float m = 0.f;
#pragma unroll
      for (int n = 0; n < NB; ++n)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = 64 * db + 32 * bi + acc_row(r, lane);
          const int e = DVB * eb + 64 * n + 32 * bj + (lane & 31);
          Sd[(int64_t)d * DV + e] = acc[n][r];
          m = fmaxf(m, fabsf(acc[n][r]));
        }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
      if (lane == 0) mdst[(int64_t)c * (NDB * NEB * 4) + wave] = m;
      const float gB = dec.pow((float)(c1 - c0));
      if (eb == 0) {
        sm.zred[zq][zd] = zpart;
        __syncthreads();
        if (tid < 64)
          zdst[(int64_t)c * DK + 64 * db + tid] = sm.zred[0][tid] + sm.zred[1][tid] + sm.zred[2][tid] + sm.zred[3][tid];
        zpart *= gB;
      }
#pragma unroll
      for (int n = 0; n < NB; ++n) acc[n] *= gB;
    }
    const int buf = t & 1;
    // registers -> LDS (A rows weighted)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = tid + u * BT, r = i >> 3, c8 = i & 7;
      const float w = g.aw[u];
      u32x4 x = g.a.v[u];
      x.x = pack_h2(h_lo(x.x) * w, h_hi(x.x) * w);
      x.y = pack_h2(h_lo(x.y) * w, h_hi(x.y) * w);
      x.z = pack_h2(h_lo(x.z) * w, h_hi(x.z) * w);
      x.w = pack_h2(h_lo(x.w) * w, h_hi(x.w) * w);
      *reinterpret_cast<u32x4*>(sm.As[buf] + r * SP + 8 * c8) = x;
      if (c8 == 0) sm.zr[buf][r] = g.az[u];
    }
#pragma unroll
    for (int u = 0; u < BPC; ++u) {
      const int i = tid + u * BT, r = i / (DVB / 8), c8 = i % (DVB / 8);
      *reinterpret_cast<u32x4*>(sm.Bs[buf] + r * BP + 8 * c8) = g.b[u];
    }
    __syncthreads();
    load_tile(t + 2, g);
    if (eb == 0)
      for (int i = 16 * zq; i < min(16 * zq + 16, nv); ++i)
        zpart += h2f(sm.As[buf][i * SP + zd]) * sm.zr[buf][i];
    // acc[d][e] += sum_row As[row][d] Bs[row][e]: both operands read transposed
#pragma unroll
    for (int n = 0; n < NB; ++n)
      mm64<true, true>(acc[n], sm.As[buf], SP, 32 * bi, sm.Bs[buf], BP, 64 * n + 32 * bj, lane);
  };

  TR g0, g1;
  load_tile(0, g0);
  load_tile(1, g1);
  for (int t = 0; t < p.nt; t += 2) {
    body(t, g0);
    if (t + 1 < p.nt) body(t + 1, g1);
  }
}

// ------------------------------------------------------------ epilogue
// an fp32 tile [64][DK + 4] in LDS -> rows of dq / dk, times gs (the 2^e of
// the head's dO) and rotated back by -p theta
template <typename TG, int DK>
__device__ __forceinline__ void store_rotated(const float* t, TG* out, const ret_strides& so, int bb, int hh, int r0,
                                              int nrows, const BwdP& p, const HeadParams& hp, float gs) {
  constexpr int PAIRS = DK / 2, RPP = BT / PAIRS, TP = DK + 4;
  const int j = threadIdx.x % PAIRS, i0 = threadIdx.x / PAIRS;
  const bool xpos = (p.flags & RET_XPOS) != 0;
  float c = 1.f, s = 0.f, c1 = 1.f, s1 = 0.f;
  if (xpos) {
    phase(p.pos0 + r0 + i0, hp.theta[j], c, s);
    phase(RPP, hp.theta[j], c1, s1);
  }
  TG* o = out + bb * so.b + hh * so.h;
  bool bad = false;
  for (int i = i0; i < nrows; i += RPP) {
    float x0 = gs * t[i * TP + 2 * j], x1 = gs * t[i * TP + 2 * j + 1];
    if (xpos) {
      rot(x0, x1, c, -s);
      advance(c, s, c1, s1);
    }
    bad |= nonfinite_as<TG>(x0) | nonfinite_as<TG>(x1);
    Out2<TG>::st(o + (int64_t)(r0 + i) * so.l + 2 * j, x0, x1);
  }
  flag_nonfinite(p.nf, bad, kNonFiniteBwd);
}

// ------------------------------------------------------------ dq
template <int DK, int DV>
struct DqSmem {
  static constexpr int PW = (Wide<DV>::N > Wide<DK>::N ? Wide<DV>::N : Wide<DK>::N) + 8;
  union {
    struct {
      uint16_t Gs[TL * (DV + 8)];
      uint16_t Es[TL * SP];
      uint16_t Ys[TL * SP];        // the decay tile (only with the row statistics)
      uint16_t Sl[2][TL * PW];     // wide slabs (the cross term's narrow slabs use pitch SP)
    } w;
    float out[TL * (DK + 4)];
  } u;
  float ra[TL], rc[TL], xi[TL];
  float red[2][2][TL];             // [den / s g.num][column half][row]
};

// With ST (score normalisation) the kernel also finds a_p and c_p: it carries
// X = diag(s) ((Gamma o T) K' + xi G R_c^T) and Y = Gamma K' + xi z_c apart, so
// that den_p = q'_p . Y_p and s_p (g_p . num_p) = q'_p . X_p, then
// dq'_p = X_p / n_p + c_p Y_p; a_p and c_p go to ra / rc for the later kernels.
template <typename TG, int DK, int DV, bool ST>
__global__ void __launch_bounds__(BT) bwd_dq_kernel(BwdP p, HeadParams hp) {
  typedef DqSmem<DK, DV> SM;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int GP = DV + 8, ND = DK / 64, NE = DV / 64;
  constexpr int NM = state_nm(DK, DV);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bi = wave >> 1, bj = wave & 1, l32 = lane & 31;
  const int bh = blockIdx.x / p.nt, tile = blockIdx.x % p.nt;
  const int bb = bh / p.h, head = bh % p.h;
  const int r0 = tile * TL, nq = min(TL, p.L - r0);
  const int c = r0 / p.B, c0 = c * p.B;
  Decay dec;
  dec.init(hp, head);
  const float qk = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;
  const uint16_t* Kr = p.Kr + (int64_t)bh * p.L * DK;
  const uint16_t* Vb = p.Vb + (int64_t)bh * p.L * DV;
  const uint16_t* Gb = p.Gb + (int64_t)bh * p.L * DV;

  if (ST) {
    if (tid < TL) {                                 // ra holds s_p until the statistics are known
      sm.ra[tid] = row_scale(dec, p.flags, qk, r0 + min(tid, nq - 1) + 1);
      sm.xi[tid] = dec.pow((float)(r0 + tid - c0 + 1));
    }
  } else {
    float a, cc;
    row_ac(p, dec, qk, bh, r0 + min(tid & 63, nq - 1), a, cc);
    if (tid < TL) {
      sm.ra[tid] = tid < nq ? a : 0.f;
      sm.rc[tid] = tid < nq ? cc : 0.f;
      sm.xi[tid] = dec.pow((float)(r0 + tid - c0 + 1));
    }
  }
  stage<DV>(sm.u.w.Gs, GP, Gb + (int64_t)r0 * DV, DV, nq, nullptr);
  f32x16 acc[ND], Y[ST ? ND : 1];
#pragma unroll
  for (int n = 0; n < ND; ++n) acc[n] = f32x16{};
#pragma unroll
  for (int n = 0; n < (ST ? ND : 1); ++n) Y[n] = f32x16{};
  int sc = 0;
  // the intra-chunk stream of wide slabs: per key tile the V slabs (columns
  // N1 at a time), then the K' slabs (N2 at a time); the next one is in flight
  constexpr int N1 = Wide<DV>::N, W1 = Wide<DV>::W, N2 = Wide<DK>::N, W2 = Wide<DK>::W, PW = SM::PW;
  const int nkt = (r0 - c0) / TL + 1;
  HW<N1> h1;
  HW<N2> h2;
  auto ld1 = [&](int j, int w) {                    // past the end: reload the last tile's slab
    const int m0 = c0 + TL * min(j, nkt - 1);
    h1.load(Vb + (int64_t)m0 * DV + N1 * w, DV, min(TL, p.L - m0));
  };
  auto ld2 = [&](int j, int w) {
    const int m0 = c0 + TL * j;
    h2.load(Kr + (int64_t)m0 * DK + N2 * w, DK, min(TL, p.L - m0));
  };
  ld1(0, 0);

  // cross: xi_p (a_p (G R_c^T)_pd + c_p z_c[d])
  if (c > 0) {
    const float* R = p.Rin + ((int64_t)bh * p.nc + c) * DK * DV;
    const float* z = p.zin + ((int64_t)bh * p.nc + c) * DK;
    const float up = state_up<NM>(p.rmax + ((int64_t)bh * p.nc + c) * NM), down = 1.f / up;
    // wide slabs R[64 ds ..][N1 ew ..], one in flight
    FW<N1> fr;
    fr.load(R, DV);
#pragma unroll
    for (int ds = 0; ds < ND; ++ds)
#pragma unroll
      for (int ew = 0; ew < W1; ++ew) {
        const int i = ds * W1 + ew, nx = min(i + 1, ND * W1 - 1);
        uint16_t* b = sm.u.w.Sl[sc++ & 1];
        fr.store(b, PW, down);
        __syncthreads();
        fr.load(R + (int64_t)(64 * (nx / W1)) * DV + N1 * (nx % W1), DV);
        // B[n = d][k = e] = R[d][e], staged [d][e]: "nt"
#pragma unroll
        for (int u = 0; u < N1 / 64; ++u)
          mm64<false, false>(acc[ds], sm.u.w.Gs + N1 * ew + 64 * u, GP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
      }
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) {
      const float zd = z[64 * ds + 32 * bj + l32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pl = 32 * bi + acc_row(r, lane);
        if (ST) {
          acc[ds][r] = sm.xi[pl] * sm.ra[pl] * up * acc[ds][r];
          Y[ds][r] = sm.xi[pl] * zd;
        } else {
          acc[ds][r] = sm.xi[pl] * (sm.ra[pl] * up * acc[ds][r] + sm.rc[pl] * zd);
        }
      }
    }
  }
  // intra-chunk key tiles up to the diagonal: V slabs (T = G V^T), E, then K' slabs
  for (int j = 0; j < nkt; ++j) {
    const int m0 = c0 + TL * j;
    f32x16 T = {};
#pragma unroll
    for (int w = 0; w < W1; ++w) {
      uint16_t* b = sm.u.w.Sl[sc++ & 1];
      h1.store(b, PW);
      __syncthreads();
      if (w + 1 < W1) ld1(j, w + 1);
      else ld2(j, 0);
#pragma unroll
      for (int u = 0; u < N1 / 64; ++u)
        mm64<false, false>(T, sm.u.w.Gs + N1 * w + 64 * u, GP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
    }
    // E[p][m] -> LDS (row p, column m)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int pl = 32 * bi + acc_row(r, lane), ml = 32 * bj + l32;
      const int row = r0 + pl, col = m0 + ml;
      const bool ok = col <= row && col < p.L && row < p.L;
      const float gm = ok ? dec.pow((float)(row - col)) : 0.f;
      if (ST) {
        sm.u.w.Es[pl * SP + ml] = f2h(gm * sm.ra[pl] * T[r]);
        sm.u.w.Ys[pl * SP + ml] = f2h(gm);
      } else {
        sm.u.w.Es[pl * SP + ml] = f2h(gm * (sm.ra[pl] * T[r] + sm.rc[pl]));
      }
    }
#pragma unroll
    for (int w = 0; w < W2; ++w) {
      uint16_t* b = sm.u.w.Sl[sc++ & 1];
      h2.store(b, PW);
      __syncthreads();
      if (w + 1 < W2) ld2(j, w + 1);
      else ld1(j + 1, 0);
      // dq'[p][d] += sum_m E[p][m] K'[m][d]; K' staged [m][d] (k = m): transposed B
#pragma unroll
      for (int u = 0; u < N2 / 64; ++u) {
        mm64<false, true>(acc[(N2 / 64) * w + u], sm.u.w.Es, SP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
        if (ST)
          mm64<false, true>(Y[ST ? (N2 / 64) * w + u : 0], sm.u.w.Ys, SP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
      }
    }
  }
  if (ST) {
    // row sums q'_p . Y_p (den_p) and q'_p . X_p (s_p g_p . num_p): q' staged
    // over the G tile (last read before the final slab's barrier), 32 columns
    // per half-wave, then the two column halves
    constexpr int QP = DK + 8;
    stage<DK>(sm.u.w.Gs, QP, p.Qr + ((int64_t)bh * p.L + r0) * DK, DK, nq, nullptr);
    __syncthreads();
    float d[16], g[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) d[r] = g[r] = 0.f;
#pragma unroll
    for (int ds = 0; ds < ND; ++ds)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float qv = h2f(sm.u.w.Gs[(32 * bi + acc_row(r, lane)) * QP + 64 * ds + 32 * bj + l32]);
        d[r] += qv * Y[ST ? ds : 0][r];
        g[r] += qv * acc[ds][r];
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) {
        d[r] += __shfl_xor(d[r], o, 64);
        g[r] += __shfl_xor(g[r], o, 64);
      }
      if (l32 == 0) {
        const int pl = 32 * bi + acc_row(r, lane);
        sm.red[0][bj][pl] = d[r];
        sm.red[1][bj][pl] = g[r];
      }
    }
    __syncthreads();
    if (tid < TL) {
      const int row = r0 + tid;
      const float den = sm.red[0][0][tid] + sm.red[0][1][tid];
      const float sg = sm.red[1][0][tid] + sm.red[1][1][tid];
      const float s = sm.ra[tid];
      const float sd = fabsf(s * den);
      const float n = fmaxf(sd, 1.f);
      const float cc = sd > 1.f ? -s * (den > 0.f ? 1.f : -1.f) * sg / (n * n) : 0.f;
      const bool ok = tid < nq;
      if (ok) {
        p.ra[(int64_t)bh * p.L + row] = s / n;
        p.rc[(int64_t)bh * p.L + row] = cc;
      }
      sm.rc[tid] = ok ? cc : 0.f;
      sm.xi[tid] = ok ? 1.f / n : 0.f;              // the factor on X
    }
    __syncthreads();
#pragma unroll
    for (int ds = 0; ds < ND; ++ds)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int pl = 32 * bi + acc_row(r, lane);
        acc[ds][r] = sm.xi[pl] * acc[ds][r] + sm.rc[pl] * Y[ST ? ds : 0][r];
      }
  }
  __syncthreads();
#pragma unroll
  for (int ds = 0; ds < ND; ++ds)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      sm.u.out[(32 * bi + acc_row(r, lane)) * (DK + 4) + 64 * ds + 32 * bj + l32] = acc[ds][r];
  __syncthreads();
  store_rotated<TG, DK>(sm.u.out, reinterpret_cast<TG*>(p.dq), p.sdq, bb, head, r0, nq, p, hp, p.gsc[bh]);
}

// ------------------------------------------------------------ dk
template <int DK, int DV>
struct DkSmem {
  static constexpr int PW = (Wide<DV>::N > Wide<DK>::N ? Wide<DV>::N : Wide<DK>::N) + 8;
  union {
    struct {
      uint16_t Vs[TL * (DV + 8)];
      uint16_t Es[TL * SP];        // E^T [m][p]
      uint16_t Sl[2][TL * PW];     // wide slabs (the cross term's narrow slabs use pitch SP)
    } w;
    float out[TL * (DK + 4)];
  } u;
  float pa[TL], pc[TL];
};

template <typename TG, int DK, int DV>
__global__ void __launch_bounds__(BT) bwd_dk_kernel(BwdP p, HeadParams hp) {
  typedef DkSmem<DK, DV> SM;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int VP = DV + 8, ND = DK / 64, NE = DV / 64;
  constexpr int NM = state_nm(DK, DV);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bi = wave >> 1, bj = wave & 1, l32 = lane & 31;
  const int bh = blockIdx.x / p.nt, tile = blockIdx.x % p.nt;
  const int bb = bh / p.h, head = bh % p.h;
  const int m0 = tile * TL, nk = min(TL, p.L - m0);
  const int c = m0 / p.B, c0 = c * p.B, c1 = min(c0 + p.B, p.L);
  Decay dec;
  dec.init(hp, head);
  const float qk = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;
  const uint16_t* Qr = p.Qr + (int64_t)bh * p.L * DK;
  const uint16_t* Vb = p.Vb + (int64_t)bh * p.L * DV;
  const uint16_t* Gb = p.Gb + (int64_t)bh * p.L * DV;

  stage<DV>(sm.u.w.Vs, VP, Vb + (int64_t)m0 * DV, DV, nk, nullptr);
  f32x16 acc[ND];
#pragma unroll
  for (int n = 0; n < ND; ++n) acc[n] = f32x16{};
  int sc = 0;
  // the intra-chunk stream of wide slabs: per query tile the dO slabs, then
  // the Q' slabs; the next one is in flight
  constexpr int N1 = Wide<DV>::N, W1 = Wide<DV>::W, N2 = Wide<DK>::N, W2 = Wide<DK>::W, PW = SM::PW;
  const int nqt = (c1 - m0 + TL - 1) / TL;
  HW<N1> h1;
  HW<N2> h2;
  auto ld1 = [&](int j, int w) {                    // past the end: reload the last tile's slab
    const int q0 = m0 + TL * min(j, nqt - 1);
    h1.load(Gb + (int64_t)q0 * DV + N1 * w, DV, min(TL, p.L - q0));
  };
  auto ld2 = [&](int j, int w) {
    const int q0 = m0 + TL * j;
    h2.load(Qr + (int64_t)q0 * DK + N2 * w, DK, min(TL, p.L - q0));
  };
  ld1(0, 0);

  // cross: gamma^(c1-m) ((V U_c^T)[m][d] + u_c[d])
  if (c + 1 < p.nc) {
    const float* U = p.Ust + ((int64_t)bh * p.nc + c) * DK * DV;
    const float* u = p.ust + ((int64_t)bh * p.nc + c) * DK;
    const float up = state_up<NM>(p.umax + ((int64_t)bh * p.nc + c) * NM), down = 1.f / up;
    // wide slabs U[64 ds ..][N1 ew ..], one in flight
    FW<N1> fr;
    fr.load(U, DV);
#pragma unroll
    for (int ds = 0; ds < ND; ++ds)
#pragma unroll
      for (int ew = 0; ew < W1; ++ew) {
        const int i = ds * W1 + ew, nx = min(i + 1, ND * W1 - 1);
        uint16_t* b = sm.u.w.Sl[sc++ & 1];
        fr.store(b, PW, down);
        __syncthreads();
        fr.load(U + (int64_t)(64 * (nx / W1)) * DV + N1 * (nx % W1), DV);
#pragma unroll
        for (int u = 0; u < N1 / 64; ++u)
          mm64<false, false>(acc[ds], sm.u.w.Vs + N1 * ew + 64 * u, VP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
      }
#pragma unroll
    for (int ds = 0; ds < ND; ++ds) {
      const float ud = u[64 * ds + 32 * bj + l32];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + 32 * bi + acc_row(r, lane);
        acc[ds][r] = dec.pow((float)(c1 - row)) * (up * acc[ds][r] + ud);
      }
    }
  }
  // intra-chunk query tiles from the diagonal to the chunk end: dO slabs (T^T = V dO^T), E^T, then Q' slabs
  for (int j = 0; j < nqt; ++j) {
    const int q0 = m0 + TL * j, nq = min(TL, p.L - q0);
    {
      float a, cc;
      row_ac(p, dec, qk, bh, q0 + min(tid & 63, nq - 1), a, cc);
      if (tid < TL) {
        sm.pa[tid] = tid < nq ? a : 0.f;
        sm.pc[tid] = tid < nq ? cc : 0.f;
      }
    }
    f32x16 T = {};
#pragma unroll
    for (int w = 0; w < W1; ++w) {
      uint16_t* b = sm.u.w.Sl[sc++ & 1];
      h1.store(b, PW);
      __syncthreads();
      if (w + 1 < W1) ld1(j, w + 1);
      else ld2(j, 0);
      // T^T[m][p] = sum_e V[m][e] G[p][e]
#pragma unroll
      for (int u = 0; u < N1 / 64; ++u)
        mm64<false, false>(T, sm.u.w.Vs + N1 * w + 64 * u, VP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = 32 * bi + acc_row(r, lane), pl = 32 * bj + l32;
      const int row = q0 + pl, col = m0 + ml;
      const bool ok = col <= row && col < p.L && row < p.L;
      const float e = ok ? dec.pow((float)(row - col)) * (sm.pa[pl] * T[r] + sm.pc[pl]) : 0.f;
      sm.u.w.Es[ml * SP + pl] = f2h(e);
    }
#pragma unroll
    for (int w = 0; w < W2; ++w) {
      uint16_t* b = sm.u.w.Sl[sc++ & 1];
      h2.store(b, PW);
      __syncthreads();
      if (w + 1 < W2) ld2(j, w + 1);
      else ld1(j + 1, 0);
      // dk'[m][d] += sum_p E^T[m][p] Q'[p][d]; Q' staged [p][d] (k = p): transposed B
#pragma unroll
      for (int u = 0; u < N2 / 64; ++u)
        mm64<false, true>(acc[(N2 / 64) * w + u], sm.u.w.Es, SP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
    }
  }
  __syncthreads();
#pragma unroll
  for (int ds = 0; ds < ND; ++ds)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      sm.u.out[(32 * bi + acc_row(r, lane)) * (DK + 4) + 64 * ds + 32 * bj + l32] = acc[ds][r];
  __syncthreads();
  store_rotated<TG, DK>(sm.u.out, reinterpret_cast<TG*>(p.dk), p.sdk, bb, head, m0, nk, p, hp, p.gsc[bh]);
}

// ------------------------------------------------------------ dv
// the d_v columns of a key tile go to two workgroups (each recomputing K' Q'^T)
// where that keeps an even number of slabs per query tile: half the
// accumulators per wave, so two workgroups fit on a CU
template <int DK, int DV> struct DvSplit {
  static constexpr int ND = DK / 64, NE = DV / 64;
  static constexpr int NEH = (NE > 1 && (ND + NE / 2) % 2 == 0) ? NE / 2 : NE;
};

template <int DK, int DV>
struct DvSmem {
  static constexpr int PW = (Wide<DK, 128>::N > Wide<DvSplit<DK, DV>::NEH * 64, 128>::N
                                 ? Wide<DK, 128>::N : Wide<DvSplit<DK, DV>::NEH * 64, 128>::N) + 8;
  uint16_t Ks[TL * (DK + 8)];
  uint16_t As[TL * SP];            // a_p A^T [m][p]
  uint16_t Sl[2][TL * PW];         // wide slabs (the cross term's narrow slabs use pitch SP)
  float pa[TL];
};

template <typename TG, int DK, int DV>
__global__ void __launch_bounds__(BT) bwd_dv_kernel(BwdP p, HeadParams hp) {
  typedef DvSmem<DK, DV> SM;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);
  constexpr int KP = DK + 8, ND = DK / 64, NE = DV / 64;
  constexpr int NM = state_nm(DK, DV);
  // the d_v columns are split over DvSplit<DK, DV>::N workgroups of NEH 64-column blocks each
  constexpr int NEH = DvSplit<DK, DV>::NEH, NSPLIT = NE / NEH;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bi = wave >> 1, bj = wave & 1, l32 = lane & 31;
  const int part = blockIdx.x % NSPLIT, wg = blockIdx.x / NSPLIT;
  const int e0 = part * NEH * 64;
  const int bh = wg / p.nt, tile = wg % p.nt;
  const int bb = bh / p.h, head = bh % p.h;
  const int m0 = tile * TL, nk = min(TL, p.L - m0);
  const int c = m0 / p.B, c0 = c * p.B, c1 = min(c0 + p.B, p.L);
  Decay dec;
  dec.init(hp, head);
  const float qk = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;
  const uint16_t* Qr = p.Qr + (int64_t)bh * p.L * DK;
  const uint16_t* Kr = p.Kr + (int64_t)bh * p.L * DK;
  const uint16_t* Gb = p.Gb + (int64_t)bh * p.L * DV;

  stage<DK>(sm.Ks, KP, Kr + (int64_t)m0 * DK, DK, nk, nullptr);
  f32x16 acc[NEH];
#pragma unroll
  for (int n = 0; n < NEH; ++n) acc[n] = f32x16{};
  int sc = 0;
  // the intra-chunk stream of wide slabs: per query tile the Q' slabs, then
  // this part's dO slabs; the next one is in flight
  constexpr int N1 = Wide<DK, 128>::N, W1 = Wide<DK, 128>::W;
  constexpr int N2 = Wide<NEH * 64, 128>::N, W2 = Wide<NEH * 64, 128>::W, PW = SM::PW;
  const int nqt = (c1 - m0 + TL - 1) / TL;
  HW<N1> h1;
  HW<N2> h2;
  auto ld1 = [&](int j, int w) {                    // past the end: reload the last tile's slab
    const int q0 = m0 + TL * min(j, nqt - 1);
    h1.load(Qr + (int64_t)q0 * DK + N1 * w, DK, min(TL, p.L - q0));
  };
  auto ld2 = [&](int j, int w) {
    const int q0 = m0 + TL * j;
    h2.load(Gb + (int64_t)q0 * DV + e0 + N2 * w, DV, min(TL, p.L - q0));
  };
  ld1(0, 0);

  // cross: gamma^(c1-m) (K' U_c)[m][e]
  if (c + 1 < p.nc) {
    const float* U = p.Ust + ((int64_t)bh * p.nc + c) * DK * DV;
    const float up = state_up<NM>(p.umax + ((int64_t)bh * p.nc + c) * NM), down = 1.f / up;
    // wide slabs U[64 ds ..][e0 + N2 eh ..], one in flight
    FW<N2> fr;
    fr.load(U + e0, DV);
#pragma unroll
    for (int ds = 0; ds < ND; ++ds)
#pragma unroll
      for (int eh = 0; eh < W2; ++eh) {
        const int i = ds * W2 + eh, nx = min(i + 1, ND * W2 - 1);
        uint16_t* b = sm.Sl[sc++ & 1];
        fr.store(b, PW, down);
        __syncthreads();
        fr.load(U + (int64_t)(64 * (nx / W2)) * DV + e0 + N2 * (nx % W2), DV);
        // B[n = e][k = d] = U[d][e], staged [d][e]: transposed B
#pragma unroll
        for (int u = 0; u < N2 / 64; ++u)
          mm64<false, true>(acc[(N2 / 64) * eh + u], sm.Ks + 64 * ds, KP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
      }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float f = up * dec.pow((float)(c1 - (m0 + 32 * bi + acc_row(r, lane))));
#pragma unroll
      for (int es = 0; es < NEH; ++es) acc[es][r] *= f;
    }
  }
  // intra-chunk query tiles from the diagonal to the chunk end: Q' slabs (S^T = K' Q'^T), a A^T, then dO slabs
  for (int j = 0; j < nqt; ++j) {
    const int q0 = m0 + TL * j, nq = min(TL, p.L - q0);
    {
      float a, cc;
      row_ac(p, dec, qk, bh, q0 + min(tid & 63, nq - 1), a, cc);
      if (tid < TL) sm.pa[tid] = tid < nq ? a : 0.f;
    }
    f32x16 S = {};
#pragma unroll
    for (int w = 0; w < W1; ++w) {
      uint16_t* b = sm.Sl[sc++ & 1];
      h1.store(b, PW);
      __syncthreads();
      if (w + 1 < W1) ld1(j, w + 1);
      else ld2(j, 0);
      // S^T[m][p] = sum_d K'[m][d] Q'[p][d]
#pragma unroll
      for (int u = 0; u < N1 / 64; ++u)
        mm64<false, false>(S, sm.Ks + N1 * w + 64 * u, KP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = 32 * bi + acc_row(r, lane), pl = 32 * bj + l32;
      const int row = q0 + pl, col = m0 + ml;
      const bool ok = col <= row && col < p.L && row < p.L;
      const float x = ok ? sm.pa[pl] * dec.pow((float)(row - col)) * S[r] : 0.f;
      sm.As[ml * SP + pl] = f2h(x);
    }
#pragma unroll
    for (int w = 0; w < W2; ++w) {
      uint16_t* b = sm.Sl[sc++ & 1];
      h2.store(b, PW);
      __syncthreads();
      if (w + 1 < W2) ld2(j, w + 1);
      else ld1(j + 1, 0);
      // dv[m][e] += sum_p (a A^T)[m][p] G[p][e]; G staged [p][e] (k = p): transposed B
#pragma unroll
      for (int u = 0; u < N2 / 64; ++u)
        mm64<false, true>(acc[(N2 / 64) * w + u], sm.As, SP, 32 * bi, b + 64 * u, PW, 32 * bj, lane);
    }
  }
  TG* o = reinterpret_cast<TG*>(p.dv) + bb * p.sdv.b + head * p.sdv.h;
  const float gs = p.gsc[bh];
  bool bad = false;
#pragma unroll
  for (int es = 0; es < NEH; ++es)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int ml = 32 * bi + acc_row(r, lane);
      if (ml < nk) {
        const float x = gs * acc[es][r];
        bad |= nonfinite_as<TG>(x);
        o[(int64_t)(m0 + ml) * p.sdv.l + e0 + 64 * es + 32 * bj + l32] = Store<TG>::cvt(x);
      }
    }
  flag_nonfinite(p.nf, bad, kNonFiniteBwd);
}

// ------------------------------------------------------------ host side
size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Carve {
  size_t qr, kr, vb, gb, rin, zin, ust, us, ra, rc, tmax, gsc, rmax, umax, total;
};

Carve carve_bwd(int b, int h, int L, int dk, int dv, int B) {
  const size_t bh = (size_t)b * h, nc = (size_t)((L + B - 1) / B);
  Carve c;
  size_t o = 0;
  c.qr = o; o += al256(bh * L * dk * 2);
  c.kr = o; o += al256(bh * L * dk * 2);
  c.vb = o; o += al256(bh * L * dv * 2);
  c.gb = o; o += al256(bh * L * dv * 2);
  c.rin = o; o += al256(bh * nc * dk * dv * 4);
  c.zin = o; o += al256(bh * nc * dk * 4);
  c.ust = o; o += al256(bh * nc * dk * dv * 4);
  c.us = o; o += al256(bh * nc * dk * 4);
  c.ra = o; o += al256(bh * L * 4);
  c.rc = o; o += al256(bh * L * 4);
  c.tmax = o; o += al256(bh * (size_t)((L + TL - 1) / TL) * 4);
  c.gsc = o; o += al256(bh * 4);
  const size_t nm = (size_t)state_nm(dk, dv);
  c.rmax = o; o += al256(bh * nc * nm * 4);
  c.umax = o; o += al256(bh * nc * nm * 4);
  c.total = o;
  return c;
}

template <typename K>
hipError_t set_smem(K k, size_t bytes) {
  return hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

template <typename T, typename TG, int DK, int DV>
hipError_t run_bwd(const BwdArgs& a, hipStream_t st) {
  BwdP p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
  p.dq = a.gq; p.dk = a.gk; p.dv = a.gv;
  p.sq = a.sq; p.sk = a.sk; p.sv = a.sv; p.sdo = a.sdo; p.sdq = a.sgq; p.sdk = a.sgk; p.sdv = a.sgv;
  p.h = a.h; p.L = a.L; p.B = a.B;
  p.nc = (a.L + a.B - 1) / a.B;
  p.nt = (a.L + TL - 1) / TL;
  p.pos0 = a.pos0; p.flags = a.flags; p.nf = a.nf;
  const Carve cv = carve_bwd(a.b, a.h, a.L, DK, DV, a.B);
  unsigned char* w = static_cast<unsigned char*>(a.ws);
  p.Qr = reinterpret_cast<uint16_t*>(w + cv.qr);
  p.Kr = reinterpret_cast<uint16_t*>(w + cv.kr);
  p.Vb = reinterpret_cast<uint16_t*>(w + cv.vb);
  p.Gb = reinterpret_cast<uint16_t*>(w + cv.gb);
  p.Rin = reinterpret_cast<float*>(w + cv.rin);
  p.zin = reinterpret_cast<float*>(w + cv.zin);
  p.Ust = reinterpret_cast<float*>(w + cv.ust);
  p.ust = reinterpret_cast<float*>(w + cv.us);
  p.ra = reinterpret_cast<float*>(w + cv.ra);
  p.rc = reinterpret_cast<float*>(w + cv.rc);
  p.tmax = reinterpret_cast<float*>(w + cv.tmax);
  p.gsc = reinterpret_cast<float*>(w + cv.gsc);
  p.rmax = reinterpret_cast<float*>(w + cv.rmax);
  p.umax = reinterpret_cast<float*>(w + cv.umax);
  const int bh = a.b * a.h;
  const HeadParams& hp = *a.hp;
  constexpr int DVB = scan_dvb(DV);
  const dim3 tiles(bh * p.nt), sgrid(bh * (DK / 64) * (DV / DVB)), blk(BT);
  hipError_t e;
  hipLaunchKernelGGL((bwd_gmax_kernel<T, DV>), tiles, blk, 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_prep_kernel<T, DK, DV>), tiles, blk, 0, st, p, hp);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    auto k = bwd_state_kernel<DK, DV, DVB, false>;
    if ((e = set_smem(k, sizeof(StateSmem<DVB>))) != hipSuccess) return e;
    hipLaunchKernelGGL(k, sgrid, blk, sizeof(StateSmem<DVB>), st, p, hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    // dq needs only the forward states; with the score normalisation it also
    // writes the a_p, c_p that the reverse scan, dk and dv read
    auto k = (a.flags & RET_NORM_SCORE) ? bwd_dq_kernel<TG, DK, DV, true> : bwd_dq_kernel<TG, DK, DV, false>;
    if ((e = set_smem(k, sizeof(DqSmem<DK, DV>))) != hipSuccess) return e;
    hipLaunchKernelGGL(k, tiles, blk, sizeof(DqSmem<DK, DV>), st, p, hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    auto k = bwd_state_kernel<DK, DV, DVB, true>;
    if ((e = set_smem(k, sizeof(StateSmem<DVB>))) != hipSuccess) return e;
    hipLaunchKernelGGL(k, sgrid, blk, sizeof(StateSmem<DVB>), st, p, hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    auto k = bwd_dk_kernel<TG, DK, DV>;
    if ((e = set_smem(k, sizeof(DkSmem<DK, DV>))) != hipSuccess) return e;
    hipLaunchKernelGGL(k, tiles, blk, sizeof(DkSmem<DK, DV>), st, p, hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    auto k = bwd_dv_kernel<TG, DK, DV>;
    if ((e = set_smem(k, sizeof(DvSmem<DK, DV>))) != hipSuccess) return e;
    constexpr int NS = (DV / 64) / DvSplit<DK, DV>::NEH;
    hipLaunchKernelGGL(k, dim3(bh * p.nt * NS), blk, sizeof(DvSmem<DK, DV>), st, p, hp);
  }
  return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t run_bwd_g(const BwdArgs& a, hipStream_t st) {
  return a.grad_dt == RET_BF16 ? run_bwd<T, bf16, DK, DV>(a, st) : run_bwd<T, float, DK, DV>(a, st);
}

#define RET_BWD_SHAPES(X) X(64, 64) X(128, 128) X(128, 256) X(256, 512)

}  // namespace

bool chunkwise_bwd_supported(int dk, int dv) {
#define X(DK, DV) if (dk == DK && dv == DV) return true;
  RET_BWD_SHAPES(X)
#undef X
  return false;
}

size_t chunkwise_bwd_workspace(int b, int h, int L, int dk, int dv, int B) {
  return carve_bwd(b, h, L, dk, dv, B).total;
}

hipError_t launch_chunkwise_bwd(const BwdArgs& a, hipStream_t st) {
#define X(DK, DV)                                                                                   \
  if (a.d_k == DK && a.d_v == DV)                                                                   \
    return a.in_dt == RET_F16 ? run_bwd_g<half, DK, DV>(a, st) : run_bwd_g<bf16, DK, DV>(a, st);
  RET_BWD_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

}  // namespace ret
