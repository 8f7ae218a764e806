// Chunkwise recurrent retention forward for large chunks (RetNet reading
// notes, §2.4, with §2.3's xPos rotation and §三.3's normalisations), split
// into three kernels whose boundaries are the only synchronisation:
//
//   delta  (one workgroup per head, chunk and half of d_v)
//          dR_i = K'_[i]^T (V_[i] (.) zeta),  dz_i = K'_[i]^T zeta
//          and, once per head and chunk, the rotated keys K' in fp16
//   scan   (one workgroup per head and block of 32 state columns)
//          R_i = gamma^(B_i) R_{i-1} + dR_i,  z_i likewise; it stores the
//          state every chunk starts from, R_{i-1}, as an fp16 operand copy
//          scaled by a power of two per block of 32 columns
//   output (one workgroup per head, chunk and 64-row query tile)
//          O = (Q'K'^T (.) D) V + (Q' R_{i-1}) (.) xi, with the row scales and
//          score normalisation, written once
//
// Chunks of at most 128 keys replace delta and scan by one state-scan kernel
// (one workgroup per head and block of 64 state columns, walking the chunks
// in order with the state in MFMA accumulators), which also rotates the keys.
//
// Every key element is rotated once (the output kernel reads the rotated fp16
// keys), and no work is repeated across d_v slices.  Operands are fp16 with fp32 accumulation.
// Shapes: d_k = 256, d_v = 512, chunk B a multiple of 64.
#include "internal.h"

namespace ret {

namespace {

constexpr int NT3 = 512;
constexpr int DK = 256, DV = 512;
constexpr int TK = 64, TR = 64;
constexpr int QP = DK + 8;     // fp16 row pitch of Qs / Ks (528 B)
constexpr int KP = TK + 8;     // fp16 row pitch of key-major tiles (144 B)
constexpr int NCB = DV / 32;   // column blocks of the state operand
// a value tile is kept in its natural [key][col] layout with unpadded 1 KB rows;
// the 16-byte column pieces of key row r are XOR-swizzled by 4 (r % 4), so the
// four key rows of one transposed read start 64 bytes apart in the bank space
// and a half-wave touches all 64 banks once
__host__ __device__ constexpr int vswz(int key, int piece) { return piece ^ ((key & 3) << 2); }

struct Work {
  half* kt;      // rotated keys       [bh][L][DK]
  half* dR;      // chunk deltas       [bh][nc][DV][DK]   (column-major: [col][d])
  float* dRs;    // delta scales       [bh][nc][2]        (2^e per d_v half)
  float* dz;     // key-sum deltas     [bh][nc][DK]
  half* Rt;      // state operands     [bh][nc][DV*DK]    (R_{i-1}, fragment order, rt_frag)
  float* Rs;     // operand scales     [bh][nc][NCB]
  float* zc;     // z_{i-1}            [bh][nc][DK]
  half* dump;    // 8 KB that masked lanes of the state scan store to (never read)
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// chunks of at most this many keys take the state-scan kernel instead of the
// delta and scan kernels (no per-chunk delta in the workspace)
constexpr int SSCAN_MAX_B = 128;

size_t carve(void* base, int bh, int L, int B, Work* w) {
  const int nc = (L + B - 1) / B;
  const bool deltas = B > SSCAN_MAX_B;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  const size_t o_kt = take((size_t)bh * L * DK * 2);
  const size_t o_dR = take(deltas ? (size_t)bh * nc * DV * DK * 2 : 0);
  const size_t o_dRs = take(deltas ? (size_t)bh * nc * 2 * 4 : 0);
  const size_t o_dz = take(deltas ? (size_t)bh * nc * DK * 4 : 0);
  const size_t o_Rt = take((size_t)bh * nc * DV * DK * 2);
  const size_t o_Rs = take((size_t)bh * nc * NCB * 4);
  const size_t o_zc = take((size_t)bh * nc * DK * 4);
  const size_t o_dump = take(deltas ? 0 : NT3 * 16);
  if (w) {
    char* b = static_cast<char*>(base);
    w->kt = reinterpret_cast<half*>(b + o_kt);
    w->dR = reinterpret_cast<half*>(b + o_dR);
    w->dRs = reinterpret_cast<float*>(b + o_dRs);
    w->dz = reinterpret_cast<float*>(b + o_dz);
    w->Rt = reinterpret_cast<half*>(b + o_Rt);
    w->Rs = reinterpret_cast<float*>(b + o_Rs);
    w->zc = reinterpret_cast<float*>(b + o_zc);
    w->dump = reinterpret_cast<half*>(b + o_dump);
  }
  return off;
}

template <typename T> struct Raw32;
template <> struct Raw32<bf16> {
  __device__ __forceinline__ static float2 f(uint32_t u) { return make_float2(lo_bf(u), hi_bf(u)); }
};
template <> struct Raw32<half> {
  __device__ __forceinline__ static float2 f(uint32_t u) {
    f16x2 v = __builtin_bit_cast(f16x2, u);
    return make_float2((float)v.x, (float)v.y);
  }
};

// eight consecutive 16-bit inputs -> float (exact) or fp16 (the MFMA operand type)
template <typename T> struct Raw16;
template <> struct Raw16<bf16> {
  __device__ __forceinline__ static void f32(u32x4 u, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo_bf(u[i]);
      x[2 * i + 1] = hi_bf(u[i]);
    }
  }
  __device__ __forceinline__ static u32x4 f16(u32x4 u) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[2 * i] = (half)lo_bf(u[i]);
      h[2 * i + 1] = (half)hi_bf(u[i]);
    }
    return __builtin_bit_cast(u32x4, h);
  }
};
template <> struct Raw16<half> {
  __device__ __forceinline__ static void f32(u32x4 u, float* x) {
    const f16x8 h = __builtin_bit_cast(f16x8, u);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)h[i];
  }
  __device__ __forceinline__ static u32x4 f16(u32x4 u) { return u; }
};

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i returns element (i & 3) of the 8-byte rows addressed by lanes
// (i >> 2), 4 + (i >> 2), 8 + (i >> 2) and 12 + (i >> 2) of its group.
__device__ __forceinline__ f16x4 lds_read_tr16(const half* p) {
  typedef short s16x4 __attribute__((__vector_size__(8)));
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(f16x4, v);
}

struct P3 {
  const void *q, *k, *v;
  void* o;
  ret_strides sq, sk, sv, so;
  int h, L, B, nc, nrt;
  int nbh;          // b * h
  int64_t pos0, n_prev;
  unsigned flags;
  const float *state_in, *z_in;
  float *state_out, *z_out;
  Work w;
};

// the workgroups of one group (same head and chunk) land on one XCD
__device__ __forceinline__ int xcd_local(int g, int n) {
  return ((n & 7) == 0) ? (g & 7) * (n >> 3) + (g >> 3) : g;
}

// offset of state operand element (col, d) within one chunk's DV x DK block,
// stored in MFMA B-fragment order: the block of 32 columns and 16 d is 1 KB,
// in which lane 32 ((d / 8) % 2) + col % 32 holds its 8 consecutive d as 16
// contiguous bytes (the fragment of a 32x32x16 MFMA with k = d)
__device__ __forceinline__ int rt_frag(int col, int d) {
  return (((col >> 5) * (DK / 16) + (d >> 4)) * 64 + ((d >> 3) & 1) * 32 + (col & 31)) * 8 + (d & 7);
}

__device__ __forceinline__ float maxabs_block(float v, float* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float m = 0.f;
  for (int i = 0; i < (int)(blockDim.x >> 6); ++i) m = fmaxf(m, red[i]);
  return m;
}

// power-of-two exponent that puts max |x| just below 2^15
__device__ __forceinline__ int scale_exp(float amax) {
  if (!(amax > 0.f) || !(amax < 3.0e38f)) return 0;
  int ex;
  frexpf(amax, &ex);
  return min(max(ex - 15, -100), 100);
}

// ---------------------------------------------------------------- delta
// natural-layout fp16 tiles ([key][d] and [key][col]); both MFMA operands
// (k = key) are read with the transposed LDS read.  Row pitch 576 bytes: the
// four key rows of one transposed read start 64 bytes apart in the bank space.
constexpr int DP = 256 + 32;
struct DeltaSmem {
  half Kz[2][TK * DP];  // zeta-scaled rotated keys [key][d], two tiles
  half Vh[2][TK * DP];  // this half of the value tile [key][col], two tiles
  float dzs[DK];
  float4 step[DK / 2];  // per pair: e^{i theta} and e^{i TK theta} as (c1, s1, cT, sT)
};

template <typename T>
__global__ void __launch_bounds__(NT3, 1) delta_kernel(P3 p, HeadParams hp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  DeltaSmem& sm = *reinterpret_cast<DeltaSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = xcd_local(blockIdx.x, gridDim.x);
  const int half_ = g & 1;
  const int c = (g >> 1) % p.nc;
  const int bh = (g >> 1) / p.nc;
  const int bb = bh / p.h, head = bh % p.h;
  const int c0 = c * p.B;
  const int Bc = min(p.B, p.L - c0);
  Decay dec;
  dec.init(hp.gamma[head]);
  const bool xpos = (p.flags & RET_XPOS) != 0;

  const T* Kg = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + head * p.sk.h + (int64_t)c0 * p.sk.l;
  const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + (int64_t)c0 * p.sv.l + half_ * 256;
  half* ktg = p.w.kt + ((int64_t)bh * p.L + c0) * DK;

  // wave tile: d rows [(wave >> 1) * 64, +64), columns [(wave & 1) * 128, +128)
  const int d0 = (wave >> 1) * 64, n0 = (wave & 1) * 128;
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // thread -> 16-byte piece cq (d or columns 8 cq .. 8 cq + 7) of keys
  // 4 (tid / 32) + 0..3 of every tile
  const int cq = tid & 31, kq = 4 * (tid >> 5);
  float dzp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // key-sum of d 8 cq .. +7
  // xPos phase of this thread's first key in the current tile for its four
  // pairs, the one-key and the one-tile steps
  float pc[4], ps[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    pc[u] = 1.f;
    ps[u] = 0.f;
    if (xpos) phase(p.pos0 + c0 + kq, hp.theta[4 * cq + u], pc[u], ps[u]);
  }
  if (xpos && tid < DK / 2) {
    float4 t;
    phase(1, hp.theta[tid], t.x, t.y);
    phase(TK, hp.theta[tid], t.z, t.w);
    sm.step[tid] = t;
  }
  __syncthreads();

  const int nkt = (Bc + TK - 1) / TK;
  u32x4 kr[4], vr[4];
  auto issue = [&](int kt) {
    const int k0 = kt * TK;
    const int kvalid = min(TK, Bc - k0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kc = min(kq + i, kvalid - 1);
      kr[i] = *reinterpret_cast<const u32x4*>(Kg + (uint32_t)((k0 + kc) * (int)p.sk.l + 8 * cq));
      vr[i] = *reinterpret_cast<const u32x4*>(Vg + (uint32_t)((k0 + kc) * (int)p.sv.l + 8 * cq));
    }
  };
  // transposed-read origin of this lane (see lds_read_tr16): key 8 (lane / 32)
  // + (lane % 16) / 4, column 16 ((lane / 16) % 2) + 4 (lane % 4)
  const int tro = (8 * (lane >> 5) + ((lane & 15) >> 2)) * DP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // ---- rotate the keys (-> workspace), scale by zeta (-> LDS, key-sum);
  // convert the values (-> LDS), tile kt into LDS buffer buf
  auto stage = [&](int kt, int buf) {
    const int k0 = kt * TK;
    const int kvalid = min(TK, Bc - k0);
    float x[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Raw16<T>::f32(kr[i], x[i]);
      if (kq + i >= kvalid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
      }
    }
    if (xpos) {
      // pair-outer: each pair's phase advances once per key
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float4 t1 = sm.step[4 * cq + u];
        float cs = pc[u], sn = ps[u];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rot(x[i][2 * u], x[i][2 * u + 1], cs, sn);
          if (i < 3) advance(cs, sn, t1.x, t1.y);
        }
        advance(pc[u], ps[u], t1.z, t1.w);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = kq + i;
      if (half_ == 0 && key < kvalid) st8(ktg + (int64_t)(k0 + key) * DK + 8 * cq, x[i]);
      const float z = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - key) * dec.lg2);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[i][e] *= z;
        dzp[e] += x[i][e];
      }
      st8(sm.Kz[buf] + key * DP + 8 * cq, x[i]);
      u32x4 v = Raw16<T>::f16(vr[i]);
      if (key >= kvalid) v = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(sm.Vh[buf] + key * DP + 8 * cq) = v;
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int kb = 0; kb < TK; kb += 16) {
      f16x8 af[2], bf[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const half* ap = sm.Kz[buf] + kb * DP + d0 + 32 * i + tro;
        const f16x4 lo = lds_read_tr16(ap), hi = lds_read_tr16(ap + 4 * DP);
        af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const half* bp = sm.Vh[buf] + kb * DP + n0 + 32 * jj + tro;
        const f16x4 lo = lds_read_tr16(bp), hi = lds_read_tr16(bp + 4 * DP);
        bf[jj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[i][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[jj], acc[i][jj], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // two LDS buffers: tile kt + 1 is staged while tile kt is multiplied (one
  // barrier per tile); tile kt + 2 is then loaded into registers
  issue(0);
  stage(0, 0);
  if (nkt > 1) issue(1);
  __syncthreads();
  // waves 4..7 (the second wave on each SIMD) stage before they multiply, so
  // the two waves of a SIMD overlap VALU staging with MFMA
  const bool stage_first = wave >= 4;
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (!stage_first) mma(kt & 1);
    if (more) {
      stage(kt + 1, (kt + 1) & 1);
      if (kt + 2 < nkt) issue(kt + 2);
    }
    if (stage_first) mma(kt & 1);
    __syncthreads();
  }

  // ---- key-sum delta: lanes l and l + 32 share a piece; the 8 waves'
  // partials are summed in a fixed order (bit-reproducible)
  if (half_ == 0) {
    float* part = reinterpret_cast<float*>(&sm.Kz[0][0]);   // [8 waves][DK], LDS free after the loop
#pragma unroll
    for (int e = 0; e < 8; ++e) dzp[e] += __shfl_xor(dzp[e], 32, 64);
    if (lane < 32) {
#pragma unroll
      for (int e = 0; e < 8; ++e) part[wave * DK + 8 * cq + e] = dzp[e];
    }
    __syncthreads();
    if (tid < DK) {
      float sum = 0.f;
#pragma unroll
      for (int w = 0; w < NT3 / 64; ++w) sum += part[w * DK + tid];
      sm.dzs[tid] = sum;
    }
  }

  // ---- store dR (scaled fp16, [col][d]) and its scale, dz
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(acc[i][jj][r]));
  amax = maxabs_block(amax, reinterpret_cast<float*>(&sm.Vh[0][0]));
  const int e = scale_exp(amax);
  const float down = ldexpf(1.f, -e);
  half* dR = p.w.dR + ((int64_t)bh * p.nc + c) * DV * DK;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int col = half_ * 256 + n0 + 32 * jj + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = d0 + 32 * i + 8 * rg + 4 * (lane >> 5);   // acc rows 4*rg .. 4*rg+3 are d .. d+3
        float x[4] = {acc[i][jj][4 * rg] * down, acc[i][jj][4 * rg + 1] * down, acc[i][jj][4 * rg + 2] * down,
                      acc[i][jj][4 * rg + 3] * down};
        st4(dR + (int64_t)col * DK + d, x);
      }
    }
  if (tid == 0) p.w.dRs[((int64_t)bh * p.nc + c) * 2 + half_] = ldexpf(1.f, e);
  if (half_ == 0 && tid < DK) p.w.dz[((int64_t)bh * p.nc + c) * DK + tid] = sm.dzs[tid];
}

// ---------------------------------------------------------------- scan
// one workgroup (256 threads) per head and block of 32 state columns; thread
// -> column cb*32 + tid/8 and 32 consecutive d
__global__ void __launch_bounds__(256) scan_kernel(P3 p, HeadParams hp) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const int cb = blockIdx.x % NCB, bh = blockIdx.x / NCB;
  const int head = bh % p.h;
  const int col = cb * 32 + (tid >> 3);
  const int dbase = (tid & 7) * 32;
  const int half_ = col >> 8;
  Decay dec;
  dec.init(hp.gamma[head]);
  float R[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    R[i] = p.state_in ? p.state_in[((int64_t)bh * DK + dbase + i) * DV + col] : 0.f;
  float z = 0.f;
  if (cb == 0 && p.z_in) z = p.z_in[(int64_t)bh * DK + tid];
  // the next chunk's delta is loaded while the current state is published
  u32x4 nx[4];
  float nds = 0.f, ndz = 0.f;
  auto load_delta = [&](int c) {
    const half* src = p.w.dR + (((int64_t)bh * p.nc + c) * DV + col) * DK + dbase;
#pragma unroll
    for (int i = 0; i < 4; ++i) nx[i] = *reinterpret_cast<const u32x4*>(src + 8 * i);
    nds = p.w.dRs[((int64_t)bh * p.nc + c) * 2 + half_];
    if (cb == 0) ndz = p.w.dz[((int64_t)bh * p.nc + c) * DK + tid];
  };
  load_delta(0);
  for (int c = 0; c < p.nc; ++c) {
    const int Bc = min(p.B, p.L - c * p.B);
    u32x4 cur[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cur[i] = nx[i];
    const float ds = nds, dzc = ndz;
    if (c + 1 < p.nc) load_delta(c + 1);
    // publish R_{c-1} and z_{c-1}
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(R[i]));
    amax = maxabs_block(amax, red);
    const int e = scale_exp(amax);
    const float down = ldexpf(1.f, -e);
    half* dst = p.w.Rt + ((int64_t)bh * p.nc + c) * DV * DK;
#pragma unroll
    for (int i = 0; i < 32; i += 8) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = R[i + u] * down;
      st8(dst + rt_frag(col, dbase + i), x);
    }
    if (tid == 0) p.w.Rs[((int64_t)bh * p.nc + c) * NCB + cb] = ldexpf(1.f, e);
    if (cb == 0) p.w.zc[((int64_t)bh * p.nc + c) * DK + tid] = z;
    // advance
    const float gB = dec.pow((float)Bc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f16x8 v = __builtin_bit_cast(f16x8, cur[i]);
#pragma unroll
      for (int u = 0; u < 8; ++u) R[8 * i + u] = gB * R[8 * i + u] + (float)v[u] * ds;
    }
    if (cb == 0) z = gB * z + dzc;
  }
  if (p.state_out) {
#pragma unroll
    for (int i = 0; i < 32; ++i) p.state_out[((int64_t)bh * DK + dbase + i) * DV + col] = R[i];
  }
  if (cb == 0 && p.z_out) p.z_out[(int64_t)bh * DK + tid] = z;
}

// ---------------------------------------------------------------- state scan (small chunks)
// For small chunks the state update of a chunk, K'_[i]^T (V_[i] (.) zeta), is
// a rank-B update.  Instead of writing it out per chunk and scanning it (the
// delta and scan kernels, whose per-chunk state traffic dominates when B is
// small), one workgroup per head and block of 64 state columns walks the
// chunks in order: it keeps its 256 x 64 block of R in fp32 MFMA accumulators,
// publishes R_{c-1} (fp16, a power of two per 32 columns) and z_{c-1} for the
// output kernel, and applies the update on MFMA from the chunk's rotated,
// zeta-scaled keys and its values.  The workgroups of column block 0 also
// write the rotated keys for the output kernel and carry the key-sum z.
constexpr int SCB = 64;             // state columns per workgroup
constexpr int VBP = SCB + 32;       // fp16 pitch of the value block [key][col] (192 bytes)
constexpr int RSP = DK + 8;         // fp16 pitch of the published block [col][d]
struct SScanSmem {
  half Kz[TK * DP];                 // zeta-scaled rotated keys of one 64-key tile [key][d]
  half Vb[TK * VBP];                // the block's value columns of the tile [key][col]
  half Rst[SCB * RSP];              // R_{c-1} operand [col][d] before it is stored
  float amaxw[NT3 / 64][2];         // per wave and 32-column block: max |R|
  float dzw[NT3 / 64][DK];          // per wave: key-sum partials of the chunk
  float4 step[DK / 2];              // per pair: e^{i theta} and e^{i TK theta}
};

// Every global load and store in the tile loop is unconditional (phantom
// tiles pad a short last chunk, masked lanes store to a scratch slot or repeat
// a value another lane stores), and the next tile is loaded into the second
// register set before any store of the current one: the waits for a tile's
// loads then never include the (write-bandwidth-bound) stores of the
// published states.  TPC = tiles per chunk (1 or 2); LEAD = column block 0.
template <typename T, int TPC>
__global__ void __launch_bounds__(NT3, 1) sscan_kernel(P3 p, HeadParams hp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SScanSmem& sm = *reinterpret_cast<SScanSmem*>(smem_raw);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31;
  constexpr int NCB64 = DV / SCB;
  const int g = xcd_local(blockIdx.x, gridDim.x);   // the column blocks of a head share an XCD
  const int cb = g % NCB64, bh = g / NCB64;
  const int bb = bh / p.h, head = bh % p.h;
  Decay dec;
  dec.init(hp.gamma[head]);
  const bool xpos = (p.flags & RET_XPOS) != 0;
  const T* Kg = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + head * p.sk.h;
  const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + cb * SCB;
  half* ktg = p.w.kt + (int64_t)bh * p.L * DK;
  half* dump = p.w.dump + tid * 8;                   // 16-byte scratch slot of this thread

  if (xpos && tid < DK / 2) {
    float4 t;
    phase(1, hp.theta[tid], t.x, t.y);
    phase(TK, hp.theta[tid], t.z, t.w);
    sm.step[tid] = t;
  }

  // R block: wave w holds d rows [32 w, +32) of column tiles jj = 0, 1
  const int d0 = 32 * wave;
  f32x16 acc[2];
#pragma unroll
  for (int jj = 0; jj < 2; ++jj)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      acc[jj][r] = p.state_in ? p.state_in[((int64_t)bh * DK + d0 + acc_row(r, lane)) * DV + cb * SCB + 32 * jj + l32]
                              : 0.f;
  // key-sum z of d = tid % 256 (threads tid and tid + 256 carry the same value)
  const int zd = tid & (DK - 1);
  float z = p.z_in ? p.z_in[(int64_t)bh * DK + zd] : 0.f;

  // staging maps: keys kq .. kq + 3, d 8 cq .. 8 cq + 7; value key vk, columns 8 vp ..
  const int cq = tid & 31, kq = 4 * (tid >> 5);
  const int vk = tid >> 3, vp = tid & 7;
  float pc[4], ps[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    pc[u] = 1.f;
    ps[u] = 0.f;
    if (xpos) phase(p.pos0 + kq, hp.theta[4 * cq + u], pc[u], ps[u]);
  }
  const int tro = (8 * (lane >> 5) + ((lane & 15) >> 2)) * DP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int trv = (8 * (lane >> 5) + ((lane & 15) >> 2)) * VBP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // 64-key tiles are numbered over the whole sequence, TPC per chunk (the
  // last chunk's missing tiles are phantoms with no valid key)
  struct Regs {
    u32x4 k[4], v;
  } ra, rb;
  const int ntiles = p.nc * TPC;
  auto issue = [&](int kt, Regs& R) {
    const int k0 = kt * TK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = min(k0 + kq + i, p.L - 1);
      R.k[i] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)key * p.sk.l + 8 * cq);
    }
    const int key = min(k0 + vk, p.L - 1);
    R.v = *reinterpret_cast<const u32x4*>(Vg + (int64_t)key * p.sv.l + 8 * vp);
  };
  issue(0, ra);
  __syncthreads();                                   // step table

  auto body = [&](auto lead_c) {
    constexpr bool LEAD = decltype(lead_c)::value;
    float dzp[8];
    float gprev = 1.f;                               // gamma^(B of the previous chunk)
    // tile s of chunk c from register set cur; the next tile goes to nxt
    auto step = [&](int c, auto s_c, Regs& cur, Regs& nxt) {
      constexpr int s = decltype(s_c)::value;
      const int kt = c * TPC + s;
      issue(min(kt + 1, ntiles - 1), nxt);
      const int c0 = c * p.B;
      const int Bc = min(p.B, p.L - c0);
      const int k0 = s * TK;                         // chunk-local first key of the tile
      const int kvalid = min(TK, Bc - k0);           // <= 0 for a phantom tile
      if (s == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dzp[e] = 0.f;
      }
      // ---- stage the tile: rotate the keys (-> workspace), scale by zeta (->
      // LDS, key-sum); convert the value block (-> LDS)
      {
        float x[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          Raw16<T>::f32(cur.k[i], x[i]);
          if (kq + i >= kvalid) {
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
          }
        }
        if (xpos) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const float4 t1 = sm.step[4 * cq + u];
            float cs = pc[u], sn = ps[u];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              rot(x[i][2 * u], x[i][2 * u + 1], cs, sn);
              if (i < 3) advance(cs, sn, t1.x, t1.y);
            }
            advance(pc[u], ps[u], t1.z, t1.w);
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = kq + i;
          if (LEAD) st8(key < kvalid ? ktg + (int64_t)(c0 + k0 + key) * DK + 8 * cq : dump, x[i]);
          const float zt = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - key) * dec.lg2);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            x[i][e] *= zt;
            dzp[e] += x[i][e];
          }
          st8(sm.Kz + key * DP + 8 * cq, x[i]);
        }
        u32x4 v = Raw16<T>::f16(cur.v);
        if (vk >= kvalid) v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm.Vb + vk * VBP + 8 * vp) = v;
      }
      if (s == 0) {
        // ---- publish R_{c-1}: per 32-column block, a power of two puts max |R| in [2^14, 2^15)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          float m = 0.f;
#pragma unroll
          for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[jj][r]));
#pragma unroll
          for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
          if (lane == 0) sm.amaxw[wave][jj] = m;
        }
      }
      __syncthreads();
      if (s == 0) {
        float down[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          float m = 0.f;
#pragma unroll
          for (int w = 0; w < NT3 / 64; ++w) m = fmaxf(m, sm.amaxw[w][jj]);
          const int e = scale_exp(m);
          down[jj] = ldexpf(1.f, -e);
          p.w.Rs[((int64_t)bh * p.nc + c) * NCB + 2 * cb + jj] = ldexpf(1.f, e);   // every thread: one value
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            // acc rows 4 rg .. 4 rg + 3 are d .. d + 3
            const int d = d0 + 8 * rg + 4 * (lane >> 5);
            float x4[4] = {acc[jj][4 * rg] * down[jj], acc[jj][4 * rg + 1] * down[jj],
                           acc[jj][4 * rg + 2] * down[jj], acc[jj][4 * rg + 3] * down[jj]};
            st4(sm.Rst + (32 * jj + l32) * RSP + d, x4);
          }
        if (LEAD) {
          // z_{c-1}: the key-sum of the previous chunk, summed over the waves in order
          if (c > 0) {
            float dz = 0.f;
#pragma unroll
            for (int w = 0; w < NT3 / 64; ++w) dz += sm.dzw[w][zd];
            z = gprev * z + dz;
          }
          p.w.zc[((int64_t)bh * p.nc + c) * DK + zd] = z;
        }
        __syncthreads();
        // fragment order: the 64 pieces of one (32 columns, 16 d) block are contiguous
        half* dst = p.w.Rt + ((int64_t)bh * p.nc + c) * DV * DK + (int64_t)cb * SCB * DK;
#pragma unroll
        for (int i = 0; i < SCB * DK / 8 / NT3; ++i) {
          const int e = tid + i * NT3;
          const int blk = e >> 6, slot = e & 63;
          const int col = (blk >> 4) * 32 + (slot & 31), d = 16 * (blk & 15) + 8 * (slot >> 5);
          *reinterpret_cast<u32x4*>(dst + (int64_t)e * 8) = *reinterpret_cast<const u32x4*>(sm.Rst + col * RSP + d);
        }
        const float gB = dec.pow((float)Bc);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) acc[jj] *= gB;
        gprev = gB;
      }
      // ---- R += (K' zeta)^T V over the tile's keys
#pragma unroll
      for (int kb = 0; kb < TK; kb += 16) {
        const half* ap = sm.Kz + kb * DP + d0 + tro;
        const f16x4 alo = lds_read_tr16(ap), ahi = lds_read_tr16(ap + 4 * DP);
        const f16x8 af = __builtin_shufflevector(alo, ahi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const half* bp = sm.Vb + kb * VBP + 32 * jj + trv;
          const f16x4 lo = lds_read_tr16(bp), hi = lds_read_tr16(bp + 4 * VBP);
          const f16x8 bf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, bf, acc[jj], 0, 0, 0);
        }
      }
      if (s == TPC - 1 && LEAD) {
        // this chunk's key-sum partials: lanes l and l + 32 share a piece
#pragma unroll
        for (int e = 0; e < 8; ++e) dzp[e] += __shfl_xor(dzp[e], 32, 64);
        if (lane < 32) {
#pragma unroll
          for (int e = 0; e < 8; ++e) sm.dzw[wave][8 * cq + e] = dzp[e];
        }
      }
      __syncthreads();
    };
    typedef std::integral_constant<int, 0> S0;
    typedef std::integral_constant<int, 1> S1;
    if (TPC == 2) {
      for (int c = 0; c < p.nc; ++c) {
        step(c, S0{}, ra, rb);
        step(c, S1{}, rb, ra);
      }
    } else {
      int c = 0;
      for (; c + 1 < p.nc; c += 2) {
        step(c, S0{}, ra, rb);
        step(c + 1, S0{}, rb, ra);
      }
      if (c < p.nc) step(c, S0{}, ra, rb);
    }
    if (LEAD) {
      float dz = 0.f;
#pragma unroll
      for (int w = 0; w < NT3 / 64; ++w) dz += sm.dzw[w][zd];
      z = gprev * z + dz;
      if (p.z_out && tid < DK) p.z_out[(int64_t)bh * DK + tid] = z;
    }
  };
  if (cb == 0) body(std::true_type{});
  else body(std::false_type{});
  if (p.state_out) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        p.state_out[((int64_t)bh * DK + d0 + acc_row(r, lane)) * DV + cb * SCB + 32 * jj + l32] = acc[jj][r];
  }
}

// ---------------------------------------------------------------- output
struct OutSmem {
  half Qs[TR * QP];
  union {
    struct {
      half Ks[TK * QP];
      half Vn[TK * DV];     // value tile [key][col] (fp16), pieces swizzled (vswz)
    } kv;
  } u;
  half Ps[TR * KP];
  float rs[TR], xs[TR], dens[TR];
  float dpart[2][TR];       // within-chunk row sums of key halves 0 / 1
  float zs[DK];
  float ginv[32];           // gamma^-m, m = 0 .. 31
};

template <typename T, typename TO>
__global__ void __launch_bounds__(NT3, 1) output_kernel(P3 p, HeadParams hp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  // Persistent schedule: one workgroup per CU walks a static list of query
  // tiles.  Every workgroup's tiles pair up as rt and nrt - 1 - rt, so all
  // workgroups carry the same work; a chunk's tiles run side by side on the
  // workgroups of one XCD (workgroup i runs on XCD i mod 8), sharing the
  // chunk's keys, values and state in that L2.
  const int NX = min(8, (int)gridDim.x);
  const int xw = blockIdx.x % NX, jw = blockIdx.x / NX;
  const int wx = ((int)gridDim.x - xw + NX - 1) / NX;      // workgroups of this XCD
  const int ngroups = p.nbh * p.nc;
  const int gx = (ngroups - xw + NX - 1) / NX;             // (head, chunk) groups of this XCD
  const int U = (p.nrt + 1) / 2;
  // teams of nrt workgroups (when the XCD has at least nrt): a team takes two
  // chunks at a time, member r query tile r of the first and nrt - 1 - r of
  // the second; otherwise units of two tiles of one chunk, round robin
  const bool teams = wx >= p.nrt;
  const int nteams = teams ? wx / p.nrt : 1, team = jw / p.nrt, mem = jw % p.nrt;
  const int npairs = (gx + 1) / 2;
  const int nk = teams ? (team < nteams ? 2 * ((npairs - team + nteams - 1) / nteams) : 0)
                       : 2 * ((gx * U - jw + wx - 1) / wx);
  // item k of this workgroup -> query tile rt of chunk c of head bh; false
  // when the slot is empty
  auto decode = [&](int k, int& rt, int& c, int& bh) -> bool {
    int m;
    if (teams) {
      m = 2 * (team + nteams * (k >> 1)) + (k & 1);
      if (m >= gx) return false;
      rt = (k & 1) ? p.nrt - 1 - mem : mem;
    } else {
      const int un = jw + wx * (k >> 1), pi = k & 1;       // unit, and which of its two tiles
      const int uu = un % U;
      if (pi == 1 && uu == p.nrt - 1 - uu) return false;   // middle tile of an odd count
      rt = pi == 0 ? p.nrt - 1 - uu : uu;                  // heavier tile first
      m = un / U;
    }
    const int grp = xw + NX * m;
    c = grp % p.nc;
    bh = grp / p.nc;
    return rt * TR < min(p.B, p.L - c * p.B);              // ragged last chunk
  };
  // the query tile of an item, as raw element pairs: thread -> pair column
  // tid % 128 of rows 16 (tid / 128) + 0..15.  The next item's tile is loaded
  // while the current item is normalised and stored.
  uint32_t qraw[16];
  auto issue_q = [&](int rt, int c, int bh) {
    const int j = threadIdx.x & 127, grp = threadIdx.x >> 7;
    const int bb = bh / p.h, head = bh % p.h;
    const int r0 = rt * TR;
    const int qvalid = min(TR, min(p.B, p.L - c * p.B) - r0);
    const T* Qg = reinterpret_cast<const T*>(p.q) + bb * p.sq.b + head * p.sq.h + (int64_t)(c * p.B + r0) * p.sq.l;
  #pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int rc = min(grp * 16 + i, qvalid - 1);
      qraw[i] = *reinterpret_cast<const uint32_t*>(Qg + (uint32_t)(rc * (int)p.sq.l + 2 * j));
    }
  };
  int k = 0, rt = 0, c = 0, bh = 0;
  while (k < nk && !decode(k, rt, c, bh)) ++k;
  if (k < nk) issue_q(rt, c, bh);
  while (k < nk) {
    int kn = k + 1, rtn = 0, cn = 0, bhn = 0;
    __syncthreads();                                       // the previous item's LDS reads are done
    {
    OutSmem& sm = *reinterpret_cast<OutSmem*>(smem_raw);
    // the thread index passes through an empty asm each item, so per-lane
    // addressing is recomputed inside the item rather than hoisted out of the
    // persistent loop (where it would stay live across the whole item)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int lh = lane >> 5, l32 = lane & 31;
    const int bb = bh / p.h, head = bh % p.h;
    const int c0 = c * p.B;
    const int Bc = min(p.B, p.L - c0);
    const int r0 = rt * TR;
    const int qvalid = min(TR, Bc - r0);
    Decay dec;
    dec.init(hp.gamma[head]);
    const bool xpos = (p.flags & RET_XPOS) != 0;
    const float qk_scale = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;

    const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + (int64_t)c0 * p.sv.l;
    // z_{c-1} (thread -> d) and the power-of-two scales of this wave's two
    // state column blocks, requested first: they are used after the query
    // rotation and after the cross term
    const int64_t ci = (int64_t)bh * p.nc + c;
    const float zpre = p.w.zc[ci * DK + (tid & (DK - 1))];
    const float up0 = p.w.Rs[ci * NCB + 2 * wave], up1 = p.w.Rs[ci * NCB + 2 * wave + 1];
    const half* Kt = p.w.kt + ((int64_t)bh * p.L + c0) * DK;
    TO* Og = reinterpret_cast<TO*>(p.o) + bb * p.so.b + head * p.so.h + (int64_t)(c0 + r0) * p.so.l;

    // ---- rotated query tile, row tables
    {
      const int j = tid & 127, grp = tid >> 7;      // 16 rows per group
      float a[16], b[16];
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = grp * 16 + i;
        const float2 x = Raw32<T>::f(qraw[i]);
        a[i] = row < qvalid ? x.x : 0.f;
        b[i] = row < qvalid ? x.y : 0.f;
      }
      float cs = 1.f, sn = 0.f, c1 = 1.f, s1 = 0.f;
      if (xpos) {
        phase(p.pos0 + c0 + r0 + grp * 16, hp.theta[j], cs, sn);
        phase(1, hp.theta[j], c1, s1);
      }
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (xpos) {
          rot(a[i], b[i], cs, sn);
          advance(cs, sn, c1, s1);
        }
        st2(sm.Qs + (grp * 16 + i) * QP + 2 * j, a[i], b[i]);
      }
      if (tid < TR) {
        float s = qk_scale;
        if (p.flags & RET_NORM_DROW) s *= dec.drow((float)(p.n_prev + c0 + r0 + tid + 1));
        sm.rs[tid] = s;
        sm.xs[tid] = s * dec.pow((float)(r0 + tid + 1));
        sm.dens[tid] = 0.f;
      }
      if (tid < DK) sm.zs[tid] = zpre;
      if (tid < 32) sm.ginv[tid] = __builtin_amdgcn_exp2f(-(float)tid * dec.lg2);
    }

    // ---- staged key / value tile registers
    u32x4 kreg[4];          // 64 keys x 256 d fp16: 2048 16-byte pieces, 4 per thread
    u32x4 vreg[8];          // 64 keys x 512 columns: 4096 16-byte pieces, 8 per thread
    auto issue_k = [&](int kt) {
      const int k0 = kt * TK;
      const int kvalid = min(TK, Bc - k0);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + i * NT3;
        const int key = min(e >> 5, kvalid - 1), piece = e & 31;
        kreg[i] = *reinterpret_cast<const u32x4*>(Kt + (int64_t)(k0 + key) * DK + piece * 8);
      }
    };
    auto issue_v = [&](int kt) {
      const int k0 = kt * TK;
      const int kvalid = min(TK, Bc - k0);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = tid + i * NT3;
        const int key = min(e >> 6, kvalid - 1), piece = e & 63;
        vreg[i] = *reinterpret_cast<const u32x4*>(Vg + (uint32_t)((k0 + key) * (int)p.sv.l + piece * 8));
      }
    };
    auto commit_k = [&](int kt) {
      const int kvalid = min(TK, Bc - kt * TK);
  #pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = tid + i * NT3;
        const int key = e >> 5, piece = e & 31;
        u32x4 v = kreg[i];
        if (key >= kvalid) v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm.u.kv.Ks + key * QP + piece * 8) = v;
      }
    };
    auto commit_v = [&](int kt) {
      const int kvalid = min(TK, Bc - kt * TK);
  #pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = tid + i * NT3;
        const int key = e >> 6, piece = e & 63;
        u32x4 v = Raw16<T>::f16(vreg[i]);
        if (key >= kvalid) v = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(sm.u.kv.Vn + key * DV + vswz(key, piece) * 8) = v;
      }
    };
    // this lane's transposed-read origin in a value tile: key 8 (lane / 32) +
    // (lane % 16) / 4, column 16 ((lane / 16) % 2) + 4 (lane % 4)
    // (swizzled: the lane's key row has r % 4 = (lane / 4) % 4)
    const int vtr_row = (8 * (lane >> 5) + ((lane & 15) >> 2)) * DV + 4 * (lane & 1);
    const int vtr_sw = ((lane >> 2) & 3) << 2, vtr_lo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);

    // output tiles of this wave: query halves {0,1} x column tiles {2w, 2w+1}
    f32x16 O[2][2];
  #pragma unroll
    for (int i = 0; i < 2; ++i)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) O[i][jj] = f32x16{};

    // ---- cross-chunk term Q' R_{c-1}.  Wave w owns state columns 64 w ..
    // 64 w + 63.  The state operand is stored in MFMA fragment order (a
    // 32-column x 16-d block is one 1 KB wave load), so each wave streams its
    // B fragments straight from global memory, XR steps ahead, with no LDS
    // staging and no barriers.  The first key / value tile is loaded meanwhile.
    issue_k(rt);
    issue_v(rt);
    __syncthreads();                                // the query tile and the row tables
    {
      constexpr int NSX = DK / 16, XR = 4;
      const half* rp = p.w.Rt + ((int64_t)bh * p.nc + c) * DV * DK + (int64_t)(2 * wave * NSX * 64 + lane) * 8;
      f16x8 rb[XR][2], qa[2][2];
  #pragma unroll
      for (int t = 0; t < XR; ++t)
  #pragma unroll
        for (int jj = 0; jj < 2; ++jj) rb[t][jj] = *reinterpret_cast<const f16x8*>(rp + (int64_t)(jj * NSX + t) * 512);
      auto load_q = [&](int t, int buf) {
  #pragma unroll
        for (int qh = 0; qh < 2; ++qh)
          qa[buf][qh] = *reinterpret_cast<const f16x8*>(sm.Qs + (qh * 32 + l32) * QP + 16 * t + 8 * lh);
      };
      load_q(0, 0);
  #pragma unroll
      for (int t = 0; t < NSX; ++t) {
        if (t + 1 < NSX) load_q(t + 1, (t + 1) & 1);
        __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
        for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            O[qh][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(qa[t & 1][qh], rb[t % XR][jj], O[qh][jj], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (t + XR < NSX) {
  #pragma unroll
          for (int jj = 0; jj < 2; ++jj)
            rb[t % XR][jj] = *reinterpret_cast<const f16x8*>(rp + (int64_t)(jj * NSX + t + XR) * 512);
        }
      }
    }
    {
      // row scale s xi and the operand's per-block power of two
  #pragma unroll
      for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = sm.xs[qh * 32 + acc_row(r, lane)];
          O[qh][0][r] *= x * up0;
          O[qh][1][r] *= x * up1;
        }
      // cross part of the score denominator, s xi (Q' . z_{c-1}): 8 threads per row
      const int row = tid >> 3, part = tid & 7;     // d 32 part .. 32 part + 31
      float acc = 0.f;
  #pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f16x8 qv = *reinterpret_cast<const f16x8*>(sm.Qs + row * QP + 32 * part + 8 * u);
        const f32x4 z0 = *reinterpret_cast<const f32x4*>(sm.zs + 32 * part + 8 * u);
        const f32x4 z1 = *reinterpret_cast<const f32x4*>(sm.zs + 32 * part + 8 * u + 4);
  #pragma unroll
        for (int e = 0; e < 4; ++e) acc += (float)qv[e] * z0[e];
  #pragma unroll
        for (int e = 0; e < 4; ++e) acc += (float)qv[4 + e] * z1[e];
      }
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      if (part == 0) sm.dens[row] = sm.xs[row] * acc;
    }

    // ---- within-chunk term, diagonal key tile first (tile order rt, 0, 1, ..)
    // Two phases per key tile, one barrier after each:
    //   1. waves 0..3 form S^T = K' Q'^T as 32 x 32 tiles (keys 32 (w / 2) ..,
    //      queries 32 (w % 2) ..) and write P; then every wave commits its
    //      share of the value tile and loads the next one
    //   2. all eight waves accumulate P V, then commit the next key tile and
    //      load the one after
    float den = 0.f;
    const int sk = wave >> 1, sqh = wave & 1;
    commit_k(rt);                                   // the key / value region is free since the item began
    if (rt > 0) issue_k(0);
    __syncthreads();
    for (int idx = 0; idx <= rt; ++idx) {
      const int kt = (idx == 0) ? rt : idx - 1;
      const bool diag = (idx == 0);
      const int k0 = kt * TK;
      if (wave < 4) {
        const bool skip = diag && sk > sqh;         // keys 32..63 vs queries 0..31 of the diagonal
        float pv[16];
        if (!skip) {
          // fragments of step s + 3 are read while step s multiplies
          const half* kp = sm.u.kv.Ks + (sk * 32 + l32) * QP + 8 * lh;
          const half* qp = sm.Qs + (sqh * 32 + l32) * QP + 8 * lh;
          constexpr int NS = DK / 16, PD = 4;
          f16x8 ka[PD], qb[PD];
  #pragma unroll
          for (int t = 0; t < PD - 1; ++t) {
            ka[t] = *reinterpret_cast<const f16x8*>(kp + 16 * t);
            qb[t] = *reinterpret_cast<const f16x8*>(qp + 16 * t);
          }
          f32x16 S = {};
  #pragma unroll
          for (int t = 0; t < NS; ++t) {
            if (t + PD - 1 < NS) {
              ka[(t + PD - 1) % PD] = *reinterpret_cast<const f16x8*>(kp + 16 * (t + PD - 1));
              qb[(t + PD - 1) % PD] = *reinterpret_cast<const f16x8*>(qp + 16 * (t + PD - 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            S = __builtin_amdgcn_mfma_f32_32x32x16_f16(ka[t % PD], qb[t % PD], S, 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);      // keep the reads ahead of the multiplies
          }
          // D = gamma^(q - k) split as gamma^base gamma^-(8i + j), base = q - (first key of the lane)
          const int base = r0 + sqh * 32 + l32 - k0 - sk * 32 - 4 * lh;
          const float gq = sm.rs[sqh * 32 + l32] * __builtin_amdgcn_exp2f((float)base * dec.lg2);
          // the causal mask q >= k only bites on the diagonal tile
          auto scale = [&](auto masked) {
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 gi = *reinterpret_cast<const float4*>(sm.ginv + 8 * i);
              const float gv[4] = {gi.x, gi.y, gi.z, gi.w};
  #pragma unroll
              for (int j = 0; j < 4; ++j) {
                float val = S[4 * i + j] * gq * gv[j];
                if (decltype(masked)::value) val = (base >= 8 * i + j) ? val : 0.f;
                den += val;
                pv[4 * i + j] = val;
              }
            }
          };
          if (diag) scale(std::true_type{});
          else scale(std::false_type{});
        } else {
  #pragma unroll
          for (int i = 0; i < 16; ++i) pv[i] = 0.f;
        }
  #pragma unroll
        for (int i = 0; i < 4; ++i) st4(sm.Ps + (sqh * 32 + l32) * KP + sk * 32 + 8 * i + 4 * lh, pv + 4 * i);
      }
      commit_v(kt);
      if (idx < rt) issue_v(idx);                   // next tile: kt = idx
      __syncthreads();
      // O += P V: the value fragment of a column tile serves both query halves
      // (rows 0..31 of P are zero against keys 32..63 of the diagonal tile);
      // the fragments of step s + 1 are read while step s multiplies
      {
        f16x8 pa[2][2], bv[2][2];
        auto load_pv = [&](int kb, int buf) {
  #pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            // keys kb + 8 (lane / 32) + 0..7 of column (2w + jj) 32 + lane % 32
            const half* vp = sm.u.kv.Vn + kb * DV + vtr_row + ((((2 * wave + jj) * 4) ^ vtr_sw) + vtr_lo) * 8;
            const f16x4 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * DV);
            bv[buf][jj] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
            pa[buf][qh] = *reinterpret_cast<const f16x8*>(sm.Ps + (qh * 32 + l32) * KP + kb + 8 * lh);
        };
        load_pv(0, 0);
  #pragma unroll
        for (int t = 0; t < TK / 16; ++t) {
          if (t + 1 < TK / 16) load_pv(16 * (t + 1), (t + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
            for (int jj = 0; jj < 2; ++jj)
              O[qh][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(pa[t & 1][qh], bv[t & 1][jj], O[qh][jj], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (idx < rt) {
        commit_k(idx);                              // next tile: kt = idx
        if (idx + 1 < rt) issue_k(idx + 1);
      }
      __syncthreads();
    }
    // the next item's query tile
    while (kn < nk && !decode(kn, rtn, cn, bhn)) ++kn;
    if (kn < nk) issue_q(rtn, cn, bhn);
    if (wave < 4) {
      den += __shfl_xor(den, 32, 64);               // lanes l and l + 32 hold the same query
      if (lh == 0) sm.dpart[sk][sqh * 32 + l32] = den;
    }
    __syncthreads();
    // cross part plus the two key halves, summed in a fixed order
    if (tid < TR) {
      const float d = sm.dens[tid] + sm.dpart[0][tid] + sm.dpart[1][tid];
      sm.rs[tid] = (p.flags & RET_NORM_SCORE) ? 1.f / fmaxf(fabsf(d), 1.f) : 1.f;
    }

    // ---- normalise and store: the whole tile is staged in LDS in the output
    // type (over the query / key / value buffers, dead by now), then written
    // with 16-byte stores
    __syncthreads();
    TO* Os = reinterpret_cast<TO*>(smem_raw);
    constexpr int OV = 16 / (int)sizeof(TO);        // elements per 16 bytes
    constexpr int OP = DV + OV;                     // staging row pitch
    static_assert(TR * OP * sizeof(TO) <= offsetof(OutSmem, Ps), "staging overlaps live LDS");
  #pragma unroll
    for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int col = (2 * wave + jj) * 32 + l32;
  #pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = qh * 32 + acc_row(r, lane);
          Os[row * OP + col] = Store<TO>::cvt(O[qh][jj][r] * sm.rs[row]);
        }
      }
    __syncthreads();
    for (int e = tid; e < TR * (DV / OV); e += NT3) {
      const int row = e / (DV / OV), cv = e % (DV / OV);
      if (row < qvalid)
        *reinterpret_cast<u32x4*>(Og + (int64_t)row * p.so.l + cv * OV) =
            *reinterpret_cast<const u32x4*>(Os + row * OP + cv * OV);
    }
    }
    k = kn;
    rt = rtn;
    c = cn;
    bh = bhn;
  }
}

static_assert(sizeof(OutSmem) <= 160 * 1024 && sizeof(DeltaSmem) <= 160 * 1024 && sizeof(SScanSmem) <= 160 * 1024,
              "LDS of one workgroup");

// workgroups of the persistent output kernel: one per CU of the current device
int persistent_workgroups() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, typename TO>
hipError_t run(const ChunkArgs& a, hipStream_t st) {
  P3 p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.sq = a.sq; p.sk = a.sk; p.sv = a.sv; p.so = a.so;
  p.h = a.h; p.L = a.L; p.B = a.B;
  p.nc = (a.L + a.B - 1) / a.B;
  p.nrt = a.B / TR;
  p.nbh = a.b * a.h;
  p.pos0 = a.pos0; p.n_prev = a.n_prev; p.flags = a.flags;
  p.state_in = a.state_in; p.z_in = a.z_in; p.state_out = a.state_out; p.z_out = a.z_out;
  const int bh = a.b * a.h;
  carve(a.ws, bh, a.L, a.B, &p.w);
  hipError_t e;
  if (a.B <= SSCAN_MAX_B) {
    auto k = a.B == 2 * TK ? sscan_kernel<T, 2> : sscan_kernel<T, 1>;
    e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(SScanSmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(bh * (DV / SCB)), dim3(NT3), sizeof(SScanSmem), st, p, *a.hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    auto k = delta_kernel<T>;
    e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(DeltaSmem));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(bh * p.nc * 2), dim3(NT3), sizeof(DeltaSmem), st, p, *a.hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(scan_kernel, dim3(bh * NCB), dim3(256), 0, st, p, *a.hp);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  {
    auto k = output_kernel<T, TO>;
    e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(OutSmem));
    if (e != hipSuccess) return e;
    const int units = bh * p.nc * ((p.nrt + 1) / 2);
    int W = min(units, persistent_workgroups());
    if (W >= 8) W -= W % 8;
    hipLaunchKernelGGL(k, dim3(W), dim3(NT3), sizeof(OutSmem), st, p, *a.hp);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t run_o(const ChunkArgs& a, hipStream_t st) {
  if (a.out_dt == RET_BF16) return run<T, bf16>(a, st);
  if (a.out_dt == RET_F16) return run<T, half>(a, st);
  return run<T, float>(a, st);
}

}  // namespace

bool three_phase_applies(ret_dtype in_dt, int dk, int dv, int B) {
  return (in_dt == RET_BF16 || in_dt == RET_F16) && dk == DK && dv == DV && B >= 64 && B % 64 == 0;
}

size_t three_phase_workspace(int b, int h, int L, int B) {
  return carve(nullptr, b * h, L, B, nullptr);
}

hipError_t launch_three_phase(const ChunkArgs& a, hipStream_t st) {
  return a.in_dt == RET_F16 ? run_o<half>(a, st) : run_o<bf16>(a, st);
}

}  // namespace ret
