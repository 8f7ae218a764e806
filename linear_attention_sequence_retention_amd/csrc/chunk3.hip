// Chunkwise recurrent retention forward for large chunks (RetNet reading
// notes, §2.4, with §2.3's xPos rotation and §三.3's normalisations), split
// into three kernels whose boundaries are the only synchronisation:
//
//   delta  (persistent; one unit of work per head, chunk and half of d_v)
//          dR_i = K'_[i]^T (V_[i] (.) zeta),  dz_i = K'_[i]^T zeta
//          and, once per head and chunk, the rotated keys K' in fp16
//   scan   (one workgroup per head and block of 32 state columns)
//          R_i = gamma^(B_i) R_{i-1} + dR_i,  z_i likewise; it stores the
//          state every chunk starts from, R_{i-1}, as an fp16 operand copy
//          scaled by a power of two per block of 32 columns
//   output (persistent; one item per head, chunk and 64-row query tile)
//          O = (Q'K'^T (.) D) V + (Q' R_{i-1}) (.) xi, with the row scales and
//          score normalisation, written once
//
// Chunks of at most 128 keys replace delta and scan by one state-scan kernel
// (one workgroup per head and block of 64 state columns, walking the chunks
// in order with the state in MFMA accumulators), which also rotates the keys.
//
// The keys are rotated only in the delta kernel (by both d_v halves of a
// chunk; the output kernel reads the rotated fp16 keys that half 0 writes),
// and no score is recomputed across d_v slices.  Operands are fp16 with fp32 accumulation.
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

// sequence length rounded up to whole 64-key tiles (the rotated-key region
// holds whole tiles, so a tile read never leaves it)
__host__ __device__ constexpr int lpad(int L) { return (L + TK - 1) / TK * TK; }
// Rotated keys are stored per 64-key tile in the A-fragment order of a
// 32x32x16 MFMA with k = d: the block of 32 keys and 16 d is 1 KB, in which
// lane 32 ((d / 8) % 2) + key % 32 holds its 8 consecutive d as 16 contiguous
// bytes, so one wave load of 1 KB is one fragment.  Offset of (key, d) from
// the head's origin (key counted over the whole sequence):
__host__ __device__ constexpr int64_t kt_off(int key, int d) {
  return (int64_t)(key >> 6) * (TK * DK) +
         (((((key >> 5) & 1) * (DK / 16) + (d >> 4)) * 64 + 32 * ((d >> 3) & 1) + (key & 31)) << 3) + (d & 7);
}

struct Work {
  half* kt;      // rotated keys       [bh][Lp/64][64*DK] (per 64-key tile, MFMA fragment order, kt_off)
  half* dR;      // chunk deltas       [bh][nc][DV][DK]   (column-major: [col][d])
  float* dRs;    // delta scales       [bh][nc][2]        (2^e per d_v half)
  float* dz;     // key-sum deltas     [bh][nc][DK]
  half* Rt;      // state operands     [bh][nc][DV*DK]    (R_{i-1}, fragment order, rt_frag)
  float* Rs;     // operand scales     [bh][nc][NCB]
  float* zc;     // z_{i-1}            [bh][nc][DK]
  half* dump;    // 8 KB that masked lanes of the state scan and output kernels store to (never read)
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
  const size_t o_kt = take((size_t)bh * lpad(L) * DK * 2);
  const size_t o_dR = take(deltas ? (size_t)bh * nc * DV * DK * 2 : 0);
  const size_t o_dRs = take(deltas ? (size_t)bh * nc * 2 * 4 : 0);
  const size_t o_dz = take(deltas ? (size_t)bh * nc * DK * 4 : 0);
  const size_t o_Rt = take((size_t)bh * nc * DV * DK * 2);
  const size_t o_Rs = take((size_t)bh * nc * NCB * 4);
  const size_t o_zc = take((size_t)bh * nc * DK * 4);
  const size_t o_dump = take(NT3 * 16);
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
  unsigned* nf;
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
  half Kz[2][TK * DP];  // rotated keys [key][d], two tiles
  half Vh[2][TK * DP];  // this half of the value tile scaled by zeta [key][col], two tiles
  float dzs[DK];
  float4 step[DK / 2];  // per pair: e^{i theta} and e^{i TK theta} as (c1, s1, cT, sT)
  double theta[DK / 2];
};

template <typename T>
__global__ void __launch_bounds__(NT3, 1) delta_kernel(P3 p, HeadParams hp) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  DeltaSmem& sm = *reinterpret_cast<DeltaSmem*>(smem_raw);
  const int tid0 = threadIdx.x;
  // Persistent: unit g = (head, chunk, half of d_v) with g = 2 (bh nc + c) +
  // half.  Workgroup i runs on XCD i mod 8; each XCD walks a contiguous range
  // of units.  Workgroups 2m and 2m + 1 of an XCD take the two halves of one
  // chunk at every step, swapping halves from step to step (half 0 also
  // writes the rotated keys, so neither falls behind the other): the two read
  // the chunk's keys at the same time, the second read from the XCD's L2.
  // The next unit's first tile is requested during the current unit's last
  // tile, so its latency and the workgroup turnover run under the current
  // unit's dR stores.
  const int U = p.nbh * p.nc * 2;
  const int NX = min(8, (int)gridDim.x);
  const int xw = blockIdx.x % NX, jw = blockIdx.x / NX;
  const int wx = ((int)gridDim.x - xw + NX - 1) / NX;      // workgroups of this XCD
  const int ulo = (int)((int64_t)xw * U / NX), uhi = (int)((int64_t)(xw + 1) * U / NX);
  const bool paired = (wx % 2 == 0) && (ulo % 2 == 0) && (uhi % 2 == 0);
  auto unit_at = [&](int i) {
    return paired ? ulo + 2 * ((jw >> 1) + (wx >> 1) * i) + ((jw ^ i) & 1) : ulo + jw + wx * i;
  };
  int step = 0, g = unit_at(0);
  if (g >= uhi) return;                                    // uniform over the workgroup
  const bool xpos = (p.flags & RET_XPOS) != 0;

  // the key rows and this half's value rows of unit g, and the chunk's length
  auto unit_src = [&](int gu, const T*& Kg_, const T*& Vg_, int& Bc_) {
    const int bhu = (gu >> 1) / p.nc, c0u = ((gu >> 1) % p.nc) * p.B;
    const int bbu = bhu / p.h, hu = bhu % p.h;
    Bc_ = min(p.B, p.L - c0u);
    Kg_ = reinterpret_cast<const T*>(p.k) + bbu * p.sk.b + hu * p.sk.h + (int64_t)c0u * p.sk.l;
    Vg_ = reinterpret_cast<const T*>(p.v) + bbu * p.sv.b + hu * p.sv.h + (int64_t)c0u * p.sv.l + (gu & 1) * 256;
  };
  u32x4 kr[4], vr[4];
  auto issue_at = [&](const T* Kg_, const T* Vg_, int Bc_, int kt) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    const int cq = t & 31, kq = 4 * (t >> 5);
    const int k0 = kt * TK;
    const int kvalid = min(TK, Bc_ - k0);
    // 64-bit tile origin; offsets inside a 64-key tile fit 32 bits (strides < 2^25)
    const T* Kt = Kg_ + (int64_t)k0 * p.sk.l;
    const T* Vt = Vg_ + (int64_t)k0 * p.sv.l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kc = min(kq + i, kvalid - 1);
      kr[i] = *reinterpret_cast<const u32x4*>(Kt + (uint32_t)(kc * (int)p.sk.l + 8 * cq));
      vr[i] = *reinterpret_cast<const u32x4*>(Vt + (uint32_t)(kc * (int)p.sv.l + 8 * cq));
    }
  };
  // per pair, once per workgroup: theta (an fp64 load from global memory
  // inside a unit would wait for the tile loads as well: the vector memory
  // counter completes in order), e^{i theta} and e^{i TK theta}
  if (xpos && tid0 < DK / 2) {
    const double th1 = hp.theta[tid0];
    float4 t;
    phase(1, th1, t.x, t.y);
    phase(TK, th1, t.z, t.w);
    sm.theta[tid0] = th1;
    sm.step[tid0] = t;
  }
  {
    const T *Kg0, *Vg0;
    int Bc0;
    unit_src(g, Kg0, Vg0, Bc0);
    issue_at(Kg0, Vg0, Bc0, 0);
  }
  for (; g < uhi; g = unit_at(++step)) {
  const int gnext = unit_at(step + 1);
  // the thread index passes through an empty asm each unit, so per-lane
  // addressing is recomputed inside the unit rather than hoisted out of the
  // persistent loop (where it would stay live across the whole unit)
  int tl = threadIdx.x;
  asm volatile("" : "+v"(tl));
  const int tid = tl, lane = tl & 63, wave = tl >> 6;
  // thread -> 16-byte piece cq (d or columns 8 cq .. 8 cq + 7) of keys
  // 4 (tid / 32) + 0..3 of every tile
  const int cq = tid & 31, kq = 4 * (tid >> 5);
  const int half_ = g & 1;
  const int c = (g >> 1) % p.nc;
  const int bh = (g >> 1) / p.nc;
  const int head = bh % p.h;
  const int c0 = c * p.B;
  const T *Kg, *Vg;
  int Bc;
  unit_src(g, Kg, Vg, Bc);
  Decay dec;
  dec.init(hp, head);
  half* kth = p.w.kt + (int64_t)bh * lpad(p.L) * DK;

  // wave tile: d rows [(wave >> 1) * 64, +64), columns [(wave & 1) * 128, +128)
  const int d0 = (wave >> 1) * 64, n0 = (wave & 1) * 128;
  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nkt = (Bc + TK - 1) / TK;
  auto issue = [&](int kt) { issue_at(Kg, Vg, Bc, kt); };
  // the unit's first tile was requested before this point (during the
  // previous unit's last tile, or above); the phase set-up runs under it
  __syncthreads();                                  // the previous unit's LDS reads; theta and the steps
  float dzp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};   // key-sum of d 8 cq .. +7
  // xPos phase of this thread's first key in the current tile for its four
  // pairs
  float pc[4], ps[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    pc[u] = 1.f;
    ps[u] = 0.f;
    if (xpos) phase(p.pos0 + c0 + kq, sm.theta[4 * cq + u], pc[u], ps[u]);
  }

  // transposed-read origin of this lane (see lds_read_tr16): key 8 (lane / 32)
  // + (lane % 16) / 4, column 16 ((lane / 16) % 2) + 4 (lane % 4)
  const int tro = (8 * (lane >> 5) + ((lane & 15) >> 2)) * DP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  // ---- rotate the keys (-> LDS; key-sum of the zeta-scaled keys); scale the
  // values by zeta (-> LDS), tile kt into LDS buffer buf.  zeta is applied to
  // the value rows rather than the keys (the same product K'^T (V (.) zeta)),
  // so the LDS key tile is the unscaled rotated keys that the output kernel
  // reads: they are written out from there in fragment order
  auto stage = [&](int kt, int buf) {
    const int k0 = kt * TK;
    const int kvalid = min(TK, Bc - k0);
    // a key past the end of a ragged chunk is zeroed; its value row (a copy
    // of the last key's, from issue) then adds nothing to dR
    float x[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Raw16<T>::f32(kr[i], x[i]);
      if (kq + i >= kvalid) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
      }
    }
    // every load of the tile is taken here, before the first store of rotated
    // keys: a later wait for a value load would also wait for those stores
    // (the vector memory counter completes in order)
#pragma unroll
    for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(vr[i]));
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
      const float z = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - key) * dec.lg2);
      if (half_ == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) dzp[e] += x[i][e] * z;
      }
      st8(sm.Kz[buf] + key * DP + 8 * cq, x[i]);
      float y[8];
      Raw16<T>::f32(vr[i], y);
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] *= z;
      st8(sm.Vh[buf] + key * DP + 8 * cq, y);
    }
  };
  // the rotated keys of tile kt (LDS buffer buf) to the workspace: thread ->
  // 16-byte pieces tid + 512 i of the tile in fragment order, so every wave
  // store is one contiguous 1 KB fragment block
  auto write_kt = [&](int kt, int buf) {
    const int k0 = kt * TK;
    const int kvalid = min(TK, Bc - k0);
    half* dst = kth + kt_off(c0 + k0, 0);
    // the lane's addressing is recomputed here rather than kept live across
    // the tile loop (the registers are needed by the accumulators)
    int t = tid;
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int i = 0; i < TK * DK / 8 / NT3; ++i) {
      const int e = t + i * NT3;
      const int blk = e >> 6, slot = e & 63;           // block (32 keys x 16 d) and its lane slot
      const int key = 32 * (blk / (DK / 16)) + (slot & 31), d = 16 * (blk % (DK / 16)) + 8 * (slot >> 5);
      if (key < kvalid)
        *reinterpret_cast<u32x4*>(dst + (int64_t)e * 8) = *reinterpret_cast<const u32x4*>(sm.Kz[buf] + key * DP + d);
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
  stage(0, 0);
  if (nkt > 1) issue(1);
  __syncthreads();
  // waves 4..7 (the second wave on each SIMD) stage before they multiply, so
  // the two waves of a SIMD overlap VALU staging with MFMA
  const bool stage_first = wave >= 4;
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (half_ == 0) write_kt(kt, kt & 1);
    if (!stage_first) mma(kt & 1);
    if (more) {
      stage(kt + 1, (kt + 1) & 1);
      if (kt + 2 < nkt) issue(kt + 2);
    } else if (gnext < uhi) {
      // the next unit's first tile (the registers are free from here on)
      const T *Kgn, *Vgn;
      int Bcn;
      unit_src(gnext, Kgn, Vgn, Bcn);
      issue_at(Kgn, Vgn, Bcn, 0);
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
  {
    // block max, the wave's slot addressed from the unit's own thread index
    // (a hoisted address would stay live across the unit)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    float* red = reinterpret_cast<float*>(&sm.Vh[0][0]);
    __syncthreads();
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = 0.f;
#pragma unroll
    for (int w = 0; w < NT3 / 64; ++w) amax = fmaxf(amax, red[w]);
  }
  const int e = scale_exp(amax);
  const float down = ldexpf(1.f, -e);
  // the workgroup's 256 columns of dR are one contiguous 128 KB block ([col][d]):
  // staged in LDS (over the dead tiles; pitch 2 mod 64 dwords, so the 32 columns
  // of a write fall in distinct bank pairs), then written with 16-byte stores
  constexpr int RP = DK + 4;
  static_assert(256 * RP * sizeof(half) <= sizeof(sm.Kz) + sizeof(sm.Vh), "dR staging exceeds the tiles");
  half* Rst = &sm.Kz[0][0];
  __syncthreads();                                  // the reductions' LDS reads are done
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int col = n0 + 32 * jj + (lane & 31);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d = d0 + 32 * i + 8 * rg + 4 * (lane >> 5);   // acc rows 4*rg .. 4*rg+3 are d .. d+3
        float x[4] = {acc[i][jj][4 * rg] * down, acc[i][jj][4 * rg + 1] * down, acc[i][jj][4 * rg + 2] * down,
                      acc[i][jj][4 * rg + 3] * down};
        st4(Rst + col * RP + d, x);
      }
    }
  __syncthreads();
  half* dR = p.w.dR + (((int64_t)bh * p.nc + c) * DV + half_ * 256) * DK;
#pragma unroll
  for (int i = 0; i < 256 * DK / 8 / NT3; ++i) {
    const int e = tid + i * NT3;
    const int col = e >> 5, piece = e & 31;
    *reinterpret_cast<u32x4*>(dR + (int64_t)e * 8) = *reinterpret_cast<const u32x4*>(Rst + col * RP + piece * 8);
  }
  if (tid == 0) p.w.dRs[((int64_t)bh * p.nc + c) * 2 + half_] = ldexpf(1.f, e);
  if (half_ == 0 && tid < DK) p.w.dz[((int64_t)bh * p.nc + c) * DK + tid] = sm.dzs[tid];
  }
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
  dec.init(hp, head);
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
    // a state that an fp16 operand overflow made non-finite is recorded as
    // such (no later chunk of this call reads it, so no output shows it)
    bool bad = false;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      p.state_out[((int64_t)bh * DK + dbase + i) * DV + col] = R[i];
      bad |= nonfinite_as<float>(R[i]);
    }
    flag_nonfinite(p.nf, bad, kNonFiniteFwd);
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
  half Kz[TK * DP];                 // rotated keys of one 64-key tile [key][d]
  half Vb[TK * VBP];                // the block's value columns of the tile scaled by zeta [key][col]
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
  dec.init(hp, head);
  const bool xpos = (p.flags & RET_XPOS) != 0;
  const T* Kg = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + head * p.sk.h;
  const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + cb * SCB;
  half* kth = p.w.kt + (int64_t)bh * lpad(p.L) * DK;
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
      // ---- stage the tile: rotate the keys (-> LDS; key-sum of the
      // zeta-scaled keys); scale the value block by zeta (-> LDS).  zeta goes
      // on the value rows (the same product K'^T (V (.) zeta)), so the LDS key
      // tile holds the unscaled rotated keys, which column block 0 writes out
      // in fragment order
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
          const float zt = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - key) * dec.lg2);
#pragma unroll
          for (int e = 0; e < 8; ++e) dzp[e] += x[i][e] * zt;
          st8(sm.Kz + key * DP + 8 * cq, x[i]);
        }
        float y[8];
        Raw16<T>::f32(cur.v, y);
        const float zv = vk < kvalid ? __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - vk) * dec.lg2) : 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= zv;
        st8(sm.Vb + vk * VBP + 8 * vp, y);
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
      if (LEAD) {
        // the tile's rotated keys to the workspace in fragment order: thread
        // -> 16-byte pieces tid + 512 i, so every wave store is one contiguous
        // 1 KB block (keys past the sequence's end go to the thread's
        // discard slot)
        half* kdst = kth + kt_off(c0 + k0, 0);
#pragma unroll
        for (int i = 0; i < TK * DK / 8 / NT3; ++i) {
          const int e = tid + i * NT3;
          const int blk = e >> 6, slot = e & 63;
          const int key = 32 * (blk / (DK / 16)) + (slot & 31), d = 16 * (blk % (DK / 16)) + 8 * (slot >> 5);
          const u32x4 v = *reinterpret_cast<const u32x4*>(sm.Kz + key * DP + d);
          *reinterpret_cast<u32x4*>(key < kvalid ? kdst + (int64_t)e * 8 : dump) = v;
        }
      }
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
      // ---- R += K'^T (V (.) zeta) over the tile's keys
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
    // a state that an fp16 operand overflow made non-finite is recorded as such
    bool bad = false;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        p.state_out[((int64_t)bh * DK + d0 + acc_row(r, lane)) * DV + cb * SCB + 32 * jj + l32] = acc[jj][r];
        bad |= nonfinite_as<float>(acc[jj][r]);
      }
    flag_nonfinite(p.nf, bad, kNonFiniteFwd);
  }
}

// ---------------------------------------------------------------- output
// Warp-specialised, one 64-row query item at a time:
//   producers (waves 0..3): wave w forms the 32 x 32 block S^T = K' Q'^T of
//     keys 32 ((w / 2) % 2) .. and queries 32 (w % 2) .. of every key tile
//     (its query fragments stay in registers for the whole item; the key
//     fragments are wave loads of the fragment-ordered rotated keys), scales
//     it by s gamma^(q - k) and writes P (fp16) to LDS, keeping fp32 row sums
//   consumers (waves 4..7): wave w owns output columns 128 (w % 4) .. + 127 of
//     all 64 rows: the cross term Q' R_{c-1} first (the state operand streamed
//     from global memory in fragment order), then P V for every key tile (a
//     bf16 value fragment is converted to fp16 in registers as it is read, so
//     P V runs on fp16 MFMA with fp16 P), then the normalised tile into LDS,
//     from where all eight waves write it with coalesced 16-byte stores; they
//     also copy the value tiles from global memory straight into LDS (16 key
//     rows per wave, no registers), the next tile's during this tile's P V
// P and the value tile are double-buffered, so the producers form the scores
// of tile j + 1 while the consumers copy its values and multiply tile j: one
// barrier per key tile.  The copies are issued from inline assembly, so the
// compiler does not drain them before every later LDS access (it cannot tell
// their destination from the buffers being read); the consumers wait for
// them explicitly before the barrier that publishes the tile.
struct OutSmem {
  half V[2][TK * DV];       // value tiles, per consumer a [key][128 col] slice (input type, pieces swizzled); the query tile overlays V[1]
  half Ps[2][TR * KP];      // P tiles [query][key]
  float rs[TR], xs[TR], dens[TR];
  float dpart[2][TR];       // within-chunk row sums of key halves 0 / 1
  float zs[DK];
  float ginv[32];           // gamma^-m, m = 0 .. 31
  // per pair, set once per workgroup: theta and e^{i theta} (an fp64 load
  // from global memory inside an item would wait for the previous item's
  // output stores as well: the vector memory counter completes in order)
  double theta[DK / 2];
  float2 step1[DK / 2];
};
static_assert(TR * QP <= TK * DV, "the query tile fits in one value buffer");

// m0 is declared clobbered by the value-tile copies (the compiler keeps no
// value in it across them)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
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
  // the role and the wave's place in it are uniform over the wave
  const int wave_u = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const bool producer = wave_u < 4;
  const int sk = (wave_u >> 1) & 1, sqh = wave_u & 1;     // producer: key half, query half
  const int cw = wave_u & 3;                               // consumer: block of 128 columns
  // the query tile of an item, as raw element pairs: thread -> pair column
  // tid % 128 of rows 16 (tid / 128) + 0..15.  The next item's tile is loaded
  // while the current item is normalised and stored, with the item's key-sum
  // z_{c-1} (thread -> d) and the power-of-two scales of the consumer's four
  // state column blocks
  uint32_t qraw[16];
  float zpre_n, up_n[4];
  auto issue_q = [&](int rt, int c, int bh) {
    const int j = threadIdx.x & 127, grp = threadIdx.x >> 7;
    const int64_t ci = (int64_t)bh * p.nc + c;
    zpre_n = p.w.zc[ci * DK + (threadIdx.x & (DK - 1))];
  #pragma unroll
    for (int jj = 0; jj < 4; ++jj) up_n[jj] = p.w.Rs[ci * NCB + 4 * cw + jj];
    const int bb = bh / p.h, head = bh % p.h;
    const int r0 = rt * TR;
    const int qvalid = min(TR, min(p.B, p.L - c * p.B) - r0);
    const char* Qg = reinterpret_cast<const char*>(reinterpret_cast<const T*>(p.q) + bb * p.sq.b + head * p.sq.h +
                                                   (int64_t)(c * p.B + r0) * p.sq.l);
    // a 32-bit byte offset from the tile origin (strides < 2^25 elements),
    // stepped one row per load and held at the tile's last valid row
    const uint32_t rowb = (uint32_t)p.sq.l * 2u;
    uint32_t off = (uint32_t)min(grp * 16, qvalid - 1) * rowb + 4u * (uint32_t)j;
  #pragma unroll
    for (int i = 0; i < 16; ++i) {
      qraw[i] = *reinterpret_cast<const uint32_t*>(Qg + off);
      if (grp * 16 + i + 1 < qvalid) off += rowb;
    }
  };
  if ((p.flags & RET_XPOS) && threadIdx.x < DK / 2) {
    OutSmem& sm = *reinterpret_cast<OutSmem*>(smem_raw);
    const double th = hp.theta[threadIdx.x];
    float2 t;
    phase(1, th, t.x, t.y);
    sm.theta[threadIdx.x] = th;
    sm.step1[threadIdx.x] = t;
  }
  int k = 0, rt = 0, c = 0, bh = 0;
  while (k < nk && !decode(k, rt, c, bh)) ++k;
  if (k < nk) issue_q(rt, c, bh);
  while (k < nk) {
    int kn = k + 1, rtn = 0, cn = 0, bhn = 0;
    while (kn < nk && !decode(kn, rtn, cn, bhn)) ++kn;
    __syncthreads();                                       // the previous item's LDS reads are done
    {
    OutSmem& sm = *reinterpret_cast<OutSmem*>(smem_raw);
    // the thread index passes through an empty asm each item, so per-lane
    // addressing is recomputed inside the item rather than hoisted out of the
    // persistent loop (where it would stay live across the whole item)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63;
    const int lh = lane >> 5, l32 = lane & 31;
    const int bb = bh / p.h, head = bh % p.h;
    const int c0 = c * p.B;
    const int Bc = min(p.B, p.L - c0);
    const int r0 = rt * TR;
    const int qvalid = min(TR, Bc - r0);
    const int n = rt + 1;                           // key tiles, taken in the order rt, 0, 1, .., rt - 1
    auto ktile = [&](int j) { return j == 0 ? rt : j - 1; };
    Decay dec;
    dec.init(hp, head);
    const bool xpos = (p.flags & RET_XPOS) != 0;
    const float qk_scale = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;
    const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + (int64_t)c0 * p.sv.l;
    const float zpre = zpre_n;
    const float up[4] = {up_n[0], up_n[1], up_n[2], up_n[3]};
    // the chunk's first tile of rotated keys (c0 is a whole number of tiles)
    const half* Kc = p.w.kt + ((int64_t)bh * lpad(p.L) + c0) * DK;
    TO* Og = reinterpret_cast<TO*>(p.o) + bb * p.so.b + head * p.so.h + (int64_t)(c0 + r0) * p.so.l;
    half* Qs = sm.V[1];
    // staging row pitch of the output tile: 16 bytes of padding per row
    constexpr int SPB = DV * (int)sizeof(TO) + 16;
    static_assert(TR * SPB <= sizeof(OutSmem::V) + sizeof(OutSmem::Ps), "the staged output tile fits");

    // a value tile's columns 128 cw .. 128 cw + 127 into consumer cw's slice
    // of LDS buffer buf ([key][16 pieces of 16 bytes], 256-byte rows, pieces
    // XOR-swizzled by 4 (key % 4) like vswz): one instruction per 4 key rows
    // (lane i lands at byte 16 i, so it fetches the piece that belongs there);
    // rows past a ragged chunk's end repeat its last key, whose P entries are
    // zero.  The copy writes no register.  Each consumer reads only its own
    // slice, so it refills a slice as soon as its own P V has read it and
    // waits for the copy only before its own next read.
    auto dma_v = [&](int kt, int buf) {
      const int k0 = kt * TK;
      const int kvalid = min(TK, Bc - k0);
      const T* Vt = Vg + (int64_t)k0 * p.sv.l + cw * 128;   // offsets inside the tile fit 32 bits
      // the lane's piece is recomputed here rather than kept live across the
      // stage loop
      int ln = threadIdx.x;
      asm volatile("" : "+v"(ln));
      const int pp = ln & 15, rq = (ln >> 4) & 3;
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 4 * i + rq;
        const int key = min(r, kvalid - 1);
        const T* src = Vt + (uint32_t)(key * (int)p.sv.l + vswz(r, pp) * 8);
        const uint32_t dst =
            (uint32_t)(uintptr_t)(__attribute__((address_space(3))) void*)(sm.V[buf] + cw * (TK * 128) + 4 * i * 128);
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" ::"s"(dst), "v"(src) : "memory", "m0");
      }
    };
    // wait for this wave's copies: all, or all but the 16 instructions of
    // the most recent one
    auto dma_wait = [] { __builtin_amdgcn_s_waitcnt(0x0F70); };        // vmcnt(0)
    auto dma_wait1 = [] { __builtin_amdgcn_s_waitcnt(0x4F70); };       // vmcnt(16)
    // ---- rotated query tile, row tables
    auto rotate_q = [&] {
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
        phase(p.pos0 + c0 + r0 + grp * 16, sm.theta[j], cs, sn);
        const float2 t = sm.step1[j];
        c1 = t.x;
        s1 = t.y;
      }
  #pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (xpos) {
          rot(a[i], b[i], cs, sn);
          advance(cs, sn, c1, s1);
        }
        st2(Qs + (grp * 16 + i) * QP + 2 * j, a[i], b[i]);
      }
      if (tid < TR) {
        float s = qk_scale;
        if (p.flags & RET_NORM_DROW) s *= dec.drow((float)(p.n_prev + c0 + r0 + tid + 1));
        sm.rs[tid] = s;
        sm.xs[tid] = s * dec.pow((float)(r0 + tid + 1));
      }
      if (tid < DK) sm.zs[tid] = zpre;
      if (tid < 32) sm.ginv[tid] = __builtin_amdgcn_exp2f(-(float)tid * dec.lg2);
    };

    constexpr int NSX = DK / 16, XR = 3;
    if (producer) {
      // the key fragments of the next score tile (16 steps of d)
      f16x8 kf[NSX];
      auto issue_kf = [&](int kt) {
        const half* kp = Kc + (int64_t)kt * (TK * DK) + (sk * NSX * 64 + lane) * 8;
  #pragma unroll
        for (int t = 0; t < NSX; ++t) kf[t] = *reinterpret_cast<const f16x8*>(kp + t * 512);
      };
      // the first tile's key fragments are requested before the query
      // rotation, which runs under them
      issue_kf(rt);
      rotate_q();
      // the first value tile, producer w copying consumer w's slice, issued
      // after the rotation's waits for the query tile: the copies are not in
      // the compiler's count of outstanding loads, so a copy issued before a
      // wait that the compiler places makes that wait cover the copy too (the
      // consumers, issuing it before their state-operand loads, waited for
      // it in the query rotation and the first cross-term step)
      dma_v(rt, 0);
      __syncthreads();                              // the query tile and the row tables
      // this wave's 32 queries as B fragments, for the whole item
      f16x8 qf[NSX];
  #pragma unroll
      for (int t = 0; t < NSX; ++t) qf[t] = *reinterpret_cast<const f16x8*>(Qs + (sqh * 32 + l32) * QP + 16 * t + 8 * lh);
      // cross part of the score denominator, s xi (Q' . z_{c-1}): 4 threads per row
      {
        const int row = tid >> 2, part = tid & 3;   // d 64 part .. 64 part + 63
        float acc = 0.f;
  #pragma unroll
        for (int u = 0; u < 8; ++u) {
          const f16x8 qv = *reinterpret_cast<const f16x8*>(Qs + row * QP + 64 * part + 8 * u);
          const f32x4 z0 = *reinterpret_cast<const f32x4*>(sm.zs + 64 * part + 8 * u);
          const f32x4 z1 = *reinterpret_cast<const f32x4*>(sm.zs + 64 * part + 8 * u + 4);
  #pragma unroll
          for (int e = 0; e < 4; ++e) acc += (float)qv[e] * z0[e];
  #pragma unroll
          for (int e = 0; e < 4; ++e) acc += (float)qv[4 + e] * z1[e];
        }
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        if (part == 0) sm.dens[row] = sm.xs[row] * acc;
      }
      float den = 0.f;
      // scores of key tile ktile(j) into P buffer buf; kf holds its key fragments
      auto score = [&](int j, int buf) {
        const int k0 = ktile(j) * TK;
        const bool diag = (j == 0);
        float pv[16];
        if (!(diag && sk > sqh)) {                  // keys 32..63 vs queries 0..31 of the diagonal: zero
          f32x16 S = {};
  #pragma unroll
          for (int t = 0; t < NSX; ++t) S = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[t], qf[t], S, 0, 0, 0);
          // D = gamma^(q - k) split as gamma^base gamma^-(8i + j), base = q - (first key of the lane)
          const int base = r0 + sqh * 32 + l32 - k0 - sk * 32 - 4 * lh;
          const float gq = sm.rs[sqh * 32 + l32] * __builtin_amdgcn_exp2f((float)base * dec.lg2);
          // the causal mask q >= k only bites on the diagonal tile (it also
          // drops the keys past a ragged chunk's end, whose fragments hold
          // whatever the workspace held)
          auto scale = [&](auto masked) {
  #pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float4 gi = *reinterpret_cast<const float4*>(sm.ginv + 8 * i);
              const float gv[4] = {gi.x, gi.y, gi.z, gi.w};
  #pragma unroll
              for (int jj = 0; jj < 4; ++jj) {
                float val = S[4 * i + jj] * gq * gv[jj];
                if (decltype(masked)::value) val = (base >= 8 * i + jj) ? val : 0.f;
                den += val;
                pv[4 * i + jj] = val;
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
        for (int i = 0; i < 4; ++i) st4(sm.Ps[buf] + (sqh * 32 + l32) * KP + sk * 32 + 8 * i + 4 * lh, pv + 4 * i);
      };
      // the diagonal tile, while the consumers form the cross term
      score(0, 0);
      dma_wait();                                   // the first value tile has landed
      if (n > 1) issue_kf(ktile(1));
      __syncthreads();
      for (int j = 0; j < n; ++j) {
        if (j + 1 < n) {
          score(j + 1, (j + 1) & 1);
          if (j + 2 < n) issue_kf(ktile(j + 2));
        } else {
          den += __shfl_xor(den, 32, 64);           // lanes l and l + 32 hold the same query
          if (lh == 0) sm.dpart[sk][sqh * 32 + l32] = den;
        }
        __syncthreads();
      }
      // the next item's query tile (requested even after the last item, then
      // the current one's again: a conditional request left the old and new
      // registers live together, and the copy between them at the join
      // waited for the loads)
      issue_q(kn < nk ? rtn : rt, kn < nk ? cn : c, kn < nk ? bhn : bh);
    } else {
      // output tiles of this wave: query halves {0,1} x column tiles 4 cw +
      // {0..3}, held transposed (the MFMAs take the column operand first):
      // lane l, register r of O[qh][jj] is query qh 32 + l % 32, column
      // (4 cw + jj) 32 + acc_row(r, l), so each lane holds runs of four
      // consecutive columns of one query row, stored straight from registers
      f32x16 O[2][4];
  #pragma unroll
      for (int i = 0; i < 2; ++i)
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) O[i][jj] = f32x16{};
      // the ring of state-operand fragments (fragment (jj, t) of this wave's
      // four column blocks at rp + (jj NSX + t) 512)
      const half* rp = p.w.Rt + ((int64_t)bh * p.nc + c) * DV * DK + (int64_t)(4 * cw * NSX * 64 + lane) * 8;
      f16x8 rb[XR * 4];
      // the head of the ring is requested before the query rotation, which
      // runs under it (the producers copy the first value tile)
  #pragma unroll
      for (int t = 0; t < XR; ++t)
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) rb[t * 4 + jj] = *reinterpret_cast<const f16x8*>(rp + (jj * NSX + t) * 512);
      rotate_q();
      __syncthreads();                              // the query tile and the row tables
      // ---- cross-chunk term Q' R_{c-1}, the state operand's fragments
      // streamed XR steps ahead with no LDS staging
      {
        f16x8 qa[2][2];
        auto load_q = [&](int t, int buf) {
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
            qa[buf][qh] = *reinterpret_cast<const f16x8*>(Qs + (qh * 32 + l32) * QP + 16 * t + 8 * lh);
        };
        load_q(0, 0);
  #pragma unroll
        for (int t = 0; t < NSX; ++t) {
          if (t + 1 < NSX) load_q(t + 1, (t + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              O[qh][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rb[(t % XR) * 4 + jj], qa[t & 1][qh], O[qh][jj], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          if (t + XR < NSX) {
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              rb[(t % XR) * 4 + jj] = *reinterpret_cast<const f16x8*>(rp + (jj * NSX + t + XR) * 512);
          }
        }
      }
      // row scale s xi and the operand's per-block power of two (the lane's
      // query row is l32 of each half)
  #pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const float x = sm.xs[qh * 32 + l32];
  #pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const float xu = x * up[jj];
  #pragma unroll
          for (int r = 0; r < 16; ++r) O[qh][jj][r] *= xu;
        }
      }
      dma_wait();
      __syncthreads();
      // this lane's transposed-read origin in a value tile: key 8 (lane / 32) +
      // (lane % 16) / 4, column 16 ((lane / 16) % 2) + 4 (lane % 4)
      // (swizzled: the lane's key row has r % 4 = (lane / 4) % 4)
      const int vtr_row = (8 * (lane >> 5) + ((lane & 15) >> 2)) * 128 + 4 * (lane & 1);
      const int vtr_sw = ((lane >> 2) & 3) << 2, vtr_lo = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      for (int j = 0; j < n; ++j) {
        // tile 1 goes to buffer 1, free of the query tile since the last
        // barrier; tile j (j >= 1) was requested a tile ago or earlier, and
        // only the copy of tile j + 1 may still be in flight
        if (j == 0) {
          if (n > 1) dma_v(ktile(1), 1);
        } else if (j + 1 < n) {
          dma_wait1();
        } else {
          dma_wait();
        }
        // O += P V (rows 0..31 of P are zero against keys 32..63 of the
        // diagonal tile); the fragments of step s + 1 are read while step s
        // multiplies
        const int buf = j & 1;
        f16x8 pa[2][2];
        u32x4 bv[2][4];                             // raw value fragments (input type)
        auto load_pv = [&](int kb, int b2) {
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            // keys kb + 8 (lane / 32) + 0..7 of column (4 cw + jj) 32 + lane % 32
            const half* vp = sm.V[buf] + cw * (TK * 128) + kb * 128 + vtr_row + (((jj * 4) ^ vtr_sw) + vtr_lo) * 8;
            const f16x4 lo = lds_read_tr16(vp), hi = lds_read_tr16(vp + 4 * 128);
            bv[b2][jj] = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
            pa[b2][qh] = *reinterpret_cast<const f16x8*>(sm.Ps[buf] + (qh * 32 + l32) * KP + kb + 8 * lh);
        };
        load_pv(0, 0);
  #pragma unroll
        for (int t = 0; t < TK / 16; ++t) {
          if (t + 1 < TK / 16) load_pv(16 * (t + 1), (t + 1) & 1);
          __builtin_amdgcn_sched_barrier(0);
          f16x8 vf[4];
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) vf[jj] = __builtin_bit_cast(f16x8, Raw16<T>::f16(bv[t & 1][jj]));
  #pragma unroll
          for (int qh = 0; qh < 2; ++qh)
  #pragma unroll
            for (int jj = 0; jj < 4; ++jj)
              O[qh][jj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[jj], pa[t & 1][qh], O[qh][jj], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        // this slice of buffer j % 2 is read: refill it with tile j + 2
        if (j + 2 < n) {
          __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): the slice's reads have returned
          dma_v(ktile(j + 2), j & 1);
        }
        __syncthreads();
      }
      // the next item's query tile (unconditional, as in the producers)
      issue_q(kn < nk ? rtn : rt, kn < nk ? cn : c, kn < nk ? bhn : bh);

      // ---- normalise into the staging tile (row pitch SPB bytes, over the
      // dead value and P buffers); lane l writes query row l % 32 of each half
      bool bad = false;
      char* stage = reinterpret_cast<char*>(&sm.V[0][0]);
  #pragma unroll
      for (int qh = 0; qh < 2; ++qh) {
        const int row = qh * 32 + l32;
        // cross part plus the two key halves, summed in a fixed order
        const float d = sm.dens[row] + sm.dpart[0][row] + sm.dpart[1][row];
        const float f = (p.flags & RET_NORM_SCORE) ? 1.f / fmaxf(fabsf(d), 1.f) : 1.f;
        const bool live = row < qvalid;
        TO* srow = reinterpret_cast<TO*>(stage + row * SPB);
        if constexpr (sizeof(TO) == 2) {
          // a 16-bit output is not finite iff its exponent field is all ones
          // (what a value at or past the type's limit rounds to): a running
          // packed 16-bit max of the stored words' magnitudes, one test per
          // row at the end (one compare and one scalar OR per value before)
          typedef __attribute__((ext_vector_type(2))) unsigned short u16x2;
          u16x2 mx = {0, 0};
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = (4 * cw + jj) * 32 + 8 * g + 4 * lh;
              float x[4];
  #pragma unroll
              for (int e = 0; e < 4; ++e) x[e] = O[qh][jj][4 * g + e] * f;
              uint2 u;
              if constexpr (std::is_same<TO, bf16>::value) {
                u.x = pack_bf2(x[0], x[1]);
                u.y = pack_bf2(x[2], x[3]);
              } else {
                u.x = __builtin_bit_cast(uint32_t, f16x2{(_Float16)x[0], (_Float16)x[1]});
                u.y = __builtin_bit_cast(uint32_t, f16x2{(_Float16)x[2], (_Float16)x[3]});
              }
              *reinterpret_cast<uint2*>(srow + col) = u;
              mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, u.x & 0x7fff7fffu));
              mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, u.y & 0x7fff7fffu));
            }
          }
          constexpr unsigned short kExp = std::is_same<TO, bf16>::value ? 0x7f80 : 0x7c00;
          bad |= live && (mx.x >= kExp || mx.y >= kExp);
        } else {
  #pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
  #pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int col = (4 * cw + jj) * 32 + 8 * g + 4 * lh;
              float x[4];
  #pragma unroll
              for (int e = 0; e < 4; ++e) {
                x[e] = O[qh][jj][4 * g + e] * f;
                bad |= live && nonfinite_as<TO>(x[e]);
              }
              store4(srow + col, x);
            }
          }
        }
      }
      flag_nonfinite(p.nf, bad, kNonFiniteFwd);
    }
    __syncthreads();                                // the staged output tile
    // ---- every wave writes the tile: 16-byte pieces, consecutive lanes along
    // a row.  Every lane issues the same stores with no branch around them (a
    // piece of a row past a ragged tile goes to the thread's own slot of the
    // workspace's discard area), so a later wait for the next item's loads is
    // not made to drain these stores.
    {
      constexpr int RPC = DV * (int)sizeof(TO) / 16;          // 16-byte pieces per row
      const char* stage = reinterpret_cast<const char*>(&sm.V[0][0]);
      char* dumpo = reinterpret_cast<char*>(p.w.dump) + tid * 16;
  #pragma unroll
      for (int i = 0; i < TR * RPC / NT3; ++i) {
        const int e = tid + i * NT3;
        const int row = e / RPC, piece = e % RPC;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + row * SPB + piece * 16);
        char* dst = row < qvalid ? reinterpret_cast<char*>(Og + (int64_t)row * p.so.l) + piece * 16 : dumpo;
        *reinterpret_cast<u32x4*>(dst) = v;
      }
    }
    }
    k = kn;
    rt = rtn;
    c = cn;
    bh = bhn;
  }
}

#pragma clang diagnostic pop

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
  p.nf = a.nf;
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
    const int units = bh * p.nc * 2;
    int W = min(units, persistent_workgroups());
    if (W >= 8) W -= W % 8;
    hipLaunchKernelGGL(k, dim3(W), dim3(NT3), sizeof(DeltaSmem), st, p, *a.hp);
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
