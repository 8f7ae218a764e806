// Projections of the gated MSR block (RetNet reading notes, §三.2 and §2.1):
// Q = X W_Q, K = X W_K, V = X W_V, G = X W_G and Out = Z W_O, as
//   C[M][N] = A[M][K] . B[N][K]^T
// with B a bf16 weight held as [out_features][in_features] (so both operands
// are contiguous along K) and fp32 accumulation.  A bf16 A is contracted on
// v_mfma_f32_32x32x16_bf16 with the operands as given; an fp16 A (the
// gated, normalised heads) on v_mfma_f32_32x32x16_f16 with B converted to
// fp16 while it is staged into LDS.
//
// Block tile 256 x 256 x 64 (x 32 when K is not a multiple of 64) on 8 waves
// (each 64 x 128 = 2 x 4 MFMA tiles); the next K slab is loaded into
// registers while the current one is multiplied out of LDS (two LDS buffers,
// one barrier per slab), and within a slab the fragments of step s + 1 are
// read while step s multiplies.  Rows and columns beyond M / N are clamped on
// load and skipped on store; K must be a multiple of 32.
//
// For M <= 128 rows (a decode step) a column-split kernel without LDS staging
// is used instead, or, when the caller brings a workspace, a split-K kernel
// with the activation rows staged in LDS (below).
//
// Epilogue options (the RetNet layer, reading notes §三.4): the exact gelu
// x Phi(x) of each output (FFN's first projection), then the addition of a
// residual (the layer's two residual connections) stored as fp32, bf16 or
// fp16 independently of the output, so that an fp32 residual stream can feed
// a bf16 result and the reverse.
#include <mutex>

#include "internal.h"

namespace ret {

namespace {

constexpr int GT = 512;          // threads
constexpr int BM = 256, BN = 256;
constexpr int WM = 64, WN = 128; // wave tile

// K slab of BK (64, or 32 when K is not a multiple of 64); LDS row pitch
// BK + 8 elements keeps the fragment reads of 16 rows on distinct banks
template <int BK> struct GemmSmem {
  static constexpr int LP = BK + 8;
  uint16_t a[2][BM * LP];
  uint16_t b[2][BN * LP];
};

// bf16 -> fp16 for eight packed values
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(u32x4 u) {
  f16x8 h;
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[2 * i] = (half)lo_bf(w[i]);
    h[2 * i + 1] = (half)hi_bf(w[i]);
  }
  return __builtin_bit_cast(u32x4, h);
}

template <typename TA> struct GemmOp;
template <> struct GemmOp<bf16> {
  typedef bf16x8 frag;
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static u32x4 cvt_b(u32x4 u) { return u; }
};
template <> struct GemmOp<half> {
  typedef f16x8 frag;
  __device__ __forceinline__ static void mma(f32x16& c, const frag& a, const frag& b) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static u32x4 cvt_b(u32x4 u) { return bf16x8_to_f16x8(u); }
};

__device__ __forceinline__ float gelu_exact(float x) { return 0.5f * x * (1.f + erff(x * 0.70710678118654752f)); }

// residual element as fp32; r_dt is uniform over the launch
__device__ __forceinline__ float ld_residual(const void* R, int r_dt, size_t i) {
  if (r_dt == RET_F32) return static_cast<const float*>(R)[i];
  if (r_dt == RET_BF16) return Elem<bf16>::ld(static_cast<const bf16*>(R) + i);
  return Elem<half>::ld(static_cast<const half*>(R) + i);
}

// C may be the residual itself (each element is read, then written, by one thread)
template <typename TA, typename TO, int BK>
__global__ void __launch_bounds__(GT, 1)
gemm_nt_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, TO* C,
               int M, int N, int K, int tiles_n, const void* R, int r_dt, int act) {
  typedef GemmOp<TA> G;
  constexpr int LP = GemmSmem<BK>::LP;
  constexpr int A_LD = BM * BK / 8 / GT;   // 16-byte loads per thread per slab
  constexpr int B_LD = BN * BK / 8 / GT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  GemmSmem<BK>& sm = *reinterpret_cast<GemmSmem<BK>*>(smem_raw);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lh = lane >> 5, l32 = lane & 31;

  // tile order: consecutive workgroups (round-robin over the XCDs) walk
  // along N first so that an XCD keeps reusing one A row panel
  const int tile = blockIdx.x;
  const int tm = tile / tiles_n, tn = tile % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int wm = (wave >> 1) * WM;       // 4 x 2 waves
  const int wn = (wave & 1) * WN;

  // loader mapping: each 16-byte load covers 8 k of one row; a slab row has
  // BK / 8 such pieces
  u32x4 ra[A_LD], rb[B_LD];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int e = tid + i * GT;
      const int row = e / (BK / 8), piece = e % (BK / 8);
      const int gr = min(m0 + row, M - 1);
      ra[i] = *reinterpret_cast<const u32x4*>(A + (size_t)gr * K + k0 + piece * 8);
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int e = tid + i * GT;
      const int row = e / (BK / 8), piece = e % (BK / 8);
      const int gr = min(n0 + row, N - 1);
      rb[i] = *reinterpret_cast<const u32x4*>(B + (size_t)gr * K + k0 + piece * 8);
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
      const int e = tid + i * GT;
      *reinterpret_cast<u32x4*>(&sm.a[buf][(e / (BK / 8)) * LP + (e % (BK / 8)) * 8]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
      const int e = tid + i * GT;
      *reinterpret_cast<u32x4*>(&sm.b[buf][(e / (BK / 8)) * LP + (e % (BK / 8)) * 8]) = G::cvt_b(rb[i]);
    }
  };

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  const int nk = K / BK;
  load_slab(0);
  store_slab(0);
  __syncthreads();
  for (int kb = 0; kb < nk; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nk) load_slab((kb + 1) * BK);
    typename G::frag af[2][2], bfr[2][4];
    auto ldf = [&](int ks, int bsel) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[bsel][i] = *reinterpret_cast<const typename G::frag*>(&sm.a[cur][(wm + i * 32 + l32) * LP + ks + 8 * lh]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[bsel][j] = *reinterpret_cast<const typename G::frag*>(&sm.b[cur][(wn + j * 32 + l32) * LP + ks + 8 * lh]);
    };
    ldf(0, 0);
#pragma unroll
    for (int t = 0; t < BK / 16; ++t) {
      if (t + 1 < BK / 16) ldf(16 * (t + 1), (t + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) G::mma(acc[i][j], af[t & 1][i], bfr[t & 1][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kb + 1 < nk) store_slab(cur ^ 1);
    __syncthreads();
  }

  // store: lane holds column l32 of each 32x32 tile, rows acc_row(r)
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn + j * 32 + l32;
      if (col < N) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = m0 + wm + i * 32 + acc_row(r, lane);
          if (row < M) {
            float v = acc[i][j][r];
            if (act) v = gelu_exact(v);
            if (R) v += ld_residual(R, r_dt, (size_t)row * N + col);
            C[(size_t)row * N + col] = Store<TO>::cvt(v);
          }
        }
      }
    }
}

template <typename TA, typename TO, int BK>
static hipError_t launch_gemm_k(const void* A, const void* B, void* C, int M, int N, int K, const void* R,
                                int r_dt, int act, hipStream_t st) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  const size_t sh = sizeof(GemmSmem<BK>);
  auto kern = gemm_nt_kernel<TA, TO, BK>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tiles_m * tiles_n), dim3(GT), sh, st, (const uint16_t*)A, (const uint16_t*)B,
                     (TO*)C, M, N, K, tiles_n, R, r_dt, act);
  return hipGetLastError();
}

template <typename TA, typename TO>
static hipError_t launch_gemm_t(const void* A, const void* B, void* C, int M, int N, int K, const void* R,
                                int r_dt, int act, hipStream_t st) {
  return K % 64 == 0 ? launch_gemm_k<TA, TO, 64>(A, B, C, M, N, K, R, r_dt, act, st)
                     : launch_gemm_k<TA, TO, 32>(A, B, C, M, N, K, R, r_dt, act, st);
}

template <typename TA>
static hipError_t launch_gemm_a(const void* A, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                                const void* R, int r_dt, int act, hipStream_t st) {
  if (c_dt == RET_BF16) return launch_gemm_t<TA, bf16>(A, B, C, M, N, K, R, r_dt, act, st);
  if (c_dt == RET_F16) return launch_gemm_t<TA, half>(A, B, C, M, N, K, R, r_dt, act, st);
  return launch_gemm_t<TA, float>(A, B, C, M, N, K, R, r_dt, act, st);
}

// ---------------------------------------------------------------- skinny
// M <= 128 rows (a decode step: one token per sequence).  The product is
// bound by reading the weight B once; the activations A (M x K) are shared by
// every workgroup and read from L2.  A workgroup owns SKN = 32 columns for all
// M rows (N / 32 workgroups) and its eight waves split K; each wave multiplies
// its activation fragments against both 16-column blocks, so a workgroup reads
// A once per 32 columns.  Every MFMA operand (16x16x32: lane l supplies row or
// column l % 16 and eight k values) is read straight from global memory.  A
// 64-deep step is two MFMAs; since the sum over k may take any order shared by
// A and B, lane l reads the 16 contiguous k values 16 (l / 16) .. + 15 of its
// row and gives the first eight to one MFMA and the rest to the other, so each
// row read covers one whole 128-byte line.  The eight partial 128 x 32 tiles
// are summed through LDS before the epilogue.
constexpr int SKM = 128, SKN = 32, SKW = 8, SKT = 64 * SKW;

template <typename TA> struct SkOp;
template <> struct SkOp<bf16> {
  __device__ __forceinline__ static void mma(f32x4& c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                0, 0, 0);
  }
  __device__ __forceinline__ static u32x4 cvt_b(u32x4 u) { return u; }
};
template <> struct SkOp<half> {
  __device__ __forceinline__ static void mma(f32x4& c, u32x4 a, u32x4 b) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0,
                                               0);
  }
  __device__ __forceinline__ static u32x4 cvt_b(u32x4 u) { return bf16x8_to_f16x8(u); }
};

template <typename TA, typename TO>
__global__ void __launch_bounds__(SKT)
gemm_skinny_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, TO* C, int M, int N, int K,
                   const void* R, int r_dt, int act) {
  __shared__ float red[SKW][SKM * SKN];
  // the wave index is wave-uniform (readfirstlane): the K loop below is then a
  // uniform loop, with exact wait counts across its back edge
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * SKN;
  const int l16 = lane & 15, kq = 16 * (lane >> 4);
  const int MB = (M + 15) / 16;                      // row blocks in use (<= 8)
  // this lane's operand rows: weight rows n0 + 16 j + l16, activation rows 16 i + l16 (clamped)
  const uint16_t* bp[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) bp[j] = B + (int64_t)min(n0 + 16 * j + l16, N - 1) * K + kq;
  const uint16_t* ap[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ap[i] = A + (int64_t)min(16 * i + l16, M - 1) * K + kq;
  f32x4 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // wave w takes the 64-deep steps w, w + SKW, ...; the next step's operands
  // are in flight while the current one is multiplied.  A 32-deep tail (K not
  // a multiple of 64) is taken by wave 0 with the lane's 8 values at 8 (l / 16).
  const int steps = K / 64;
  u32x4 bn[2][2] = {}, an[8][2];
  auto load = [&](int st, u32x4 (&b2)[2][2], u32x4 (&a8)[8][2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 2; ++j) b2[j][h] = *reinterpret_cast<const u32x4*>(bp[j] + 64 * st + 8 * h);
#pragma unroll
      for (int i = 0; i < 8; ++i) a8[i][h] = *reinterpret_cast<const u32x4*>(ap[i] + 64 * st + 8 * h);
    }
  };
  int s = wave;
  if (s < steps) load(s, bn, an);
  for (; s < steps; s += SKW) {
    u32x4 bc[2][2], ac[8][2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int j = 0; j < 2; ++j) bc[j][h] = SkOp<TA>::cvt_b(bn[j][h]);
#pragma unroll
      for (int i = 0; i < 8; ++i) ac[i][h] = an[i][h];
    }
    load(min(s + SKW, steps - 1), bn, an);          // past the end: reload the last step
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < MB)
#pragma unroll
          for (int j = 0; j < 2; ++j) SkOp<TA>::mma(acc[i][j], ac[i][h], bc[j][h]);
  }
  if ((K % 64) && wave == 0) {
    const int kt = 64 * steps - kq + 8 * (lane >> 4);   // this lane's 8 values of the tail
    u32x4 bt[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) bt[j] = SkOp<TA>::cvt_b(*reinterpret_cast<const u32x4*>(bp[j] + kt));
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < MB) {
        const u32x4 at = *reinterpret_cast<const u32x4*>(ap[i] + kt);
#pragma unroll
        for (int j = 0; j < 2; ++j) SkOp<TA>::mma(acc[i][j], at, bt[j]);
      }
  }
  // partial tiles -> LDS: lane l holds column l % 16, rows 4 (l / 16) + r of each block
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) red[wave][(16 * i + 4 * (lane >> 4) + r) * SKN + 16 * j + l16] = acc[i][j][r];
  __syncthreads();
  for (int e = tid; e < SKM * SKN; e += SKT) {
    const int m = e / SKN, n = n0 + e % SKN;
    if (m < M && n < N) {
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < SKW; ++w) v += red[w][e];
      if (act) v = gelu_exact(v);
      if (R) v += ld_residual(R, r_dt, (size_t)m * N + n);
      C[(size_t)m * N + n] = Store<TO>::cvt(v);
    }
  }
}

template <typename TA, typename TO>
static hipError_t launch_skinny_t(const void* A, const void* B, void* C, int M, int N, int K, const void* R, int r_dt,
                                  int act, hipStream_t st) {
  hipLaunchKernelGGL((gemm_skinny_kernel<TA, TO>), dim3((N + SKN - 1) / SKN), dim3(SKT), 0, st,
                     (const uint16_t*)A, (const uint16_t*)B, (TO*)C, M, N, K, R, r_dt, act);
  return hipGetLastError();
}

template <typename TA>
static hipError_t launch_skinny_a(const void* A, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                                  const void* R, int r_dt, int act, hipStream_t st) {
  if (c_dt == RET_BF16) return launch_skinny_t<TA, bf16>(A, B, C, M, N, K, R, r_dt, act, st);
  if (c_dt == RET_F16) return launch_skinny_t<TA, half>(A, B, C, M, N, K, R, r_dt, act, st);
  return launch_skinny_t<TA, float>(A, B, C, M, N, K, R, r_dt, act, st);
}

// ---------------------------------------------------------------- split-K
// M <= 128 rows with a workspace.  Every workgroup that works on a column
// block reads all M rows of A over its K range, so the activation bytes moved
// from L2 are (N / columns per workgroup) x |A|: at 32 columns per workgroup
// and K = 4096 that is 4x the weight bytes.  Here a workgroup owns SPN = 128
// columns and one of KS slices of K; the slice's A rows are staged through LDS
// (SPK = 128 deep, two buffers, one barrier per step) and shared by the eight
// waves, each of which owns 16 columns and reads its weight fragments straight
// from global memory (lane l: column l % 16, the eight k values 8 (l / 16) of
// each 32-deep block, a contiguous 64 bytes per column and block).  Each slice
// writes its fp32 partial tile; a second kernel sums the KS partials in slice
// order (so the result does not depend on scheduling) and applies the
// epilogue.
constexpr int SPN = 128, SPK = 128, SPT = 512, SPP = SPK + 8;

// slices: the most (up to 8) that keep at least 128 x 128 per workgroup
// and at most ~512 workgroups
__host__ inline int splitk_slices(int N, int K) {
  const int nb = (N + SPN - 1) / SPN;
  int ks = 1;
  while (ks < 8 && nb * ks * 2 <= 512 && K % (SPK * ks * 2) == 0) ks *= 2;
  return ks;
}

template <typename TA>
__global__ void __launch_bounds__(SPT)
gemm_splitk_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, float* __restrict__ P, int M,
                   int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t As[2][SKM * SPP];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n0 = blockIdx.x * SPN, KL = K / gridDim.y, k0 = blockIdx.y * KL;
  const int l16 = lane & 15, kq = 8 * (lane >> 4);
  const uint16_t* bp = B + (int64_t)min(n0 + 16 * wave + l16, N - 1) * K + k0 + kq;
  // A staging: 128 rows x 128 k = 2048 pieces of 16 bytes, 4 per thread (row e / 16, piece e % 16)
  const uint16_t* apc[4];
  int aoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = tid + i * SPT, r = e >> 4, c = e & 15;
    apc[i] = A + (int64_t)min(r, M - 1) * K + k0 + 8 * c;
    aoff[i] = r * SPP + 8 * c;
  }
  const int steps = KL / SPK;
  u32x4 an[4], bn[4];
  auto load = [&](int st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) an[i] = *reinterpret_cast<const u32x4*>(apc[i] + SPK * st);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bn[kb] = *reinterpret_cast<const u32x4*>(bp + SPK * st + 32 * kb);
  };
  f32x4 acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  load(0);
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&As[0][aoff[i]]) = an[i];
  __syncthreads();
  for (int st = 0; st < steps; ++st) {
    u32x4 bc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) bc[kb] = SkOp<TA>::cvt_b(bn[kb]);
    load(min(st + 1, steps - 1));                   // past the end: reload the last step
    const uint16_t* a = As[st & 1];
    // all eight row blocks, also past M (rows clamped on staging, never
    // stored): a branch per block would copy the accumulators at every join
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const u32x4 af = *reinterpret_cast<const u32x4*>(a + (16 * i + l16) * SPP + 32 * kb + kq);
        SkOp<TA>::mma(acc[i], af, bc[kb]);
      }
    // the other buffer was last read in step st - 1, before this step's barrier
#pragma unroll
    for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&As[(st + 1) & 1][aoff[i]]) = an[i];
    __syncthreads();
  }
  // partial tile: lane l holds column 16 w + l % 16, rows 16 i + 4 (l / 16) + r
  const int n = n0 + 16 * wave + l16;
  float* pp = P + (int64_t)blockIdx.y * M * N;
  if (n < N) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = 16 * i + 4 * (lane >> 4) + r;
        if (m < M) pp[(int64_t)m * N + n] = acc[i][r];
      }
  }
}

// four consecutive outputs per thread (16-byte partial loads) when M N is a
// multiple of 4, else one
template <typename TO, int V>
__global__ void __launch_bounds__(256)
gemm_splitk_reduce(const float* __restrict__ P, int ks, TO* C, int M, int N, const void* R, int r_dt, int act) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * V, mn = (int64_t)M * N;
  if (e >= mn) return;
  float v[V];
#pragma unroll
  for (int u = 0; u < V; ++u) v[u] = 0.f;
  for (int y = 0; y < ks; ++y) {
    if (V == 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(P + y * mn + e);
#pragma unroll
      for (int u = 0; u < V; ++u) v[u] += x[u];
    } else {
      v[0] += P[y * mn + e];
    }
  }
#pragma unroll
  for (int u = 0; u < V; ++u) {
    float w = v[u];
    if (act) w = gelu_exact(w);
    if (R) w += ld_residual(R, r_dt, (size_t)(e + u));
    C[e + u] = Store<TO>::cvt(w);
  }
}

template <typename TA, typename TO>
static hipError_t launch_splitk_t(const void* A, const void* B, void* C, int M, int N, int K, const void* R,
                                  int r_dt, int act, float* P, hipStream_t st) {
  const int ks = splitk_slices(N, K);
  hipLaunchKernelGGL((gemm_splitk_kernel<TA>), dim3((N + SPN - 1) / SPN, ks), dim3(SPT), 0, st,
                     (const uint16_t*)A, (const uint16_t*)B, P, M, N, K);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t mn = (int64_t)M * N;
  if (mn % 4 == 0)
    hipLaunchKernelGGL((gemm_splitk_reduce<TO, 4>), dim3((unsigned)((mn / 4 + 255) / 256)), dim3(256), 0, st, P,
                       ks, (TO*)C, M, N, R, r_dt, act);
  else
    hipLaunchKernelGGL((gemm_splitk_reduce<TO, 1>), dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, st, P, ks,
                       (TO*)C, M, N, R, r_dt, act);
  return hipGetLastError();
}

template <typename TA>
static hipError_t launch_splitk_a(const void* A, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                                  const void* R, int r_dt, int act, float* P, hipStream_t st) {
  if (c_dt == RET_BF16) return launch_splitk_t<TA, bf16>(A, B, C, M, N, K, R, r_dt, act, P, st);
  if (c_dt == RET_F16) return launch_splitk_t<TA, half>(A, B, C, M, N, K, R, r_dt, act, P, st);
  return launch_splitk_t<TA, float>(A, B, C, M, N, K, R, r_dt, act, P, st);
}

}  // namespace

hipError_t launch_gemm(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                       const void* R, ret_dtype r_dt, int act, hipStream_t st) {
  if (M <= SKM)
    return a_dt == RET_F16 ? launch_skinny_a<half>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, st)
                           : launch_skinny_a<bf16>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, st);
  return a_dt == RET_F16 ? launch_gemm_a<half>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, st)
                         : launch_gemm_a<bf16>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, st);
}

size_t gemm_workspace_bytes(int M, int N, int K) {
  if (M > SKM || K % SPK) return 0;
  return (size_t)splitk_slices(N, K) * M * N * sizeof(float);
}

hipError_t launch_gemm_ws(const void* A, ret_dtype a_dt, const void* B, void* C, ret_dtype c_dt, int M, int N, int K,
                          const void* R, ret_dtype r_dt, int act, void* ws, hipStream_t st) {
  if (gemm_workspace_bytes(M, N, K) == 0) return launch_gemm(A, a_dt, B, C, c_dt, M, N, K, R, r_dt, act, st);
  float* P = static_cast<float*>(ws);
  return a_dt == RET_F16 ? launch_splitk_a<half>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, P, st)
                         : launch_splitk_a<bf16>(A, B, C, c_dt, M, N, K, R, (int)r_dt, act, P, st);
}

// ---------------------------------------------------------------- scratch
// The split-K partials of msr_gemm_scratch live in this static device array
// (each device holds its own copy).  Host code uses the device address looked
// up with hipGetSymbolAddress, never the array's name (a host-side stand-in).
namespace {
static __device__ __align__(256) float scratch[MSR_GEMM_SCRATCH_BYTES / sizeof(float)];
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];
}  // namespace

hipError_t gemm_scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ret
