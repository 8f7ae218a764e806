// Chunkwise recurrent retention forward (RetNet reading notes, §2.4), with the
// xPos rotation of §2.3 and the normalisations of §三.3.
//
// Work decomposition: one persistent workgroup per (batch*head, d_v slice of
// SV columns).  It walks the chunks in order and keeps its slice of the state
// R (d_k x SV, float32) in MFMA accumulators for the whole sequence, so R
// never touches HBM.  Inside a chunk the rows are processed in tiles of TR
// queries; for each query tile the key tiles up to the diagonal are streamed
// through LDS:
//   S^T = K' Q'^T           (MFMA, fp32 accumulate)            intra scores
//   P   = s_i S^T gamma^(i-j) masked to j <= i; row sums of P (den) in fp32
//   O  += P V[:, slice]     (P rounded to the operand type)    intra output
// then the cross-chunk term with the previous chunk's state,
//   Oc += (s xi (.) Q') R_{c-1}[:, slice],  den += s xi (Q' . z_{c-1}),
// and the tile o = (O + Oc) / max(|den|, 1) is stored (the division only
// with the score normalisation).  s_i is the positive row scale of the
// 1/sqrt(d_k) and D-row normalisations, folded into the operands so that the
// fp16 operands carry normalised scores.  The diagonal key tile of each query
// tile also feeds the state update R += K'^T (zeta (.) V[:, slice]) (after R
// was scaled by gamma^(B_c) at chunk start; the cross term reads an operand
// copy of R_{c-1} in LDS, scaled by a power of two that puts its largest
// element just below 2^15, and Oc is scaled back exactly).  The decay mask,
// zeta, xi and the xPos phases are generated in registers.  Scores are
// recomputed once per d_v slice.
//
// Operand types: float inputs are contracted in fp32 MFMA; bf16 inputs in
// fp16 MFMA (see OpOf).  The fp16 operands require |q|, |k| < 2^15 and
// |v| < 2^16 elementwise and normalised scores s_i |q'_i . k'_j| < 2^16.
#include "internal.h"

namespace ret {

constexpr int NT = 256;   // threads per workgroup (4 waves)
constexpr int TR = 64;    // query rows per tile
constexpr int TK = 64;    // keys per tile

template <typename OP> struct Pad { static constexpr int v = 16 / sizeof(OP); };

template <typename OP, int DK, int SV>
struct Smem {
  static constexpr int P = Pad<OP>::v;
  static constexpr int QP = DK + P;      // pitch of Qs / Ks / Rt rows
  static constexpr int KP = TK + P;      // pitch of Vt / Vz / Ps rows
  OP Qs[TR * QP];
  OP Ks[TK * QP];
  OP Rt[SV * QP];      // scaled R_{c-1}^T for this slice: [col][d]
  OP Vt[SV * KP];      // V^T tile: [col][key]
  OP Vz[SV * KP];      // zeta-scaled V^T tile (diagonal tiles only)
  OP Ps[TR * KP];      // P tile: [query][key]
  float zs[DK];        // z_{c-1}
  float dens[TR];      // scaled score row sums of the current query tile
  float rscale[TR];    // s_i of the current query tile
  float wmax[NT / 64]; // per-wave max |R| for the operand copy scale
};

struct KParams {
  const void *q, *k, *v;
  void* o;
  ret_strides sq, sk, sv, so;
  int h, L, B, nslice;
  int64_t pos0, n_prev;
  unsigned flags;
  const float *state_in, *z_in;
  float *state_out, *z_out;
};

// Load TR rows x DK columns of Q or K (rows >= nvalid are zero), rotating each
// pair (2j, 2j+1) of row i by the phase of absolute position pos_first + i.
// Thread -> pair j, rows i0, i0 + RPP, ...; the phase of row i0 comes from a
// float64-reduced fp32 sincos and advances by e^{i RPP theta_j} per step.
template <typename T, typename OP, int DK>
__device__ __forceinline__ void load_rot_tile(OP* __restrict__ dst, const T* __restrict__ src, int64_t rs,
                                              int nvalid, int64_t pos_first, bool xpos,
                                              const double* __restrict__ theta) {
  constexpr int PAIRS = DK / 2;
  constexpr int RPP = NT / PAIRS;
  constexpr int NPASS = TR / RPP;
  constexpr int QP = DK + Pad<OP>::v;
  const int tid = threadIdx.x;
  const int j = tid % PAIRS;
  const int i0 = tid / PAIRS;
  float2 x[NPASS];
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int i = i0 + p * RPP;
    x[p] = (i < nvalid) ? Elem<T>::ld2(src + (int64_t)i * rs + 2 * j) : make_float2(0.f, 0.f);
  }
  float c = 1.f, s = 0.f, c1 = 1.f, s1 = 0.f;
  if (xpos) {
    phase(pos_first + i0, theta[j], c, s);
    phase(RPP, theta[j], c1, s1);
  }
#pragma unroll
  for (int p = 0; p < NPASS; ++p) {
    const int i = i0 + p * RPP;
    float a = x[p].x, b = x[p].y;
    if (xpos) {
      rot(a, b, c, s);
      advance(c, s, c1, s1);
    }
    st2(dst + i * QP + 2 * j, a, b);
  }
}

// Load TK keys x SV columns of V transposed into vt[col][key] (keys >= nvalid
// are zero); when vz is given also store zeta_key * v with
// zeta_key = gamma^(zeta_top - key) (the chunk-level zeta of the state update).
template <typename T, typename OP, int SV>
__device__ __forceinline__ void load_v_tile(OP* __restrict__ vt, OP* __restrict__ vz, const T* __restrict__ src,
                                            int64_t rs, int nvalid, const Decay& dec, int zeta_top) {
  constexpr int CP = SV / 2;           // column pairs
  constexpr int KG = NT / CP;          // key groups of 8 per pass
  constexpr int KP = TK + Pad<OP>::v;
  const int tid = threadIdx.x;
  const int cp = tid % CP;
  const int kg = tid / CP;
  for (int kk = 8 * kg; kk < TK; kk += 8 * KG) {
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int key = kk + e;
      float2 x = (key < nvalid) ? Elem<T>::ld2(src + (int64_t)key * rs + 2 * cp) : make_float2(0.f, 0.f);
      a[e] = x.x;
      b[e] = x.y;
    }
    st8(vt + (2 * cp) * KP + kk, a);
    st8(vt + (2 * cp + 1) * KP + kk, b);
    if (vz != nullptr) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float zt = dec.pow((float)(zeta_top - (kk + e)));
        a[e] *= zt;
        b[e] *= zt;
      }
      st8(vz + (2 * cp) * KP + kk, a);
      st8(vz + (2 * cp + 1) * KP + kk, b);
    }
  }
}

// A fragment of K'^T (rows = d, k = keys) gathered from the row-major key tile.
template <typename OP, int DK>
__device__ __forceinline__ typename Mfma<OP>::frag load_kT_frag(const OP* __restrict__ Ks, int key0, int d) {
  constexpr int QP = DK + Pad<OP>::v;
  const int h = (threadIdx.x & 32) ? 1 : 0;
  typename Mfma<OP>::frag f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = Ks[(key0 + 8 * h + e) * QP + d];
  return f;
}

template <typename T, typename TO, int DK, int DV, int SV>
__global__ void __launch_bounds__(NT, 1) chunkwise_kernel(KParams p, HeadParams hp) {
  typedef typename OpOf<T>::type OP;
  typedef Smem<OP, DK, SV> SM;
  typedef Mfma<OP> M;
  constexpr int QP = SM::QP;
  constexpr int KP = SM::KP;
  constexpr int NDT = DK / 32;               // d tiles of the state
  constexpr int NCT = SV / 32;               // column tiles of the slice
  constexpr int NST = NDT * NCT;             // state tiles
  constexpr int SPW = (NST + 3) / 4;         // state tiles per wave
  constexpr int NOT = (TR / 32) * NCT;       // output tiles per query tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lh = lane >> 5;      // lane half
  const int l32 = lane & 31;

  // workgroup -> (bh, slice); the slices of one head are kept on one XCD
  // (consecutive workgroup ids are dealt round-robin over the 8 XCDs)
  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if ((nwg & 7) == 0) wg = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int bh = wg / p.nslice;
  const int slice = wg % p.nslice;
  const int bb = bh / p.h;
  const int head = bh % p.h;
  const int s0 = slice * SV;

  Decay dec;
  dec.init(hp.gamma[head]);
  const bool xpos = (p.flags & RET_XPOS) != 0;
  const float qk_scale = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;

  const T* Qg = reinterpret_cast<const T*>(p.q) + bb * p.sq.b + head * p.sq.h;
  const T* Kg = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + head * p.sk.h;
  const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + s0;
  TO* Og = reinterpret_cast<TO*>(p.o) + bb * p.so.b + head * p.so.h + s0;

  // ---- state slice R[d][s0 + col] in accumulators, key-sum z[d] per thread
  f32x16 R[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    const int st = wave + 4 * t;
    const int dt = st / NCT, ct = st % NCT;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float val = 0.f;
      if (st < NST && p.state_in) {
        const int d = dt * 32 + acc_row(r, lane);
        val = p.state_in[((int64_t)bh * DK + d) * DV + s0 + ct * 32 + l32];
      }
      R[t][r] = val;
    }
  }
  float zreg = 0.f;   // z[tid] for tid < DK
  if (tid < DK && p.z_in) zreg = p.z_in[(int64_t)bh * DK + tid];

  const int my_ot = wave;                          // output tile of this wave
  const int ot_q = my_ot / NCT, ot_c = my_ot % NCT;
  const int sq_k = wave >> 1, sq_q = wave & 1;     // S^T tile: key half, query half

  const int nchunks = (p.L + p.B - 1) / p.B;
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * p.B;
    const int Bc = min(p.B, p.L - c0);
    const float gB = dec.pow((float)Bc);

    // ---- operand copy of R_{c-1} (transposed, scaled by 2^-e so that its
    //      largest element lies in [2^14, 2^15)), z_{c-1}; then scale the
    //      carried state by gamma^(B_c)
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < SPW; ++t)
      if (wave + 4 * t < NST)
#pragma unroll
        for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(R[t][r]));
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    __syncthreads();
    if (lane == 0) sm.wmax[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(sm.wmax[0], sm.wmax[1]), fmaxf(sm.wmax[2], sm.wmax[3]));
    int rexp = 0;
    if (amax > 0.f && amax < 3.0e38f) {
      int ex;
      frexpf(amax, &ex);          // amax in [2^(ex-1), 2^ex)
      rexp = ex - 15;
    }
    const float rdown = ldexpf(1.f, -rexp), rup = ldexpf(1.f, rexp);
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      const int st = wave + 4 * t;
      if (st < NST) {
        const int dt = st / NCT, ct = st % NCT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = dt * 32 + acc_row(r, lane);
          sm.Rt[(ct * 32 + l32) * QP + d] = to_op<OP>(R[t][r] * rdown);
          R[t][r] *= gB;
        }
      }
    }
    if (tid < DK) {
      sm.zs[tid] = zreg;
      zreg *= gB;
    }

    const int nrt = (Bc + TR - 1) / TR;
    for (int rt = 0; rt < nrt; ++rt) {
      const int r0 = rt * TR;
      const int qvalid = min(TR, Bc - r0);
      __syncthreads();
      load_rot_tile<T, OP, DK>(sm.Qs, Qg + (int64_t)(c0 + r0) * p.sq.l, p.sq.l, qvalid, p.pos0 + c0 + r0, xpos,
                               hp.theta);
      if (tid < TR) {
        sm.dens[tid] = 0.f;
        float s = qk_scale;
        if (p.flags & RET_NORM_DROW) s *= dec.drow((float)(p.n_prev + c0 + r0 + tid + 1));
        sm.rscale[tid] = s;
      }
      // row scale of this lane's S^T query column
      float s_q = qk_scale;
      if (p.flags & RET_NORM_DROW) s_q *= dec.drow((float)(p.n_prev + c0 + r0 + sq_q * 32 + l32 + 1));

      f32x16 O = {};
      float den = 0.f;

      for (int kt = 0; kt <= rt; ++kt) {
        const int k0 = kt * TK;
        const int kvalid = min(TK, Bc - k0);
        const bool diag = (kt == rt);
        if (kt > 0) __syncthreads();
        load_rot_tile<T, OP, DK>(sm.Ks, Kg + (int64_t)(c0 + k0) * p.sk.l, p.sk.l, kvalid, p.pos0 + c0 + k0, xpos,
                                 hp.theta);
        load_v_tile<T, OP, SV>(sm.Vt, diag ? sm.Vz : nullptr, Vg + (int64_t)(c0 + k0) * p.sv.l, p.sv.l, kvalid,
                               dec, Bc - 1 - k0);
        __syncthreads();

        // S^T tile (32 keys x 32 queries) of this wave
        f32x16 S = {};
#pragma unroll 4
        for (int kb = 0; kb < DK; kb += 16) {
          auto a = M::load(sm.Ks + (sq_k * 32 + l32) * QP + kb + 8 * lh);
          auto b = M::load(sm.Qs + (sq_q * 32 + l32) * QP + kb + 8 * lh);
          M::mma(S, a, b);
        }
        // decay mask and row scale, fp32 row sums, P -> LDS
        {
          const int qi = r0 + sq_q * 32 + l32;   // chunk-local query
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float pv[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              const int r = 4 * i + jj;
              const int ki = k0 + sq_k * 32 + acc_row(r, lane);
              float val = 0.f;
              if (ki <= qi) val = S[r] * (s_q * dec.pow((float)(qi - ki)));
              den += val;
              pv[jj] = val;
            }
            st4(sm.Ps + (sq_q * 32 + l32) * KP + sq_k * 32 + 8 * i + 4 * lh, pv);
          }
        }
        __syncthreads();
        // O += P V[:, slice]
        if (my_ot < NOT) {
#pragma unroll
          for (int kb = 0; kb < TK; kb += 16) {
            auto a = M::load(sm.Ps + (ot_q * 32 + l32) * KP + kb + 8 * lh);
            auto b = M::load(sm.Vt + (ot_c * 32 + l32) * KP + kb + 8 * lh);
            M::mma(O, a, b);
          }
        }
        // state update from the diagonal key tile: R += K'^T (zeta V)
        if (diag) {
#pragma unroll
          for (int t = 0; t < SPW; ++t) {
            const int st = wave + 4 * t;
            if (st < NST) {
              const int dt = st / NCT, ct = st % NCT;
#pragma unroll
              for (int kb = 0; kb < TK; kb += 16) {
                auto a = load_kT_frag<OP, DK>(sm.Ks, kb, dt * 32 + l32);
                auto b = M::load(sm.Vz + (ct * 32 + l32) * KP + kb + 8 * lh);
                M::mma(R[t], a, b);
              }
            }
          }
          if (tid < DK) {
            float zacc = 0.f;
            for (int key = 0; key < kvalid; ++key)
              zacc += dec.pow((float)(Bc - 1 - k0 - key)) * from_op<OP>(sm.Ks[key * QP + tid]);
            zreg += zacc;
          }
        }
      }

      // score row sums of this query tile: lanes l and l^32 share a query,
      // waves (0,q) and (1,q) cover the two key halves
      den += __shfl_xor(den, 32, 64);
      if (lh == 0) atomicAdd(&sm.dens[sq_q * 32 + l32], den);

      // cross-chunk term: scale query rows by s xi (xi = gamma^(i+1)), then
      // Oc = (s xi Q') (2^-e R_{c-1}),  den += s xi (Q' . z_{c-1})
      __syncthreads();
      for (int e = tid; e < TR * DK; e += NT) {
        const int i = e / DK, d = e % DK;
        const float f = sm.rscale[i] * dec.pow((float)(r0 + i + 1));
        sm.Qs[i * QP + d] = to_op<OP>(from_op<OP>(sm.Qs[i * QP + d]) * f);
      }
      __syncthreads();
      {
        // 4 threads per query row for Q' . z
        const int i = tid >> 2, part = tid & 3;
        float acc = 0.f;
        for (int d = part; d < DK; d += 4) acc += from_op<OP>(sm.Qs[i * QP + d]) * sm.zs[d];
        acc += __shfl_xor(acc, 1, 64);
        acc += __shfl_xor(acc, 2, 64);
        if (part == 0) atomicAdd(&sm.dens[i], acc);
      }
      f32x16 Oc = {};
      if (my_ot < NOT) {
#pragma unroll 4
        for (int kb = 0; kb < DK; kb += 16) {
          auto a = M::load(sm.Qs + (ot_q * 32 + l32) * QP + kb + 8 * lh);
          auto b = M::load(sm.Rt + (ot_c * 32 + l32) * QP + kb + 8 * lh);
          M::mma(Oc, a, b);
        }
      }
      __syncthreads();
      // normalise and store
      if (my_ot < NOT) {
        const int col = ot_c * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qi = ot_q * 32 + acc_row(r, lane);
          if (qi < qvalid) {
            const int64_t t_abs = c0 + r0 + qi;
            float val = O[r] + Oc[r] * rup;
            if (p.flags & RET_NORM_SCORE) val = val / fmaxf(fabsf(sm.dens[qi]), 1.f);
            Og[t_abs * p.so.l + col] = Store<TO>::cvt(val);
          }
        }
      }
    }
  }

  // ---- final state
  if (p.state_out) {
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      const int st = wave + 4 * t;
      if (st < NST) {
        const int dt = st / NCT, ct = st % NCT;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int d = dt * 32 + acc_row(r, lane);
          p.state_out[((int64_t)bh * DK + d) * DV + s0 + ct * 32 + l32] = R[t][r];
        }
      }
    }
  }
  if (p.z_out && slice == 0 && tid < DK) p.z_out[(int64_t)bh * DK + tid] = zreg;
}

template <typename T, typename TO, int DK, int DV, int SV>
static hipError_t launch_t(const ChunkArgs& a, hipStream_t st) {
  static_assert(DK / 2 <= NT, "pairs per row exceed the workgroup");
  static_assert((TR / 32) * (SV / 32) <= 4, "one output tile per wave");
  KParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.sq = a.sq; p.sk = a.sk; p.sv = a.sv; p.so = a.so;
  p.h = a.h; p.L = a.L; p.B = a.B; p.nslice = DV / SV;
  p.pos0 = a.pos0; p.n_prev = a.n_prev; p.flags = a.flags;
  p.state_in = a.state_in; p.z_in = a.z_in; p.state_out = a.state_out; p.z_out = a.z_out;
  const size_t sh = sizeof(Smem<typename OpOf<T>::type, DK, SV>);
  auto kern = chunkwise_kernel<T, TO, DK, DV, SV>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sh);
  if (e != hipSuccess) return e;
  dim3 grid(a.b * a.h * (DV / SV));
  hipLaunchKernelGGL(kern, grid, dim3(NT), sh, st, p, *a.hp);
  return hipGetLastError();
}

template <typename T, int DK, int DV, int SV>
static hipError_t launch_o(const ChunkArgs& a, hipStream_t st) {
  return a.out_dt == RET_BF16 ? launch_t<T, bf16, DK, DV, SV>(a, st) : launch_t<T, float, DK, DV, SV>(a, st);
}

#define RET_SHAPES(X)                       \
  X(bf16, 32, 32, 32)                       \
  X(bf16, 64, 64, 64)                       \
  X(bf16, 128, 128, 64)                     \
  X(bf16, 128, 256, 64)                     \
  X(bf16, 256, 256, 64)                     \
  X(bf16, 256, 512, 64)                     \
  X(float, 32, 32, 32)                      \
  X(float, 64, 64, 64)

bool chunkwise_supported(ret_dtype in_dt, int dk, int dv) {
#define X(T, DK, DV, SV) \
  if ((in_dt == RET_BF16) == (sizeof(T) == 2) && dk == DK && dv == DV) return true;
  RET_SHAPES(X)
#undef X
  return false;
}

size_t chunkwise_workspace(int, int, int, int, int, int, unsigned) { return 0; }

hipError_t launch_chunkwise(const ChunkArgs& a, hipStream_t st, bool* supported) {
  *supported = true;
#define X(T, DK, DV, SV) \
  if ((a.in_dt == RET_BF16) == (sizeof(T) == 2) && a.dk == DK && a.dv == DV) return launch_o<T, DK, DV, SV>(a, st);
  RET_SHAPES(X)
#undef X
  *supported = false;
  return hipSuccess;
}

}  // namespace ret
