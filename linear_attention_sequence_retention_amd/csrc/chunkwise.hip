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

constexpr int NT = 512;   // threads per workgroup: 4 score waves + 4 state waves
constexpr int TR = 64;    // query rows per tile
constexpr int TK = 64;    // keys per tile

template <typename OP> struct Pad { static constexpr int v = 16 / sizeof(OP); };

template <typename OP, int DK, int SV>
struct Smem {
  static constexpr int P = Pad<OP>::v;
  static constexpr int QP = DK + P;      // pitch of Qs / Ks / Rt rows
  static constexpr int KP = TK + P;      // pitch of Vt / Vz / Ps rows
  static constexpr int CP = SV + 4;      // pitch of the fp32 cross-term tile
  OP Qs[TR * QP];      // rotated query tile [row][d]
  OP Ks[TK * QP];      // rotated key tile [key][d]
  OP Rt[SV * QP];      // scaled R_{c-1}^T for this slice: [col][d]
  OP Vt[SV * KP];      // V^T tile: [col][key]
  OP Vz[SV * KP];      // zeta-scaled V^T tile (diagonal tiles only)
  OP Ps[TR * KP];      // P tile: [query][key]; reused to stage the output
  float Oc[TR * CP];   // scaled cross term of the query tile
  float zs[DK];        // z_{c-1}
  float zeta[TK];      // zeta of the keys of the diagonal tile
  float dens[TR];      // scaled score row sums of the query tile (cross part)
  float dpart[2][TR];  // within-chunk row sums of key halves 0 / 1
  float rs[TR];        // s_i of the query tile
  float xs[TR];        // s_i xi_i (cross-term row factor)
  float wmax[NT / 64];
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
  unsigned* nf;
};

// Raw pair loads (two consecutive input elements) kept in one register
// between the global load and the LDS store.
template <typename T> struct Raw;
template <> struct Raw<bf16> {
  typedef uint32_t type;
  __device__ __forceinline__ static type ld(const bf16* p) { return *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ static float2 f(type u) { return make_float2(lo_bf(u), hi_bf(u)); }
  __device__ __forceinline__ static type zero() { return 0u; }
};
template <> struct Raw<half> {
  typedef uint32_t type;
  __device__ __forceinline__ static type ld(const half* p) { return *reinterpret_cast<const uint32_t*>(p); }
  __device__ __forceinline__ static float2 f(type u) {
    f16x2 v = __builtin_bit_cast(f16x2, u);
    return make_float2((float)v.x, (float)v.y);
  }
  __device__ __forceinline__ static type zero() { return 0u; }
};
template <> struct Raw<float> {
  typedef float2 type;
  __device__ __forceinline__ static type ld(const float* p) { return *reinterpret_cast<const float2*>(p); }
  __device__ __forceinline__ static float2 f(type u) { return u; }
  __device__ __forceinline__ static type zero() { return make_float2(0.f, 0.f); }
};

// Staged global data of one job (a key tile, plus the query tile on the
// diagonal), loaded into registers one job ahead of its use.
template <typename T, int DK, int SV>
struct Stage {
  static constexpr int PAIRS = DK / 2;
  static constexpr int RPP = NT / PAIRS;          // rows per pass of the Q/K loader
  static constexpr int NPASS = TR / RPP;
  static constexpr int VCP = SV / 2;              // V column pairs
  static constexpr int VKG = NT / VCP;            // V key groups of 4
  static constexpr int VPASS = (TK + 4 * VKG - 1) / (4 * VKG);
  typename Raw<T>::type k[NPASS];
  typename Raw<T>::type q[NPASS];
  typename Raw<T>::type v[VPASS][4];

  // issue the loads (rows >= nvalid read as zero).  Bases are uniform
  // (scalar registers); per-lane offsets are 32-bit and clamped to the last
  // valid row, so the loads are branch-free and in bounds.
  __device__ __forceinline__ void load(const T* __restrict__ Qrow, int qs, const T* __restrict__ Krow, int ks,
                                       const T* __restrict__ Vrow, int vs, int nvalid, bool with_q) {
    const int tid = threadIdx.x;
    const int j = tid % PAIRS, i0 = tid / PAIRS;
#pragma unroll
    for (int p = 0; p < NPASS; ++p) {
      const int i = i0 + p * RPP;
      const int ic = min(i, nvalid - 1);
      const uint32_t ko = (uint32_t)(ic * ks + 2 * j);
      typename Raw<T>::type kv = Raw<T>::ld(Krow + ko);
      k[p] = (i < nvalid) ? kv : Raw<T>::zero();
      if (with_q) {
        const uint32_t qo = (uint32_t)(ic * qs + 2 * j);
        typename Raw<T>::type qv = Raw<T>::ld(Qrow + qo);
        q[p] = (i < nvalid) ? qv : Raw<T>::zero();
      }
    }
    const int cp = tid % VCP, kg = tid / VCP;
#pragma unroll
    for (int p = 0; p < VPASS; ++p) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = 4 * (kg + p * VKG) + e;
        const int kc = min(key, nvalid - 1);
        typename Raw<T>::type vv = Raw<T>::ld(Vrow + (uint32_t)(kc * vs + 2 * cp));
        v[p][e] = (key < nvalid) ? vv : Raw<T>::zero();
      }
    }
  }
};

template <typename T, typename TO, int DK, int DV, int SV>
__global__ void __launch_bounds__(NT, 1) chunkwise_kernel(KParams p, HeadParams hp) {
  typedef typename OpOf<T>::type OP;
  typedef Smem<OP, DK, SV> SM;
  typedef Stage<T, DK, SV> ST;
  typedef Mfma<OP> M;
  constexpr int QP = SM::QP;
  constexpr int KP = SM::KP;
  constexpr int CPITCH = SM::CP;
  constexpr int NDT = DK / 32;               // d tiles of the state
  constexpr int NCT = SV / 32;               // column tiles of the slice
  constexpr int NST = NDT * NCT;             // state tiles
  constexpr int SPW = (NST + 7) / 8;         // state tiles per wave
  constexpr int NOT = (TR / 32) * NCT;       // output tiles per query tile (<= 4)
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  SM& sm = *reinterpret_cast<SM*>(smem_raw);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool score_wave = wave < 4;
  const int w4 = wave & 3;
  const int lh = lane >> 5;
  const int l32 = lane & 31;

  // workgroup -> (bh, slice); the slices of one head are kept on one XCD
  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if ((nwg & 7) == 0) wg = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int bh = wg / p.nslice;
  const int slice = wg % p.nslice;
  const int bb = bh / p.h;
  const int head = bh % p.h;
  const int s0 = slice * SV;

  Decay dec;
  dec.init(hp, head);
  const bool xpos = (p.flags & RET_XPOS) != 0;
  const bool drow = (p.flags & RET_NORM_DROW) != 0;
  const float qk_scale = (p.flags & RET_SCALE_QK) ? rsqrtf((float)DK) : 1.f;

  const T* Qg = reinterpret_cast<const T*>(p.q) + bb * p.sq.b + head * p.sq.h;
  const T* Kg = reinterpret_cast<const T*>(p.k) + bb * p.sk.b + head * p.sk.h;
  const T* Vg = reinterpret_cast<const T*>(p.v) + bb * p.sv.b + head * p.sv.h + s0;
  TO* Og = reinterpret_cast<TO*>(p.o) + bb * p.so.b + head * p.so.h + s0;

  // ---- state slice R[d][s0 + col] spread over all 8 waves (tile
  //      wave + 8t), key-sum z[d] on thread tid - 256 of the state waves
  f32x16 R[SPW];
#pragma unroll
  for (int t = 0; t < SPW; ++t) {
    const int st = wave + 8 * t;
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
  const int zd = tid - 256;             // d owned by this state-wave thread
  float zreg = 0.f;
  if (!score_wave && zd < DK && p.z_in) zreg = p.z_in[(int64_t)bh * DK + zd];

  // ---- flattened job list: per chunk, per query tile: the diagonal key
  //      tile first (loaded together with the query tile), then the earlier
  //      key tiles
  const int nchunks = (p.L + p.B - 1) / p.B;
  auto rows_in = [&](int c) { return min(p.B, p.L - c * p.B); };
  struct Job { int c, rt, kt; };
  auto next_job = [&](Job j) -> Job {
    const int nrt = (rows_in(j.c) + TR - 1) / TR;
    // order within a row tile: kt = rt, 0, 1, ..., rt-1
    int nk;
    if (j.kt == j.rt) nk = (j.rt > 0) ? 0 : -1;
    else nk = (j.kt + 1 < j.rt) ? j.kt + 1 : -1;
    if (nk >= 0) return Job{j.c, j.rt, nk};
    if (j.rt + 1 < nrt) return Job{j.c, j.rt + 1, j.rt + 1};
    return Job{j.c + 1, 0, 0};
  };

  ST stg;
  auto issue = [&](Job j) {
    if (j.c >= nchunks) return;
    const int c0 = j.c * p.B, Bc = rows_in(j.c);
    const int k0 = j.kt * TK;
    const int nvalid = min(TK, Bc - k0);
    const bool diag = (j.kt == j.rt);
    stg.load(Qg + (int64_t)(c0 + k0) * p.sq.l, (int)p.sq.l, Kg + (int64_t)(c0 + k0) * p.sk.l, (int)p.sk.l,
             Vg + (int64_t)(c0 + k0) * p.sv.l, (int)p.sv.l, nvalid, diag);
  };

  const int ot_q = w4 / NCT, ot_c = w4 % NCT;      // output / cross tile of wave w4
  const int sq_k = w4 >> 1, sq_q = w4 & 1;         // S^T tile of score wave w4

  Job job{0, 0, 0};
  issue(job);
  f32x16 O = {};
  float den = 0.f;
  int cur_chunk = -1;
  float rup = 1.f;

  while (job.c < nchunks) {
    const int c0 = job.c * p.B;
    const int Bc = rows_in(job.c);
    const int r0 = job.rt * TR;
    const int k0 = job.kt * TK;
    const int qvalid = min(TR, Bc - r0);
    const int kvalid = min(TK, Bc - k0);
    const bool diag = (job.kt == job.rt);

    __syncthreads();   // previous job done with the LDS tiles
    if (job.c != cur_chunk) {
      // ---- chunk start: operand copy of R_{c-1} (transposed, scaled by
      //      2^-e so its largest element lies in [2^14, 2^15)) and z_{c-1};
      //      then scale the carried state by gamma^(B_c)
      cur_chunk = job.c;
      float amax = 0.f;
#pragma unroll
      for (int t = 0; t < SPW; ++t)
        if (wave + 8 * t < NST)
#pragma unroll
          for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(R[t][r]));
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      if (lane == 0) sm.wmax[wave] = amax;
      __syncthreads();
      amax = 0.f;
#pragma unroll
      for (int w = 0; w < NT / 64; ++w) amax = fmaxf(amax, sm.wmax[w]);
      int rexp = 0;
      if (amax > 0.f && amax < 3.0e38f) {
        int ex;
        frexpf(amax, &ex);
        rexp = min(max(ex - 15, -100), 100);
      }
      const float rdown = ldexpf(1.f, -rexp);
      rup = ldexpf(1.f, rexp);
      const float gB = dec.pow((float)Bc);
#pragma unroll
      for (int t = 0; t < SPW; ++t) {
        const int st = wave + 8 * t;
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
      if (!score_wave && zd < DK) {
        sm.zs[zd] = zreg;
        zreg *= gB;
      }
    }

    // ---- staged registers -> LDS (rotation of Q/K, transposition of V)
    {
      constexpr int PAIRS = ST::PAIRS, RPP = ST::RPP, NPASS = ST::NPASS;
      const int j = tid % PAIRS, i0 = tid / PAIRS;
      float c = 1.f, s = 0.f, c1 = 1.f, s1 = 0.f;
      if (xpos) {
        phase(p.pos0 + c0 + k0 + i0, hp.theta[j], c, s);
        phase(RPP, hp.theta[j], c1, s1);
      }
#pragma unroll
      for (int pp = 0; pp < NPASS; ++pp) {
        const int i = i0 + pp * RPP;
        float2 kk = Raw<T>::f(stg.k[pp]);
        float2 qq = Raw<T>::f(stg.q[pp]);
        if (xpos) {
          rot(kk.x, kk.y, c, s);
          if (diag) rot(qq.x, qq.y, c, s);
          advance(c, s, c1, s1);
        }
        st2(sm.Ks + i * QP + 2 * j, kk.x, kk.y);
        if (diag) st2(sm.Qs + i * QP + 2 * j, qq.x, qq.y);
      }
      constexpr int VCP = ST::VCP, VKG = ST::VKG, VPASS = ST::VPASS;
      const int cp = tid % VCP, kg = tid / VCP;
#pragma unroll
      for (int pp = 0; pp < VPASS; ++pp) {
        const int key0 = 4 * (kg + pp * VKG);
        if (key0 < TK) {
          float a[4], b[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float2 x = Raw<T>::f(stg.v[pp][e]);
            a[e] = x.x;
            b[e] = x.y;
          }
          st4(sm.Vt + (2 * cp) * KP + key0, a);
          st4(sm.Vt + (2 * cp + 1) * KP + key0, b);
          if (diag) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float zt = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - key0 - e) * dec.lg2);
              a[e] *= zt;
              b[e] *= zt;
            }
            st4(sm.Vz + (2 * cp) * KP + key0, a);
            st4(sm.Vz + (2 * cp + 1) * KP + key0, b);
          }
        }
      }
      if (diag && tid < TK) sm.zeta[tid] = __builtin_amdgcn_exp2f((float)(Bc - 1 - k0 - tid) * dec.lg2);
      if (diag && tid < TR) {
        // row tables of the query tile: s_i, s_i xi_i 2^e, and den = 0
        float sc = qk_scale;
        if (drow) sc *= dec.drow((float)(p.n_prev + c0 + r0 + tid + 1));
        sm.rs[tid] = sc;
        sm.xs[tid] = sc * dec.pow((float)(r0 + tid + 1));
        sm.dens[tid] = 0.f;
        sm.dpart[0][tid] = 0.f;
        sm.dpart[1][tid] = 0.f;
      }
    }
    __syncthreads();
    // ---- prefetch the next job while this one computes
    const Job nj = next_job(job);
    issue(nj);

    if (score_wave) {
      if (diag) {
        O = f32x16{};
        den = 0.f;
      }
      // S^T tile (32 keys x 32 queries); on the diagonal tile the block of
      // keys 32..63 against queries 0..31 is entirely masked
      const bool skip = diag && sq_k > sq_q;
      const int qi = r0 + sq_q * 32 + l32;          // chunk-local query of this lane
      if (!skip) {
        f32x16 S = {};
#pragma unroll 2
        for (int kb = 0; kb < DK; kb += 16) {
          auto a = M::load(sm.Ks + (sq_k * 32 + l32) * QP + kb + 8 * lh);
          auto b = M::load(sm.Qs + (sq_q * 32 + l32) * QP + kb + 8 * lh);
          M::mma(S, a, b);
        }
        const float s_q = sm.rs[sq_q * 32 + l32];
        const float base = (float)(qi - k0 - sq_k * 32 - 4 * lh);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float pv[4];
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int r = 4 * i + jj;
            const float dist = base - (float)(8 * i + jj);     // qi - ki
            float val = 0.f;
            if (dist >= 0.f) val = S[r] * s_q * __builtin_amdgcn_exp2f(dist * dec.lg2);
            den += val;
            pv[jj] = val;
          }
          st4(sm.Ps + (sq_q * 32 + l32) * KP + sq_k * 32 + 8 * i + 4 * lh, pv);
        }
      } else {
        float zero4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) st4(sm.Ps + (sq_q * 32 + l32) * KP + sq_k * 32 + 8 * i + 4 * lh, zero4);
      }
    } else {
      if (diag) {
        if (zd < DK) {
          float zacc = 0.f;
          for (int key = 0; key < kvalid; ++key) zacc += sm.zeta[key] * from_op<OP>(sm.Ks[key * QP + zd]);
          zreg += zacc;
        }
        // cross-chunk term of this query tile: Oc = Q' (2^-e R_{c-1}), and
        // Q' . z_{c-1}; the row factors s xi (and 2^e for Oc) are applied here
        if (w4 < NOT) {
          f32x16 Oc = {};
#pragma unroll 2
          for (int kb = 0; kb < DK; kb += 16) {
            auto a = M::load(sm.Qs + (ot_q * 32 + l32) * QP + kb + 8 * lh);
            auto b = M::load(sm.Rt + (ot_c * 32 + l32) * QP + kb + 8 * lh);
            M::mma(Oc, a, b);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int qrow = ot_q * 32 + acc_row(r, lane);
            sm.Oc[qrow * CPITCH + ot_c * 32 + l32] = Oc[r] * (sm.xs[qrow] * rup);
          }
        }
        {
          // 4 threads per query row for Q' . z_{c-1}
          const int i = (tid - 256) >> 2, part = tid & 3;
          float acc = 0.f;
          for (int d = part; d < DK; d += 4) acc += from_op<OP>(sm.Qs[i * QP + d]) * sm.zs[d];
          acc += __shfl_xor(acc, 1, 64);
          acc += __shfl_xor(acc, 2, 64);
          if (part == 0) atomicAdd(&sm.dens[i], acc * sm.xs[i]);
        }
      }
    }
    if (diag) {
      // state update from the diagonal key tile: R += K'^T (zeta V), all waves
#pragma unroll
      for (int t = 0; t < SPW; ++t) {
        const int st = wave + 8 * t;
        if (st < NST) {
          const int dt = st / NCT, ct = st % NCT;
#pragma unroll
          for (int kb = 0; kb < TK; kb += 16) {
            typename M::frag a;
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = sm.Ks[(kb + 8 * lh + e) * QP + dt * 32 + l32];
            auto b = M::load(sm.Vz + (ct * 32 + l32) * KP + kb + 8 * lh);
            M::mma(R[t], a, b);
          }
        }
      }
    }
    __syncthreads();
    // O += P V[:, slice] (on the diagonal tile, queries 0..31 only see keys 0..31)
    if (score_wave && w4 < NOT) {
      const int kend = (diag && ot_q == 0) ? 32 : TK;
      for (int kb = 0; kb < kend; kb += 16) {
        auto a = M::load(sm.Ps + (ot_q * 32 + l32) * KP + kb + 8 * lh);
        auto b = M::load(sm.Vt + (ot_c * 32 + l32) * KP + kb + 8 * lh);
        M::mma(O, a, b);
      }
    }

    // ---- end of a query tile: combine, normalise, store
    const bool last_of_rt = !(nj.c == job.c && nj.rt == job.rt);
    if (last_of_rt) {
      if (score_wave) {
        den += __shfl_xor(den, 32, 64);
        if (lh == 0) sm.dpart[sq_k][sq_q * 32 + l32] = den;
      }
      __syncthreads();
      // cross part plus the two key halves, summed in a fixed order
      if (tid < TR) sm.dens[tid] += sm.dpart[0][tid] + sm.dpart[1][tid];
      __syncthreads();
      if (score_wave && w4 < NOT) {
        const int col = ot_c * 32 + l32;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qrow = ot_q * 32 + acc_row(r, lane);
          float val = O[r] + sm.Oc[qrow * CPITCH + col];
          if (p.flags & RET_NORM_SCORE) val = val / fmaxf(fabsf(sm.dens[qrow]), 1.f);
          sm.Oc[qrow * CPITCH + col] = val;
        }
      }
      __syncthreads();
      // coalesced store: each thread writes 4 consecutive columns of a row
      constexpr int C4 = SV / 4;
      bool bad = false;
      for (int e = tid; e < TR * C4; e += NT) {
        const int row = e / C4, c4 = e % C4;
        if (row < qvalid) {
          const float* src = sm.Oc + row * CPITCH + 4 * c4;
          bad |= nonfinite_as<TO>(src[0]) | nonfinite_as<TO>(src[1]) | nonfinite_as<TO>(src[2]) |
                 nonfinite_as<TO>(src[3]);
          store4(Og + (int64_t)(c0 + r0 + row) * p.so.l + 4 * c4, src);
        }
      }
      flag_nonfinite(p.nf, bad, kNonFiniteFwd);
    }
    job = nj;
  }

  // ---- final state
  if (p.state_out) {
#pragma unroll
    for (int t = 0; t < SPW; ++t) {
      const int st = wave + 8 * t;
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
  if (p.z_out && slice == 0 && !score_wave && zd < DK) p.z_out[(int64_t)bh * DK + zd] = zreg;
}
// n floats from src to dst (the key-sum snapshot of an in-place continuation)
__global__ void __launch_bounds__(256) copy_f32_kernel(const float* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

template <typename T, typename TO, int DK, int DV, int SV>
static hipError_t launch_t(const ChunkArgs& a, hipStream_t st) {
  static_assert(DK / 2 <= NT, "pairs per row exceed the workgroup");
  static_assert((TR / 32) * (SV / 32) <= 4, "one output tile per wave");
  static_assert(sizeof(Smem<typename OpOf<T>::type, DK, SV>) <= 160 * 1024, "LDS of one workgroup");
  KParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.sq = a.sq; p.sk = a.sk; p.sv = a.sv; p.so = a.so;
  p.h = a.h; p.L = a.L; p.B = a.B; p.nslice = DV / SV;
  p.pos0 = a.pos0; p.n_prev = a.n_prev; p.flags = a.flags;
  p.state_in = a.state_in; p.z_in = a.z_in; p.state_out = a.state_out; p.z_out = a.z_out;
  p.nf = a.nf;
  if (fused_z_snapshot(a)) {
    // every d_v slice of a head reads z_in, and slice 0 writes z_out when it
    // ends: with z_out over z_in, a slice that starts after its head's slice 0
    // has finished would read the new key-sum.  The slices read a copy.
    const int n = a.b * a.h * a.dk;
    float* snap = static_cast<float*>(a.ws);
    hipLaunchKernelGGL(copy_f32_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.z_in, snap, n);
    p.z_in = snap;
  }
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
  if (a.out_dt == RET_BF16) return launch_t<T, bf16, DK, DV, SV>(a, st);
  if (a.out_dt == RET_F16) return launch_t<T, half, DK, DV, SV>(a, st);
  return launch_t<T, float, DK, DV, SV>(a, st);
}

template <typename T> constexpr ret_dtype dt_of();
template <> constexpr ret_dtype dt_of<bf16>() { return RET_BF16; }
template <> constexpr ret_dtype dt_of<half>() { return RET_F16; }
template <> constexpr ret_dtype dt_of<float>() { return RET_F32; }

#define RET_SHAPES(X)                       \
  X(bf16, 32, 32, 32)                       \
  X(bf16, 64, 64, 64)                       \
  X(bf16, 128, 128, 64)                     \
  X(bf16, 128, 256, 64)                     \
  X(bf16, 256, 256, 64)                     \
  X(bf16, 256, 512, 64)                     \
  X(half, 128, 256, 64)                     \
  X(half, 256, 512, 64)                     \
  X(float, 32, 32, 32)                      \
  X(float, 64, 64, 64)

bool chunkwise_supported(ret_dtype in_dt, int dk, int dv) {
#define X(T, DK, DV, SV) \
  if (in_dt == dt_of<T>() && dk == DK && dv == DV) return true;
  RET_SHAPES(X)
#undef X
  return false;
}

size_t chunkwise_workspace(int b, int h, int L, int dk, int dv, int B, unsigned) {
  // the workspace query has no dtype: the large-chunk path serves bf16 / f16
  // inputs, and no f32 kernel exists for its shape.  The fused kernel needs
  // room for a snapshot of the key-sums (used only when z_out overlaps z_in).
  if (three_phase_applies(RET_BF16, dk, dv, B)) return three_phase_workspace(b, h, L, B);
  return ((size_t)b * h * dk * sizeof(float) + 255) & ~(size_t)255;
}

bool fused_z_snapshot(const ChunkArgs& a) {
  if (three_phase_applies(a.in_dt, a.dk, a.dv, a.B) || !a.z_in || !a.z_out) return false;
  const size_t n = (size_t)a.b * a.h * a.dk * sizeof(float);
  const uintptr_t x = (uintptr_t)a.z_in, y = (uintptr_t)a.z_out;
  return x < y + n && y < x + n;
}

hipError_t launch_chunkwise(const ChunkArgs& a, hipStream_t st, bool* supported) {
  *supported = true;
  if (three_phase_applies(a.in_dt, a.dk, a.dv, a.B)) return launch_three_phase(a, st);
#define X(T, DK, DV, SV) \
  if (a.in_dt == dt_of<T>() && a.dk == DK && a.dv == DV) return launch_o<T, DK, DV, SV>(a, st);
  RET_SHAPES(X)
#undef X
  *supported = false;
  return hipSuccess;
}

}  // namespace ret
