// Chunked causal prefill for OAL attention on gfx950.
//
// The prefix sum of the OAL paper's Eq. (6) is split at chunk starts: for a
// query i in chunk c,
//     u~_i = phi_q(q_i)^T S_c + sum_{j in c, j <= i} kappa(q_i, k_j) [v_j, 1]
// with S_c the state of Eq. (5) accumulated over all tokens before chunk c.
// The second term is the direct pairwise form of the paper's sec. 4.4,
// restricted to one chunk.
//
// Kernel 1 (scan): one CTA per (16-feature tiles x 4, batch*KV head) walks the
// chunks in order, keeping its slice of S in MFMA accumulators (fp32).  Before
// adding chunk c it writes S_c to a snapshot buffer in the internal K-blocked
// layout (bf16 for bf16 inputs, fp32 otherwise); the update itself is
// S += phi_k(K_c)^T [V_c | 1] on MFMA.
//
// Kernel 2 (out): one CTA per (chunk, query head, batch) computes
//   * the inter-chunk read phi_q(Q_c) . S_c on MFMA, the four waves splitting
//     the feature (K) dimension and reducing through LDS;
//   * the intra-chunk block: group score tiles S_g = Q K_g^T on MFMA, the
//     grouped polynomial and the causal mask in registers, P . [V | 1] on MFMA;
//   * the normalisation y = num / den.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

constexpr int DV = 64;       // value head dimension handled by these kernels
constexpr int NCOL = DV + 1; // value columns + normaliser column

// --------------------------------------------------------------------------
// staging helpers
// --------------------------------------------------------------------------

// Loads rows [row0, row0 + nrows) of a [N, DH] activation slab into `dst`
// (fp32, row stride `ld`), zero-filling rows at or beyond N.  All threads of
// the block take part.
template <typename T, int DH>
__device__ __forceinline__ void stage_rows_f32(const T* __restrict__ src, int row0, int nrows, int N,
                                               float* dst, int ld) {
  for (int idx = threadIdx.x; idx < nrows * DH; idx += blockDim.x) {
    const int rr = idx / DH, cc = idx % DH;
    const int row = row0 + rr;
    dst[rr * ld + cc] = row < N ? to_f32(src[(long)row * DH + cc]) : 0.f;
  }
}

// ReBased pre-map in place on `nrows` fp32 rows of length DH (stride ld):
// x <- gamma * (x - mean) / sqrt(var + eps) + beta, biased variance.
// Rows at or beyond `nvalid` are left untouched (they are zero padding).
template <int DH>
__device__ __forceinline__ void premap_rows(float* rows, int ld, int nrows, int nvalid,
                                            const float* __restrict__ gamma,
                                            const float* __restrict__ beta, float eps) {
  for (int rr = threadIdx.x; rr < nrows; rr += blockDim.x) {
    if (rr >= nvalid) continue;
    float* x = rows + rr * ld;
    float mu = 0.f;
    for (int c = 0; c < DH; ++c) mu += x[c];
    mu *= 1.f / DH;
    float var = 0.f;
    for (int c = 0; c < DH; ++c) {
      const float t = x[c] - mu;
      var += t * t;
    }
    var *= 1.f / DH;
    const float inv = 1.f / sqrtf(var + eps);
    for (int c = 0; c < DH; ++c) x[c] = gamma[c] * (x[c] - mu) * inv + beta[c];
  }
}

// --------------------------------------------------------------------------
// kernel 1: chunk scan (state update + snapshots)
// --------------------------------------------------------------------------

template <typename T, int DH, int C, bool PREMAP>
__global__ __launch_bounds__(256) void scan_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                   const float* __restrict__ gamma_k,
                                                   const float* __restrict__ beta_k, float ln_eps,
                                                   const float* __restrict__ state_in,
                                                   float* __restrict__ state_out,
                                                   typename FragStore<T>::type* __restrict__ snap,
                                                   int Hkv, int N, int nchunks) {
  typedef typename FragStore<T>::type ST;
  constexpr bool BF = IsBf16<T>::value;
  constexpr int KB = n_kblocks(DH);
  constexpr int NQ = nq_kblocks(DH);
  constexpr int NL = nl_kblocks(DH);
  constexpr int MT = 2 * KB;          // 16-feature M tiles
  constexpr int KROWS = 32 * NL;      // dims, the ones row (index DH), zeros
  constexpr int CP = C + 4;           // fp32 row stride of kT
  constexpr int VP = C + 8;           // row stride of vT (16-byte multiple)
  constexpr long D = packed_features(DH);
  constexpr long SF = D * NCOL;
  constexpr int ZROW = KROWS - 1;     // always zero

  __shared__ float kT[KROWS * CP];    // transposed keys (+ ones row)
  __shared__ ST vT[DV * VP];          // transposed values
  __shared__ float kraw[C * (DH + 1)];  // row-major staging for the pre-map

  const int bh = blockIdx.y;
  const int kvh = bh % Hkv;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const int mt = blockIdx.x * 4 + wave;
  const bool active = mt < MT;
  const int kb = active ? mt / 2 : 0, half = mt % 2;

  // the feature owned by this lane's A row: kT[r_row] * kT[t_row]
  int r_row = ZROW, t_row = ZROW;
  if (active) {
    if (kb < NQ) {
      int rb, tb;
      pair_of(DH, 2 * kb + half, rb, tb);
      if (rb >= 0) {
        r_row = 4 * rb + l16 / 4;
        t_row = 4 * tb + l16 % 4;
      }
    } else {
      const int u = 32 * (kb - NQ) + 16 * half + l16;
      r_row = u < KROWS ? u : ZROW;
      t_row = DH;  // the ones row
    }
  }

  // initial state (ABI layout) -> accumulators
  f32x4 acc[5];
#pragma unroll
  for (int nt = 0; nt < 5; ++nt) acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const long sbase = (long)bh * SF;
  if (active && state_in != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool canon;
      const long f = abi_feature(DH, kb, 16 * half + 4 * lg + e, canon);
      if (f < 0) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt][e] = state_in[sbase + f * DV + 16 * nt + l16];
      if (l16 == 0) acc[4][e] = state_in[sbase + D * DV + f];
    }
  }

  const T* kb_ptr = k + (long)bh * N * DH;
  const T* vb_ptr = v + (long)bh * N * DV;

  for (int c = 0; c < nchunks; ++c) {
    // snapshot S_c (state before chunk c) in the internal layout
    if (active) {
      ST* sp = snap + (((long)c * gridDim.y + bh) * KB + kb) * NCOL * 32 + 16 * half + 4 * lg;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) store4(sp + (16 * nt + l16) * 32, acc[nt]);
      if (l16 == 0) store4(sp + DV * 32, acc[4]);
    }

    // stage K_c (transposed, + ones row) and V_c (transposed)
    const int j0 = c * C;
    const int nvalid = min(C, N - j0);
    if (PREMAP) {
      stage_rows_f32<T, DH>(kb_ptr, j0, C, N, kraw, DH + 1);
      __syncthreads();
      premap_rows<DH>(kraw, DH + 1, C, nvalid, gamma_k + kvh * DH, beta_k + kvh * DH, ln_eps);
      __syncthreads();
      for (int idx = threadIdx.x; idx < KROWS * C; idx += blockDim.x) {
        const int rr = idx / C, jj = idx % C;
        float val = 0.f;
        if (rr < DH) val = kraw[jj * (DH + 1) + rr];
        else if (rr == DH) val = jj < nvalid ? 1.f : 0.f;
        kT[rr * CP + jj] = val;
      }
    } else {
      // rows > DH stay zero from the first chunk on
      for (int idx = threadIdx.x; idx < C * DH; idx += blockDim.x) {
        const int jj = idx / DH, rr = idx % DH;
        kT[rr * CP + jj] = jj < nvalid ? to_f32(kb_ptr[(long)(j0 + jj) * DH + rr]) : 0.f;
      }
      for (int jj = threadIdx.x; jj < C; jj += blockDim.x) kT[DH * CP + jj] = jj < nvalid ? 1.f : 0.f;
      if (c == 0)
        for (int idx = threadIdx.x; idx < (KROWS - DH - 1) * C; idx += blockDim.x)
          kT[(DH + 1 + idx / C) * CP + idx % C] = 0.f;
    }
    for (int idx = threadIdx.x; idx < DV * C; idx += blockDim.x) {
      const int nn = idx % DV, jj = idx / DV;
      ST val = ST(0);
      if (jj < nvalid) val = vb_ptr[(long)(j0 + jj) * DV + nn];
      vT[nn * VP + jj] = val;
    }
    __syncthreads();

    if (active) {
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        const int jb = 32 * ks + 8 * lg;
        float av[8];
        {
          const float4* pr = reinterpret_cast<const float4*>(&kT[r_row * CP + jb]);
          const float4* pt = reinterpret_cast<const float4*>(&kT[t_row * CP + jb]);
          const float4 r0 = pr[0], r1 = pr[1], t0 = pt[0], t1 = pt[1];
          av[0] = r0.x * t0.x; av[1] = r0.y * t0.y; av[2] = r0.z * t0.z; av[3] = r0.w * t0.w;
          av[4] = r1.x * t1.x; av[5] = r1.y * t1.y; av[6] = r1.z * t1.z; av[7] = r1.w * t1.w;
        }
        float ones[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ones[e] = l16 == 0 ? kT[DH * CP + jb + e] : 0.f;
        const Frag<BF> O1 = frag_from<BF>(ones);
        const Frag<BF> A = frag_from<BF>(av);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) mma(acc[nt], A, frag_load(&vT[(16 * nt + l16) * VP + jb]));
        mma(acc[4], A, O1);
        if constexpr (BF) {
          // a product of two bf16 values has at most 16 significant bits, so
          // hi + lo (both bf16) carries it exactly: the update is then exact
          // up to fp32 accumulation, like the fp32 path.
          float lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) lo[e] = av[e] - (float)A.v[e];
          const Frag<BF> Al = frag_from<BF>(lo);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) mma(acc[nt], Al, frag_load(&vT[(16 * nt + l16) * VP + jb]));
          mma(acc[4], Al, O1);
        }
      }
    }
    __syncthreads();
  }

  // final state -> ABI layout (each packed entry written once)
  if (active && state_out != nullptr) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bool canon;
      const long f = abi_feature(DH, kb, 16 * half + 4 * lg + e, canon);
      if (f < 0 || !canon) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) state_out[sbase + f * DV + 16 * nt + l16] = acc[nt][e];
      if (l16 == 0) state_out[sbase + D * DV + f] = acc[4][e];
    }
  }
}

// --------------------------------------------------------------------------
// kernel 2: chunk readout + intra-chunk block + normalisation
// --------------------------------------------------------------------------

template <typename T, int DH, int C, int NG, bool PREMAP>
__global__ __launch_bounds__(256) void out_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ group_of_dim, const float* __restrict__ ca,
    const float* __restrict__ cb, const float* __restrict__ cc, int G,
    const float* __restrict__ gamma_q, const float* __restrict__ beta_q,
    const float* __restrict__ gamma_k, const float* __restrict__ beta_k, float ln_eps,
    const typename FragStore<T>::type* __restrict__ snap, T* __restrict__ y, int Hq, int Hkv,
    int N, int nchunks) {
  typedef typename FragStore<T>::type ST;
  constexpr bool BF = IsBf16<T>::value;
  constexpr int KB = n_kblocks(DH);
  constexpr int NQ = nq_kblocks(DH);
  constexpr int NL = nl_kblocks(DH);
  constexpr int QS = 32 * NL + 4;           // fp32 q-hat row stride
  constexpr int ZQ = 32 * NL - 4;           // 4 zero entries of every q-hat row
  constexpr int DS = DH < 32 ? 32 : DH;     // score K depth (padded to 32)
  constexpr int STEPS = DS / 32;
  constexpr int DP = DS + 8;                // row stride of qi/ki
  constexpr int VP = C + 8;
  constexpr int RS = 84;                    // row stride of the reduction buffer
  constexpr int T16 = C / 16;               // 16-token tiles per chunk

  __shared__ float qh[C * QS];
  __shared__ float coef[KB * 32];
  __shared__ ST qi[C * DP];
  __shared__ ST ki[C * DP];
  __shared__ ST vT[DV * VP];
  __shared__ float red[C * RS];
  __shared__ float kst[C * (DH + 1)];
  __shared__ int gm[DH];
  __shared__ float pc[1 + NG + NG * NG];   // a, b_g/sqrt(d), sym(c)_gh/d
  __shared__ int bad;

  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int rep = Hq / Hkv;
  const int kvh = h / rep;
  const int bh = b * Hkv + kvh;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const int j0 = c * C;
  const int nvalid = min(C, N - j0);
  const float inv_sqrt_d = 1.f / sqrtf((float)DH);

  // ---- prologue: coefficients of this query head (row a2) ----
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int r = threadIdx.x; r < DH; r += blockDim.x) {
    const int g = group_of_dim[h * DH + r];
    gm[r] = g;
    if (g < 0 || g >= G) atomicOr(&bad, 1);
  }
  for (int idx = threadIdx.x; idx < 1 + NG + NG * NG; idx += blockDim.x) {
    float val = 0.f;
    if (idx == 0) {
      val = ca[h];
    } else if (idx <= NG) {
      const int g = idx - 1;
      val = g < G ? cb[h * G + g] * inv_sqrt_d : 0.f;
    } else {
      const int gh = idx - 1 - NG, g = gh / NG, hh = gh % NG;
      val = (g < G && hh < G) ? 0.5f * (cc[(h * G + g) * G + hh] + cc[(h * G + hh) * G + g]) / DH : 0.f;
    }
    pc[idx] = val;
  }
  __syncthreads();
  // phi_q coefficient of every internal feature
  for (int idx = threadIdx.x; idx < KB * 32; idx += blockDim.x) {
    const int kbi = idx / 32, kk = idx % 32;
    float val = 0.f;
    if (!bad) {
      if (kbi < NQ) {
        int rb, tb;
        pair_of(DH, 2 * kbi + kk / 16, rb, tb);
        if (rb >= 0) {
          const int r = 4 * rb + (kk % 16) / 4, t = 4 * tb + kk % 4;
          const float m = rb < tb ? 2.f : 1.f;
          val = m * pc[1 + NG + gm[r] * NG + gm[t]];
        }
      } else {
        const int u = 32 * (kbi - NQ) + kk;
        if (u < DH) val = pc[1 + gm[u]];
        else if (u == DH) val = pc[0];
      }
    }
    coef[idx] = val;
  }

  // ---- stage Q_c, K_c, V_c ----
  const T* qp = q + ((long)(b * Hq + h) * N) * DH;
  const T* kp = k + ((long)bh * N) * DH;
  const T* vp = v + ((long)bh * N) * DV;
  stage_rows_f32<T, DH>(qp, j0, C, N, kst, DH + 1);
  __syncthreads();
  if (PREMAP) {
    premap_rows<DH>(kst, DH + 1, C, nvalid, gamma_q + h * DH, beta_q + h * DH, ln_eps);
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < C * QS; idx += blockDim.x) {
    const int ii = idx / QS, cc2 = idx % QS;
    float val = 0.f;
    if (ii < nvalid) {
      if (cc2 < DH) val = kst[ii * (DH + 1) + cc2];
      else if (cc2 == DH) val = 1.f;
    }
    qh[idx] = val;
  }
  for (int idx = threadIdx.x; idx < C * DP; idx += blockDim.x) {
    const int ii = idx / DP, cc2 = idx % DP;
    const float val = (ii < nvalid && cc2 < DH) ? kst[ii * (DH + 1) + cc2] : 0.f;
    if constexpr (BF) qi[idx] = bf16_bits(val);
    else qi[idx] = val;
  }
  __syncthreads();
  stage_rows_f32<T, DH>(kp, j0, C, N, kst, DH + 1);
  __syncthreads();
  if (PREMAP) {
    premap_rows<DH>(kst, DH + 1, C, nvalid, gamma_k + kvh * DH, beta_k + kvh * DH, ln_eps);
    __syncthreads();
  }
  for (int idx = threadIdx.x; idx < C * DP; idx += blockDim.x) {
    const int ii = idx / DP, cc2 = idx % DP;
    const float val = (ii < nvalid && cc2 < DH) ? kst[ii * (DH + 1) + cc2] : 0.f;
    if constexpr (BF) ki[idx] = bf16_bits(val);
    else ki[idx] = val;
  }
  for (int idx = threadIdx.x; idx < DV * C; idx += blockDim.x) {
    const int nn = idx % DV, jj = idx / DV;
    ST val = ST(0);
    if (jj < nvalid) val = vp[(long)(j0 + jj) * DV + nn];
    vT[nn * VP + jj] = val;
  }
  __syncthreads();

  // ---- inter-chunk read: phi_q(Q_c) . S_c, K split over the four waves ----
  f32x4 acc[T16][5];
#pragma unroll
  for (int mt = 0; mt < T16; ++mt)
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const ST* sbase = snap + ((long)c * gridDim.z * Hkv + bh) * KB * NCOL * 32;
  const int kb_lo = (KB * wave) / 4, kb_hi = (KB * (wave + 1)) / 4;
  for (int kbi = kb_lo; kbi < kb_hi; ++kbi) {
    const ST* sp = sbase + (long)kbi * NCOL * 32 + 8 * lg;
    Frag<BF> Bf[5];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) Bf[nt] = frag_load(sp + (16 * nt + l16) * 32);
    Bf[4] = l16 == 0 ? frag_load(sp + DV * 32) : frag_zero<BF>();
    float cf[8];
    {
      const float4 c0 = *reinterpret_cast<const float4*>(&coef[kbi * 32 + 8 * lg]);
      const float4 c1 = *reinterpret_cast<const float4*>(&coef[kbi * 32 + 8 * lg + 4]);
      cf[0] = c0.x; cf[1] = c0.y; cf[2] = c0.z; cf[3] = c0.w;
      cf[4] = c1.x; cf[5] = c1.y; cf[6] = c1.z; cf[7] = c1.w;
    }
    if (kbi < NQ) {
      int rb, tb;
      pair_of(DH, 2 * kbi + lg / 2, rb, tb);
      const int ra = rb >= 0 ? 4 * rb + 2 * (lg % 2) : ZQ;
      const int t0 = rb >= 0 ? 4 * tb : ZQ;
#pragma unroll
      for (int mt = 0; mt < T16; ++mt) {
        const float* row = &qh[(16 * mt + l16) * QS];
        const float2 rp = *reinterpret_cast<const float2*>(row + ra);
        const float4 tq = *reinterpret_cast<const float4*>(row + t0);
        float f[8];
        f[0] = rp.x * tq.x * cf[0]; f[1] = rp.x * tq.y * cf[1];
        f[2] = rp.x * tq.z * cf[2]; f[3] = rp.x * tq.w * cf[3];
        f[4] = rp.y * tq.x * cf[4]; f[5] = rp.y * tq.y * cf[5];
        f[6] = rp.y * tq.z * cf[6]; f[7] = rp.y * tq.w * cf[7];
        const Frag<BF> A = frag_from<BF>(f);
#pragma unroll
        for (int nt = 0; nt < 5; ++nt) mma(acc[mt][nt], A, Bf[nt]);
      }
    } else {
      const int u0 = 32 * (kbi - NQ) + 8 * lg;
#pragma unroll
      for (int mt = 0; mt < T16; ++mt) {
        const float* row = &qh[(16 * mt + l16) * QS + u0];
        const float4 x0 = *reinterpret_cast<const float4*>(row);
        const float4 x1 = *reinterpret_cast<const float4*>(row + 4);
        float f[8];
        f[0] = x0.x * cf[0]; f[1] = x0.y * cf[1]; f[2] = x0.z * cf[2]; f[3] = x0.w * cf[3];
        f[4] = x1.x * cf[4]; f[5] = x1.y * cf[5]; f[6] = x1.z * cf[6]; f[7] = x1.w * cf[7];
        const Frag<BF> A = frag_from<BF>(f);
#pragma unroll
        for (int nt = 0; nt < 5; ++nt) mma(acc[mt][nt], A, Bf[nt]);
      }
    }
  }

  // ---- reduce the four partial reads in LDS (fixed order: deterministic) ----
  for (int w = 0; w < 4; ++w) {
    if (wave == w) {
#pragma unroll
      for (int mt = 0; mt < T16; ++mt)
#pragma unroll
        for (int nt = 0; nt < 5; ++nt) {
          const int col = 16 * nt + l16;
          if (col >= NCOL) continue;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float* dst = &red[(16 * mt + 4 * lg + e) * RS + col];
            *dst = (w == 0 ? 0.f : *dst) + acc[mt][nt][e];
          }
        }
    }
    __syncthreads();
  }

  // ---- intra-chunk block ----
  // group masks of this lane's score dims (32 s + 8 lg + e)
  int gid[STEPS][8];
#pragma unroll
  for (int s = 0; s < STEPS; ++s)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int dd = 32 * s + 8 * lg + e;
      gid[s][e] = dd < DH ? gm[dd] : -1;
    }
  float pcr[1 + NG + NG * NG];
#pragma unroll
  for (int i2 = 0; i2 < 1 + NG + NG * NG; ++i2) pcr[i2] = pc[i2];

  for (int pass = 0; pass < 2; ++pass) {
    int it;
    if (T16 == 8) it = pass == 0 ? wave : 7 - wave;
    else it = pass == 0 ? wave : -1;
    if (it < 0 || it >= T16) continue;
    const int irow = 16 * it + l16;  // query row (N index of the scores)
    // masked query fragments per group
    Frag<BF> Bq[NG][STEPS];
#pragma unroll
    for (int s = 0; s < STEPS; ++s) {
      float base[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (BF) base[e] = to_f32(qi[irow * DP + 32 * s + 8 * lg + e]);
        else base[e] = qi[irow * DP + 32 * s + 8 * lg + e];
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float mv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) mv[e] = gid[s][e] == g ? base[e] : 0.f;
        Bq[g][s] = frag_from<BF>(mv);
      }
    }
    f32x4 iacc[5];
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) iacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int jt0 = 0; jt0 <= it; jt0 += 2) {
      float p[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jt = jt0 + hh;
        if (jt > it) {
#pragma unroll
          for (int e = 0; e < 4; ++e) p[4 * hh + e] = 0.f;
          continue;
        }
        Frag<BF> Ak[STEPS];
#pragma unroll
        for (int s = 0; s < STEPS; ++s) Ak[s] = frag_load(&ki[(16 * jt + l16) * DP + 32 * s + 8 * lg]);
        f32x4 sg[NG];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          sg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < STEPS; ++s) mma(sg[g], Ak[s], Bq[g][s]);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // kappa = a + sum_g s_g (b_g + c_gg s_g + 2 sum_{h>g} c_gh s_h)
          float kap = pcr[0];
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            float inner = pcr[1 + g] + pcr[1 + NG + g * NG + g] * sg[g][e];
#pragma unroll
            for (int hg = g + 1; hg < NG; ++hg) inner += 2.f * pcr[1 + NG + g * NG + hg] * sg[hg][e];
            kap += sg[g][e] * inner;
          }
          const int jrow = 16 * jt + 4 * lg + e;  // key row (M index)
          p[4 * hh + e] = (jt == it && jrow > irow) ? 0.f : kap;
        }
      }
      const Frag<BF> A = frag_from<BF>(p);
      const int ja = 16 * jt0 + 4 * lg, jb = ja + 16;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const ST* vr = &vT[(16 * nt + l16) * VP];
        float vb[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (BF) {
            vb[e] = to_f32(vr[ja + e]);
            vb[4 + e] = to_f32(vr[jb + e]);
          } else {
            vb[e] = vr[ja + e];
            vb[4 + e] = vr[jb + e];
          }
        }
        mma(iacc[nt], A, frag_from<BF>(vb));
      }
      float ones[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ones[e] = l16 == 0 ? 1.f : 0.f;
      mma(iacc[4], A, frag_from<BF>(ones));
    }
    // rows of tile `it` belong to this wave alone
#pragma unroll
    for (int nt = 0; nt < 5; ++nt) {
      const int col = 16 * nt + l16;
      if (col >= NCOL) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) red[(16 * it + 4 * lg + e) * RS + col] += iacc[nt][e];
    }
  }
  __syncthreads();

  // ---- normalise and store ----
  T* yp = y + ((long)(b * Hq + h) * N + j0) * DV;
  const float nanv = __builtin_nanf("");
  for (int idx = threadIdx.x; idx < nvalid * DV; idx += blockDim.x) {
    const int ii = idx / DV, nn = idx % DV;
    const float val = bad ? nanv : red[ii * RS + nn] / red[ii * RS + DV];
    store_elem(&yp[(long)ii * DV + nn], val);
  }
}

// --------------------------------------------------------------------------
// host launchers
// --------------------------------------------------------------------------

template <typename T, int DH, int C>
static hipError_t launch_fwd_t(const FwdLaunch& a, int stages, hipStream_t stream) {
  typedef typename FragStore<T>::type ST;
  const int nchunks = (a.N + C - 1) / C;
  const int BH = a.B * a.Hkv;
  constexpr int MT = 2 * n_kblocks(DH);
  ST* snap = reinterpret_cast<ST*>(a.workspace);
  const T* qq = reinterpret_cast<const T*>(a.q);
  const T* kk = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  T* yy = reinterpret_cast<T*>(a.y);
  if (stages & 1) {
    dim3 grid((MT + 3) / 4, BH);
    if (a.premap)
      hipLaunchKernelGGL((scan_kernel<T, DH, C, true>), grid, dim3(256), 0, stream, kk, vv, a.gamma_k,
                         a.beta_k, a.ln_eps, a.state_in, a.state_out, snap, a.Hkv, a.N, nchunks);
    else
      hipLaunchKernelGGL((scan_kernel<T, DH, C, false>), grid, dim3(256), 0, stream, kk, vv, nullptr,
                         nullptr, 0.f, a.state_in, a.state_out, snap, a.Hkv, a.N, nchunks);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(stages & 2)) return hipSuccess;
  dim3 grid(nchunks, a.Hq, a.B);
#define OAL_OUT(NGV, PM)                                                                              \
  hipLaunchKernelGGL((out_kernel<T, DH, C, NGV, PM>), grid, dim3(256), 0, stream, qq, kk, vv,         \
                     a.group_of_dim, a.ca, a.cb, a.cc, a.G, a.gamma_q, a.beta_q, a.gamma_k, a.beta_k, \
                     a.ln_eps, snap, yy, a.Hq, a.Hkv, a.N, nchunks)
  const int ng = a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : 8;
  if (a.premap) {
    switch (ng) {
      case 1: OAL_OUT(1, true); break;
      case 2: OAL_OUT(2, true); break;
      case 4: OAL_OUT(4, true); break;
      default: OAL_OUT(8, true); break;
    }
  } else {
    switch (ng) {
      case 1: OAL_OUT(1, false); break;
      case 2: OAL_OUT(2, false); break;
      case 4: OAL_OUT(4, false); break;
      default: OAL_OUT(8, false); break;
    }
  }
#undef OAL_OUT
  return hipGetLastError();
}

// state_out <- state_in (or zeros) for an empty sequence; a plain kernel so
// that callers may capture it in a graph.
__global__ void state_passthrough_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_passthrough(const float* src, float* dst, long n, hipStream_t stream) {
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(state_passthrough_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, src, dst, n);
  return hipGetLastError();
}

size_t fwd_workspace_bytes(int B, int Hkv, int N, int d_h, int dtype) {
  const int C = kChunk;
  const long nchunks = (N + C - 1) / C;
  const size_t elem = dtype == 1 ? 2 : 4;
  return (size_t)nchunks * B * Hkv * snap_elems(d_h, DV) * elem;
}

hipError_t launch_fwd(const FwdLaunch& a, int stages, hipStream_t stream) {
  if (a.dtype == 1) {
    switch (a.d_h) {
      case 16: return launch_fwd_t<uint16_t, 16, kChunk>(a, stages, stream);
      case 32: return launch_fwd_t<uint16_t, 32, kChunk>(a, stages, stream);
      default: return launch_fwd_t<uint16_t, 64, kChunk>(a, stages, stream);
    }
  }
  switch (a.d_h) {
    case 16: return launch_fwd_t<float, 16, kChunk>(a, stages, stream);
    case 32: return launch_fwd_t<float, 32, kChunk>(a, stages, stream);
    default: return launch_fwd_t<float, 64, kChunk>(a, stages, stream);
  }
}

}  // namespace oal
