// Chunked causal prefill for OAL attention on gfx950 (kernels; instantiated
// per head dimension by oal_prefill_d16/32/64.hip).
//
// The prefix sum of the OAL paper's Eq. (6) is split at chunk starts: for a
// query i in chunk c,
//     u~_i = phi_q(q_i)^T S_c + sum_{j in c, j <= i} kappa(q_i, k_j) [v_j, 1]
// with S_c the state of Eq. (5) accumulated over all tokens before chunk c.
// The second term is the direct pairwise form of the paper's sec. 4.4,
// restricted to one chunk.
//
// Kernel 1 (scan): one CTA per (four K-blocks of features, batch x KV head)
// walks the chunks in order.  Each wave keeps one K-block of S (32 features x
// 65 columns) in fp32 MFMA accumulators, writes it to the chunk's snapshot
// at every chunk start and adds S += phi_k(K_c)^T [V_c | 1] on MFMA.
//
// Kernel 2 (readout): one CTA per (chunk, batch x KV head) serves every
// query head of that KV head (GQA): the snapshot S_c is staged through LDS
// one K-block pair at a time and read by all heads, so it leaves HBM once
// per chunk.  Wave w owns rows 16w..16w+15 of the chunk for all heads.  It
// builds phi_q for its rows on the fly (two multiplies per feature pair in
// packed fp16), reads phi_q . S_c on MFMA, adds the within-chunk pairs
// (group score tiles on MFMA, the grouped polynomial and causal mask in
// registers, P . [V | 1] on MFMA) and normalises.
//
// Number formats.  For bf16 activations the features and the snapshots are
// fp16 and every product accumulates in fp32; fp32 activations use fp32
// MFMA throughout.  fp16 needs scaling, all by powers of two so that it is
// exact bookkeeping:
//  * scan: keys and values of a chunk are divided by 2^Ek and 2^Ev, running
//    maxima of the chunk exponents (|k_hat|, |v_hat| <= 1); the accumulators
//    hold S in those units and are rescaled when an exponent grows;
//  * snapshot: each K-block is further divided by 2^beta with beta from its
//    largest entry, so the stored values stay below 2^15;
//  * readout: q rows are divided by 2^f (f from the row maximum), the
//    coefficients by 2^c_h, and the per-K-block factors are folded into the
//    generated feature values relative to the largest K-block, so every
//    fp16 operand is at most 2^15.  Linear-feature K-blocks run first and
//    their partial sums are rescaled once before the quadratic K-blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

namespace {

constexpr int DV = 64;        // value head dimension handled by these kernels
constexpr int NCOL = DV + 1;  // value columns + normaliser column
constexpr int C = kChunk;     // tokens per chunk
// LDS column pitch (elements) of a staged snapshot K-block: 80 bytes (fp16)
// or 144 bytes (fp32), so that 16 lanes reading 16 bytes each hit distinct banks
// Snapshot K-blocks the readout stages per pipeline step: two, or three for
// fp16 snapshots read by a single head slot per pass.  There a two-block
// stage is 8 KB, so the per-stage wait and barrier rather than the bytes set
// the pace; three blocks still leave room for two workgroups per compute unit.
__host__ __device__ constexpr int stage_kblocks(int rmax, int esize) { return rmax == 1 && esize == 2 ? 3 : 2; }
// Elements of one staged group of kg snapshot K-blocks in LDS: kg value
// blocks of 64 columns x 32 features, then kg z blocks of 32.
__host__ __device__ constexpr int stage_elems(int kg) {
  return kg * (DV * 32 + 32);
}
constexpr int kNegExp = -200; // exponent of an all-zero block

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));

// ---- compute element of the feature GEMMs per activation type ----
template <typename T>
struct Cx;
template <>
struct Cx<uint16_t> {  // bf16 activations: fp16 features and snapshots
  typedef _Float16 E;
  struct Frag {
    h8 v;
  };
};
template <>
struct Cx<float> {  // fp32 activations: fp32 throughout
  typedef float E;
  struct Frag {
    float v[8];
  };
};

__device__ __forceinline__ void mma(f32x4& acc, const Cx<uint16_t>::Frag& a, const Cx<uint16_t>::Frag& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Cx<float>::Frag& a, const Cx<float>::Frag& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

__device__ __forceinline__ void frag_zero(Cx<uint16_t>::Frag& f) {
  f.v = h8{0, 0, 0, 0, 0, 0, 0, 0};
}
__device__ __forceinline__ void frag_zero(Cx<float>::Frag& f) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = 0.f;
}
__device__ __forceinline__ void frag_ones_if(Cx<uint16_t>::Frag& f, bool on) {
  const _Float16 x = on ? (_Float16)1.f : (_Float16)0.f;
  f.v = h8{x, x, x, x, x, x, x, x};
}
__device__ __forceinline__ void frag_ones_if(Cx<float>::Frag& f, bool on) {
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = on ? 1.f : 0.f;
}
// eight consecutive elements (16-byte aligned for fp16, 32-byte for fp32)
__device__ __forceinline__ void frag_ld(Cx<uint16_t>::Frag& f, const _Float16* p) {
  f.v = *reinterpret_cast<const h8*>(p);
}
__device__ __forceinline__ void frag_ld(Cx<float>::Frag& f, const float* p) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}
__device__ __forceinline__ void frag_st(_Float16* p, const float (&x)[8]) {
  h8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (_Float16)x[e];
  *reinterpret_cast<h8*>(p) = v;
}
__device__ __forceinline__ void frag_st(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// x, hidden from the optimiser when ON (an empty asm that "modifies" it), so
// that values derived from it are recomputed where they are used instead of
// being hoisted and kept live in registers.
template <bool ON>
__device__ __forceinline__ int opaque(int x) {
  if constexpr (ON) asm volatile("" : "+v"(x));
  return x;
}

// The lane's index within its wave, recomputed from the hardware (bit count
// of a full mask below the lane) where it is used: a volatile asm is neither
// hoisted nor merged, so no register holds the index in between.
__device__ __forceinline__ int lane_now() {
  int x;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
  return x;
}

// s_waitcnt immediate that waits for vector-memory count <= n (other counters
// untouched): vmcnt in bits 3:0 and 15:14, expcnt 6:4 = 7, lgkmcnt 11:8 = 15.
template <int n>
constexpr int kWaitVm = (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8);
// ... and, in the same instruction, for every LDS operation (lgkmcnt = 0)
template <int n>
constexpr int kWaitVmLds = (n & 15) | ((n >> 4) << 14) | (7 << 4);

// Workgroup barrier for LDS producer/consumer steps whose global-to-LDS
// loads are waited for explicitly: the wait (vector-memory count <= N, all
// LDS operations done) precedes the barrier, and the empty asm with a memory
// clobber keeps the compiler from moving memory operations across it (a
// __syncthreads() would also wait for the loads of later stages).
template <int N>
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kWaitVmLds<N>);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---- power-of-two helpers ----
// e with |x| < 2^e for x != 0 (kNegExp for zero or non-finite maxima)
__device__ __forceinline__ int exp_above(float m) {
  if (!(m > 0.f) || !(m < 3.0e38f)) return m > 0.f ? 128 : kNegExp;
  int e;
  frexpf(m, &e);
  return e;
}
__device__ __forceinline__ float pow2(int e) { return ldexpf(1.f, e); }


// n consecutive activations (n a multiple of 4) starting at p -> floats
template <int n>
__device__ __forceinline__ void load_vals(const uint16_t* p, float* out) {
#pragma unroll
  for (int i = 0; i < n; i += 8) {
    if (n - i >= 8) {
      const uint4 w = *reinterpret_cast<const uint4*>(p + i);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        out[i + 2 * j] = __uint_as_float(ws[j] << 16);
        out[i + 2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
      }
    } else {
      const uint2 w = *reinterpret_cast<const uint2*>(p + i);
      out[i] = __uint_as_float(w.x << 16);
      out[i + 1] = __uint_as_float(w.x & 0xffff0000u);
      out[i + 2] = __uint_as_float(w.y << 16);
      out[i + 3] = __uint_as_float(w.y & 0xffff0000u);
    }
  }
}
template <int n>
__device__ __forceinline__ void load_vals(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < n; i += 4) {
    const float4 w = *reinterpret_cast<const float4*>(p + i);
    out[i] = w.x; out[i + 1] = w.y; out[i + 2] = w.z; out[i + 3] = w.w;
  }
}

// Pre-map (normalisation of kind pn, then the affine) of a row split over 4
// consecutive lanes, each holding n values at dimension offset d0.
template <int DH, int n>
__device__ __forceinline__ void premap4(float* x, int d0, const float* __restrict__ gamma,
                                        const float* __restrict__ beta, float eps, PremapNorm pn) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) s += x[i];
  s = quad_sum(s);
  const float mu = s * pn.mean_w;
  float v2 = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) {
    const float t = x[i] - mu;
    v2 += t * t;
  }
  v2 = quad_sum(v2);
  const float inv = 1.f / sqrtf(v2 * pn.var_w + eps);
#pragma unroll
  for (int i = 0; i < n; ++i) x[i] = gamma[d0 + i] * (x[i] - mu) * inv + beta[d0 + i];
}

}  // namespace

// --------------------------------------------------------------------------
// kernel 1: chunk scan (state update + snapshots)
// --------------------------------------------------------------------------

// One CTA per (NCW K-blocks, batch x KV head), twelve waves in two roles:
//  * compute waves 0..NCW-1 (NCW = 4 or 8): wave w keeps K-block
//    NCW blockIdx.x + w of S in fp32 MFMA accumulators (the wave after the
//    last K-block keeps the constant feature's row [sum v, n]); per chunk it
//    writes the snapshot S_c and adds phi_k(K_c)^T [V_c | 1].  They issue
//    only stores to global memory.
//  * loader waves: the first half keys, the second half values; they load
//    chunks ahead, reduce the chunk maxima that set the scaling exponents,
//    apply the pre-map, and write the scaled tiles transposed into LDS
//    (double-buffered).  They issue only loads, so their waits never cover
//    the snapshot stores.
// One barrier per chunk separates staging chunk c+1 from reading chunk c.
// NCW = 4 keeps the MFMA work per SIMD and chunk at one K-block and splits
// the staging eight ways; it takes twice the CTAs of NCW = 8, which the host
// picks when the NCW = 4 grid would not fit on the compute units at once.
constexpr int kScanWaves = 12;

// Eight consecutive activations of one row, as loaded.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
  uint4 w;
};
template <>
struct Raw8<float> {
  float4 a, b;
};
__device__ __forceinline__ void ld8(Raw8<uint16_t>& r, const uint16_t* p) { r.w = *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void ld8(Raw8<float>& r, const float* p) {
  r.a = reinterpret_cast<const float4*>(p)[0];
  r.b = reinterpret_cast<const float4*>(p)[1];
}
__device__ __forceinline__ void zero8(Raw8<uint16_t>& r) { r.w = make_uint4(0u, 0u, 0u, 0u); }
__device__ __forceinline__ void zero8(Raw8<float>& r) {
  r.a = make_float4(0.f, 0.f, 0.f, 0.f);
  r.b = r.a;
}
__device__ __forceinline__ void unpack8(const Raw8<uint16_t>& r, float (&x)[8]) {
  const uint32_t ws[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(ws[j] << 16);
    x[2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float (&x)[8]) {
  x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
  x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
}

// Chunk exponents (one CTA per chunk and batch x KV head): ek, ev with
// |k| < 2^ek over the chunk's keys (after the pre-map) and |v| < 2^ev over its
// values (kNegExp for all zeros).  The scan reads them from this table
// instead of every CTA of a sequence reducing the same chunk maxima.
template <typename T, int DH, bool PREMAP>
__global__ __launch_bounds__(256) void chunk_exp_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                        const float* __restrict__ gamma_k,
                                                        const float* __restrict__ beta_k, float ln_eps,
                                                        PremapNorm pn, int2* __restrict__ kvexp, int Hkv, int N,
                                                        int nchunks, const int32_t* __restrict__ seq_lens) {
  constexpr int QD = DH / 4, QV = DV / 4;
  __shared__ float wm[2][4];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int kvh = bh % Hkv;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int srow = tid / 4, sq = tid % 4;  // token of the chunk, quarter of its dimensions
  const int row = c * C + srow;
  const bool valid = row < seq_len_of(seq_lens, bh / Hkv, N);  // rows of the sequence (stride N)
  float kx[QD], vx[QV];
#pragma unroll
  for (int i = 0; i < QD; ++i) kx[i] = 0.f;
#pragma unroll
  for (int i = 0; i < QV; ++i) vx[i] = 0.f;
  if (valid) {
    load_vals<QD>(k + ((long)bh * N + row) * DH + sq * QD, kx);
    load_vals<QV>(v + ((long)bh * N + row) * DV + sq * QV, vx);
  }
  if (PREMAP) {
    premap4<DH, QD>(kx, sq * QD, gamma_k + kvh * DH, beta_k + kvh * DH, ln_eps, pn);
    if (!valid)
#pragma unroll
      for (int i = 0; i < QD; ++i) kx[i] = 0.f;
  }
  float mk = 0.f, mv = 0.f;
#pragma unroll
  for (int i = 0; i < QD; ++i) mk = fmaxf(mk, fabsf(kx[i]));
#pragma unroll
  for (int i = 0; i < QV; ++i) mv = fmaxf(mv, fabsf(vx[i]));
  mk = wave_max(mk);
  mv = wave_max(mv);
  if (lane == 0) {
    wm[0][wave] = mk;
    wm[1][wave] = mv;
  }
  __syncthreads();
  if (tid == 0) {
    mk = fmaxf(fmaxf(wm[0][0], wm[0][1]), fmaxf(wm[0][2], wm[0][3]));
    mv = fmaxf(fmaxf(wm[1][0], wm[1][1]), fmaxf(wm[1][2], wm[1][3]));
    kvexp[(long)bh * nchunks + c] = make_int2(exp_above(mk), exp_above(mv));
  }
}

template <typename T, int DH, bool PREMAP, int NCW>
__global__ __launch_bounds__(64 * kScanWaves) void scan_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const float* __restrict__ gamma_k,
    const float* __restrict__ beta_k, float ln_eps, PremapNorm pn, const float* __restrict__ state_in,
    float* __restrict__ state_out, typename Cx<T>::E* __restrict__ snap, int* __restrict__ sexp,
    float* __restrict__ sconst, const int2* __restrict__ kvexp, int Hkv, int NS, int nchunks,
    const int32_t* __restrict__ seq_lens) {
  typedef typename Cx<T>::E E;
  typedef typename Cx<T>::Frag F;
  constexpr int KB = n_kblocks(DH);
  constexpr int NQ = nq_kblocks(DH);
  constexpr long D = packed_features(DH);
  constexpr long SF = D * NCOL;
  constexpr int KP = C + 8;                // row pitch of the transposed tiles (elements)
  constexpr int ONE = DH, ZERO = DH + 1;   // rows of ones / zeros after the key rows
  constexpr int VROW = DH + 2;             // first value row
  constexpr int BUF = (DH + 2 + DV) * KP;  // elements per staging buffer
  constexpr int KUL = DH / 16;             // key units (8 dimensions) per loader lane
  constexpr int UL = DV / 16;              // value units per loader lane (>= KUL)
  constexpr int NR = IsBf16<T>::value ? 3 : 2;  // chunks held in loader registers
  constexpr int kScanCompute = NCW;
  constexpr int kScanLoad = kScanWaves - NCW;
  constexpr int LWR = kScanLoad / 2;           // loader waves per role (keys, values)
  constexpr int TPL = 8 / LWR;                 // tokens per loader lane without the pre-map
  static_assert(NCW == 4 || NCW == 8, "four or eight compute waves");
  __shared__ __align__(16) E tile[2][BUF];
  __shared__ float wmx[2][kScanLoad];      // [slot][loader wave]: max |k| (first half), |v| (second half)
  __shared__ float wm_in[kScanCompute];
  __shared__ __align__(16) float gb[2][DH];  // pre-map gamma, beta of the KV head

  const int bh = blockIdx.y, BH = gridDim.y;
  const int kvh = bh % Hkv;
  // rows of this sequence (its own length with seq_lens; the row stride is NS)
  const int N = seq_len_of(seq_lens, bh / Hkv, NS);
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const bool loader = wave >= kScanCompute;
  // compute role
  const int kb = blockIdx.x * kScanCompute + wave;
  const bool active = !loader && kb < KB;  // a K-block of S
  const bool cwave = !loader && kb == KB;  // the constant feature's row
  const int nu = kb < NQ ? 2 : (kb < KB ? 1 : 0);  // key-exponent multiplicity of the wave's features
  const bool lead = blockIdx.x == 0 && tid == 0;
  const long nsnap = (long)nchunks * BH;  // snapshots in the workspace
  // loader role.  With the pre-map: the first two loader waves of each role,
  // token ltok, units lhalf + 2 i (dimensions 8 unit ..), so that a token's
  // statistics stay in two lanes; further loader waves idle.  Without it:
  // tokens TPL tg .. TPL tg + TPL - 1 of unit lu, so that each staged row
  // segment of TPL tokens leaves the lane as one store.
  const int lw = wave - kScanCompute;
  const bool kload = loader && lw < LWR;
  const bool lidle = PREMAP && loader && (lw % LWR) >= 2;
  const int ltok = 32 * ((lw % LWR) & 1) + (lane & 31);
  const int lhalf = lane >> 5;
  const int lsid = 64 * (lw % LWR) + lane;
  const int tg = lsid % (64 / TPL), lu = lsid / (64 / TPL);
  const bool ulive = lu < (kload ? DH : DV) / 8;
  static_assert(UL == 4, "four units per pre-map loader lane");

  if (PREMAP)
    for (int i = tid; i < 2 * DH; i += blockDim.x) gb[i / DH][i % DH] = (i < DH ? gamma_k : beta_k)[kvh * DH + i % DH];

  // A operand (phi_k) rows of this lane: the features of accumulator row l16
  int ar[2], at[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    int r = 0, t = 0, mu = 0;
    if (active && kfeature(DH, kb, acc_position(m, l16), r, t, mu)) {
      ar[m] = r;
      at[m] = t;
    } else if (cwave && m == 0 && l16 == 0) {
      ar[m] = ONE;
      at[m] = ONE;
    } else {
      ar[m] = ZERO;
      at[m] = ZERO;
    }
  }
  f32x4 acc[2][5];
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 5; ++n) acc[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

  const long sbase = (long)bh * SF;
  const T* kp = k + (long)bh * NS * DH;
  const T* vp = v + (long)bh * NS * DV;

  // ---- loader helpers ----
  struct RawSet {
    Raw8<T> u[PREMAP ? UL : TPL];  // units of one token (pre-map) or one unit of TPL tokens
    float mu, inv;                  // pre-map statistics of the token (keys)
  };
  auto fetch = [&](int c) __attribute__((always_inline)) {
    RawSet r;
    // Rows past the sequence end load the last row (in bounds) and are
    // zeroed where the values are used: a select right after the load would
    // make every prefetch wait for its data.
    if constexpr (!PREMAP) {
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const int row = c * C + TPL * tg + i;
        const long rr = row < N ? row : max(N - 1, 0);
        if (ulive) {
          ld8(r.u[i], kload ? kp + rr * DH + 8 * lu : vp + rr * DV + 8 * lu);
        } else {
          zero8(r.u[i]);
        }
      }
      r.mu = 0.f;
      r.inv = 0.f;
      return r;
    }
    const int row = c * C + ltok;
    const long rr = row < N ? row : max(N - 1, 0);
#pragma unroll
    for (int i = 0; i < UL; ++i) {
      const int unit = lhalf + 2 * i;
      if (!lidle && (kload ? i < KUL : true)) {
        ld8(r.u[i], kload ? kp + rr * DH + 8 * unit : vp + rr * DV + 8 * unit);
      } else {
        zero8(r.u[i]);
      }
    }
    r.mu = 0.f;
    r.inv = 0.f;
    return r;
  };
  // values of unit i with the pre-map applied (keys)
  auto values = [&](const RawSet& r, int i, float (&x)[8]) __attribute__((always_inline)) {
    unpack8(r.u[i], x);
    if (PREMAP && kload) {
      const int d0 = 8 * (lhalf + 2 * i);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = gb[0][d0 + e] * (x[e] - r.mu) * r.inv + gb[1][d0 + e];
    }
  };
  // pre-map statistics and this wave's maximum into wmx[slot]
  auto convert = [&](RawSet& r, int c, int slot) __attribute__((always_inline)) {
    if constexpr (!PREMAP) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < TPL; ++i) {
        const bool valid = c * C + TPL * tg + i < N;
        float x[8];
        unpack8(r.u[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) m = fmaxf(m, valid ? fabsf(x[e]) : 0.f);
      }
      m = wave_max(m);
      if (lane == 0) wmx[slot][lw] = m;
      return;
    }
    const bool valid = !lidle && c * C + ltok < N;
    if (PREMAP && kload) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < KUL; ++i) {
        float x[8];
        unpack8(r.u[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) s += x[e];
      }
      s += __shfl_xor(s, 32);
      const float mu = s * pn.mean_w;
      float q2 = 0.f;
#pragma unroll
      for (int i = 0; i < KUL; ++i) {
        float x[8];
        unpack8(r.u[i], x);
#pragma unroll
        for (int e = 0; e < 8; ++e) q2 += (x[e] - mu) * (x[e] - mu);
      }
      q2 += __shfl_xor(q2, 32);
      r.mu = mu;
      r.inv = valid ? 1.f / sqrtf(q2 * pn.var_w + ln_eps) : 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < UL; ++i) {
      if (kload && i >= KUL) continue;
      float x[8];
      values(r, i, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, valid ? fabsf(x[e]) : 0.f);
    }
    m = wave_max(m);
    if (lane == 0) wmx[slot][lw] = m;
  };
  // scaled chunk -> staging buffer: k / 2^ekx, v / 2^evx, transposed
  auto stage = [&](const RawSet& r, int c, int buf, int ekx, int evx) __attribute__((always_inline)) {
    E* tb = tile[buf];
    const float sc = pow2(kload ? -ekx : -evx);
    if constexpr (!PREMAP) {
      typedef E EV __attribute__((ext_vector_type(TPL)));
      if (ulive) {
        float x[TPL][8];
#pragma unroll
        for (int i = 0; i < TPL; ++i) {
          unpack8(r.u[i], x[i]);
          if (c * C + TPL * tg + i >= N)
#pragma unroll
            for (int e = 0; e < 8; ++e) x[i][e] = 0.f;
        }
        const int r0 = (kload ? 0 : VROW) + 8 * lu;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          EV o;
#pragma unroll
          for (int i = 0; i < TPL; ++i) o[i] = (E)(x[i][e] * sc);
          *reinterpret_cast<EV*>(&tb[(r0 + e) * KP + TPL * tg]) = o;
        }
      }
      if (kload && lu < 2) {  // the row of ones (valid tokens) and the row of zeros
        EV o;
#pragma unroll
        for (int i = 0; i < TPL; ++i) o[i] = (lu == 0 && c * C + TPL * tg + i < N) ? (E)1.f : (E)0.f;
        *reinterpret_cast<EV*>(&tb[(lu == 0 ? ONE : ZERO) * KP + TPL * tg]) = o;
      }
      return;
    }
    if (lidle) return;
    const bool valid = c * C + ltok < N;
#pragma unroll
    for (int i = 0; i < UL; ++i) {
      if (kload && i >= KUL) continue;
      float x[8];
      values(r, i, x);
      const int r0 = (kload ? 0 : VROW) + 8 * (lhalf + 2 * i);
#pragma unroll
      for (int e = 0; e < 8; ++e) tb[(r0 + e) * KP + ltok] = valid ? (E)(x[e] * sc) : (E)0.f;
    }
    if (kload) tb[(lhalf ? ZERO : ONE) * KP + ltok] = (!lhalf && valid) ? (E)1.f : (E)0.f;
  };
  // exponents of chunk c, from the chunk exponent table
  auto chunk_exps = [&](int c, int& ek, int& ev) __attribute__((always_inline)) {
    const int2 e = kvexp[(long)bh * nchunks + c];
    ek = e.x;
    ev = e.y;
  };

  // ---- prologue: chunk 0 staged, maxima of chunk 1 reduced ----
  RawSet R[NR];
  // Every fetch, convert and stage is issued unconditionally (chunk indices
  // past the end are clamped for loads, and rows past the end stage as
  // zeros into a buffer nobody reads), and the loader and compute roles run
  // separate loops: straight-line code lets the compiler's memory-counter
  // waits cover exactly the chunk being staged, so NR chunks stay in flight.
  if (loader) {
#pragma unroll
    for (int i = 0; i < NR; ++i) R[i] = fetch(min(i, nchunks - 1));
    if (PREMAP) convert(R[0], 0, 0);  // the pre-map statistics of the keys
  }
  __syncthreads();
  int Ek = 0, Ev = 0, beta = 0;
  {
    int ek, ev;
    chunk_exps(0, ek, ev);
    Ek = ek == kNegExp ? 0 : ek;
    Ev = ev == kNegExp ? 0 : ev;
    // initial state in units 2^(nu Ek + Ev) (2^(nu Ek) for z); the fixed
    // snapshot exponent beta bounds every later entry: |acc| <= N + M_in
    float m_in = 0.f;
    if (state_in != nullptr && (active || cwave)) {
      const float sh = pow2(-(nu * Ek + Ev)), sz = pow2(-nu * Ek);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          long f;
          int r = 0, t = 0, mu = 0;
          if (active) {
            if (!kfeature(DH, kb, acc_position(m, 4 * lg + e), r, t, mu)) continue;
            f = abi_index(DH, r, t);
          } else {
            if (m != 0 || lg != 0 || e != 0) continue;
            f = 0;
          }
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[m][n][e] = state_in[sbase + f * DV + 16 * n + l16] * sh;
          if (l16 == 0) acc[m][4][e] = state_in[sbase + D * DV + f] * sz;
        }
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 5; ++n)
#pragma unroll
          for (int e = 0; e < 4; ++e) m_in = fmaxf(m_in, fabsf(acc[m][n][e]));
    }
    if (!loader) {
      m_in = wave_max(m_in);
      if (lane == 0) wm_in[wave] = m_in;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < kScanCompute; ++w) m_in = fmaxf(m_in, wm_in[w]);
    beta = exp_above((float)NS + m_in) - 15;
    const float sb = pow2(-beta);
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int n = 0; n < 5; ++n) acc[m][n] *= sb;
  }
  if (loader) {
    stage(R[0], 0, 0, Ek, Ev + beta);
    if (PREMAP) convert(R[1], 1, 1);
    R[0] = fetch(min(NR, nchunks - 1));
  }
  __syncthreads();

  F ones;
  if constexpr (IsBf16<T>::value) {
    const _Float16 o = l16 == 0 ? (_Float16)pow2(-beta) : (_Float16)0.f;
    ones.v = h8{o, o, o, o, o, o, o, o};
  } else {
    const float o = l16 == 0 ? pow2(-beta) : 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones.v[e] = o;
  }

  // Chunk c.  Loader registers: rs = chunk c+1 (staged now, then refilled
  // with chunk c+1+NR), rc = chunk c+2 (maxima reduced now).
  auto step = [&](auto role, int c, RawSet& rs, RawSet& rc) __attribute__((always_inline)) {
    constexpr bool LOADER = decltype(role)::value;
    int Ek1 = Ek, Ev1 = Ev;  // exponents of chunk c+1
    if (c + 1 < nchunks) {
      int ek, ev;
      chunk_exps(c + 1, ek, ev);
      Ek1 = max(Ek, ek);
      Ev1 = max(Ev, ev);
    }
    if constexpr (LOADER) {
      stage(rs, c + 1, (c + 1) & 1, Ek1, Ev1 + beta);
      if (PREMAP) convert(rc, c + 2, c & 1);
      rs = fetch(min(c + 1 + NR, nchunks - 1));
    } else {
      // ---- snapshot S_c: raw = stored * 2^(beta + nu Ek) (* 2^Ev for H) ----
      const long sidx = (long)c * BH + bh;
      if (active) {
        E* sp = snap + (sidx * KB + kb) * DV * 32 + 8 * lg;
        E* sz = snap + nsnap * KB * DV * 32 + (sidx * KB + kb) * 32 + 8 * lg;
#pragma unroll
        for (int n = 0; n < 5; ++n) {
          if (n == 4 && l16 != 0) continue;
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = acc[0][n][e];
            x[4 + e] = acc[1][n][e];
          }
          frag_st(n < 4 ? sp + (16 * n + l16) * 32 : sz, x);
        }
        if (lane == 0) sexp[sidx * (KB + 2) + kb] = beta;
      } else if (cwave && lg == 0) {
        const float sh = pow2(Ev + beta);
#pragma unroll
        for (int n = 0; n < 4; ++n) sconst[sidx * NCOL + 16 * n + l16] = acc[0][n][0] * sh;
        if (l16 == 0) sconst[sidx * NCOL + DV] = acc[0][4][0] * pow2(beta);
      }
      if (lead) {
        sexp[sidx * (KB + 2) + KB] = Ek;
        sexp[sidx * (KB + 2) + KB + 1] = Ev;
      }
      // ---- S += phi_k(K_c)^T [V_c | 1] ----
      if (active || cwave) {
        const E* kT = tile[c & 1];
        const E* vT = kT + VROW * KP;
#pragma unroll
        for (int ks = 0; ks < C / 32; ++ks) {
          const int jb = 32 * ks + 8 * lg;
          F A[2];
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            F a0, a1;
            frag_ld(a0, &kT[ar[m] * KP + jb]);
            frag_ld(a1, &kT[at[m] * KP + jb]);
            if constexpr (IsBf16<T>::value) {
              A[m].v = a0.v * a1.v;
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) A[m].v[e] = a0.v[e] * a1.v[e];
            }
          }
          F Bv[4];
#pragma unroll
          for (int n = 0; n < 4; ++n) frag_ld(Bv[n], &vT[(16 * n + l16) * KP + jb]);
#pragma unroll
          for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int n = 0; n < 4; ++n) mma(acc[m][n], A[m], Bv[n]);
            mma(acc[m][4], A[m], ones);
          }
        }
      }
      // ---- units of chunk c+1 ----
      if (Ek1 > Ek || Ev1 > Ev) {
        const int dk = Ek1 - Ek, dv = Ev1 - Ev;
        const float sh = pow2(-(nu * dk + dv)), sz = pow2(-nu * dk);
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
          for (int n = 0; n < 4; ++n) acc[m][n] *= sh;
          acc[m][4] *= sz;
        }
      }
    }
    Ek = Ek1;
    Ev = Ev1;
    __syncthreads();
  };
  auto run = [&](auto role) __attribute__((always_inline)) {
    int c0 = 0;
    for (; c0 + NR <= nchunks; c0 += NR) {
#pragma unroll
      for (int i = 0; i < NR; ++i) step(role, c0 + i, R[(i + 1) % NR], R[(i + 2) % NR]);
    }
#pragma unroll
    for (int i = 0; i + 1 < NR; ++i)
      if (c0 + i < nchunks) step(role, c0 + i, R[(i + 1) % NR], R[(i + 2) % NR]);
  };
  if (loader) run(std::true_type{});
  else run(std::false_type{});

  // ---- final state -> ABI layout (raw moments, each packed entry once) ----
  if (state_out != nullptr) {
    if (active) {
      const float sh = pow2(nu * Ek + Ev + beta), sz = pow2(nu * Ek + beta);
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          int r = 0, t = 0, mu = 0;
          if (!kfeature(DH, kb, acc_position(m, 4 * lg + e), r, t, mu)) continue;
          if (t != DH && r > t) continue;  // the (t, r) copy of a diagonal block writes it
          const long f = abi_index(DH, r, t);
#pragma unroll
          for (int n = 0; n < 4; ++n) state_out[sbase + f * DV + 16 * n + l16] = acc[m][n][e] * sh;
          if (l16 == 0) state_out[sbase + D * DV + f] = acc[m][4][e] * sz;
        }
    } else if (cwave && lg == 0) {
      const float sh = pow2(Ev + beta);
#pragma unroll
      for (int n = 0; n < 4; ++n) state_out[sbase + 16 * n + l16] = acc[0][n][0] * sh;
      if (l16 == 0) state_out[sbase + D * DV] = acc[0][4][0] * pow2(beta);
    }
  }
}

// Value of a bad head's coefficient exponent (a group id out of range): the
// readout writes NaN for every output of that head.
constexpr int kBadHead = 1 << 20;

template <int NG>
__host__ __device__ constexpr int npc() {
  return 1 + NG + NG * NG;
}

// Feature position -> (r, t, multiplicity) of the K-blocked layout.
template <int DH>
__device__ constexpr KPosTable<DH> kpos_dev = make_kpos_table<DH>();

// --------------------------------------------------------------------------
// kernel 2: chunk readout + intra-chunk block + normalisation
// --------------------------------------------------------------------------

// Readout CTAs have NW = 4 or 8 waves: wave w owns rows 16 (w % 4) .. of the
// chunk and the heads hh with hh % (NW / 4) == w / 4.  Eight waves give two
// waves per SIMD but only 256 registers each (up to four heads per wave
// fit); four waves give 512 registers each (seven heads per wave).

// Dynamic LDS layout of the readout kernel (bytes), for RG heads per pass.
struct ReadoutLds {
  long qh, coef, kh, vt, bst, total;
};
template <typename T, int DH>
__host__ __device__ inline ReadoutLds readout_lds(int RG) {
  typedef typename Cx<T>::E E;
  constexpr int KB = n_kblocks(DH);
  constexpr int DHP = DH + 8;
  ReadoutLds L;
  L.qh = 0;
  L.coef = L.qh + (long)RG * C * DHP * sizeof(E);
  L.kh = L.coef + (long)RG * (KB + 1) * 32 * sizeof(E);
  L.vt = L.kh + (long)C * DHP * sizeof(E);
  L.bst = L.vt + (long)DV * (C + 8) * sizeof(T);
  // three stage buffers of stage_kblocks K-blocks: value columns, then z
  L.total = L.bst + 3L * stage_elems(stage_kblocks(RG, (int)sizeof(E))) * sizeof(E);
  return L;
}

// With one head slot a workgroup is four waves and its LDS leaves room for a
// second one on the compute unit; the register budget of two waves per SIMD
// lets both run.
template <typename T, int DH, int RMAX, int NG, bool PREMAP, int NW>
__global__ __launch_bounds__(64 * NW, (RMAX == 1 && IsBf16<T>::value) ? 2 : 1) void readout_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const float* __restrict__ ca, const float* __restrict__ cb, const float* __restrict__ cc, int G,
    const float* __restrict__ gamma_q, const float* __restrict__ beta_q, const float* __restrict__ gamma_k,
    const float* __restrict__ beta_k, float ln_eps, PremapNorm pn, const int32_t* __restrict__ group_of_dim,
    const typename Cx<T>::E* __restrict__ snap, const int* __restrict__ sexp, const float* __restrict__ sconst,
    int has_state_in, T* __restrict__ y, int Hq, int Hkv, int NS, int nchunks, int RG,
    const int32_t* __restrict__ seq_lens) {
  typedef typename Cx<T>::E E;
  typedef typename Cx<T>::Frag F;
  typedef Frag<IsBf16<T>::value> PF;  // P . V operands (bf16 or fp32)
  constexpr int KB = n_kblocks(DH);
  constexpr int NQ = nq_kblocks(DH);
  constexpr int NL = nl_kblocks(DH);
  constexpr int DHP = DH + 8;
  constexpr int VP = C + 8;
  constexpr int STEPS = (DH + 31) / 32;  // K steps of the score GEMM
  constexpr int NPC = npc<NG>();
  constexpr int QD = DH / 4;
  constexpr int NT = 64 * NW;
  constexpr int HS = NW / 4;  // head split between the waves of a row tile
  constexpr int KG = stage_kblocks(RMAX, (int)sizeof(typename Cx<T>::E));  // K-blocks per stage

  extern __shared__ __align__(16) unsigned char lds[];
  const ReadoutLds LL = readout_lds<T, DH>(RMAX);
  E* qh = reinterpret_cast<E*>(lds + LL.qh);      // [RG][C][DHP] q / 2^f
  E* coef = reinterpret_cast<E*>(lds + LL.coef);  // [RG][KB + 1][32] coefficients * kscale / 2^c_h
  E* kh = reinterpret_cast<E*>(lds + LL.kh);      // [C][DHP] k / 2^aK
  T* vTi = reinterpret_cast<T*>(lds + LL.vt);     // [DV][VP] raw values, transposed
  E* bst = reinterpret_cast<E*>(lds + LL.bst);    // [2][KG][NCOL][32]
  __shared__ int qexp[RMAX][C];
  __shared__ float kscale[KB];  // per-K-block fold factor 2^(15 + tau - tau_max(type))
  __shared__ int gm[RMAX][DH];
  __shared__ float pc[RMAX][NPC];
  __shared__ int cexp[RMAX];
  __shared__ float cst[NCOL];
  __shared__ float wmx[NW];
  __shared__ int sc_int[3];  // aK, tau_quad_max, tau_lin_max
  __shared__ float wtau[2][2];
  __shared__ __align__(16) int zdummy[NW][4];  // sink of the waves' padding z loads

  const int c = blockIdx.x, bh = blockIdx.y, BH = gridDim.y;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int R = Hq / Hkv;
  // rows of this sequence (its own length with seq_lens; the row stride is NS):
  // chunks past its end have nothing to do
  const int N = seq_len_of(seq_lens, b, NS);
  if (c * C >= N) return;
  // Builds with eight head slots, and the eight-group builds with one slot
  // (held to two waves per SIMD) or four, run short of registers (measured
  // gains: one slot 899 -> 830 us on the 32k-token prefill, four slots
  // 96 -> 76 us; the two-slot eight-group build is faster without, 49 us
  // against 54, although it spills 124 bytes per lane): there the wave
  // index is made scalar and the lanes' LDS offsets are recomputed per stage
  // (values hidden from loop-invariant hoisting), which keeps the spills out
  // of the stage loop (one reload is left in the eight-slot eight-group
  // build).  Other builds keep the offsets live.
  constexpr bool kTight = RMAX >= 8 || (NG == 8 && IsBf16<T>::value && (RMAX == 1 || RMAX == 4));
  // The eight-slot eight-group build still spilled the lane index out of the
  // stage loop; there it is re-derived from the hardware at each use
  // (measured: 116-117 -> 111-112 us; the four-group build lost 2 us with it).
  constexpr bool kLaneHw = RMAX >= 8 && NG >= 8;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = kTight ? __builtin_amdgcn_readfirstlane(tid / kWave) : tid / kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const int rt = wave % 4, kpar = wave / 4;  // row tile, head class
  const int j0 = c * C;
  const int nvalid = min(C, N - j0);
  const bool inter = c > 0 || has_state_in;
  const long sidx = (long)c * BH + bh;
  const int srow = (tid / 4) % C, sq = tid % 4;  // staging (threads < 256): row, quarter
  const bool stager = tid < 4 * C;

  // ---- snapshot staging: KG K-blocks per stage, stage 0 = the linear ones ----
  // Stages go straight from global memory into LDS (16 bytes per lane, the
  // lane's bytes landing at the wave's base + 16 lane).  In LDS the column
  // parts (eight features) are swizzled, part' = (part + col/2 + col/8) % 4,
  // so that the 16 lanes of a lane group read their B fragments without
  // bank conflicts.
  const E* sv0 = snap + sidx * KB * DV * 32;                     // value blocks
  const E* sz0 = snap + (long)nchunks * BH * KB * DV * 32 + sidx * KB * 32;  // z blocks
  constexpr int VE = 16 / sizeof(E);            // elements per 16-byte vector
  constexpr int VH = sizeof(E) / 2;             // vectors per eight-element part
  constexpr int VPB = DV * 32 / VE;             // value vectors per K-block
  constexpr int LPT = KG * VPB / NT;            // value vectors per thread and stage
  constexpr int ZV = KG * 32 / VE;              // z vectors per stage (wave 0)
  static_assert(KG * VPB % NT == 0 && ZV <= kWave, "stage split");
  constexpr int SE = stage_elems(KG);
  static_assert(NL <= KG, "one linear stage");
  constexpr int NSTAGE = 1 + (NQ + KG - 1) / KG;
  auto kb_at = [&](int sg, int slot) __attribute__((always_inline)) {
    // padding slots map to a real K-block; their scale is forced to zero
    return sg == 0 ? NQ + min(slot, NL - 1) : min((sg - 1) * KG + slot, NQ - 1);
  };
  auto slot_live = [&](int sg, int slot) __attribute__((always_inline)) {
    return sg == 0 ? slot < NL : (sg - 1) * KG + slot < NQ;
  };
  // LDS element offset of (column, part) inside a value block
  auto swz = [](int col, int part) __attribute__((always_inline)) {
    return (4 * col + ((part + col / 2 + col / 8) & 3)) * 8;
  };
  typedef __attribute__((address_space(3))) void lds_void;
  typedef const __attribute__((address_space(1))) void gbl_void;
  auto issue = [&](int sg, int buf) __attribute__((always_inline)) {
    E* dst = bst + (long)buf * SE;
    const int tid_o = kLaneHw ? wave * kWave + lane_now() : opaque<kTight>(tid);
    const int lane_o = tid_o % kWave, wave_o = tid_o / kWave;
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int w = tid_o + NT * i;               // LDS vector of this lane
      const int slot = w / VPB, wl = w % VPB;
      const int pu = wl / VH, half = wl % VH;
      const int col = pu / 4, pp = pu % 4;
      const int part = (pp - col / 2 - col / 8) & 3;
      const E* src = sv0 + (long)kb_at(sg, slot) * DV * 32 + ((4 * col + part) * VH + half) * VE;
      __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)(dst + (long)(w - lane_o) * VE), 16, 0, 0);
    }
    // z vectors: lanes < ZV of wave 0; every other wave issues the same
    // instruction with only lane 0 live, into its own 16-byte dummy slot, so
    // that all waves count the same number of outstanding loads
    if (lane_o < (wave_o == 0 ? ZV : 1)) {
      const int slot = lane_o / (32 / VE), part = lane_o % (32 / VE);
      const E* src = sz0 + (long)kb_at(sg, slot) * 32 + part * VE;
      void* zd = wave_o == 0 ? (void*)(dst + KG * DV * 32) : (void*)&zdummy[wave_o][0];
      __builtin_amdgcn_global_load_lds((gbl_void*)src, (lds_void*)zd, 16, 0, 0);
    }
  };
  // barrier after which the stages issued before the last issue are in LDS
  // (one_left: the wave's most recent stage issue may still be in flight)
  auto stage_sync = [&](bool one_left) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    if (one_left) {
      lds_barrier<LPT + 1>();
    } else {
      lds_barrier<0>();
    }
  };
  // the first two stages are requested before anything else
  if (inter) {
    issue(0, 0);
    issue(1, 1);
  }

  // ---- chunk-wide prologue: K (scores), V (P . V), snapshot scales ----
  {
    float kx[QD];
    const T* kp = k + ((long)bh * NS + j0) * DH;
    const T* vp = v + ((long)bh * NS + j0) * DV;
#pragma unroll
    for (int i = 0; i < QD; ++i) kx[i] = 0.f;
    if (stager) {
      if (srow < nvalid) {
        load_vals<QD>(kp + (long)srow * DH + sq * QD, kx);
#pragma unroll
        for (int i = 0; i < 16; i += 8) {
          // raw copy of the values into the transposed tile
          if constexpr (IsBf16<T>::value) {
            const uint4 w = *reinterpret_cast<const uint4*>(vp + (long)srow * DV + sq * 16 + i);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              vTi[(sq * 16 + i + 2 * jj) * VP + srow] = (uint16_t)(ws[jj] & 0xffffu);
              vTi[(sq * 16 + i + 2 * jj + 1) * VP + srow] = (uint16_t)(ws[jj] >> 16);
            }
          } else {
            float t8[8];
            load_vals<8>(vp + (long)srow * DV + sq * 16 + i, t8);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) vTi[(sq * 16 + i + jj) * VP + srow] = t8[jj];
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) vTi[(sq * 16 + i) * VP + srow] = T(0);
      }
      if (PREMAP) {
        premap4<DH, QD>(kx, sq * QD, gamma_k + kvh * DH, beta_k + kvh * DH, ln_eps, pn);
        if (srow >= nvalid)
#pragma unroll
          for (int i = 0; i < QD; ++i) kx[i] = 0.f;
      }
    }
    float mk = 0.f;
#pragma unroll
    for (int i = 0; i < QD; ++i) mk = fmaxf(mk, fabsf(kx[i]));
    mk = wave_max(mk);
    if (lane == 0) wmx[wave] = mk;
    if (tid < NCOL) cst[tid] = inter ? sconst[sidx * NCOL + tid] : 0.f;
    // snapshot exponents: tau of K-block tid, maxima per feature type
    int tau_me = kNegExp;
    if (inter && tid < KB) {
      const int* ex = sexp + sidx * (KB + 2);
      tau_me = ex[tid] + (tid < NQ ? 2 : 1) * ex[KB];
    }
    static_assert(KB <= 2 * kWave, "two waves reduce the K-block exponents");
    if (wave < 2) {
      const float tqw = wave_max(tid < NQ ? (float)tau_me : (float)kNegExp);
      const float tlw = wave_max(tid >= NQ && tid < KB ? (float)tau_me : (float)kNegExp);
      if (lane == 0) {
        wtau[0][wave] = tqw;
        wtau[1][wave] = tlw;
      }
    }
    __syncthreads();
    const int tq = (int)fmaxf(wtau[0][0], wtau[0][1]), tl = (int)fmaxf(wtau[1][0], wtau[1][1]);
    if (tid == 0) {
      sc_int[1] = tq;
      sc_int[2] = tl;
    }
    float mall = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) mall = fmaxf(mall, wmx[w]);
    int aK = exp_above(mall);
    if (aK == kNegExp) aK = 0;
    if (stager) {
      const float sk = pow2(-aK);
#pragma unroll
      for (int i = 0; i < QD; ++i) kh[srow * DHP + sq * QD + i] = (E)(kx[i] * sk);
    }
    if (tid == 0) sc_int[0] = aK;
    if (tid < KB) kscale[tid] = inter ? pow2(15 + tau_me - (tid < NQ ? tq : tl)) : 0.f;
  }
  __syncthreads();
  const int aK = sc_int[0];
  const int tau_q = sc_int[1] != kNegExp ? sc_int[1] : (sc_int[2] != kNegExp ? sc_int[2] : 0);
  const int tau_l = sc_int[2] != kNegExp ? sc_int[2] : tau_q;
  const int Ev = inter ? sexp[sidx * (KB + 2) + KB + 1] : 0;
  const int row = 16 * rt + l16;  // A-operand row of this lane

  for (int h0 = 0; h0 < R; h0 += RMAX) {
    constexpr int nh = RMAX;         // head slots per pass
    const int nreal = min(RMAX, R - h0);  // slots beyond are dead: zero features, no output
    __syncthreads();  // previous head group done with qh / coef / bst
    if (inter && h0 > 0) {
      issue(0, 0);
      issue(1, 1);
    }
    // ---- per-head tables: polynomial [a, b_g / sqrt(d), sym(c)_gh / d],
    // exponent c_h with 2^c_h above every feature coefficient (kBadHead for
    // a group id out of range), feature coefficients / 2^c_h ----
    for (int idx = tid; idx < nh * DH; idx += NT) {
      const int hh = idx / DH, r = idx % DH;
      gm[hh][r] = hh < nreal ? group_of_dim[(kvh * R + h0 + hh) * DH + r] : 0;
    }
    for (int idx = tid; idx < nh * NPC; idx += NT) {
      const int hh = idx / NPC, i2 = idx % NPC, h = kvh * R + h0 + hh;
      float val = 0.f;
      if (hh < nreal) {
        if (i2 == 0) {
          val = ca[h];
        } else if (i2 <= NG) {
          const int g = i2 - 1;
          val = g < G ? cb[h * G + g] * (1.f / sqrtf((float)DH)) : 0.f;
        } else {
          const int gh = i2 - 1 - NG, g = gh / NG, g2 = gh % NG;
          val = (g < G && g2 < G) ? 0.5f * (cc[(h * G + g) * G + g2] + cc[(h * G + g2) * G + g]) / DH : 0.f;
        }
      }
      pc[hh][i2] = val;
    }
    __syncthreads();
    if (wave < nh) {  // one wave per head slot
      const bool bad = lane < DH && (unsigned)gm[wave][lane] >= (unsigned)G;
      float mx = 0.f;
      for (int i2 = 1 + lane; i2 < NPC; i2 += kWave) mx = fmaxf(mx, (i2 <= NG ? 1.f : 2.f) * fabsf(pc[wave][i2]));
      mx = wave_max(mx);
      const bool anybad = __ballot(bad) != 0;
      if (lane == 0) {
        const int e = exp_above(mx);
        cexp[wave] = wave >= nreal ? 0 : anybad ? kBadHead : e == kNegExp ? 0 : e;
      }
    }
    __syncthreads();
    // position-major: one table entry per thread and position, all slots
#pragma unroll
    for (int it = 0; it < ((KB + 1) * 32 + NT - 1) / NT; ++it) {
      const int pos = tid + NT * it;
      if (pos < (KB + 1) * 32) {
        // block KB is all zeros: padding slots of the last stage read it
        const unsigned short fe = pos < KB * 32 ? kpos_dev<DH>.e[pos] : kPadFeature;
        const float ks = pos < KB * 32 ? kscale[pos / 32] : 0.f;
        const int r = fe & 127, t = (fe >> 7) & 127;
        const float mu = (float)(fe >> 14);
#pragma unroll
        for (int hh = 0; hh < nh; ++hh) {
          if (hh >= nreal) break;  // dead slots are never read
          const int ce = cexp[hh];
          float val = 0.f;
          if (fe != kPadFeature && ce != kBadHead) {
            const int gr = gm[hh][r];
            val = t == DH ? pc[hh][1 + gr] : mu * pc[hh][1 + NG + gr * NG + gm[hh][t]];
          }
          coef[hh * (KB + 1) * 32 + pos] = (E)(val * pow2(-ce) * ks);
        }
      }
    }
    // ---- stage q rows of the head group (pre-map, row exponent) ----
#pragma unroll 1
    for (int it0 = 0; it0 < nh; it0 += NT / (4 * C)) {
      const int it = it0 + tid / (4 * C);
      const bool live = it < nreal;
      const int h = kvh * R + h0 + (live ? it : 0);
      float qx[QD];
      if (live && srow < nvalid) {
        load_vals<QD>(q + ((long)(b * Hq + h) * NS + j0 + srow) * DH + sq * QD, qx);
      } else {
#pragma unroll
        for (int i = 0; i < QD; ++i) qx[i] = 0.f;
      }
      if (PREMAP) premap4<DH, QD>(qx, sq * QD, gamma_q + h * DH, beta_q + h * DH, ln_eps, pn);
      float mq = 0.f;
#pragma unroll
      for (int i = 0; i < QD; ++i) mq = fmaxf(mq, fabsf(qx[i]));
      mq = quad_max(mq);
      int f = exp_above(mq);
      if (f == kNegExp || srow >= nvalid) f = 0;
      const float s = pow2(-f);
      if (it < nh) {
#pragma unroll
        for (int i = 0; i < QD; ++i)
          qh[((long)it * C + srow) * DHP + sq * QD + i] = live && srow < nvalid ? (E)(qx[i] * s) : (E)0.f;
        if (sq == 0) qexp[it][srow] = f;
      }
    }
    __syncthreads();

    // ---- accumulators: this wave serves the heads hh = HS j + kpar ----
    // acc[j] holds, per row, (intra part + constant feature) pre-scaled into
    // the units of the inter partial sums, to which the inter read then adds;
    // units (value columns / normaliser) are 2^(f + c_h + tau_l - 15 + Ev) /
    // 2^(f + c_h + tau_l - 15) during the linear K-blocks and, after one
    // rescale by 2^(tau_l - tau_q - f), 2^(2 f + c_h + tau_q - 15 + Ev) /
    // 2^(2 f + c_h + tau_q - 15).  y = num / den then only needs 2^Ev.
    constexpr int HOWN = (RMAX + HS - 1) / HS;
    f32x4 acc[HOWN][5];
#pragma unroll
    for (int j = 0; j < HOWN; ++j)
#pragma unroll
      for (int n = 0; n < 5; ++n) acc[j][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- intra-chunk block (one head at a time) ----
#pragma unroll 1
    for (int j = 0; j < HOWN; ++j) {
      const int hh = HS * j + kpar;
      if (hh >= nreal) break;  // dead slots (wave-uniform): no work, zero accumulators
      const float* pcr = pc[hh];  // LDS
      // masked query fragments per group (B operand of the transposed scores)
      F Bq[NG][STEPS];
      {
        const E* qrow = qh + ((long)hh * C + row) * DHP;
#pragma unroll
        for (int s = 0; s < STEPS; ++s) {
          F base;
          const int d0 = 32 * s + 8 * lg;
          if (d0 < DH) frag_ld(base, qrow + d0);
          else frag_zero(base);
#pragma unroll
          for (int g = 0; g < NG; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int dd = d0 + e;
              const bool in = dd < DH && gm[hh][dd] == g;
              if constexpr (IsBf16<T>::value) Bq[g][s].v[e] = in ? base.v[e] : (_Float16)0.f;
              else Bq[g][s].v[e] = in ? base.v[e] : 0.f;
            }
          }
        }
      }
      // raw dot products: q / 2^f_row times k / 2^aK (the polynomial table
      // carries the 1/sqrt(d) and 1/d of the scores)
      const float sfac = pow2(qexp[hh][row] + aK);
      f32x4 cur[5];
#pragma unroll
      for (int n = 0; n < 5; ++n) cur[n] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int jt0 = 0; jt0 <= rt; jt0 += 2) {
        // With eight groups the 45 distinct polynomial coefficients, hoisted
        // out of this loop, would sit in registers for the whole block and
        // push the build into spills; there they are re-read from LDS per
        // key tile (the row pointer is hidden from loop-invariant hoisting).
        const float* pck = NG >= 8 ? pc[opaque<true>(hh)] : pcr;
        float p[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int jt = jt0 + half;
          if (jt > rt) {
#pragma unroll
            for (int e = 0; e < 4; ++e) p[4 * half + e] = 0.f;
            continue;
          }
          F Ak[STEPS];
#pragma unroll
          for (int s = 0; s < STEPS; ++s) {
            const int d0 = 32 * s + 8 * lg;
            if (d0 < DH) frag_ld(Ak[s], kh + (16 * jt + l16) * DHP + d0);
            else frag_zero(Ak[s]);
          }
          f32x4 sg[NG];
#pragma unroll
          for (int g = 0; g < NG; ++g) {
            sg[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < STEPS; ++s) mma(sg[g], Ak[s], Bq[g][s]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // kappa = a + sum_g s_g (b_g + c_gg s_g + 2 sum_{g2>g} c_gg2 s_g2)
            float sv[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) sv[g] = sg[g][e] * sfac;
            float kap = pck[0];
#pragma unroll
            for (int g = 0; g < NG; ++g) {
              float inner = pck[1 + g] + pck[1 + NG + g * NG + g] * sv[g];
#pragma unroll
              for (int g2 = g + 1; g2 < NG; ++g2) inner += 2.f * pck[1 + NG + g * NG + g2] * sv[g2];
              kap += sv[g] * inner;
            }
            const int key = 16 * jt + 4 * lg + e;
            p[4 * half + e] = key > row ? 0.f : kap;
          }
        }
        const PF A = frag_from<IsBf16<T>::value>(p);
        const int ja = 16 * jt0 + 4 * lg, jb = ja + 16;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          // values of keys ja..ja+3 and jb..jb+3, straight from the tile
          const T* vr = vTi + (16 * n + l16) * VP;
          PF Bv;
          if constexpr (IsBf16<T>::value) {
            const uint2 lo = *reinterpret_cast<const uint2*>(vr + ja);
            const uint2 hi = *reinterpret_cast<const uint2*>(vr + jb);
            Bv.v = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
          } else {
            const float4 lo = *reinterpret_cast<const float4*>(vr + ja);
            const float4 hi = *reinterpret_cast<const float4*>(vr + jb);
            Bv.v[0] = lo.x; Bv.v[1] = lo.y; Bv.v[2] = lo.z; Bv.v[3] = lo.w;
            Bv.v[4] = hi.x; Bv.v[5] = hi.y; Bv.v[6] = hi.z; Bv.v[7] = hi.w;
          }
          mma(cur[n], A, Bv);
        }
        float ones[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) ones[e] = l16 == 0 ? 1.f : 0.f;
        mma(cur[4], A, frag_from<IsBf16<T>::value>(ones));
      }
      // constant feature and pre-scaling into the linear-block units
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int rr = 16 * rt + 4 * lg + e;
        const float uz = inter ? pow2(-(qexp[hh][rr] + cexp[hh] + tau_l - 15)) : 1.f;
        const float uh = inter ? uz * pow2(-Ev) : 1.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) cur[n][e] = (cur[n][e] + pcr[0] * cst[16 * n + l16]) * uh;
        cur[4][e] = (cur[4][e] + pcr[0] * cst[DV]) * uz;
      }
      // static placement keeps every accumulator set in registers
#pragma unroll
      for (int jj = 0; jj < HOWN; ++jj)
        if (jj == j)
#pragma unroll
          for (int n = 0; n < 5; ++n) acc[jj][n] = cur[n];
    }

    // ---- inter-chunk read: phi_q(Q_c) . S_c ----
    if (inter) {
      // The lane's LDS offsets, recomputed at the start of every stage in
      // tight builds (a few integer operations).
      struct LaneOff {
        int row;      // A-operand row of the lane
        int lgo;      // lane group
        int b[4];     // B fragments of value columns 16 n + l16 (swizzled)
        bool zlane;   // the lane that carries the normaliser column
      };
      auto lane_offsets = [&]() __attribute__((always_inline)) {
        const int ln = kLaneHw ? lane_now() : opaque<kTight>(lane);
        LaneOff o;
        o.row = 16 * rt + ln % 16;
        o.lgo = ln / 16;
#pragma unroll
        for (int n = 0; n < 4; ++n) o.b[n] = swz(16 * n + ln % 16, ln / 16);
        o.zlane = ln % 16 == 0;
        return o;
      };
      auto load_b = [&](F (&Bf)[5], int buf, int slot, const LaneOff& o) __attribute__((always_inline)) {
        const E* bp = bst + (long)buf * SE + slot * DV * 32;
#pragma unroll
        for (int n = 0; n < 4; ++n) frag_ld(Bf[n], bp + o.b[n]);
        if (o.zlane) frag_ld(Bf[4], bst + (long)buf * SE + KG * DV * 32 + slot * 32 + 8 * o.lgo);
        else frag_zero(Bf[4]);
      };
      // linear K-blocks: (q_u ks) coef; their row factor 2^-f (the row's
      // "one") is applied when the partial sums are rescaled
      auto compute_lin = [&](int buf) __attribute__((always_inline)) {
        const LaneOff lo = lane_offsets();
#pragma unroll
        for (int slot = 0; slot < NL; ++slot) {
          const int kk = NQ + slot;
          F Bf[5];
          load_b(Bf, buf, slot, lo);
          const int u0 = 32 * slot + 8 * lg;
          const int uo = u0 < DH ? u0 : 0;  // padding features have zero coefficients
#pragma unroll
          for (int j = 0; j < HOWN; ++j) {
            const int hh = HS * j + kpar;
            if (hh >= nreal) break;  // dead slots (wave-uniform)
            const E* qrow = qh + ((long)hh * C + row) * DHP;
            const E* cf = coef + ((long)hh * (KB + 1) + kk) * 32 + 8 * lg;
            F A;
            if constexpr (IsBf16<T>::value) {
              A.v = *reinterpret_cast<const h8*>(qrow + uo) * *reinterpret_cast<const h8*>(cf);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) A.v[e] = qrow[uo + e] * cf[e];
            }
#pragma unroll
            for (int n = 0; n < 5; ++n) mma(acc[j][n], A, Bf[n]);
          }
        }
      };
      // quadratic K-blocks: (q_r ks) q_t coef for r in {r0, r0 + 1}, t in
      // t0..t0+3; branch-free so that the accumulators update in place
      // (prb, ptb): block pair of slot 0 of the next quadratic K-block
      // (pairs are listed tb-major; K-block kk holds pairs 2 kk, 2 kk + 1)
      int prb = 0, ptb = 0;
      auto next_pair = [](int& rb, int& tb) __attribute__((always_inline)) {
        if (rb == tb) {
          ++tb;
          rb = 0;
        } else {
          ++rb;
        }
      };
      auto compute_quad = [&](int sg, int buf) __attribute__((always_inline)) {
        const LaneOff lo = lane_offsets();
#pragma unroll 1
        for (int slot = 0; slot < KG; ++slot) {
          const bool live = slot_live(sg, slot);
          const int kk = live ? kb_at(sg, slot) : KB;  // KB: the zero block
          F Bf[5];
          load_b(Bf, buf, slot, lo);
          int rb1 = prb, tb1 = ptb;
          next_pair(rb1, tb1);
          // a padding slot reads row offset 0 (finite values times zero coefficients)
          const int r0 = live ? 4 * (lg < 2 ? prb : rb1) + 2 * (lg & 1) : 0;
          const int t0 = live ? 4 * (lg < 2 ? ptb : tb1) : 0;
          prb = rb1;
          ptb = tb1;
          next_pair(prb, ptb);
          // head slot HS j + kpar sits HS j whole blocks after slot kpar
          const E* qr = qh + ((long)kpar * C + lo.row) * DHP + r0;
          const E* qt = qh + ((long)kpar * C + lo.row) * DHP + t0;
          const E* cb = coef + ((long)kpar * (KB + 1) + kk) * 32 + 8 * lo.lgo;
#pragma unroll
          for (int j = 0; j < HOWN; ++j) {
            if (HS * j + kpar >= nreal) break;  // dead slots (wave-uniform)
            const E* qrow = qh + ((long)(HS * j + kpar) * C + row) * DHP;
            const E* cf = cb + HS * j * (KB + 1) * 32;
            F A;
            if constexpr (IsBf16<T>::value) {
              const h8 cv = *reinterpret_cast<const h8*>(cf);
              const h2 rs = *reinterpret_cast<const h2*>(qr + HS * j * C * DHP);
              const h4 tq = *reinterpret_cast<const h4*>(qt + HS * j * C * DHP);
              const h2 t01 = h2{tq[0], tq[1]}, t23 = h2{tq[2], tq[3]};
              const h2 e0 = (rs.xx * t01) * h2{cv[0], cv[1]};
              const h2 e1 = (rs.xx * t23) * h2{cv[2], cv[3]};
              const h2 e2 = (rs.yy * t01) * h2{cv[4], cv[5]};
              const h2 e3 = (rs.yy * t23) * h2{cv[6], cv[7]};
              A.v = h8{e0[0], e0[1], e1[0], e1[1], e2[0], e2[1], e3[0], e3[1]};
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) A.v[e] = qrow[r0 + e / 4] * qrow[t0 + e % 4] * cf[e];
            }
#pragma unroll
            for (int n = 0; n < 5; ++n) mma(acc[j][n], A, Bf[n]);
          }
        }
      };
      // pipeline over three LDS buffers: stage sg is read from buffer sg % 3
      // while stage sg + 2 loads into buffer (sg + 2) % 3; before the barrier
      // that ends step sg, each wave waits for its loads of stage sg + 1
      // (issued one step earlier).  Stages 0 and 1 were issued at the start.
      auto inter_step = [&](int sg) __attribute__((always_inline)) {
        if (sg + 2 < NSTAGE) issue(sg + 2, (sg + 2) % 3);
        if (sg == 0) compute_lin(0);
        else compute_quad(sg, sg % 3);
        stage_sync(sg + 2 < NSTAGE);
      };
      stage_sync(false);
      inter_step(0);
      // linear K-blocks done: to quadratic units, 2^(tau_l - tau_q - f) per row
#pragma unroll
      for (int j = 0; j < HOWN; ++j) {
        const int hh = HS * j + kpar;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float fr = pow2(tau_l - tau_q - qexp[hh][16 * rt + 4 * lg + e]);
#pragma unroll
          for (int n = 0; n < 5; ++n) acc[j][n][e] *= fr;
        }
      }
      for (int sg = 1; sg < NSTAGE; ++sg) inter_step(sg);
    }

    // ---- normalise and store (one head at a time) ----
    const float sev = inter ? pow2(Ev) : 1.f;
    const float nanv = __builtin_nanf("");
    // the wave's 16 x 64 output tile goes through its own LDS slice (the
    // stage buffers are free now) and leaves as 16-byte row segments
    T* yt = reinterpret_cast<T*>(bst) + wave * 16 * DV;
#pragma unroll 1
    for (int j = 0; j < HOWN; ++j) {
      const int hh = HS * j + kpar;
      if (hh >= nreal) break;
      const int h = kvh * R + h0 + hh;
      f32x4 cur[5];
#pragma unroll
      for (int n = 0; n < 5; ++n) cur[n] = acc[0][n];
#pragma unroll
      for (int jj = 1; jj < HOWN; ++jj)
        if (jj == j)
#pragma unroll
          for (int n = 0; n < 5; ++n) cur[n] = acc[jj][n];
      const bool badh = cexp[hh] == kBadHead;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float den = __shfl(cur[4][e], (lane & ~15));  // column 64 lives in lane l16 == 0
        // bf16 outputs: one reciprocal per row (its rounding is far below the
        // output's); fp32 outputs: IEEE division
        const float rden = IsBf16<T>::value ? sev / den : 0.f;
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const float val = badh ? nanv : (IsBf16<T>::value ? cur[n][e] * rden : (cur[n][e] * sev) / den);
          store_elem(&yt[(4 * lg + e) * DV + 16 * n + l16], val);
        }
      }
      {
        constexpr int VPR = DV * sizeof(T) / 16;  // 16-byte vectors per row
        T* yp = y + ((long)(b * Hq + h) * NS + j0 + 16 * rt) * DV;
#pragma unroll
        for (int u = 0; u < 16 * VPR / 64; ++u) {
          const int vi = lane + 64 * u, r = vi / VPR, cv = vi % VPR;
          const uint4 w = reinterpret_cast<const uint4*>(yt)[vi];
          if (16 * rt + r < nvalid) reinterpret_cast<uint4*>(yp + (long)r * DV)[cv] = w;
        }
      }
    }
  }
}

// --------------------------------------------------------------------------
// host launchers
// --------------------------------------------------------------------------

namespace {

template <typename T, int DH>
struct FwdWs {
  long snap_bytes, exp_off, const_off, kvexp_off, total;
};

template <typename T, int DH>
FwdWs<T, DH> fwd_ws(int B, int Hq, int Hkv, int N) {
  typedef typename Cx<T>::E E;
  constexpr int KB = n_kblocks(DH);
  const long nchunks = (N + C - 1) / C;
  const long snaps = nchunks * B * Hkv;
  auto up = [](long x) { return (x + 255) / 256 * 256; };
  FwdWs<T, DH> w;
  w.snap_bytes = snaps * KB * NCOL * 32 * (long)sizeof(E);
  w.exp_off = up(w.snap_bytes);
  w.const_off = w.exp_off + up(snaps * (KB + 2) * 4);
  w.kvexp_off = w.const_off + up(snaps * NCOL * 4);
  w.total = w.kvexp_off + up(snaps * 8);  // chunk exponents
  return w;
}

// Query heads per KV head served in one pass: 8 or 4 (four or two per wave;
// eight waves), 2, or 1; the last pass of a head count that is not a multiple
// carries dead slots.  fp32 activations use at most 2.
template <typename T, int DH>
int pick_rg(int R) {
  // dynamic LDS limit: 160 KiB per workgroup less the static tables (< 9 KiB)
  constexpr long lim = 151 * 1024 + 512 * 5;
  if (R >= 5 && IsBf16<T>::value && readout_lds<T, DH>(8).total <= lim) return 8;
  if (R >= 3 && IsBf16<T>::value && readout_lds<T, DH>(4).total <= lim) return 4;
  if (R >= 2 && readout_lds<T, DH>(2).total <= lim) return 2;
  return 1;
}

}  // namespace

template <typename T, int DH>
hipError_t launch_fwd_t(const FwdLaunch& a, int stages, hipStream_t stream) {
  typedef typename Cx<T>::E E;
  const int nchunks = (a.N + C - 1) / C;
  const int BH = a.B * a.Hkv;
  constexpr int KB = n_kblocks(DH);
  const FwdWs<T, DH> w = fwd_ws<T, DH>(a.B, a.Hq, a.Hkv, a.N);
  const PremapNorm pn = premap_norm(a.premap_kind, DH);
  unsigned char* ws = reinterpret_cast<unsigned char*>(a.workspace);
  E* snap = reinterpret_cast<E*>(ws);
  int* sexp = reinterpret_cast<int*>(ws + w.exp_off);
  float* sconst = reinterpret_cast<float*>(ws + w.const_off);
  const T* qq = reinterpret_cast<const T*>(a.q);
  const T* kk = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  T* yy = reinterpret_cast<T*>(a.y);
  if (stages & 1) {
    int2* kvexp = reinterpret_cast<int2*>(ws + w.kvexp_off);
    {
      const dim3 egrid(nchunks, BH);
      if (a.premap)
        hipLaunchKernelGGL((chunk_exp_kernel<T, DH, true>), egrid, dim3(256), 0, stream, kk, vv, a.gamma_k, a.beta_k,
                           a.ln_eps, pn, kvexp, a.Hkv, a.N, nchunks, a.seq_lens);
      else
        hipLaunchKernelGGL((chunk_exp_kernel<T, DH, false>), egrid, dim3(256), 0, stream, kk, vv, nullptr, nullptr,
                           0.f, pn, kvexp, a.Hkv, a.N, nchunks, a.seq_lens);
      hipError_t e0 = hipGetLastError();
      if (e0 != hipSuccess) return e0;
    }
    // four compute waves per CTA when that grid fits on the 256 compute
    // units in one round (one CTA per unit), else eight
    const bool four = (long)((KB + 1 + 3) / 4) * BH <= 256;
    const int ncw = four ? 4 : 8;
    dim3 grid((KB + 1 + ncw - 1) / ncw, BH);  // K-blocks + the constant row
#define OAL_SCAN(PM, NC)                                                                                       \
    hipLaunchKernelGGL((scan_kernel<T, DH, PM, NC>), grid, dim3(64 * kScanWaves), 0, stream, kk, vv,            \
                       PM ? a.gamma_k : nullptr, PM ? a.beta_k : nullptr, PM ? a.ln_eps : 0.f, pn, a.state_in, \
                       a.state_out, snap, sexp, sconst, kvexp, a.Hkv, a.N, nchunks, a.seq_lens)
    if (a.premap) {
      if (four) OAL_SCAN(true, 4);
      else OAL_SCAN(true, 8);
    } else {
      if (four) OAL_SCAN(false, 4);
      else OAL_SCAN(false, 8);
    }
#undef OAL_SCAN
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  if (!(stages & 2)) return hipSuccess;
  const int R = a.Hq / a.Hkv;
  const int rg = pick_rg<T, DH>(R);
  const size_t shm = (size_t)readout_lds<T, DH>(rg).total;
  dim3 grid(nchunks, BH);
  const int has_in = a.state_in != nullptr;
#define OAL_OUT(RM, NGV, PM)                                                                                    \
  do {                                                                                                          \
    constexpr int NWV = RM % 2 == 0 ? 8 : 4;                                                                         \
    auto fn = readout_kernel<T, DH, RM, NGV, PM, NWV>;                                                          \
    hipError_t e2 = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),                                      \
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);                  \
    if (e2 != hipSuccess) return e2;                                                                            \
    hipLaunchKernelGGL(fn, grid, dim3(64 * NWV), shm, stream, qq, kk, vv, a.ca, a.cb, a.cc, a.G, a.gamma_q,             \
                       a.beta_q, a.gamma_k, a.beta_k, a.ln_eps, pn, a.group_of_dim, snap, sexp, sconst, has_in, yy, \
                       a.Hq, a.Hkv, a.N, nchunks, rg, a.seq_lens);                                              \
  } while (0)
#define OAL_OUT_NG(RM, PM)                 \
  do {                                     \
    switch (ng) {                          \
      case 1: OAL_OUT(RM, 1, PM); break;   \
      case 4: OAL_OUT(RM, 4, PM); break;   \
      default: OAL_OUT(RM, 8, PM); break;  \
    }                                      \
  } while (0)
  const int ng = a.G <= 1 ? 1 : a.G <= 4 ? 4 : 8;
#define OAL_OUT_RG(PM)                       \
  do {                                       \
    switch (rg) {                            \
      case 1: OAL_OUT_NG(1, PM); break;      \
      case 2: OAL_OUT_NG(2, PM); break;      \
      case 4: OAL_OUT_NG(4, PM); break;      \
      default: OAL_OUT_NG(8, PM); break;     \
    }                                        \
  } while (0)
  if constexpr (IsBf16<T>::value) {
    if (a.premap) OAL_OUT_RG(true);
    else OAL_OUT_RG(false);
  } else {
    if (rg == 2) {
      if (a.premap) OAL_OUT_NG(2, true);
      else OAL_OUT_NG(2, false);
    } else {
      if (a.premap) OAL_OUT_NG(1, true);
      else OAL_OUT_NG(1, false);
    }
  }
#undef OAL_OUT_RG
#undef OAL_OUT_NG
#undef OAL_OUT
  return hipGetLastError();
}

}  // namespace oal
