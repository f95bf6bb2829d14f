// Causal prefill for small feature spaces, where the whole prefix state of
// the OAL paper's Eq. (5) fits in the MFMA accumulators of one CTA:
//
//  * the dimension-wise form  kappa = a + sum_r b_g(r) x_r + sum_r c_g(r)g(r) x_r^2
//    (x_r = q_r k_r / sqrt(d_h)), the grouped kernel of sec. 4.2 when every
//    group is one dimension and c is diagonal -- the ReBased feature map read
//    as an elementwise square ("Linear Transformers with Learnable Kernel
//    Functions", the section on the learnable parabola).  Features
//    [1, k_r, k_r^2]: F = 1 + 2 d_h.
//  * (template only) the full grouped kernel at d_h = 16 (the packed
//    features of App. D, F = 153).  That instantiation passed parity but ran
//    slower than the chunk kernels on the Based workload, so the library does
//    not build or dispatch it; DIAG = false is kept for that experiment.
//
// The query-side feature of (r, t) carries the kernel coefficient: a for the
// constant, b_g(r) / sqrt(d) for the linear term r, and for a pair the
// symmetric c of the two groups / d, twice off the diagonal (Eq. (6)).
//
// Work split: a sequence is cut into `nseg` contiguous segments of whole
// chunks.  Kernel 1 (one CTA per segment but the last, and per batch x KV
// head) sums phi_K(k_j) [v_j, 1] over its segment into the workspace.
// Kernel 2 (one CTA per segment and batch x KV head) starts from the
// incoming state plus the sums of the earlier segments and walks its chunks:
// stage phi_K (row-major and transposed), V and ones; snapshot S into LDS;
// S += phi_K^T [V | 1] on MFMA; then for every query head stage phi_Q and,
// per 16-row tile, compute the within-chunk scores phi_K phi_Q^T (causal
// mask), P [V | 1] and phi_Q S, normalise and store.  Without a workspace
// the whole sequence is one segment.
// bf16 activations use bf16 features and bf16 MFMA (fp32 accumulation, the
// state snapshot rounded to bf16 for the readout); fp32 activations use fp32
// MFMA and half-length chunks to fit the tiles in LDS.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

namespace {

constexpr int DV = 64;
constexpr int NCOL = DV + 1;

// Feature list of a small space: (r, t) over k_hat = [k_0 .. k_{d-1}, 1, 0]
// (index d is the constant 1, d + 1 a zero used for padding).  Internal
// order: the full space keeps the library's packed order (constant, linear
// terms, pairs r <= t row-major); the dimension-wise space lists the linear
// terms, then the squares, then the constant (LIN, SQ, CF below), so that a
// thread's dimensions map to contiguous features.
template <int DH, bool DIAG>
struct SmallSpace {
  static constexpr int F = DIAG ? 1 + 2 * DH : (int)packed_features(DH);
  static constexpr int FP = (F + 31) / 32 * 32;
  static constexpr int LIN = DIAG ? 0 : 1;   // feature of linear term r: LIN + r
  static constexpr int SQ = DH;              // dimension-wise: square of r at SQ + r
  static constexpr int CF = DIAG ? 2 * DH : 0;  // the constant feature
  unsigned char r[FP], t[FP];
};
template <int DH, bool DIAG>
constexpr SmallSpace<DH, DIAG> make_space() {
  typedef SmallSpace<DH, DIAG> S;
  S s{};
  s.r[S::CF] = DH;
  s.t[S::CF] = DH;
  for (int r = 0; r < DH; ++r) {
    s.r[S::LIN + r] = (unsigned char)r;
    s.t[S::LIN + r] = DH;
  }
  int f = DIAG ? S::SQ : 1 + DH;
  for (int r = 0; r < DH; ++r)
    for (int t = r; t < (DIAG ? r + 1 : DH); ++t, ++f) {
      s.r[f] = (unsigned char)r;
      s.t[f] = (unsigned char)t;
    }
  for (f = S::F; f < S::FP; ++f) {
    s.r[f] = DH + 1;
    s.t[f] = DH + 1;
  }
  return s;
}
template <int DH, bool DIAG>
__device__ constexpr SmallSpace<DH, DIAG> space_dev = make_space<DH, DIAG>();

template <typename T>
constexpr int small_chunk() {
  return IsBf16<T>::value ? 64 : 32;
}

// LDS layout (elements of E) of one CTA.
template <typename T, int DH, bool DIAG>
struct SmallLds {
  typedef typename std::conditional<IsBf16<T>::value, uint16_t, float>::type E;
  static constexpr int C = small_chunk<T>();
  static constexpr int FP = SmallSpace<DH, DIAG>::FP;
  static constexpr int FPP = FP + 8;  // row pitch of feature-major tiles
  static constexpr int CP = C + 8;    // row pitch of token-major tiles
  static constexpr int KH = DH + 1;   // row pitch of k_hat / q_hat (floats; odd: no bank conflicts)
  static constexpr long kf = 0;                        // [C][FPP]   phi_K rows
  static constexpr long kft = kf + (long)C * FPP;      // [FP][CP]   phi_K transposed
  static constexpr long qf = kft + (long)FP * CP;      // [C][FPP]   phi_Q rows of one head
  static constexpr long vt = qf + (long)C * FPP;       // [NCOL][CP] values and ones, transposed
  static constexpr long st = vt + (long)NCOL * CP;     // [NCOL][FPP] state snapshot, transposed
  static constexpr long yt = st + (long)NCOL * FPP;    // [4][16][DV] output tiles
  static constexpr long end = yt + 4L * 16 * DV;
  static constexpr long hat_bytes = (long)C * KH * 4;  // k_hat / q_hat rows (floats), full space only
  static constexpr long bytes = end * (long)sizeof(E) + (DIAG ? 0 : hat_bytes);
};

__device__ __forceinline__ uint16_t to_e(float x, uint16_t) { return bf16_bits(x); }
__device__ __forceinline__ float to_e(float x, float) { return x; }
__device__ __forceinline__ Frag<true> dload(const uint16_t* p) { return frag_load(p); }
__device__ __forceinline__ Frag<false> dload(const float* p) { return frag_load(p); }

// n consecutive elements of T as raw 32-bit words, moved with 16-byte (or,
// for 8 bytes, one 8-byte) vector loads; p is 8- or 16-byte aligned.
template <typename T, int n>
struct RawRow {
  static constexpr int NW = n * (int)sizeof(T) / 4;
  static_assert(NW == 2 || NW % 4 == 0, "row part of 8 or 16k bytes");
  uint32_t w[NW];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (NW == 2) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      w[0] = x.x;
      w[1] = x.y;
    } else {
#pragma unroll
      for (int i = 0; i < NW / 4; ++i) {
        const uint4 x = reinterpret_cast<const uint4*>(p)[i];
        w[4 * i] = x.x;
        w[4 * i + 1] = x.y;
        w[4 * i + 2] = x.z;
        w[4 * i + 3] = x.w;
      }
    }
  }
  // element i as float, or 0 when !ok
  __device__ __forceinline__ float get(int i, bool ok) const {
    float x;
    if constexpr (sizeof(T) == 2) x = __uint_as_float(i % 2 ? w[i / 2] & 0xffff0000u : w[i / 2] << 16);
    else x = __uint_as_float(w[i]);
    return ok ? x : 0.f;
  }
};

// Workgroup barrier for the LDS tiles: waits for this wave's LDS operations
// only, so global loads issued earlier (the next chunk's rows) stay in flight
// (__syncthreads() would wait for them too).  The empty asm statements keep
// the compiler from moving memory operations across it.
__device__ __forceinline__ void lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf | (7 << 4) | (3 << 14));  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// n floats as n consecutive elements (bf16 bits or float) with 8- and
// 16-byte stores; p is aligned to the run's size (at most 16 bytes).
template <int n>
__device__ __forceinline__ void store_run(uint16_t* p, const float (&x)[n]) {
  static_assert(n % 4 == 0, "runs of 4k elements");
  if constexpr (n % 8 == 0) {
#pragma unroll
    for (int i = 0; i < n; i += 8) {
      uint4 w;
      w.x = (uint32_t)bf16_bits(x[i]) | ((uint32_t)bf16_bits(x[i + 1]) << 16);
      w.y = (uint32_t)bf16_bits(x[i + 2]) | ((uint32_t)bf16_bits(x[i + 3]) << 16);
      w.z = (uint32_t)bf16_bits(x[i + 4]) | ((uint32_t)bf16_bits(x[i + 5]) << 16);
      w.w = (uint32_t)bf16_bits(x[i + 6]) | ((uint32_t)bf16_bits(x[i + 7]) << 16);
      *reinterpret_cast<uint4*>(p + i) = w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < n; i += 4) store4(p + i, f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]});
  }
}
template <int n>
__device__ __forceinline__ void store_run(float* p, const float (&x)[n]) {
  static_assert(n % 2 == 0, "runs of 2k elements");
  if constexpr (n % 4 == 0) {
#pragma unroll
    for (int i = 0; i < n; i += 4) store4(p + i, f32x4{x[i], x[i + 1], x[i + 2], x[i + 3]});
  } else {
#pragma unroll
    for (int i = 0; i < n; i += 2) *reinterpret_cast<float2*>(p + i) = make_float2(x[i], x[i + 1]);
  }
}

// sum over the TPR consecutive lanes that share a token row (TPR = 4 or 8)
template <int TPR>
__device__ __forceinline__ float row_sum(float s) {
  s = quad_sum(s);
  if constexpr (TPR == 8) s += __shfl_xor(s, 4);
  return s;
}

// Pre-map (normalisation of kind pn, then the affine) of a row split over
// TPR consecutive lanes (n values each).
template <int DH, int TPR, int n>
__device__ __forceinline__ void premap_row(float (&x)[n], int d0, const float* __restrict__ gamma,
                                           const float* __restrict__ beta, float eps, PremapNorm pn, bool valid) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) s += x[i];
  s = row_sum<TPR>(s);
  const float mu = s * pn.mean_w;
  float v2 = 0.f;
#pragma unroll
  for (int i = 0; i < n; ++i) v2 += (x[i] - mu) * (x[i] - mu);
  v2 = row_sum<TPR>(v2);
  const float inv = 1.f / sqrtf(v2 * pn.var_w + eps);
#pragma unroll
  for (int i = 0; i < n; ++i) x[i] = valid ? gamma[d0 + i] * (x[i] - mu) * inv + beta[d0 + i] : 0.f;
}

}  // namespace

size_t small_segment_bytes(int d_h, bool diagonal) {
  const int F = diagonal ? 1 + 2 * d_h : (int)packed_features(d_h);
  return (size_t)F * NCOL * sizeof(float);
}

// OUT = false: segment sums (kernel 1); OUT = true: outputs (kernel 2).
template <typename T, int DH, bool DIAG, bool PREMAP, bool OUT>
__global__ __launch_bounds__(256, 2) void small_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ group_of_dim, const float* __restrict__ ca, const float* __restrict__ cb,
    const float* __restrict__ cc, int G, const float* __restrict__ gamma_q, const float* __restrict__ beta_q,
    const float* __restrict__ gamma_k, const float* __restrict__ beta_k, float ln_eps, PremapNorm pn,
    const float* __restrict__ state_in, float* __restrict__ state_out, float* __restrict__ segsum,
    T* __restrict__ y, int Hq, int Hkv, int N, int seg_chunks) {
  typedef SmallLds<T, DH, DIAG> L;
  typedef typename L::E E;
  typedef Frag<IsBf16<T>::value> F;
  typedef SmallSpace<DH, DIAG> SP;
  constexpr int C = L::C, FP = L::FP, FPP = L::FPP, CP = L::CP, KH = L::KH;
  constexpr int F0 = SP::F;
  constexpr int KS = FP / 32;        // K steps over the features
  constexpr int MT = FP / 16;        // feature row tiles of the state
  constexpr int MTW = (MT + 3) / 4;  // state row tiles per wave
  constexpr int RT = C / 16;         // row tiles of a chunk
  constexpr int TPR = 256 / C;       // staging threads per token row (4 or 8)
  constexpr int QD = DH / TPR;       // dimensions staged per thread
  constexpr int VD = DV / TPR;       // value columns staged per thread
  constexpr long D = packed_features(DH);
  constexpr long SF = D * NCOL;
  static_assert(QD >= 1 && QD * TPR == DH, "staging split");
  extern __shared__ __align__(16) unsigned char lds_raw[];
  E* lds = reinterpret_cast<E*>(lds_raw);
  E* kf = lds + L::kf;
  E* kft = lds + L::kft;
  E* qf = lds + L::qf;
  E* vt = lds + L::vt;
  E* st = lds + L::st;
  E* yt = lds + L::yt;
  float* hat = reinterpret_cast<float*>(lds_raw + L::end * sizeof(E));  // [C][KH], full space only
  __shared__ float coefq[8][FP];  // query-side coefficient of every feature, per head slot
  __shared__ int bad[8];

  const int seg = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv, R = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const int srow = tid / TPR, sq = tid % TPR;  // staging: token row, part
  const int nchunks = (N + C - 1) / C;
  const int c_begin = seg * seg_chunks, c_end = min(c_begin + seg_chunks, nchunks);
  const long sbase = (long)bh * SF;
  const float nanv = __builtin_nanf("");

  // packed (library) index of feature f of the space
  auto abi_f = [](int f) __attribute__((always_inline)) {
    if constexpr (!DIAG) return (long)f;
    return f < DH ? 1L + f : f < 2 * DH ? abi_index(DH, f - DH, f - DH) : 0L;
  };

  // ---- query-side coefficients of every head of the KV head ----
  if (OUT) {
    for (int i = tid; i < R * FP; i += blockDim.x) {
      const int hh = i / FP, f = i % FP, h = kvh * R + hh;
      const int r = space_dev<DH, DIAG>.r[f], t = space_dev<DH, DIAG>.t[f];
      float cf = 0.f;
      if (f < F0) {
        if (r == DH) {
          cf = ca[h];
        } else {
          const int g1 = min(max(group_of_dim[h * DH + r], 0), G - 1);
          if (t == DH) {
            cf = cb[h * G + g1] * (1.f / sqrtf((float)DH));
          } else {
            const int g2 = min(max(group_of_dim[h * DH + t], 0), G - 1);
            cf = (cc[(h * G + g1) * G + g2] + cc[(h * G + g2) * G + g1]) * (0.5f / DH);
            if (r != t) cf *= 2.f;
          }
        }
      }
      coefq[hh][f] = cf;
    }
    if (wave == 0)
      for (int hh = 0; hh < R; ++hh) {
        const int h = kvh * R + hh;
        bool badg = false;
        if (lane < DH) {
          const int g = group_of_dim[h * DH + lane];
          badg = g < 0 || g >= G;
        }
        const bool anyb = __ballot(badg) != 0;
        if (lane == 0) bad[hh] = anyb ? 1 : 0;
      }
  }

  // ---- state accumulators: rows 16 m + 4 lg + e, columns 16 n + l16 (n < 4) and z ----
  f32x4 acc[MTW][5];
#pragma unroll
  for (int i = 0; i < MTW; ++i)
#pragma unroll
    for (int n = 0; n < 5; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (OUT) {
    // incoming state plus the sums of the earlier segments
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        if (f >= F0) continue;
        const long af = abi_f(f);
        float x[4] = {0.f, 0.f, 0.f, 0.f}, z = 0.f;
        if (state_in != nullptr) {
#pragma unroll
          for (int n = 0; n < 4; ++n) x[n] = state_in[sbase + af * DV + 16 * n + l16];
          z = state_in[sbase + D * DV + af];
        }
        for (int s = 0; s < seg; ++s) {
          const float* sp = segsum + ((long)bh * gridDim.x + s) * F0 * NCOL + (long)f * NCOL;
#pragma unroll
          for (int n = 0; n < 4; ++n) x[n] += sp[16 * n + l16];
          z += sp[DV];
        }
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n][e] = x[n];
        if (l16 == 0) acc[i][4][e] = z;
      }
    }
  }

  // padding features stay zero in every tile
  for (int i = tid; i < C * (FP - F0); i += blockDim.x) {
    const int r = i / (FP - F0), f = F0 + i % (FP - F0);
    kf[r * FPP + f] = to_e(0.f, E());
    qf[r * FPP + f] = to_e(0.f, E());
    kft[f * CP + r] = to_e(0.f, E());
  }

  // ---- raw loads of a chunk (one token row part per thread); rows past the
  // segment or the sequence read row 0 (in bounds) and are zeroed on use ----
  struct Raw {
    RawRow<T, QD> k, q;
    RawRow<T, VD> v;
    bool ok;
  };
  auto fetch = [&](int c) __attribute__((always_inline)) {
    Raw r;
    const int row = c * C + srow;
    r.ok = c < c_end && row < N;
    const long rr = r.ok ? row : 0;
    r.k.load(k + ((long)bh * N + rr) * DH + sq * QD);
    r.v.load(v + ((long)bh * N + rr) * DV + sq * VD);
    if (OUT) r.q.load(q + ((long)(b * Hq + kvh * R) * N + rr) * DH + sq * QD);
    return r;
  };
  // Features of the chunk from this thread's pre-mapped values x: phi_K
  // (coef == null) or phi_Q (coefficients of a head slot), written into a
  // row-major tile and/or a transposed one (either may be null).  The linear
  // (and, in the dimension-wise space, squared) features of the thread's own
  // dimensions are written directly; the pair features of the full space are
  // formed from the rows gathered in LDS, wave-uniform feature by feature.
  auto feats = [&](float (&x)[QD], E* rows, E* cols, const float* coef) __attribute__((always_inline)) {
    if constexpr (DIAG) {
      // the thread's QD dimensions are contiguous runs of features, stored as
      // 8- or 16-byte vectors in the row-major tile
      float lin[QD], sqv[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        const int r = sq * QD + i;
        lin[i] = coef ? coef[SP::LIN + r] * x[i] : x[i];
        sqv[i] = coef ? coef[SP::SQ + r] * x[i] * x[i] : x[i] * x[i];
      }
      if (rows) {
        store_run<QD>(rows + srow * FPP + SP::LIN + sq * QD, lin);
        store_run<QD>(rows + srow * FPP + SP::SQ + sq * QD, sqv);
      }
      if (cols)
#pragma unroll
        for (int i = 0; i < QD; ++i) {
          const int r = sq * QD + i;
          cols[(SP::LIN + r) * CP + srow] = to_e(lin[i], E());
          cols[(SP::SQ + r) * CP + srow] = to_e(sqv[i], E());
        }
    } else {
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        const int r = sq * QD + i;
        const E lin = to_e(coef ? coef[SP::LIN + r] * x[i] : x[i], E());
        if (rows) rows[srow * FPP + SP::LIN + r] = lin;
        if (cols) cols[(SP::LIN + r) * CP + srow] = lin;
      }
#pragma unroll
      for (int i = 0; i < QD; ++i) hat[srow * KH + sq * QD + i] = x[i];
      lds_sync();
      // pair f = 1 + DH + p is (r, t), p-th in row-major upper-triangle
      // order; this thread takes p = fg, fg + NFG, ... (wave-uniform)
      constexpr int NFG = 256 / C;
      const int row = tid % C, fg = tid / C;
      int r = 0, t = fg;
      for (int f = 1 + DH + fg; f < F0; f += NFG) {
        const E pv = to_e((coef ? coef[f] : 1.f) * hat[row * KH + r] * hat[row * KH + t], E());
        if (rows) rows[row * FPP + f] = pv;
        if (cols) cols[f * CP + row] = pv;
        t += NFG;
        // past the end of row r: continue on the diagonal of row r + 1 (stops
        // at r = DH, after the last pair)
        while (t >= DH && r < DH) {
          ++r;
          t += r - DH;
        }
      }
      lds_sync();  // hat is rewritten by the next staging
    }
  };

  Raw cur = fetch(c_begin);
  for (int c = c_begin; c < c_end; ++c) {
    const int j0 = c * C, nvalid = min(C, N - j0);
    const bool okrow = srow < nvalid;
    // ---- stage phi_K (rows for the scores, transposed for the update), V, ones ----
    {
      float kx[QD];
#pragma unroll
      for (int i = 0; i < QD; ++i) kx[i] = cur.k.get(i, cur.ok);
      if (PREMAP) premap_row<DH, TPR, QD>(kx, kvh * DH + sq * QD, gamma_k, beta_k, ln_eps, pn, okrow);
      feats(kx, OUT ? kf : nullptr, kft, nullptr);  // kernel 1 needs only the transposed tile
      if (sq == 0) {
        const E one = to_e(okrow ? 1.f : 0.f, E());
        if (OUT) kf[srow * FPP + SP::CF] = one;
        kft[SP::CF * CP + srow] = one;
        vt[DV * CP + srow] = one;
      }
#pragma unroll
      for (int i = 0; i < VD; ++i) vt[(sq * VD + i) * CP + srow] = to_e(cur.v.get(i, cur.ok), E());
    }
    Raw nxt = fetch(c + 1);  // in flight during this chunk
    lds_sync();
    // ---- snapshot S (before this chunk), transposed, for the readout ----
    if (OUT) {
#pragma unroll
      for (int i = 0; i < MTW; ++i) {
        const int m = wave + 4 * i;
        if (m >= MT) continue;
        // a lane's four rows 4 lg + e are consecutive features: one store each
        const int f0 = 16 * m + 4 * lg;
#pragma unroll
        for (int n = 0; n < 4; ++n) store4(&st[(16 * n + l16) * FPP + f0], acc[i][n]);
        if (l16 == 0) store4(&st[DV * FPP + f0], acc[i][4]);
      }
    }
    // ---- S += phi_K^T [V | 1] ----
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        const F A = dload(&kft[(16 * m + l16) * CP + 32 * ks + 8 * lg]);
#pragma unroll
        for (int n = 0; n < 4; ++n) mma(acc[i][n], A, dload(&vt[(16 * n + l16) * CP + 32 * ks + 8 * lg]));
        F B1 = dload(&vt[DV * CP + 32 * ks + 8 * lg]);
        if (l16 != 0) B1 = frag_zero<IsBf16<T>::value>();
        mma(acc[i][4], A, B1);
      }
    }

    if (OUT) {
      for (int hh = 0; hh < R; ++hh) {
        const int h = kvh * R + hh;
        lds_sync();  // snapshot written; previous head done with qf
        // ---- phi_Q rows of the head ----
        {
          float qx[QD];
          if (hh == 0) {
#pragma unroll
            for (int i = 0; i < QD; ++i) qx[i] = cur.q.get(i, cur.ok);
          } else {
            RawRow<T, QD> qr;
            qr.load(q + ((long)(b * Hq + h) * N + j0 + (okrow ? srow : 0)) * DH + sq * QD);
#pragma unroll
            for (int i = 0; i < QD; ++i) qx[i] = qr.get(i, okrow);
          }
          if (PREMAP) premap_row<DH, TPR, QD>(qx, h * DH + sq * QD, gamma_q, beta_q, ln_eps, pn, okrow);
          feats(qx, qf, nullptr, coefq[hh]);
          if (sq == 0) qf[srow * FPP + SP::CF] = to_e(okrow ? coefq[hh][SP::CF] : 0.f, E());
        }
        lds_sync();
        for (int rt = wave; rt < RT; rt += 4) {
          // ---- inter: phi_Q S (S before this chunk) ----
          f32x4 yacc[5];
#pragma unroll
          for (int n = 0; n < 5; ++n) yacc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const F A = dload(&qf[(16 * rt + l16) * FPP + 32 * ks + 8 * lg]);
#pragma unroll
            for (int n = 0; n < 4; ++n) mma(yacc[n], A, dload(&st[(16 * n + l16) * FPP + 32 * ks + 8 * lg]));
            F B1 = dload(&st[DV * FPP + 32 * ks + 8 * lg]);
            if (l16 != 0) B1 = frag_zero<IsBf16<T>::value>();
            mma(yacc[4], A, B1);
          }
          // ---- within-chunk pairs: scores phi_K(key) . phi_Q(row); a lane
          // holds keys 4 lg + e of query row `row` ----
          const int row = 16 * rt + l16;
          F Bq[KS];
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) Bq[ks] = dload(&qf[row * FPP + 32 * ks + 8 * lg]);
          for (int jt0 = 0; jt0 <= rt; jt0 += 2) {
            float p[8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const int jt = jt0 + half;
              f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
              if (jt <= rt) {
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                  mma(sc, dload(&kf[(16 * jt + l16) * FPP + 32 * ks + 8 * lg]), Bq[ks]);
              }
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int key = 16 * jt + 4 * lg + e;
                p[4 * half + e] = (jt <= rt && key <= row) ? sc[e] : 0.f;
              }
            }
            const F A = frag_from<IsBf16<T>::value>(p);
            const int ja = 16 * jt0 + 4 * lg, jb = ja + 16;
#pragma unroll
            for (int n = 0; n < 5; ++n) {
              // values of keys ja..ja+3 and jb..jb+3, straight from the tile
              const E* vr = vt + (n < 4 ? 16 * n + l16 : DV) * CP;
              const bool live = n < 4 || l16 == 0;
              F Bv;
              if constexpr (IsBf16<T>::value) {
                uint2 lo = *reinterpret_cast<const uint2*>(vr + ja);
                uint2 hi = *reinterpret_cast<const uint2*>(vr + jb);
                if (!live) lo = hi = make_uint2(0u, 0u);
                Bv.v = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
              } else {
                const float4 lo = *reinterpret_cast<const float4*>(vr + ja);
                const float4 hi = *reinterpret_cast<const float4*>(vr + jb);
                const float vb[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) Bv.v[e] = live ? vb[e] : 0.f;
              }
              mma(yacc[n], A, Bv);
            }
          }
          // ---- y = num / den via the wave's output tile ----
          E* ytw = yt + wave * 16 * DV;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float den = __shfl(yacc[4][e], lane & ~15);
#pragma unroll
            for (int n = 0; n < 4; ++n)
              ytw[(4 * lg + e) * DV + 16 * n + l16] = to_e(bad[hh] ? nanv : yacc[n][e] / den, E());
          }
          constexpr int VPR = DV * sizeof(E) / 16;  // 16-byte vectors per output row
          T* yp = y + ((long)(b * Hq + h) * N + j0 + 16 * rt) * DV;
#pragma unroll
          for (int u = 0; u < 16 * VPR / 64; ++u) {
            const int vi = lane + 64 * u, r = vi / VPR, cv = vi % VPR;
            const uint4 w = reinterpret_cast<const uint4*>(ytw)[vi];
            if (16 * rt + r < nvalid) reinterpret_cast<uint4*>(yp + (long)r * DV)[cv] = w;
          }
        }
      }
    }
    lds_sync();  // every tile of this chunk consumed
    cur = nxt;
  }

  // ---- results: segment sum (kernel 1) or, for the last segment, the state ----
  const bool last = seg == (int)gridDim.x - 1;
  if (!OUT || (last && state_out != nullptr)) {
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        if (f >= F0) continue;
        if (!OUT) {
          // gridDim.x of kernel 1 is nseg - 1; segment sums are strided by nseg
          float* sp = segsum + ((long)bh * (gridDim.x + 1) + seg) * F0 * NCOL + (long)f * NCOL;
#pragma unroll
          for (int n = 0; n < 4; ++n) sp[16 * n + l16] = acc[i][n][e];
          if (l16 == 0) sp[DV] = acc[i][4][e];
        } else {
          const long af = abi_f(f);
#pragma unroll
          for (int n = 0; n < 4; ++n) state_out[sbase + af * DV + 16 * n + l16] = acc[i][n][e];
          if (l16 == 0) state_out[sbase + D * DV + af] = acc[i][4][e];
        }
      }
    }
  }
}

// Segments for a sequence of nchunks chunks: enough CTAs for the chip (about
// two per compute unit), each segment at least two chunks, limited by the
// workspace.
static int small_segments(int BH, int nchunks, size_t seg_bytes_per_bh, size_t workspace_bytes) {
  int nseg = (512 + BH - 1) / BH;
  nseg = std::min(nseg, std::max(1, nchunks / 2));
  if (seg_bytes_per_bh > 0) {
    const long fit = (long)(workspace_bytes / (seg_bytes_per_bh * (size_t)BH));
    nseg = (int)std::min<long>(nseg, std::max<long>(1, fit));
  }
  return std::max(nseg, 1);
}

template <typename T, int DH, bool DIAG>
static hipError_t launch_small_t(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  typedef SmallLds<T, DH, DIAG> L;
  const size_t shm = (size_t)L::bytes;
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + L::C - 1) / L::C;
  const size_t segb = small_segment_bytes(DH, DIAG);
  const int nseg = small_segments(BH, nchunks, segb, a.workspace ? workspace_bytes : 0);
  const int seg_chunks = (nchunks + nseg - 1) / nseg;
  const int nseg_used = (nchunks + seg_chunks - 1) / seg_chunks;
  const T* qq = reinterpret_cast<const T*>(a.q);
  const T* kk = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  T* yy = reinterpret_cast<T*>(a.y);
  float* segsum = reinterpret_cast<float*>(a.workspace);
  const PremapNorm pn = premap_norm(a.premap_kind, DH);
#define OAL_SMALL(PM)                                                                                         \
  do {                                                                                                        \
    auto f1 = small_fwd_kernel<T, DH, DIAG, PM, false>;                                                       \
    auto f2 = small_fwd_kernel<T, DH, DIAG, PM, true>;                                                        \
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(f1),                                     \
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);                 \
    if (e == hipSuccess)                                                                                      \
      e = hipFuncSetAttribute(reinterpret_cast<const void*>(f2), hipFuncAttributeMaxDynamicSharedMemorySize,  \
                              (int)shm);                                                                      \
    if (e != hipSuccess) return e;                                                                            \
    if (nseg_used > 1)                                                                                        \
      hipLaunchKernelGGL(f1, dim3(nseg_used - 1, BH), dim3(256), shm, stream, qq, kk, vv, a.group_of_dim,     \
                         a.ca, a.cb, a.cc, a.G, a.gamma_q, a.beta_q, a.gamma_k, a.beta_k, a.ln_eps, pn,       \
                         a.state_in, a.state_out, segsum, yy, a.Hq, a.Hkv, a.N, seg_chunks);                  \
    hipLaunchKernelGGL(f2, dim3(nseg_used, BH), dim3(256), shm, stream, qq, kk, vv, a.group_of_dim, a.ca,     \
                       a.cb, a.cc, a.G, a.gamma_q, a.beta_q, a.gamma_k, a.beta_k, a.ln_eps, pn, a.state_in,   \
                       a.state_out, segsum, yy, a.Hq, a.Hkv, a.N, seg_chunks);                                \
  } while (0)
  if (a.premap) OAL_SMALL(true);
  else OAL_SMALL(false);
#undef OAL_SMALL
  return hipGetLastError();
}

size_t small_workspace_bytes(int B, int Hkv, int N, int d_h, bool diagonal, int dtype) {
  const int C = dtype == 1 ? small_chunk<uint16_t>() : small_chunk<float>();
  const int BH = B * Hkv;
  const int nchunks = (N + C - 1) / C;
  const int nseg = small_segments(BH, nchunks, 0, 0);
  return nseg > 1 ? (size_t)nseg * BH * small_segment_bytes(d_h, diagonal) : 0;
}

size_t small_workspace_bytes_for(int B, int Hq, int Hkv, int N, int d_h, bool diagonal, int dtype) {
  const size_t cta = small_workspace_bytes(B, Hkv, N, d_h, diagonal, dtype);
  return dimw_supported(d_h, dtype, diagonal, Hq, Hkv) ? std::max(cta, dimw_workspace_bytes(B, Hkv, N)) : cta;
}

bool small_path_supported(int d_h, bool diagonal, int Hq, int Hkv) {
  (void)d_h;
  return Hq / Hkv <= 8 && diagonal;
}

hipError_t launch_fwd_small(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  if (!a.diagonal) return hipErrorInvalidValue;  // only the dimension-wise form is dispatched here
  if (dimw_supported(a.d_h, a.dtype, a.diagonal, a.Hq, a.Hkv)) return launch_dimw(a, workspace_bytes, stream);
  if (a.dtype == 1) {
    switch (a.d_h) {
      case 16: return launch_small_t<uint16_t, 16, true>(a, workspace_bytes, stream);
      case 32: return launch_small_t<uint16_t, 32, true>(a, workspace_bytes, stream);
      default: return launch_small_t<uint16_t, 64, true>(a, workspace_bytes, stream);
    }
  }
  switch (a.d_h) {
    case 16: return launch_small_t<float, 16, true>(a, workspace_bytes, stream);
    case 32: return launch_small_t<float, 32, true>(a, workspace_bytes, stream);
    default: return launch_small_t<float, 64, true>(a, workspace_bytes, stream);
  }
}

}  // namespace oal
