// Causal prefill for the dimension-wise form of the grouped kernel:
//
//     kappa(q, k) = a + sum_r b_g(r) x_r + sum_r c_g(r)g(r) x_r^2,  x_r = q_r k_r / sqrt(d_h)
//
// which is the grouped kernel of the OAL paper (sec. 4.2) when every group is
// a single dimension and c is diagonal: the ReBased feature map read as an
// elementwise square ("Linear Transformers with Learnable Kernel Functions",
// the section on the learnable parabola: phi(x) = (gamma norm(x) + beta)^2
// elementwise, so kappa = sum_r q_r^2 k_r^2 with a = b = 0, c = d_h I).  Its
// separable features are only F = 1 + 2 d_h wide,
//     phi_K(k) = [1, k_r, k_r^2],   phi_Q(q) = [a, b_g(r) q_r / sqrt(d), c_g(r)g(r) q_r^2 / d],
// so the prefix state of Eq. (5) is F x (d_v + 1) and a whole sequence is
// walked by one CTA per (batch x KV head, 16 value columns) with the state in
// MFMA accumulators:
//   per chunk of 64 tokens: stage phi_K (row-major and transposed), V and
//   ones; snapshot S into LDS; S += phi_K^T [V | 1]; then for every query head
//   of the KV head stage phi_Q and compute, per 16-row tile of the chunk,
//   the within-chunk scores phi_K phi_Q^T (causal mask), P [V | 1] and
//   phi_Q S, and normalise.
// bf16 activations use bf16 features and bf16 MFMA (fp32 accumulation);
// fp32 activations use fp32 MFMA.  The state in memory uses the packed layout
// of the library (App. D order); only its constant, linear and squared
// entries are read and written.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

namespace {

constexpr int DV = 64;
constexpr int C = kChunk;
constexpr int NCG = DV / 16;  // value-column groups (one CTA each)

template <int DH>
__host__ __device__ constexpr int dfeat() {
  return 1 + 2 * DH;
}
template <int DH>
__host__ __device__ constexpr int dfeat_pad() {
  return (dfeat<DH>() + 31) / 32 * 32;
}

// LDS layout (elements of E) for one CTA.
template <typename E, int DH>
struct DiagLds {
  static constexpr int FP = dfeat_pad<DH>();
  static constexpr int FPP = FP + 8;  // row pitch of feature-major tiles
  static constexpr int CP = C + 8;    // row pitch of token-major tiles
  static constexpr long kf = 0;                      // [C][FPP]   phi_K rows
  static constexpr long kft = kf + (long)C * FPP;    // [FP][CP]   phi_K transposed
  static constexpr long qf = kft + (long)FP * CP;    // [C][FPP]   phi_Q rows of one head
  static constexpr long vt = qf + (long)C * FPP;     // [17][CP]   value columns and ones, transposed
  static constexpr long st = vt + 17L * CP;          // [17][FPP]  state snapshot, transposed
  static constexpr long total = st + 17L * FPP;
};

template <typename T>
struct DiagFrag;
template <>
struct DiagFrag<uint16_t> {
  typedef Frag<true> F;
  typedef uint16_t E;
};
template <>
struct DiagFrag<float> {
  typedef Frag<false> F;
  typedef float E;
};

__device__ __forceinline__ uint16_t to_e(float x, uint16_t) { return bf16_bits(x); }
__device__ __forceinline__ float to_e(float x, float) { return x; }

// eight consecutive elements of a tile as an MFMA operand
__device__ __forceinline__ Frag<true> dload(const uint16_t* p) { return frag_load(p); }
__device__ __forceinline__ Frag<false> dload(const float* p) { return frag_load(p); }

}  // namespace

template <typename T, int DH, bool PREMAP>
__global__ __launch_bounds__(256) void diag_fwd_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ group_of_dim, const float* __restrict__ ca, const float* __restrict__ cb,
    const float* __restrict__ cc, int G, const float* __restrict__ gamma_q, const float* __restrict__ beta_q,
    const float* __restrict__ gamma_k, const float* __restrict__ beta_k, float ln_eps,
    const float* __restrict__ state_in, float* __restrict__ state_out, T* __restrict__ y, int Hq, int Hkv,
    int N) {
  typedef typename DiagFrag<T>::F F;
  typedef typename DiagFrag<T>::E E;
  typedef DiagLds<E, DH> L;
  constexpr int F0 = dfeat<DH>();
  constexpr int FP = L::FP, FPP = L::FPP, CP = L::CP;
  constexpr int KS = FP / 32;        // K steps over the features
  constexpr int MT = FP / 16;        // feature row tiles of the state
  constexpr int MTW = (MT + 3) / 4;  // state row tiles per wave
  constexpr int QD = DH / 4;         // staged dimensions per thread
  constexpr long D = packed_features(DH);
  constexpr long SF = D * (DV + 1);
  extern __shared__ __align__(16) unsigned char lds_raw[];
  E* lds = reinterpret_cast<E*>(lds_raw);
  E* kf = lds + L::kf;
  E* kft = lds + L::kft;
  E* qf = lds + L::qf;
  E* vt = lds + L::vt;
  E* st = lds + L::st;
  __shared__ float coefq[DH + 1][3];  // per head: [r][0] = b_g(r)/sqrt(d), [r][1] = c_gg/d; [DH][0] = a
  __shared__ int bad;

  const int cg = blockIdx.x, bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv, R = Hq / Hkv;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int lg = lane / 16, l16 = lane % 16;
  const int rt = wave;                    // row tile of the chunk
  const int srow = tid / 4, sq = tid % 4;  // staging: token row, quarter
  const int nchunks = (N + C - 1) / C;
  const long sbase = (long)bh * SF;

  // ---- state accumulators: S rows 16 m + 4 lg + e, columns (16 cg + l16 | z) ----
  f32x4 acc[MTW][2];
#pragma unroll
  for (int i = 0; i < MTW; ++i) acc[i][0] = acc[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  // packed (library) index of state feature f: 0 const, 1 + r linear, 1 + d + r square
  auto abi_f = [](int f) __attribute__((always_inline)) {
    return f <= DH ? (long)f : abi_index(DH, f - 1 - DH, f - 1 - DH);
  };
  if (state_in != nullptr) {
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        if (f >= F0) continue;
        const long af = abi_f(f);
        acc[i][0][e] = state_in[sbase + af * DV + 16 * cg + l16];
        if (l16 == 0) acc[i][1][e] = state_in[sbase + D * DV + af];
      }
    }
  }

  // padding features (F0 .. FP - 1) stay zero in every tile
  for (int i = tid; i < C * (FP - F0); i += blockDim.x) {
    const int r = i / (FP - F0), f = F0 + i % (FP - F0);
    kf[r * FPP + f] = to_e(0.f, E());
    qf[r * FPP + f] = to_e(0.f, E());
    kft[f * CP + r] = to_e(0.f, E());
  }
  for (int f = F0 + tid; f < FP; f += blockDim.x) {
    for (int cc2 = 0; cc2 < 17; ++cc2) st[cc2 * FPP + f] = to_e(0.f, E());
  }

  for (int c = 0; c < nchunks; ++c) {
    const int j0 = c * C, nvalid = min(C, N - j0);
    // ---- stage phi_K (both layouts), values of this column group, ones ----
    {
      float kx[QD];
      const bool ok = srow < nvalid;
      if (ok) {
        const T* kp = k + ((long)bh * N + j0 + srow) * DH + sq * QD;
#pragma unroll
        for (int i = 0; i < QD; ++i) kx[i] = to_f32(kp[i]);
      } else {
#pragma unroll
        for (int i = 0; i < QD; ++i) kx[i] = 0.f;
      }
      if (PREMAP) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) s += kx[i];
        s = quad_sum(s);
        const float mu = s * (1.f / DH);
        float v2 = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) v2 += (kx[i] - mu) * (kx[i] - mu);
        v2 = quad_sum(v2);
        const float inv = 1.f / sqrtf(v2 * (1.f / DH) + ln_eps);
#pragma unroll
        for (int i = 0; i < QD; ++i) {
          const int d = sq * QD + i;
          kx[i] = ok ? gamma_k[kvh * DH + d] * (kx[i] - mu) * inv + beta_k[kvh * DH + d] : 0.f;
        }
      }
#pragma unroll
      for (int i = 0; i < QD; ++i) {
        const int r = sq * QD + i;
        const E lin = to_e(kx[i], E()), sqv = to_e(kx[i] * kx[i], E());
        kf[srow * FPP + 1 + r] = lin;
        kf[srow * FPP + 1 + DH + r] = sqv;
        kft[(1 + r) * CP + srow] = lin;
        kft[(1 + DH + r) * CP + srow] = sqv;
      }
      if (sq == 0) {
        const E one = to_e(ok ? 1.f : 0.f, E());
        kf[srow * FPP] = one;
        kft[srow] = one;
        vt[16 * CP + srow] = one;
      }
      const T* vp = v + ((long)bh * N + j0 + srow) * DV + 16 * cg + 4 * sq;
#pragma unroll
      for (int i = 0; i < 4; ++i) vt[(4 * sq + i) * CP + srow] = to_e(ok ? to_f32(vp[i]) : 0.f, E());
    }
    // ---- snapshot S (before this chunk) into LDS, transposed ----
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        st[l16 * FPP + f] = to_e(acc[i][0][e], E());
        if (l16 == 0) st[16 * FPP + f] = to_e(acc[i][1][e], E());
      }
    }
    __syncthreads();
    // ---- S += phi_K^T [V | 1] ----
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int ks = 0; ks < C / 32; ++ks) {
        const F A = dload(&kft[(16 * m + l16) * CP + 32 * ks + 8 * lg]);
        const F B0 = dload(&vt[l16 * CP + 32 * ks + 8 * lg]);
        F B1 = dload(&vt[16 * CP + 32 * ks + 8 * lg]);
        if (l16 != 0) B1 = frag_zero<IsBf16<T>::value>();
        mma(acc[i][0], A, B0);
        mma(acc[i][1], A, B1);
      }
    }

    // ---- every query head of the KV head ----
    for (int hh = 0; hh < R; ++hh) {
      const int h = kvh * R + hh;
      __syncthreads();  // previous head done with qf / coefq / bad
      if (wave == 0) {  // DH <= 64: one lane per dimension
        bool badg = false;
        if (lane < DH) {
          const int g = group_of_dim[h * DH + lane];
          badg = g < 0 || g >= G;
          const int gg = badg ? 0 : g;
          coefq[lane][0] = cb[h * G + gg] * (1.f / sqrtf((float)DH));
          coefq[lane][1] = cc[(h * G + gg) * G + gg] * (1.f / DH);
        }
        const bool anyb = __ballot(badg) != 0;
        if (lane == 0) {
          bad = anyb ? 1 : 0;
          coefq[DH][0] = ca[h];
        }
      }
      __syncthreads();
      // phi_Q rows of the head
      {
        float qx[QD];
        const bool ok = srow < nvalid;
        if (ok) {
          const T* qp = q + ((long)(b * Hq + h) * N + j0 + srow) * DH + sq * QD;
#pragma unroll
          for (int i = 0; i < QD; ++i) qx[i] = to_f32(qp[i]);
        } else {
#pragma unroll
          for (int i = 0; i < QD; ++i) qx[i] = 0.f;
        }
        if (PREMAP) {
          float s = 0.f;
#pragma unroll
          for (int i = 0; i < QD; ++i) s += qx[i];
          s = quad_sum(s);
          const float mu = s * (1.f / DH);
          float v2 = 0.f;
#pragma unroll
          for (int i = 0; i < QD; ++i) v2 += (qx[i] - mu) * (qx[i] - mu);
          v2 = quad_sum(v2);
          const float inv = 1.f / sqrtf(v2 * (1.f / DH) + ln_eps);
#pragma unroll
          for (int i = 0; i < QD; ++i) {
            const int d = sq * QD + i;
            qx[i] = ok ? gamma_q[h * DH + d] * (qx[i] - mu) * inv + beta_q[h * DH + d] : 0.f;
          }
        }
#pragma unroll
        for (int i = 0; i < QD; ++i) {
          const int r = sq * QD + i;
          qf[srow * FPP + 1 + r] = to_e(coefq[r][0] * qx[i], E());
          qf[srow * FPP + 1 + DH + r] = to_e(coefq[r][1] * qx[i] * qx[i], E());
        }
        if (sq == 0) qf[srow * FPP] = to_e(ok ? coefq[DH][0] : 0.f, E());
      }
      __syncthreads();

      // ---- row tile rt: inter (phi_Q S) + within-chunk pairs ----
      f32x4 yacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      const int row = 16 * rt + l16;  // query row of this lane in the score tiles
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const F A = dload(&qf[(16 * rt + l16) * FPP + 32 * ks + 8 * lg]);
        const F B0 = dload(&st[l16 * FPP + 32 * ks + 8 * lg]);
        F B1 = dload(&st[16 * FPP + 32 * ks + 8 * lg]);
        if (l16 != 0) B1 = frag_zero<IsBf16<T>::value>();
        mma(yacc[0], A, B0);
        mma(yacc[1], A, B1);
      }
      // scores phi_K(key) . phi_Q(row): A = key rows, B = query rows, so a
      // lane holds keys 4 lg + e of query row `row`
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
            for (int ks = 0; ks < KS; ++ks) mma(sc, dload(&kf[(16 * jt + l16) * FPP + 32 * ks + 8 * lg]), Bq[ks]);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int key = 16 * jt + 4 * lg + e;
            p[4 * half + e] = (jt <= rt && key <= row) ? sc[e] : 0.f;
          }
        }
        const F A = frag_from<IsBf16<T>::value>(p);
        const int ja = 16 * jt0 + 4 * lg, jb = ja + 16;
        float vb[8], ob[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vb[e] = to_f32(vt[l16 * CP + ja + e]);
          vb[4 + e] = to_f32(vt[l16 * CP + jb + e]);
          ob[e] = l16 == 0 ? to_f32(vt[16 * CP + ja + e]) : 0.f;
          ob[4 + e] = l16 == 0 ? to_f32(vt[16 * CP + jb + e]) : 0.f;
        }
        mma(yacc[0], A, frag_from<IsBf16<T>::value>(vb));
        mma(yacc[1], A, frag_from<IsBf16<T>::value>(ob));
      }
      // ---- y = num / den (den lives in lane l16 == 0 of each lane group) ----
      const float nanv = __builtin_nanf("");
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float den = __shfl(yacc[1][e], lane & ~15);
        const int rr = 16 * rt + 4 * lg + e;
        if (rr < nvalid) {
          const float val = bad ? nanv : yacc[0][e] / den;
          store_elem(&y[((long)(b * Hq + h) * N + j0 + rr) * DV + 16 * cg + l16], val);
        }
      }
    }
    __syncthreads();  // chunk done with every tile before the next stage
  }

  // ---- final state: constant, linear and squared entries ----
  if (state_out != nullptr) {
#pragma unroll
    for (int i = 0; i < MTW; ++i) {
      const int m = wave + 4 * i;
      if (m >= MT) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        if (f >= F0) continue;
        const long af = abi_f(f);
        state_out[sbase + af * DV + 16 * cg + l16] = acc[i][0][e];
        if (cg == 0 && l16 == 0) state_out[sbase + D * DV + af] = acc[i][1][e];
      }
    }
  }
}

template <typename T, int DH>
static hipError_t launch_diag_t(const FwdLaunch& a, hipStream_t stream) {
  typedef typename DiagFrag<T>::E E;
  const size_t shm = (size_t)DiagLds<E, DH>::total * sizeof(E);
  dim3 grid(NCG, a.B * a.Hkv);
  const T* qq = reinterpret_cast<const T*>(a.q);
  const T* kk = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  T* yy = reinterpret_cast<T*>(a.y);
  auto fn = a.premap ? diag_fwd_kernel<T, DH, true> : diag_fwd_kernel<T, DH, false>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)shm);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, grid, dim3(256), shm, stream, qq, kk, vv, a.group_of_dim, a.ca, a.cb, a.cc, a.G,
                     a.gamma_q, a.beta_q, a.gamma_k, a.beta_k, a.ln_eps, a.state_in, a.state_out, yy, a.Hq,
                     a.Hkv, a.N);
  return hipGetLastError();
}

hipError_t launch_fwd_diag(const FwdLaunch& a, hipStream_t stream) {
  if (a.dtype == 1) {
    switch (a.d_h) {
      case 16: return launch_diag_t<uint16_t, 16>(a, stream);
      case 32: return launch_diag_t<uint16_t, 32>(a, stream);
      default: return launch_diag_t<uint16_t, 64>(a, stream);
    }
  }
  switch (a.d_h) {
    case 16: return launch_diag_t<float, 16>(a, stream);
    case 32: return launch_diag_t<float, 32>(a, stream);
    default: return launch_diag_t<float, 64>(a, stream);
  }
}

}  // namespace oal
