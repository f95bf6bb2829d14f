// Backward pass of the causal normalised OAL attention at d_h = 16, d_v = 64,
// for heads with their own keys and values: the gradients of a loss L with
// dL/dy given, with respect to q, k, v and the kernel coefficients
// (a, b_g, c_gh).  The calibration of the OAL paper fits L (App. B, Eq. (20),
// the output-matching objective) and its adaptation trains the coefficients
// jointly with LoRA (App. F.2); both need these gradients through the causal
// evaluation of Eqs. (5)-(6).
//
// In the packed feature space of the forward pass (App. D: 153 features
// [1, x_r, x_r x_t (r <= t)] at d_h = 16) the kernel is
//     kappa(q, k) = sum_f coef_f m_f(q) m_f(k),
// m_f the feature's monomial (1, x_r or x_r x_t) and coef_f = a, b_g(r) /
// sqrt(d) or (c_g(r)g(t) + c_g(t)g(r)) / d (c_g(r)g(r) / d on the diagonal).
// With u_j = [v_j, 1], y_i = num_i / den_i and g_i = dL/d[num_i, den_i] =
// [dy_i / den_i, -(dy_i . y_i) / den_i]:
//     dkappa_ij    = g_i . u_j                                (j <= i)
//     dL/dPhiQ_i   = sum_{j<=i} dkappa_ij m(k_j)  = S_i g_i,   S_i = sum_{j<=i} m(k_j) u_j^T
//     dL/dPhiK_j   = sum_{i>=j} dkappa_ij coef m(q_i) = R_j u_j, R_j = sum_{i>=j} coef m(q_i) g_i^T
//     dL/du_j      = sum_{i>=j} kappa_ij g_i = R_j^T m(k_j)
//     dL/dcoef_f   = sum_i m_f(q_i) [dL/dPhiQ_i]_f
// and dq, dk follow through the monomials (PhiQ = coef * m(q), PhiK = m(k)).
//
// Two passes over 64-token chunks, one workgroup per (sequence, head):
//  * forward direction: S before the chunk (held in the registers of its
//    owner threads, written to LDS per chunk) recomputes num, den and y of
//    the chunk's queries (inter part against S, within-chunk pairs from
//    the definition) and gives g (written to the workspace), dq, and the
//    per-feature coefficient gradient; then S takes the chunk's keys;
//  * reverse direction: R after the chunk (likewise) gives dk and dv of the
//    chunk's keys with the within-chunk pairs; then R takes the chunk's
//    queries and their g.
// A last kernel maps the per-feature sums to da, db, dc (summed over the
// batch).  All arithmetic is fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <utility>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {
namespace {
namespace bw {

constexpr int DH = 16;
constexpr int DV = 64;
constexpr int NU = DV + 1;  // [v, 1]
constexpr int C = 64;       // tokens per chunk
constexpr int D = 153;      // packed features at d_h = 16
constexpr int NT = 256;     // threads per workgroup: four waves
constexpr int XE = DH + 1;  // a row with the constant 1 appended (index 16)

// Feature f of the library's packed order as a pair of indices into the
// augmented row [x_0 .. x_15, 1]: f = 0 the constant (16, 16), f = 1 + r the
// linear term (r, 16), then the pairs r <= t row by row.
struct Feat {
  int r, t;
};
__host__ __device__ constexpr Feat feat16(int f) {
  if (f == 0) return Feat{DH, DH};
  if (f <= DH) return Feat{f - 1, DH};
  int idx = f - 1 - DH, r = 0;
  while (idx >= DH - r) {
    idx -= DH - r;
    ++r;
  }
  return Feat{r, r + idx};
}

// Features f = W, W + 4, W + 8, ... (the share of wave W), unrolled with
// compile-time indices.
template <int W, typename F, int... M>
__device__ __forceinline__ void for_share_impl(F&& fn, std::integer_sequence<int, M...>) {
  (fn(std::integral_constant<int, W + 4 * M>{}), ...);
}
template <int W>
constexpr int kShare = (D - W + 3) / 4;  // 39, 38, 38, 38
template <int W, typename F>
__device__ __forceinline__ void for_share(F&& fn) {
  for_share_impl<W>(fn, std::make_integer_sequence<int, kShare<W>>{});
}
template <typename F, int... M>
__device__ __forceinline__ void for_all_impl(F&& fn, std::integer_sequence<int, M...>) {
  (fn(std::integral_constant<int, M>{}), ...);
}
template <typename F>
__device__ __forceinline__ void for_all(F&& fn) {
  for_all_impl(fn, std::make_integer_sequence<int, D>{});
}
// run fn<W>() for the wave-uniform W
template <typename F>
__device__ __forceinline__ void by_wave(int w, F&& fn) {
  switch (w) {
    case 0: fn(std::integral_constant<int, 0>{}); break;
    case 1: fn(std::integral_constant<int, 1>{}); break;
    case 2: fn(std::integral_constant<int, 2>{}); break;
    default: fn(std::integral_constant<int, 3>{}); break;
  }
}

struct BwdArgs {
  const void *q, *k, *v, *dy;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  int G, H, N, nchunks;
  float* g;      // [B, H, N, 65] workspace: dL/d[num, den] per query row
  float* P;      // [B, H, D] workspace: dL/dcoef_f per sequence and head
  float *dq, *dk, *dv;
};

__device__ __forceinline__ float ld_act(const void* p, long i, bool bf16) {
  if (bf16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  return reinterpret_cast<const float*>(p)[i];
}

// group of dimension r of head h; -1 when the id is outside [0, G)
__device__ __forceinline__ int group_or_bad(const BwdArgs& p, int h, int r) {
  const int g = p.group_of_dim[h * DH + r];
  return g >= 0 && g < p.G ? g : -1;
}

// coef_f of head h (thread-parallel fill of an LDS table); a group id
// outside [0, G) makes every coefficient of the head NaN, so that all of its
// outputs are NaN
__device__ void fill_coef(const BwdArgs& p, int h, float* coef) {
  bool bad = false;
  for (int r = 0; r < DH; ++r) bad |= group_or_bad(p, h, r) < 0;
  for (int f = threadIdx.x; f < D; f += NT) {
    const Feat ft = feat16(f);
    float cf;
    if (bad) {
      cf = __builtin_nanf("");
    } else if (ft.r == DH) {
      cf = p.ca[h];
    } else {
      const int g1 = group_or_bad(p, h, ft.r);
      if (ft.t == DH) {
        cf = p.cb[h * p.G + g1] * 0.25f;  // 1 / sqrt(16)
      } else {
        const int g2 = group_or_bad(p, h, ft.t);
        cf = p.cc[(h * p.G + g1) * p.G + g2];
        if (ft.r != ft.t) cf += p.cc[(h * p.G + g2) * p.G + g1];
        cf *= 1.f / 16.f;  // 1 / d
      }
    }
    coef[f] = cf;
  }
}

struct __align__(16) LdsB {
  float st[D][NU];        // S before the chunk (forward) or R after it (reverse)
  float x[C][XE + 3];     // query rows (augmented, padded)
  float kk[C][XE + 3];    // key rows (augmented, padded)
  float u[C][NU];         // [v, 1] (zero rows past the end)
  float gg[C][NU];        // g rows (forward: computed here; reverse: from the workspace)
  float dy[C][DV];        // dL/dy rows (forward)
  float kap[C][C + 1];    // kappa_ij
  float dkap[C][C + 1];   // dkappa_ij
  float part[4][C][XE];   // per-wave partial gradients of q or k rows; also the dy . y partials
  float coef[D];
};

}  // namespace bw

// ---- forward direction: g, dq, dL/dcoef ----
template <bool BF16>
__global__ __launch_bounds__(bw::NT, 1) void bwd16_fwd_kernel(const bw::BwdArgs p) {
  using namespace bw;
  __shared__ LdsB sh;
  const int bh = blockIdx.x, h = bh % p.H;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int N = p.N;
  fill_coef(p, h, sh.coef);

  // S stays in LDS; thread (w, lane) is the only writer of S[f][lane] (and
  // lane 0 of S[f][64]) for the wave's features f = w, w + 4, ...
  for (int e = tid; e < D * NU; e += NT) (&sh.st[0][0])[e] = 0.f;
  float Pacc[kShare<0>];
#pragma unroll
  for (int m = 0; m < kShare<0>; ++m) Pacc[m] = 0.f;

  const long rb = (long)bh * N;
  for (int c = 0; c < p.nchunks; ++c) {
    const int j0 = c * C, nv = min(C, N - j0);
    // ---- stage the chunk ----
    for (int e = tid; e < C * XE; e += NT) {
      const int r = e / XE, d = e % XE;
      const bool ok = r < nv;
      sh.x[r][d] = d == DH ? (ok ? 1.f : 0.f) : (ok ? ld_act(p.q, (rb + j0 + r) * DH + d, BF16) : 0.f);
      sh.kk[r][d] = d == DH ? (ok ? 1.f : 0.f) : (ok ? ld_act(p.k, (rb + j0 + r) * DH + d, BF16) : 0.f);
    }
    for (int e = tid; e < C * NU; e += NT) {
      const int r = e / NU, d = e % NU;
      const bool ok = r < nv;
      sh.u[r][d] = !ok ? 0.f : d == DV ? 1.f : ld_act(p.v, (rb + j0 + r) * DV + d, BF16);
      if (d < DV) sh.dy[r][d] = ok ? ld_act(p.dy, (rb + j0 + r) * DV + d, BF16) : 0.f;
    }
    __syncthreads();

    // ---- per query row i = lane (a wave takes a quarter of the work) ----
    const int i = lane;
    float xq[XE];
#pragma unroll
    for (int d = 0; d < XE; ++d) xq[d] = sh.x[i][d];
    float cq[D];  // coef_f m_f(q_i)
    for_all([&](auto FC) {
      constexpr int f = decltype(FC)::value;
      constexpr Feat ft = feat16(f);
      cq[f] = sh.coef[f] * xq[ft.r] * xq[ft.t];
    });
    // kappa_ij for keys j = w, w + 4, ... up to i
    for (int j = w; j < C; j += 4) {
      float kap = 0.f;
      if (j <= i) {
        float xk[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xk[d] = sh.kk[j][d];
        for_all([&](auto FC) {
          constexpr int f = decltype(FC)::value;
          constexpr Feat ft = feat16(f);
          kap = fmaf(cq[f], xk[ft.r] * xk[ft.t], kap);
        });
      }
      sh.kap[i][j] = kap;
    }
    __syncthreads();
    // num over columns 16 w .. 16 w + 15, and den
    float num[16], den = 0.f;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) num[cc] = 0.f;
    for_all([&](auto FC) {
      constexpr int f = decltype(FC)::value;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) num[cc] = fmaf(cq[f], sh.st[f][16 * w + cc], num[cc]);
      den = fmaf(cq[f], sh.st[f][DV], den);
    });
    for (int j = 0; j <= i; ++j) {
      const float kij = sh.kap[i][j];
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) num[cc] = fmaf(kij, sh.u[j][16 * w + cc], num[cc]);
      den += kij;
    }
    const bool qok = i < nv;
    const float rden = qok ? 1.f / den : 0.f;
    float dyy = 0.f;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) dyy = fmaf(sh.dy[i][16 * w + cc], num[cc] * rden, dyy);
    sh.part[w][i][0] = dyy;
    __syncthreads();
    const float dden = qok ? -(sh.part[0][i][0] + sh.part[1][i][0] + sh.part[2][i][0] + sh.part[3][i][0]) * rden : 0.f;
#pragma unroll
    for (int cc = 0; cc < 16; ++cc) sh.gg[i][16 * w + cc] = sh.dy[i][16 * w + cc] * rden;
    if (w == 0) sh.gg[i][DV] = dden;
    if (qok) {
      float* gr = p.g + (rb + j0 + i) * NU;
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) gr[16 * w + cc] = sh.dy[i][16 * w + cc] * rden;
      if (w == 0) gr[DV] = dden;
    }
    __syncthreads();
    // dkappa_ij = g_i . u_j for keys j = w, w + 4, ... up to i
    for (int j = w; j < C; j += 4) {
      float dk = 0.f;
      if (j <= i)
        for (int cc = 0; cc < NU; ++cc) dk = fmaf(sh.gg[i][cc], sh.u[j][cc], dk);
      sh.dkap[i][j] = dk;
    }
    __syncthreads();
    // dL/dPhiQ_{i,f} for the wave's features: S g_i + sum_{j<=i} dkappa_ij m_f(k_j)
    float dqp[XE];
#pragma unroll
    for (int d = 0; d < XE; ++d) dqp[d] = 0.f;
    by_wave(w, [&](auto WC) {
      constexpr int W = decltype(WC)::value;
      float dphi[kShare<W>];
      {
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          float s = 0.f;
          for (int cc = 0; cc < NU; ++cc) s = fmaf(sh.st[f][cc], sh.gg[i][cc], s);
          dphi[m] = s;
        });
      }
      for (int j = 0; j <= i; ++j) {
        const float dk = sh.dkap[i][j];
        float xk[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xk[d] = sh.kk[j][d];
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          constexpr Feat ft = feat16(f);
          dphi[m] = fmaf(dk, xk[ft.r] * xk[ft.t], dphi[m]);
        });
      }
      for_share<W>([&](auto FC) {
        constexpr int f = decltype(FC)::value, m = (f - W) / 4;
        constexpr Feat ft = feat16(f);
        const float gd = qok ? dphi[m] : 0.f;
        Pacc[m] = fmaf(xq[ft.r] * xq[ft.t], gd, Pacc[m]);
        const float cg = sh.coef[f] * gd;
        // d m_f / d x_r = x_t (and d / d x_t = x_r); the appended 1 takes none
        dqp[ft.r] = fmaf(cg, xq[ft.t], dqp[ft.r]);
        dqp[ft.t] = fmaf(cg, xq[ft.r], dqp[ft.t]);
      });
    });
#pragma unroll
    for (int d = 0; d < DH; ++d) sh.part[w][i][d] = dqp[d];
    __syncthreads();
    if (qok)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int dd = 4 * w + d;
        p.dq[(rb + j0 + i) * DH + dd] = sh.part[0][i][dd] + sh.part[1][i][dd] + sh.part[2][i][dd] + sh.part[3][i][dd];
      }
    // ---- S takes the chunk's keys (owner: column lane, the wave's features) ----
    by_wave(w, [&](auto WC) {
      constexpr int W = decltype(WC)::value;
      float Sreg[kShare<W>], Zreg[kShare<W>];
      for_share<W>([&](auto FC) {
        constexpr int m = (decltype(FC)::value - W) / 4;
        Sreg[m] = Zreg[m] = 0.f;
      });
      for (int j = 0; j < nv; ++j) {
        float xk[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xk[d] = sh.kk[j][d];
        const float uj = sh.u[j][lane];
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          constexpr Feat ft = feat16(f);
          const float mk = xk[ft.r] * xk[ft.t];
          Sreg[m] = fmaf(mk, uj, Sreg[m]);
          Zreg[m] += mk;
        });
      }
      for_share<W>([&](auto FC) {
        constexpr int f = decltype(FC)::value, m = (f - W) / 4;
        sh.st[f][lane] += Sreg[m];
        if (lane == 0) sh.st[f][DV] += Zreg[m];
      });
    });
    __syncthreads();
  }
  // ---- dL/dcoef_f of this (sequence, head): the wave's 64 rows summed ----
  by_wave(w, [&](auto WC) {
    constexpr int W = decltype(WC)::value;
    for_share<W>([&](auto FC) {
      constexpr int f = decltype(FC)::value, m = (f - W) / 4;
      sh.st[f][lane] = Pacc[m];
    });
  });
  __syncthreads();
  for (int f = tid; f < D; f += NT) {
    float s = 0.f;
    for (int r = 0; r < kWave; ++r) s += sh.st[f][r];
    p.P[(long)bh * D + f] = s;
  }
}

// ---- reverse direction: dk, dv ----
template <bool BF16>
__global__ __launch_bounds__(bw::NT, 1) void bwd16_rev_kernel(const bw::BwdArgs p) {
  using namespace bw;
  __shared__ LdsB sh;
  const int bh = blockIdx.x, h = bh % p.H;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int N = p.N;
  fill_coef(p, h, sh.coef);

  // R stays in LDS; thread (w, lane) is the only writer of R[f][lane] (and
  // lane 0 of R[f][64]) for the wave's features f = w, w + 4, ...
  for (int e = tid; e < D * NU; e += NT) (&sh.st[0][0])[e] = 0.f;

  const long rb = (long)bh * N;
  for (int c = p.nchunks - 1; c >= 0; --c) {
    const int j0 = c * C, nv = min(C, N - j0);
    for (int e = tid; e < C * XE; e += NT) {
      const int r = e / XE, d = e % XE;
      const bool ok = r < nv;
      sh.x[r][d] = d == DH ? (ok ? 1.f : 0.f) : (ok ? ld_act(p.q, (rb + j0 + r) * DH + d, BF16) : 0.f);
      sh.kk[r][d] = d == DH ? (ok ? 1.f : 0.f) : (ok ? ld_act(p.k, (rb + j0 + r) * DH + d, BF16) : 0.f);
    }
    for (int e = tid; e < C * NU; e += NT) {
      const int r = e / NU, d = e % NU;
      const bool ok = r < nv;
      sh.u[r][d] = !ok ? 0.f : d == DV ? 1.f : ld_act(p.v, (rb + j0 + r) * DV + d, BF16);
      sh.gg[r][d] = ok ? p.g[(rb + j0 + r) * NU + d] : 0.f;
    }
    __syncthreads();

    // ---- per key row j = lane ----
    const int j = lane;
    float xk[XE];
#pragma unroll
    for (int d = 0; d < XE; ++d) xk[d] = sh.kk[j][d];
    float ck[D];  // coef_f m_f(k_j)
    for_all([&](auto FC) {
      constexpr int f = decltype(FC)::value;
      constexpr Feat ft = feat16(f);
      ck[f] = sh.coef[f] * xk[ft.r] * xk[ft.t];
    });
    // kappa_ij and dkappa_ij for queries i = w, w + 4, ... from j on
    for (int i = w; i < C; i += 4) {
      float kap = 0.f, dk = 0.f;
      if (i >= j) {
        float xq[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xq[d] = sh.x[i][d];
        for_all([&](auto FC) {
          constexpr int f = decltype(FC)::value;
          constexpr Feat ft = feat16(f);
          kap = fmaf(ck[f], xq[ft.r] * xq[ft.t], kap);
        });
        for (int cc = 0; cc < NU; ++cc) dk = fmaf(sh.gg[i][cc], sh.u[j][cc], dk);
      }
      sh.kap[j][i] = kap;
      sh.dkap[j][i] = dk;
    }
    __syncthreads();
    // dv_j, columns 16 w .. 16 w + 15: R^T m(k_j) + sum_{i>=j} kappa_ij g_i
    const bool kok = j < nv;
    {
      float du[16];
#pragma unroll
      for (int cc = 0; cc < 16; ++cc) du[cc] = 0.f;
      for_all([&](auto FC) {
        constexpr int f = decltype(FC)::value;
        constexpr Feat ft = feat16(f);
        const float mk = xk[ft.r] * xk[ft.t];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) du[cc] = fmaf(mk, sh.st[f][16 * w + cc], du[cc]);
      });
      for (int i = j; i < C; ++i) {
        const float kij = sh.kap[j][i];
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) du[cc] = fmaf(kij, sh.gg[i][16 * w + cc], du[cc]);
      }
      if (kok)
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) p.dv[(rb + j0 + j) * DV + 16 * w + cc] = du[cc];
    }
    // dL/dPhiK_{j,f} for the wave's features: R u_j + coef_f sum_{i>=j} dkappa_ij m_f(q_i)
    float dkp[XE];
#pragma unroll
    for (int d = 0; d < XE; ++d) dkp[d] = 0.f;
    by_wave(w, [&](auto WC) {
      constexpr int W = decltype(WC)::value;
      float dphi[kShare<W>];
      for_share<W>([&](auto FC) { dphi[(decltype(FC)::value - W) / 4] = 0.f; });
      for (int i = j; i < C; ++i) {
        const float dk = sh.dkap[j][i];
        float xq[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xq[d] = sh.x[i][d];
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          constexpr Feat ft = feat16(f);
          dphi[m] = fmaf(dk, xq[ft.r] * xq[ft.t], dphi[m]);
        });
      }
      for_share<W>([&](auto FC) {
        constexpr int f = decltype(FC)::value, m = (f - W) / 4;
        dphi[m] *= sh.coef[f];
      });
      for (int cc = 0; cc < NU; ++cc) {
        const float uc = sh.u[j][cc];
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          dphi[m] = fmaf(sh.st[f][cc], uc, dphi[m]);
        });
      }
      for_share<W>([&](auto FC) {
        constexpr int f = decltype(FC)::value, m = (f - W) / 4;
        constexpr Feat ft = feat16(f);
        const float gd = kok ? dphi[m] : 0.f;
        dkp[ft.r] = fmaf(gd, xk[ft.t], dkp[ft.r]);
        dkp[ft.t] = fmaf(gd, xk[ft.r], dkp[ft.t]);
      });
    });
#pragma unroll
    for (int d = 0; d < DH; ++d) sh.part[w][j][d] = dkp[d];
    __syncthreads();
    if (kok)
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const int dd = 4 * w + d;
        p.dk[(rb + j0 + j) * DH + dd] = sh.part[0][j][dd] + sh.part[1][j][dd] + sh.part[2][j][dd] + sh.part[3][j][dd];
      }
    // ---- R takes the chunk's queries: coef_f m_f(q_i) g_i^T ----
    by_wave(w, [&](auto WC) {
      constexpr int W = decltype(WC)::value;
      float Rreg[kShare<W>], Rz[kShare<W>];
      for_share<W>([&](auto FC) {
        constexpr int m = (decltype(FC)::value - W) / 4;
        Rreg[m] = Rz[m] = 0.f;
      });
      for (int i = 0; i < nv; ++i) {
        float xq[XE];
#pragma unroll
        for (int d = 0; d < XE; ++d) xq[d] = sh.x[i][d];
        const float gi = sh.gg[i][lane], gz = sh.gg[i][DV];
        for_share<W>([&](auto FC) {
          constexpr int f = decltype(FC)::value, m = (f - W) / 4;
          constexpr Feat ft = feat16(f);
          const float mq = sh.coef[f] * xq[ft.r] * xq[ft.t];
          Rreg[m] = fmaf(mq, gi, Rreg[m]);
          Rz[m] = fmaf(mq, gz, Rz[m]);
        });
      }
      for_share<W>([&](auto FC) {
        constexpr int f = decltype(FC)::value, m = (f - W) / 4;
        sh.st[f][lane] += Rreg[m];
        if (lane == 0) sh.st[f][DV] += Rz[m];
      });
    });
    __syncthreads();
  }
}

// ---- dL/dcoef_f -> da, db, dc, summed over the batch (one workgroup per head) ----
__global__ __launch_bounds__(256) void bwd16_coef_kernel(const bw::BwdArgs p, int B, float* __restrict__ da,
                                                         float* __restrict__ db, float* __restrict__ dc) {
  using namespace bw;
  __shared__ float Ps[D];
  __shared__ int gr[DH];
  __shared__ int nbad;
  const int h = blockIdx.x, G = p.G;
  if (threadIdx.x == 0) nbad = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < D; f += blockDim.x) {
    float s = 0.f;
    for (int b = 0; b < B; ++b) s += p.P[((long)b * p.H + h) * D + f];
    Ps[f] = s;
  }
  if (threadIdx.x < DH) {
    gr[threadIdx.x] = group_or_bad(p, h, threadIdx.x);
    if (gr[threadIdx.x] < 0) atomicAdd(&nbad, 1);
  }
  __syncthreads();
  // entry e: 0 -> a; 1 .. G -> b_g; then c_gh (ordered)
  for (int e = threadIdx.x; e < 1 + G + G * G; e += blockDim.x) {
    float s = 0.f;
    if (e == 0) {
      s = Ps[0];
    } else if (e <= G) {
      const int g = e - 1;
      for (int r = 0; r < DH; ++r)
        if (gr[r] == g) s += Ps[1 + r];
      s *= 0.25f;  // 1 / sqrt(d)
    } else {
      const int g = (e - 1 - G) / G, hh = (e - 1 - G) % G;
      for (int f = 1 + DH; f < D; ++f) {
        const Feat ft = feat16(f);
        const int g1 = gr[ft.r], g2 = gr[ft.t];
        float mult = (g1 == g && g2 == hh) ? 1.f : 0.f;
        if (ft.r != ft.t && g2 == g && g1 == hh) mult += 1.f;
        s = fmaf(mult, Ps[f], s);
      }
      s *= 1.f / 16.f;  // 1 / d
    }
    if (nbad > 0) s = __builtin_nanf("");
    if (e == 0) da[h] = s;
    else if (e <= G) db[h * G + e - 1] = s;
    else dc[h * G * G + (e - 1 - G)] = s;
  }
}

}  // namespace

bool bwd16_supported(int d_h, int d_v, int dtype, bool diagonal, int G, int Hq, int Hkv) {
  return d_h == 16 && d_v == 64 && (dtype == 0 || dtype == 1) && !diagonal && G >= 1 && G <= 16 && Hq == Hkv;
}

size_t bwd16_workspace_bytes(int B, int H, int N) {
  const size_t g = (size_t)B * H * N * bw::NU * sizeof(float);
  return (g + 255) / 256 * 256 + (size_t)B * H * bw::D * sizeof(float);
}

hipError_t launch_bwd16(const BwdLaunch& a, hipStream_t stream) {
  bw::BwdArgs p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.dy = a.dy;
  p.group_of_dim = a.group_of_dim; p.ca = a.ca; p.cb = a.cb; p.cc = a.cc;
  p.G = a.G; p.H = a.H; p.N = a.N;
  p.nchunks = (a.N + bw::C - 1) / bw::C;
  const size_t gbytes = ((size_t)a.B * a.H * a.N * bw::NU * sizeof(float) + 255) / 256 * 256;
  p.g = reinterpret_cast<float*>(a.workspace);
  p.P = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + gbytes);
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv;
  const dim3 grid(a.B * a.H);
  // with no sequences only the coefficient kernel runs (it writes zeros)
  if (a.B > 0 && a.dtype == 1) {
    hipLaunchKernelGGL((bwd16_fwd_kernel<true>), grid, dim3(bw::NT), 0, stream, p);
    hipLaunchKernelGGL((bwd16_rev_kernel<true>), grid, dim3(bw::NT), 0, stream, p);
  } else if (a.B > 0) {
    hipLaunchKernelGGL((bwd16_fwd_kernel<false>), grid, dim3(bw::NT), 0, stream, p);
    hipLaunchKernelGGL((bwd16_rev_kernel<false>), grid, dim3(bw::NT), 0, stream, p);
  }
  hipLaunchKernelGGL(bwd16_coef_kernel, dim3(a.H), dim3(256), 0, stream, p, a.B, a.da, a.db, a.dc);
  return hipGetLastError();
}

}  // namespace oal
