// Backward pass of the causal normalised OAL attention at d_h = 16, d_v = 64,
// for heads with their own keys and values: the gradients of a loss L with
// dL/dy given, with respect to q, k, v and the kernel coefficients
// (a, b_g, c_gh).  The calibration of the OAL paper fits L (App. B, Eq. (20),
// the output-matching objective) and its adaptation trains the coefficients
// jointly with LoRA (App. F.2); both need these gradients through the causal
// evaluation of Eqs. (5)-(6).
//
// In the packed feature space of the forward pass (App. D: 153 features
// [1, x_r, x_r x_t (r <= t)] at d_h = 16, padded here to 160) the kernel is
//     kappa(q, k) = sum_f coef_f m_f(q) m_f(k),
// m_f the feature's monomial (1, x_r or x_r x_t) and coef_f = a, b_g(r) /
// sqrt(d) or (c_g(r)g(t) + c_g(t)g(r)) / d (c_g(r)g(r) / d on the diagonal).
// With Phi = coef * m(q) per query row, M = m(k) per key row, u_j = [v_j, 1],
// y_i = num_i / den_i and g_i = dL/d[num_i, den_i] =
// [dy_i / den_i, -(dy_i . y_i) / den_i]:
//     dkappa_ij   = g_i . u_j                          (j <= i)
//     dL/dPhi_i   = S_i g_i,  S_i = sum_{j<=i} m(k_j) u_j^T     -> dq, dL/dcoef
//     dL/dm(k_j)  = R_j u_j,  R_j = sum_{i>=j} Phi_i g_i^T      -> dk
//     dL/du_j     = R_j^T m(k_j)                               -> dv
//     dL/dcoef_f  = sum_i m_f(q_i) [dL/dPhi_i]_f
// and dq, dk follow through the monomials.
//
// Work is cut into 32-token chunks and every contraction of a chunk runs on
// fp32 matrix cores (v_mfma_f32_16x16x4_f32; all operands staged in LDS):
//   forward direction, per chunk: kappa = Phi M^T, num = Phi S + kappa U,
//     dkappa = G U^T + gden, dL/dPhi = G S^T + dkappa M + gden z^T, S += M^T U;
//   reverse direction: kappa, dkappa as above, dL/du = M R + kappa^T G,
//     dL/dm(k) = U R^T + dkappa^T Phi + Rz^T, R += Phi^T G.
// The normaliser columns (z = sum m(k), Rz = sum Phi gden, den) and the chain
// rule through the monomials are vector work.  Sequences are cut into
// segments that run in parallel: a segment starts from the sum of the
// earlier segments' key sums (forward direction) or the later segments'
// query sums (reverse direction), which two short passes compute first.  A
// last kernel maps the per-feature sums to da, db, dc (summed over the
// batch).  All arithmetic is fp32.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {
namespace {
namespace bw {

constexpr int DH = 16;
constexpr int DV = 64;
constexpr int C = 32;       // tokens per chunk
constexpr int D = 153;      // packed features at d_h = 16
constexpr int DP = 160;     // padded to ten 16-row blocks
constexpr int NFB = DP / 16;
constexpr int NT = 256;     // four waves
constexpr int XS = 20;      // augmented row [x_0 .. x_15, 1, 0, 0, 0]
constexpr int XONE = 16;    // index of the constant 1
constexpr int XZERO = 17;   // index of a constant 0 (padding features)
constexpr int FS = 164;     // row stride of [C][DP] tiles
constexpr int VS = 68;      // row stride of [C][DV] tiles
constexpr int SS = 68;      // row stride of the [DP][DV] state
constexpr int KS = 36;      // row stride of [C][C] tiles
constexpr int SEGF = DP * (DV + 1);  // one segment sum: [DP][DV] then [DP]
constexpr int kMaxSeg = 8;

typedef float f4 __attribute__((ext_vector_type(4)));

// one 16x16x4 fp32 product: lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16]; the accumulator holds D[4 (l / 16) + r][l % 16]
__device__ __forceinline__ f4 mma(float a, float b, f4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Operands along K: a K-block kb of 16 is taken as four steps e = 0..3 in
// which lane group g = lane / 16 supplies k = 16 kb + 4 g + e, so an operand
// stored contiguously along K loads as one 16-byte LDS read per four
// products, and an accumulator tile (lane group g holds rows 4 g .. 4 g + 3)
// is, unchanged, the B operand of the K-block it covers.
__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float el(const float4& v, int e) { return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w; }

// Feature f of the library's packed order as a pair of indices into the
// augmented row: f = 0 the constant (16, 16), f = 1 + r the linear term
// (r, 16), then the pairs r <= t row by row; padding features (17, 17).
struct Feat {
  int r, t;
};
__host__ __device__ constexpr Feat feat16(int f) {
  if (f >= D) return Feat{XZERO, XZERO};
  if (f == 0) return Feat{XONE, XONE};
  if (f <= DH) return Feat{f - 1, XONE};
  int idx = f - 1 - DH, r = 0;
  while (idx >= DH - r) {
    idx -= DH - r;
    ++r;
  }
  return Feat{r, r + idx};
}
// feature of the pair (r, t), r <= t
__device__ __forceinline__ int pair_feature(int r, int t) { return 1 + DH + DH * r - r * (r - 1) / 2 + (t - r); }

struct BwdArgs {
  const void *q, *k, *v, *dy;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  int G, H, N, nchunks, nseg, cps;  // cps: chunks per segment
  int nsub, cpsub;                  // parts per segment in the segment sums, chunks per part
  float* g;     // [B H, N, 64] workspace: dL/dnum rows
  float* gden;  // [B H, N] workspace: dL/dden
  float* seg;   // [B H, nseg, nsub, SEGF] workspace: segment sums (S, then R)
  float* P;     // [B H, nseg, DP] workspace: dL/dcoef_f per segment
  float *dq, *dk, *dv;
};

// group of dimension r of head h; -1 when the id is outside [0, G)
__device__ __forceinline__ int group_or_bad(const BwdArgs& p, int h, int r) {
  const int g = p.group_of_dim[h * DH + r];
  return g >= 0 && g < p.G ? g : -1;
}

// coef_f of head h (thread-parallel);
// a group id outside [0, G) makes every coefficient of the head NaN, so that
// all of its outputs are NaN
__device__ void fill_tables(const BwdArgs& p, int h, float* coef) {
  bool bad = false;
  for (int r = 0; r < DH; ++r) bad |= group_or_bad(p, h, r) < 0;
  for (int f = threadIdx.x; f < DP; f += NT) {
    const Feat fe = feat16(f);
    float cf;
    if (f >= D) {
      cf = 0.f;
    } else if (bad) {
      cf = __builtin_nanf("");
    } else if (fe.r == XONE) {
      cf = p.ca[h];
    } else {
      const int g1 = group_or_bad(p, h, fe.r);
      if (fe.t == XONE) {
        cf = p.cb[h * p.G + g1] * 0.25f;  // 1 / sqrt(16)
      } else {
        const int g2 = group_or_bad(p, h, fe.t);
        cf = p.cc[(h * p.G + g1) * p.G + g2];
        if (fe.r != fe.t) cf += p.cc[(h * p.G + g2) * p.G + g1];
        cf *= 1.f / 16.f;  // 1 / d
      }
    }
    coef[f] = cf;
  }
}

// Four elements of an activation row, fetched into registers ahead of use
// (bf16: two words; fp32: four) and unpacked when stored to LDS.
template <bool BF16>
struct Raw4 {
  uint32_t w[BF16 ? 2 : 4];
};

template <bool BF16>
__device__ __forceinline__ void fetch4(Raw4<BF16>& d, const void* base, long e, bool ok) {
#pragma unroll
  for (int k = 0; k < (BF16 ? 2 : 4); ++k) d.w[k] = 0u;
  if (!ok) return;
  if (BF16) {
    const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(base) + e);
    d.w[0] = x.x;
    d.w[1] = x.y;
  } else {
    const uint4 x = *reinterpret_cast<const uint4*>(reinterpret_cast<const float*>(base) + e);
    d.w[0] = x.x; d.w[1] = x.y; d.w[2] = x.z; d.w[3] = x.w;
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack4(const Raw4<BF16>& d, float* dst) {
  if (BF16) {
    dst[0] = __uint_as_float(d.w[0] << 16);
    dst[1] = __uint_as_float(d.w[0] & 0xffff0000u);
    dst[2] = __uint_as_float(d.w[1] << 16);
    dst[3] = __uint_as_float(d.w[1] & 0xffff0000u);
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) dst[k] = __uint_as_float(d.w[k]);
  }
}

// Shared staging of a chunk: query rows, key rows and the value rows (rows
// at and past nv are zero, including the constant 1 of the augmented rows).
struct __align__(16) Rows {
  float xq[C][XS], xk[C][XS];
  float phq[C][FS];  // coef * m(q); forward direction later coef * dL/dPhi
  float mk[C][FS];   // m(k); reverse direction later dL/dm(k)
  float u[C][VS];    // v
  float gg[C][VS];   // dL/dnum rows
};

template <bool BF16>
__device__ __forceinline__ void fetch_qk(Raw4<BF16>& d, const BwdArgs& p, long row0, int nv, bool want_q,
                                         bool want_k) {
  const int t = threadIdx.x & 127;
  const bool isk = threadIdx.x >= 128;
  const int r = t >> 2, d0 = (t & 3) * 4;
  fetch4<BF16>(d, isk ? p.k : p.q, (row0 + r) * DH + d0, r < nv && (isk ? want_k : want_q));
}

template <bool BF16>
__device__ __forceinline__ void store_qk(Rows& s, const Raw4<BF16>& d, int nv) {
  const int t = threadIdx.x & 127;
  const bool isk = threadIdx.x >= 128;
  const int r = t >> 2, d0 = (t & 3) * 4;
  float x[4];
  unpack4<BF16>(d, x);
  float* dst = isk ? s.xk[r] : s.xq[r];
#pragma unroll
  for (int e = 0; e < 4; ++e) dst[d0 + e] = x[e];
  dst[XONE + (t & 3)] = (t & 3) == 0 && r < nv ? 1.f : 0.f;
}

// eight elements of row threadIdx / 8 of a [C][64] operand
template <bool BF16>
__device__ __forceinline__ void fetch_v64(Raw4<BF16> (&d)[2], const void* src, long row0, int nv) {
  const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 8;
  fetch4<BF16>(d[0], src, (row0 + r) * DV + c0, r < nv);
  fetch4<BF16>(d[1], src, (row0 + r) * DV + c0 + 4, r < nv);
}

template <bool BF16>
__device__ __forceinline__ void store_v64(float (*dst)[VS], const Raw4<BF16> (&d)[2]) {
  const int r = threadIdx.x >> 3, c0 = (threadIdx.x & 7) * 8;
  float x[8];
  unpack4<BF16>(d[0], x);
  unpack4<BF16>(d[1], x + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) dst[r][c0 + e] = x[e];
}

__device__ __forceinline__ float fetch_gden(const BwdArgs& p, long row0, int nv) {
  return (int)threadIdx.x < nv ? p.gden[row0 + threadIdx.x] : 0.f;
}

// The index pairs of every padded feature, as a compile-time table.
struct FeatTable {
  Feat e[DP];
};
constexpr FeatTable make_feat_table() {
  FeatTable t{};
  for (int f = 0; f < DP; ++f) t.e[f] = feat16(f);
  return t;
}
constexpr FeatTable kFeat = make_feat_table();

// Features [40 QQ, 40 QQ + 40) of one staged row x (20 floats in LDS) into
// dst, scaled by coef when asked (the plain monomials also into dst2 when
// given): the row is read once into registers and every product has its
// operand indices fixed at compile time, so the lanes of a wave (one row
// each) run one instruction stream.
template <int QQ>
__device__ __forceinline__ void features_quarter(const float* x, const float* coef, bool scale, float* dst,
                                                 float* dst2) {
  float xr[XS];
#pragma unroll
  for (int e = 0; e < XS; e += 4) {
    const float4 v = *reinterpret_cast<const float4*>(x + e);
    xr[e] = v.x; xr[e + 1] = v.y; xr[e + 2] = v.z; xr[e + 3] = v.w;
  }
#pragma unroll
  for (int e = 0; e < 40; e += 4) {
    float m[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = xr[kFeat.e[40 * QQ + e + k].r] * xr[kFeat.e[40 * QQ + e + k].t];
    const float4 cf = *reinterpret_cast<const float4*>(coef + 40 * QQ + e);
    const float4 o = scale ? make_float4(cf.x * m[0], cf.y * m[1], cf.z * m[2], cf.w * m[3])
                           : make_float4(m[0], m[1], m[2], m[3]);
    *reinterpret_cast<float4*>(dst + 40 * QQ + e) = o;
    if (dst2 != nullptr) *reinterpret_cast<float4*>(dst2 + 40 * QQ + e) = make_float4(m[0], m[1], m[2], m[3]);
  }
}

// Phi (coef-scaled query features, and the plain query monomials into mq
// when given) and/or M (key features) of the staged rows: wave w takes the
// feature quarter w, lanes 0..31 the query rows and 32..63 the key rows.
__device__ __forceinline__ void build_features(Rows& s, const float* coef, bool want_q, bool want_k,
                                               float (*mq)[FS] = nullptr) {
  const int lane = threadIdx.x & 63, i = lane & 31;
  const bool isk = lane >= 32;
  if (isk ? !want_k : !want_q) return;
  const float* x = isk ? s.xk[i] : s.xq[i];
  float* dst = isk ? s.mk[i] : s.phq[i];
  float* dst2 = !isk && mq != nullptr ? mq[i] : nullptr;
  switch (__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)) {
    case 0: features_quarter<0>(x, coef, !isk, dst, dst2); break;
    case 1: features_quarter<1>(x, coef, !isk, dst, dst2); break;
    case 2: features_quarter<2>(x, coef, !isk, dst, dst2); break;
    default: features_quarter<3>(x, coef, !isk, dst, dst2); break;
  }
}

// Sums over aligned groups of 8 or 16 consecutive lanes by DPP moves
// (quad swaps, then the half-row and row mirrors).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp_mov<0xb1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4e>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  return x;
}
__device__ __forceinline__ float sum16(float x) {
  x = sum8(x);
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// kappa (Phi M^T) tile (rb, cb) of the chunk, masked to j <= i, into kap;
// the all-masked tile (0, 1) is written as zeros
__device__ __forceinline__ void kappa_tile(const Rows& s, float (*kap)[KS], int rb, int cb, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
  if (rb == 0 && cb == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) kap[4 * g + r][16 + i16] = 0.f;
    return;
  }
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 5
  for (int kb = 0; kb < NFB; ++kb) {
    const float4 a = ld4(&s.phq[16 * rb + i16][16 * kb + 4 * g]), b = ld4(&s.mk[16 * cb + i16][16 * kb + 4 * g]);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mma(el(a, e), el(b, e), acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * rb + 4 * g + r, j = 16 * cb + i16;
    kap[i][j] = j <= i ? acc[r] : 0.f;
  }
}

// dkappa tile (rb, cb) = G U^T + gden_i [j valid], masked to j <= i; gd4:
// gden of the lane's four rows 16 rb + 4 (lane / 16) + r
__device__ __forceinline__ void dkappa_tile(const Rows& s, const float (&gd4)[4], float (*dkap)[KS], int rb, int cb,
                                            int nv, int lane) {
  const int i16 = lane & 15, g = lane >> 4;
  if (rb == 0 && cb == 1) {
#pragma unroll
    for (int r = 0; r < 4; ++r) dkap[4 * g + r][16 + i16] = 0.f;
    return;
  }
  f4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < DV / 16; ++kb) {
    const float4 a = ld4(&s.gg[16 * rb + i16][16 * kb + 4 * g]), b = ld4(&s.u[16 * cb + i16][16 * kb + 4 * g]);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = mma(el(a, e), el(b, e), acc);
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int i = 16 * rb + 4 * g + r, j = 16 * cb + i16;
    dkap[i][j] = j <= i && j < nv ? acc[r] + gd4[r] : 0.f;
  }
}

// chain rule through the monomials: w[f] = dL/dm_f of row x (d m_f/d x_r =
// x_t and d/d x_t = x_r; the constant 1 and the padding take none)
__device__ __forceinline__ float chain_rule(const float* w, const float* x, int r) {
  float s = w[1 + r];  // linear feature (r, 1)
#pragma unroll
  for (int t = 0; t < DH; ++t) {
    const int f = t < r ? pair_feature(t, r) : pair_feature(r, t);
    s = fmaf(t == r ? 2.f * w[f] : w[f], x[t], s);
  }
  return s;
}

struct __align__(16) LdsFwd {
  Rows rows;
  float mq[C][FS];   // m(q) of the chunk's queries
  float st[DP][SS];  // S before the chunk (v columns)
  float z[DP];       // its normaliser column
  float dy[C][VS];
  float kap[C][KS], dkap[C][KS];
  float rden[C], gden[C];
  float red[4][C];
  float coef[DP];
};

struct __align__(16) LdsRev {
  Rows rows;
  float st[DP][SS];  // R after the chunk (v columns)
  float z[DP];       // its normaliser column Rz
  float kap[C][KS], dkap[C][KS];
  float gden[C];
  float coef[DP];
};

struct __align__(16) LdsSeg {
  Rows rows;
  float gden[C];
  float coef[DP];
};

}  // namespace bw

// ---- segment sums: S (MODE 0, key sums, for every segment but the last) or
// R (MODE 1, query sums with g, for every segment but the first), each
// segment cut into nsub parts summed by their own workgroups ----
template <int MODE, bool BF16>
__global__ __launch_bounds__(bw::NT, 1) void bwd16_segsum_kernel(const bw::BwdArgs p) {
  using namespace bw;
  __shared__ LdsSeg sh;
  const int sub = blockIdx.x % p.nsub, seg = (blockIdx.x / p.nsub) % p.nseg, bh = blockIdx.x / (p.nsub * p.nseg);
  const int h = bh % p.H;
  if (MODE == 0 ? seg == p.nseg - 1 : seg == 0) return;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int i16 = lane & 15, g = lane >> 4;
  fill_tables(p, h, sh.coef);
  const int send = min(seg * p.cps + p.cps, p.nchunks);
  const int c0 = min(seg * p.cps + sub * p.cpsub, send), c1 = min(c0 + p.cpsub, send);
  const long rbase = (long)bh * p.N;
  f4 acc[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) acc[fb] = f4{0.f, 0.f, 0.f, 0.f};
  float zacc = 0.f;  // thread f < DP: the normaliser column
  Raw4<BF16> fqk, fv[2];
  Raw4<false> fg[2];
  float fgd = 0.f;
  auto fetch = [&](int c) {
    const int nv = min(C, p.N - c * C);
    const long row0 = rbase + (long)c * C;
    fetch_qk<BF16>(fqk, p, row0, nv, MODE == 1, MODE == 0);
    if (MODE == 0) {
      fetch_v64<BF16>(fv, p.v, row0, nv);
    } else {
      fetch_v64<false>(fg, p.g, row0, nv);
      fgd = fetch_gden(p, row0, nv);
    }
  };
  if (c0 < c1) fetch(c0);
  for (int c = c0; c < c1; ++c) {
    const int nv = min(C, p.N - c * C);
    __syncthreads();  // the previous chunk's reads are done
    store_qk<BF16>(sh.rows, fqk, nv);
    if (MODE == 0) {
      store_v64<BF16>(sh.rows.u, fv);
    } else {
      store_v64<false>(sh.rows.gg, fg);
      if (tid < C) sh.gden[tid] = fgd;
    }
    if (c + 1 < c1) fetch(c + 1);
    __syncthreads();
    build_features(sh.rows, sh.coef, MODE == 1, MODE == 0);
    __syncthreads();
    // columns 16 w .. 16 w + 15 of sum_j feat_j w_j^T over the chunk
    const float(*fe)[FS] = MODE == 0 ? sh.rows.mk : sh.rows.phq;
    const float(*wv)[VS] = MODE == 0 ? sh.rows.u : sh.rows.gg;
#pragma unroll
    for (int ks = 0; ks < C / 4; ++ks) {
      const float b = wv[4 * ks + g][16 * w + i16];
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) acc[fb] = mma(fe[4 * ks + g][16 * fb + i16], b, acc[fb]);
    }
    if (tid < DP) {
      float s = 0.f;  // rows past nv are zero in both feature tiles
      for (int j = 0; j < C; ++j) s = fmaf(fe[j][tid], MODE == 0 ? 1.f : sh.gden[j], s);
      zacc += s;
    }
  }
  float* out = p.seg + (((long)bh * p.nseg + seg) * p.nsub + sub) * SEGF;
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[(16 * fb + 4 * g + r) * DV + 16 * w + i16] = acc[fb][r];
  if (tid < DP) out[DP * DV + tid] = zacc;
}

// the sums of segments [s0, s1) (all their parts) into this wave's columns
// of a [DP][DV] state held as accumulators, and the normaliser column
__device__ __forceinline__ void gather_segments(const bw::BwdArgs& p, int bh, int s0, int s1, bw::f4 (&acc)[bw::NFB],
                                                float& zs, int w, int lane) {
  using namespace bw;
  const int i16 = lane & 15, g = lane >> 4;
  for (int s = s0 * p.nsub; s < s1 * p.nsub; ++s) {
    const float* src = p.seg + ((long)bh * p.nseg * p.nsub + s) * SEGF;
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[fb][r] += src[(16 * fb + 4 * g + r) * DV + 16 * w + i16];
    if (threadIdx.x < DP) zs += src[DP * DV + threadIdx.x];
  }
}

// ---- forward direction: g, dq, dL/dcoef ----
template <bool BF16>
__global__ __launch_bounds__(bw::NT, 1) void bwd16_fwd_kernel(const bw::BwdArgs p) {
  using namespace bw;
  __shared__ LdsFwd sh;
  Rows& R = sh.rows;
  const int bh = blockIdx.x / p.nseg, seg = blockIdx.x % p.nseg, h = bh % p.H;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int i16 = lane & 15, g = lane >> 4;
  fill_tables(p, h, sh.coef);
  const int c0 = seg * p.cps, c1 = min(c0 + p.cps, p.nchunks);
  const long rbase = (long)bh * p.N;

  // S at the segment start: the earlier segments' key sums; wave w keeps
  // columns 16 w .. 16 w + 15 in its accumulators
  f4 accS[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) accS[fb] = f4{0.f, 0.f, 0.f, 0.f};
  float zs = 0.f;
  gather_segments(p, bh, 0, seg, accS, zs, w, lane);
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sh.st[16 * fb + 4 * g + r][16 * w + i16] = accS[fb][r];
  if (tid < DP) sh.z[tid] = zs;

  // tiles of this wave: kappa / dkappa (krb, kcb); the outputs' column block
  // w; dL/dPhi rows prb, feature blocks (w >> 1) + 2 m
  const int krb = w >> 1, kcb = w & 1, prb = w & 1;
  float pacc[5] = {0.f, 0.f, 0.f, 0.f, 0.f};

  Raw4<BF16> fqk, fv[2], fd[2];
  auto fetch = [&](int c) {
    const int nv = min(C, p.N - c * C);
    const long row0 = rbase + (long)c * C;
    fetch_qk<BF16>(fqk, p, row0, nv, true, true);
    fetch_v64<BF16>(fv, p.v, row0, nv);
    fetch_v64<BF16>(fd, p.dy, row0, nv);
  };
  if (c0 < c1) fetch(c0);
  for (int c = c0; c < c1; ++c) {
    const int j0 = c * C, nv = min(C, p.N - j0);
    const long row0 = rbase + j0;
    __syncthreads();  // the previous chunk is done with every tile
    store_qk<BF16>(R, fqk, nv);
    store_v64<BF16>(R.u, fv);
    store_v64<BF16>(sh.dy, fd);
    if (c + 1 < c1) fetch(c + 1);
    __syncthreads();
    build_features(R, sh.coef, true, true, sh.mq);
    __syncthreads();
    // kappa; num against S before the chunk
    kappa_tile(R, sh.kap, krb, kcb, lane);
    f4 accY[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb) {  // B: this wave's columns of S, from its accumulators
      const float4 a0 = ld4(&R.phq[i16][16 * fb + 4 * g]), a1 = ld4(&R.phq[16 + i16][16 * fb + 4 * g]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        accY[0] = mma(el(a0, e), accS[fb][e], accY[0]);
        accY[1] = mma(el(a1, e), accS[fb][e], accY[1]);
      }
    }
    __syncthreads();
    // num += kappa U over the chunk; den = Phi z + sum_j kappa_ij
#pragma unroll
    for (int ks = 0; ks < C / 4; ++ks) {
      const float b = R.u[4 * ks + g][16 * w + i16];
      if (ks < 4) accY[0] = mma(sh.kap[i16][4 * ks + g], b, accY[0]);
      accY[1] = mma(sh.kap[16 + i16][4 * ks + g], b, accY[1]);
    }
    {
      const int i = tid >> 3, pp = tid & 7;
      float s = 0.f;
#pragma unroll
      for (int m = 0; m < DP / 8; ++m) s = fmaf(R.phq[i][pp + 8 * m], sh.z[pp + 8 * m], s);
#pragma unroll
      for (int m = 0; m < C / 8; ++m) s += sh.kap[i][pp + 8 * m];
      s = sum8(s);
      if (pp == 0) sh.rden[i] = i < nv ? 1.f / s : 0.f;
    }
    __syncthreads();
    // y, dy . y, g = dy / den
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * rb + 4 * g + r, col = 16 * w + i16;
        const float rd = sh.rden[i], dyv = sh.dy[i][col];
        const float part = sum16(dyv * (accY[rb][r] * rd));
        if (i16 == 0) sh.red[w][i] = part;
        const float gv = dyv * rd;
        R.gg[i][col] = gv;
        if (i < nv) p.g[(row0 + i) * DV + col] = gv;
      }
    __syncthreads();
    // gden = -(dy . y) / den, by every lane for the rows of its tiles
    {
      auto gden_of = [&](int i) {
        return -(sh.red[0][i] + sh.red[1][i] + sh.red[2][i] + sh.red[3][i]) * sh.rden[i];
      };
      float gd4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) gd4[r] = gden_of(16 * krb + 4 * g + r);
      dkappa_tile(R, gd4, sh.dkap, krb, kcb, nv, lane);
      if (tid < C) {
        const float gd = gden_of(tid);  // zero past nv (rden is zero there)
        sh.gden[tid] = gd;
        if (tid < nv) p.gden[row0 + tid] = gd;
      }
    }
    __syncthreads();
    // dL/dPhi = G S^T + dkappa M + gden z^T; P += m(q) . dL/dPhi; coef * dL/dPhi -> phq
    {
      f4 acc[5];
#pragma unroll
      for (int m = 0; m < 5; ++m) acc[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < DV / 16; ++cb) {
        const float4 a = ld4(&R.gg[16 * prb + i16][16 * cb + 4 * g]);
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const float4 b = ld4(&sh.st[16 * ((w >> 1) + 2 * m) + i16][16 * cb + 4 * g]);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[m] = mma(el(a, e), el(b, e), acc[m]);
        }
      }
      for (int ks = 0; ks < 4 * (prb + 1); ++ks) {
        const float a = sh.dkap[16 * prb + i16][4 * ks + g];
#pragma unroll
        for (int m = 0; m < 5; ++m) acc[m] = mma(a, R.mk[4 * ks + g][16 * ((w >> 1) + 2 * m) + i16], acc[m]);
      }
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const int f = 16 * ((w >> 1) + 2 * m) + i16;
        const float zf = sh.z[f], cf = sh.coef[f];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * prb + 4 * g + r;
          const float dphi = fmaf(sh.gden[i], zf, acc[m][r]);
          pacc[m] = fmaf(sh.mq[i][f], dphi, pacc[m]);
          R.phq[i][f] = cf * dphi;
        }
      }
    }
    __syncthreads();
    // dq through the monomials
    {
      const int i = tid >> 3;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = (tid & 7) * 2 + e;
        const float s = chain_rule(R.phq[i], R.xq[i], r);
        if (i < nv) p.dq[(row0 + i) * DH + r] = s;
      }
    }
    // S += M^T U (the chunk's keys), z += sum_j m(k_j)
#pragma unroll
    for (int ks = 0; ks < C / 4; ++ks) {
      const float b = R.u[4 * ks + g][16 * w + i16];
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) accS[fb] = mma(R.mk[4 * ks + g][16 * fb + i16], b, accS[fb]);
    }
    if (tid < DP) {
      float s = 0.f;
      for (int j = 0; j < C; ++j) s += R.mk[j][tid];
      sh.z[tid] += s;
    }
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.st[16 * fb + 4 * g + r][16 * w + i16] = accS[fb][r];
  }
  // dL/dcoef_f of this (sequence, head, segment): rows summed over the lanes
  // and the two waves that share each feature block
  __syncthreads();
  float* scr = &sh.kap[0][0];  // free after the last chunk: 4 waves x 80 entries
#pragma unroll
  for (int m = 0; m < 5; ++m) {
    float s = pacc[m];
    s += __shfl_xor(s, 16);
    s += __shfl_xor(s, 32);
    if (g == 0) scr[w * 80 + 16 * m + i16] = s;
  }
  __syncthreads();
  if (tid < DP) {
    // feature block fb belongs to waves 2 (fb & 1) and 2 (fb & 1) + 1 as their m = fb >> 1
    const int fb = tid >> 4, m = fb >> 1, w0 = 2 * (fb & 1), e = 16 * m + (tid & 15);
    p.P[((long)bh * p.nseg + seg) * DP + tid] = scr[w0 * 80 + e] + scr[(w0 + 1) * 80 + e];
  }
}

// ---- reverse direction: dk, dv ----
template <bool BF16>
__global__ __launch_bounds__(bw::NT, 1) void bwd16_rev_kernel(const bw::BwdArgs p) {
  using namespace bw;
  __shared__ LdsRev sh;
  Rows& R = sh.rows;
  const int bh = blockIdx.x / p.nseg, seg = blockIdx.x % p.nseg, h = bh % p.H;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int i16 = lane & 15, g = lane >> 4;
  fill_tables(p, h, sh.coef);
  const int c0 = seg * p.cps, c1 = min(c0 + p.cps, p.nchunks);
  const long rbase = (long)bh * p.N;

  // R at the segment end: the later segments' query sums
  f4 accR[NFB];
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb) accR[fb] = f4{0.f, 0.f, 0.f, 0.f};
  float zs = 0.f;
  gather_segments(p, bh, seg + 1, p.nseg, accR, zs, w, lane);
#pragma unroll
  for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sh.st[16 * fb + 4 * g + r][16 * w + i16] = accR[fb][r];
  if (tid < DP) sh.z[tid] = zs;

  const int krb = w >> 1, kcb = w & 1, pjb = w & 1;
  Raw4<BF16> fqk, fv[2];
  Raw4<false> fg[2];
  float fgd = 0.f;
  auto fetch = [&](int c) {
    const int nv = min(C, p.N - c * C);
    const long row0 = rbase + (long)c * C;
    fetch_qk<BF16>(fqk, p, row0, nv, true, true);
    fetch_v64<BF16>(fv, p.v, row0, nv);
    fetch_v64<false>(fg, p.g, row0, nv);
    fgd = fetch_gden(p, row0, nv);
  };
  if (c0 < c1) fetch(c1 - 1);
  for (int c = c1 - 1; c >= c0; --c) {
    const int j0 = c * C, nv = min(C, p.N - j0);
    const long row0 = rbase + j0;
    __syncthreads();
    store_qk<BF16>(R, fqk, nv);
    store_v64<BF16>(R.u, fv);
    store_v64<false>(R.gg, fg);
    if (tid < C) sh.gden[tid] = fgd;
    if (c > c0) fetch(c - 1);
    __syncthreads();
    build_features(R, sh.coef, true, true);
    __syncthreads();
    kappa_tile(R, sh.kap, krb, kcb, lane);
    {
      float gd4[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) gd4[r] = sh.gden[16 * krb + 4 * (lane >> 4) + r];
      dkappa_tile(R, gd4, sh.dkap, krb, kcb, nv, lane);
    }
    __syncthreads();
    // dL/du = M R + kappa^T G (v columns 16 w ..): dv
    {
      f4 acc[2] = {f4{0.f, 0.f, 0.f, 0.f}, f4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) {  // B: this wave's columns of R, from its accumulators
        const float4 a0 = ld4(&R.mk[i16][16 * fb + 4 * g]), a1 = ld4(&R.mk[16 + i16][16 * fb + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[0] = mma(el(a0, e), accR[fb][e], acc[0]);
          acc[1] = mma(el(a1, e), accR[fb][e], acc[1]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < C / 4; ++ks) {
        const float b = R.gg[4 * ks + g][16 * w + i16];
        acc[0] = mma(sh.kap[4 * ks + g][i16], b, acc[0]);
        if (ks >= 4) acc[1] = mma(sh.kap[4 * ks + g][16 + i16], b, acc[1]);
      }
#pragma unroll
      for (int jb = 0; jb < 2; ++jb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jb + 4 * g + r;
          if (j < nv) p.dv[(row0 + j) * DV + 16 * w + i16] = acc[jb][r];
        }
    }
    // dL/dm(k) = U R^T + dkappa^T Phi (+ Rz for valid keys), rows pjb,
    // feature blocks (w >> 1) + 2 m
    f4 accK[5];
#pragma unroll
    for (int m = 0; m < 5; ++m) accK[m] = f4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int cb = 0; cb < DV / 16; ++cb) {
      const float4 a = ld4(&R.u[16 * pjb + i16][16 * cb + 4 * g]);
#pragma unroll
      for (int m = 0; m < 5; ++m) {
        const float4 b = ld4(&sh.st[16 * ((w >> 1) + 2 * m) + i16][16 * cb + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) accK[m] = mma(el(a, e), el(b, e), accK[m]);
      }
    }
    for (int ks = 4 * pjb; ks < C / 4; ++ks) {
      const float a = sh.dkap[4 * ks + g][16 * pjb + i16];
#pragma unroll
      for (int m = 0; m < 5; ++m) accK[m] = mma(a, R.phq[4 * ks + g][16 * ((w >> 1) + 2 * m) + i16], accK[m]);
    }
    __syncthreads();  // every read of M, R and Rz for this chunk is done
#pragma unroll
    for (int m = 0; m < 5; ++m) {
      const int f = 16 * ((w >> 1) + 2 * m) + i16;
      const float rz = sh.z[f];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * pjb + 4 * g + r;
        R.mk[j][f] = j < nv ? accK[m][r] + rz : 0.f;
      }
    }
    // R += Phi^T G (the chunk's queries), Rz += Phi^T gden
#pragma unroll
    for (int ks = 0; ks < C / 4; ++ks) {
      const float b = R.gg[4 * ks + g][16 * w + i16];
#pragma unroll
      for (int fb = 0; fb < NFB; ++fb) accR[fb] = mma(R.phq[4 * ks + g][16 * fb + i16], b, accR[fb]);
    }
    float rz = 0.f;
    if (tid < DP)
      for (int i = 0; i < C; ++i) rz = fmaf(R.phq[i][tid], sh.gden[i], rz);
    __syncthreads();
    if (tid < DP) sh.z[tid] += rz;
#pragma unroll
    for (int fb = 0; fb < NFB; ++fb)
#pragma unroll
      for (int r = 0; r < 4; ++r) sh.st[16 * fb + 4 * g + r][16 * w + i16] = accR[fb][r];
    // dk through the monomials
    {
      const int j = tid >> 3;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = (tid & 7) * 2 + e;
        const float s = chain_rule(R.mk[j], R.xk[j], r);
        if (j < nv) p.dk[(row0 + j) * DH + r] = s;
      }
    }
  }
}

// ---- dL/dcoef_f -> da, db, dc, summed over the batch (one workgroup per head) ----
__global__ __launch_bounds__(256) void bwd16_coef_kernel(const bw::BwdArgs p, int B, float* __restrict__ da,
                                                         float* __restrict__ db, float* __restrict__ dc) {
  using namespace bw;
  __shared__ float Ps[DP];
  __shared__ int gr[DH];
  __shared__ int nbad;
  const int h = blockIdx.x, G = p.G;
  if (threadIdx.x == 0) nbad = 0;
  __syncthreads();
  for (int f = threadIdx.x; f < DP; f += blockDim.x) {
    float s = 0.f;
    for (int b = 0; b < B; ++b)
      for (int sg = 0; sg < p.nseg; ++sg) s += p.P[(((long)b * p.H + h) * p.nseg + sg) * DP + f];
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

struct BwdPlan {
  int nchunks, nseg, cps, nsub, cpsub;
};

// Segments per sequence: enough (sequence x head, segment) workgroups to
// give every compute unit of a 256-CU device one, at most kMaxSeg, at most
// one per chunk, no empty segment.  The segment sums split each segment
// into parts so that about 1024 workgroups share them.
BwdPlan bwd_plan(int BH, int N) {
  BwdPlan pl{};
  pl.nchunks = (N + bw::C - 1) / bw::C;
  int nseg = BH > 0 ? 256 / BH : 1;
  nseg = std::max(1, std::min({nseg, bw::kMaxSeg, std::max(pl.nchunks, 1)}));
  pl.cps = pl.nchunks > 0 ? (pl.nchunks + nseg - 1) / nseg : 1;
  pl.nseg = pl.nchunks > 0 ? (pl.nchunks + pl.cps - 1) / pl.cps : 1;
  int nsub = BH > 0 ? (1024 + BH * pl.nseg - 1) / (BH * pl.nseg) : 1;
  nsub = std::max(1, std::min({nsub, bw::kMaxSeg, pl.cps}));
  pl.cpsub = (pl.cps + nsub - 1) / nsub;
  pl.nsub = (pl.cps + pl.cpsub - 1) / pl.cpsub;
  return pl;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

bool bwd16_supported(int d_h, int d_v, int dtype, bool diagonal, int G, int Hq, int Hkv) {
  return d_h == 16 && d_v == 64 && (dtype == 0 || dtype == 1) && !diagonal && G >= 1 && G <= 16 && Hq == Hkv;
}

size_t bwd16_workspace_bytes(int B, int H, int N) {
  const size_t BH = (size_t)B * H;
  const BwdPlan pl = bwd_plan((int)BH, N);
  return align256(BH * N * bw::DV * sizeof(float)) + align256(BH * N * sizeof(float)) +
         align256(BH * pl.nseg * pl.nsub * bw::SEGF * sizeof(float)) + BH * pl.nseg * bw::DP * sizeof(float);
}

hipError_t launch_bwd16(const BwdLaunch& a, hipStream_t stream) {
  const int BH = a.B * a.H;
  const BwdPlan pl = bwd_plan(BH, a.N);
  bw::BwdArgs p{};
  p.q = a.q; p.k = a.k; p.v = a.v; p.dy = a.dy;
  p.group_of_dim = a.group_of_dim; p.ca = a.ca; p.cb = a.cb; p.cc = a.cc;
  p.G = a.G; p.H = a.H; p.N = a.N;
  p.nchunks = pl.nchunks; p.nseg = pl.nseg; p.cps = pl.cps; p.nsub = pl.nsub; p.cpsub = pl.cpsub;
  char* ws = reinterpret_cast<char*>(a.workspace);
  p.g = reinterpret_cast<float*>(ws);
  ws += align256((size_t)BH * a.N * bw::DV * sizeof(float));
  p.gden = reinterpret_cast<float*>(ws);
  ws += align256((size_t)BH * a.N * sizeof(float));
  p.seg = reinterpret_cast<float*>(ws);
  ws += align256((size_t)BH * pl.nseg * pl.nsub * bw::SEGF * sizeof(float));
  p.P = reinterpret_cast<float*>(ws);
  p.dq = a.dq; p.dk = a.dk; p.dv = a.dv;
  const dim3 grid(BH * pl.nseg), sgrid(BH * pl.nseg * pl.nsub), block(bw::NT);
  // with no sequences only the coefficient kernel runs (it writes zeros)
  if (BH > 0) {
    if (a.dtype == 1) {
      if (pl.nseg > 1) hipLaunchKernelGGL((bwd16_segsum_kernel<0, true>), sgrid, block, 0, stream, p);
      hipLaunchKernelGGL((bwd16_fwd_kernel<true>), grid, block, 0, stream, p);
      if (pl.nseg > 1) hipLaunchKernelGGL((bwd16_segsum_kernel<1, true>), sgrid, block, 0, stream, p);
      hipLaunchKernelGGL((bwd16_rev_kernel<true>), grid, block, 0, stream, p);
    } else {
      if (pl.nseg > 1) hipLaunchKernelGGL((bwd16_segsum_kernel<0, false>), sgrid, block, 0, stream, p);
      hipLaunchKernelGGL((bwd16_fwd_kernel<false>), grid, block, 0, stream, p);
      if (pl.nseg > 1) hipLaunchKernelGGL((bwd16_segsum_kernel<1, false>), sgrid, block, 0, stream, p);
      hipLaunchKernelGGL((bwd16_rev_kernel<false>), grid, block, 0, stream, p);
    }
  }
  hipLaunchKernelGGL(bwd16_coef_kernel, dim3(a.H), dim3(256), 0, stream, p, a.B, a.da, a.db, a.dc);
  return hipGetLastError();
}

}  // namespace oal
