// Causal prefill of the dimension-wise form at d_h = 64 with bfloat16
// activations, for heads with their own keys and values (as many query heads
// as KV heads), one wavefront per (sequence x head, segment of the sequence).
//
// The kernel is the grouped kernel of the OAL paper (sec. 4.2) with one
// group per dimension and a diagonal c,
//     kappa(q, k) = a + sum_r b_r x_r + sum_r c_rr x_r^2,  x_r = q_r k_r / sqrt(d_h),
// which is the ReBased feature map read as an elementwise square ("Linear
// Transformers with Learnable Kernel Functions are Better In-Context
// Models", the section on letting training place the parabola), optionally
// after its pre-map gamma * LayerNorm(x) + beta on queries and keys.  Its
// feature space is [k_r, k_r^2, 1] (129 features), so the prefix state of
// Eq. (5) -- nine accumulator tiles of sixteen feature rows (tiles 0-3 the
// linear terms of dims 16 m + l, tiles 4-7 their squares, tile 8 row 0 the
// constant) times the 64 value columns and z -- fits in the MFMA
// accumulators of one wave (180 registers).  Per 32-token chunk:
//
//  1. the chunk's rows (loaded into registers one chunk ahead) are mapped
//     (LayerNorm over each row's 64 dims, eight lanes per row, then the
//     affine) and written to the wave's LDS tiles in bf16;
//  2. every 16-token query tile builds its query features times their
//     coefficients (a, b_r / sqrt(d), c_rr / d) once and uses them twice:
//     for the readout phi_Q^T [H | z] against the state before the chunk
//     (rounded once per chunk to bf16 operands), and for the within-chunk
//     scores kappa = phi_K . (coef * phi_Q) on MFMA, with the causal mask in
//     registers and V^T P^T on MFMA (the value fragments of the update);
//  3. the state update S += phi_K^T [V | 1].
//
// Segments as in the d_h = 16 one-wave kernel: a first kernel sums
// phi_K^T [V | 1] over each segment but the last, a scan turns the sums into
// prefix sums over segments, and the outputs kernel starts segment s from
// the initial state plus the prefix of segments 0 .. s - 1.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "oal_device.h"
#include "oal_internal.h"
#include "oal_layout.h"
#include "oal_onepass16.h"

namespace oal {
namespace {
namespace dw {

constexpr int D = 64;          // d_h
constexpr int C = 32;          // tokens per chunk
constexpr int NT = 9;          // accumulator tiles
constexpr int NKBW = 5;         // K-blocks of 32 feature rows (the last: tile 8 and a zero tile)
constexpr int NBS = 34;        // float4 rows of 64 lanes per segment sum (below)
constexpr int kSegTarget = 1024;
constexpr int kSegMax = 8;
constexpr long PF = packed_features(D);  // rows of the library's packed state

struct __align__(16) Lds {
  uint16_t q[C * D];   // mapped query rows [32][64] bf16, 16-byte pieces permuted (vswz16)
  uint16_t k[C * D];   // mapped key rows, same layout; rows past the end zero
  uint16_t k2[C * D];  // their elementwise squares (rounded once from fp32), same layout
  uint16_t v[C * DV];  // value rows, same layout
  float coef[4][32];   // query-side coefficient of K-block kb's row p (kb 0, 1: linear; 2, 3: squares)
  float gq[D], bq[D], gk[D], bk[D];  // pre-map affine of the head
  float a;             // constant coefficient
  int bad;             // a group id outside [0, G)
};

// 16-byte pieces of the next chunk's rows held by one lane: piece lane + 64 u
// of each [32][64] bf16 tile (row (lane + 64 u) / 8, dims 8 (lane % 8) ..).
struct Pre {
  uint4 q[4], k[4], v[4];
};

// bf16 element offset of dims 4 i .. 4 i + 3 of row r in a permuted tile
__device__ __forceinline__ int piece4_offset(int r, int i) {
  return r * D + 8 * ((i >> 1) ^ vswz16(r)) + 4 * (i & 1);
}

// sum over the eight lanes 8 s .. 8 s + 7 (a row's pieces): quad swaps, then
// the half-row mirror
__device__ __forceinline__ float sum8(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0xb1, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x4e, 0xf, 0xf, true));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x141, 0xf, 0xf, true));
  return x;
}

}  // namespace dw

template <bool OUT, bool PREMAP>
__global__ __launch_bounds__(64, 1) void dimw_kernel(const Args16 p) {
  using namespace dw;
  __shared__ Lds sh;
  const int seg = blockIdx.x, bh = blockIdx.y, BH = gridDim.y;
  const int lane = threadIdx.x, lg = lane / 16, l = lane % 16;
  const int N = p.N;
  const int nchunks = (N + C - 1) / C;
  const int c_begin = seg * p.seg_chunks, c_end = min(c_begin + p.seg_chunks, nchunks);
  const long rowbase = (long)bh * N;
  const int h = bh % p.Hq;  // query head = KV head
  constexpr long SF = PF * (DV + 1);

  // ---- prefix of the earlier segments (segment sums in the compact layout:
  // rows 4 m + n: S[m][n] of tiles 0..7; row 32, lane (lg, m): z of tile m,
  // rows 4 lg ..; row 33, lane (0, l): row 0 of tile 8 at columns 16 n + l).
  // Issued first so that the loads overlap the table set-up. ----
  f32x4 P[8][4], PZ[NT], P8;
  if (OUT && seg > 0) {
    const auto rb = buf_rsrc(reinterpret_cast<const float4*>(p.blocksum) + ((long)(seg - 1) * BH + bh) * NBS * kWave,
                             NBS * kWave * 16);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n)
        P[m][n] = __builtin_bit_cast(f32x4, buf_load16(rb, 16 * lane + (4 * m + n) * kWave * 16));
#pragma unroll
    for (int m = 0; m < NT; ++m) PZ[m] = __builtin_bit_cast(f32x4, buf_load16(rb, (32 * kWave + 16 * lg + m) * 16));
    P8 = __builtin_bit_cast(f32x4, buf_load16(rb, (33 * kWave + l) * 16));
  }

  // ---- per-head tables ----
  {
    const float rs = 0.125f, rd = 1.f / 64.f;  // 1/sqrt(d), 1/d at d = 64
    for (int i = lane; i < 128; i += kWave) {
      const int kb = i / 32, pr = i % 32;
      const int r = (kb & 1) * 32 + pr;
      const int g = min(max(p.group_of_dim[h * D + r], 0), p.G - 1);
      sh.coef[kb][pr] = kb < 2 ? p.cb[h * p.G + g] * rs : p.cc[(h * p.G + g) * p.G + g] * rd;
    }
    if (PREMAP) {
      sh.gq[lane] = p.gamma_q[h * D + lane];
      sh.bq[lane] = p.beta_q[h * D + lane];
      sh.gk[lane] = p.gamma_k[h * D + lane];
      sh.bk[lane] = p.beta_k[h * D + lane];
    }
    const int g = p.group_of_dim[h * D + lane];
    const bool anyb = __ballot(g < 0 || g >= p.G) != 0;
    if (lane == 0) {
      sh.a = p.ca[h];
      sh.bad = anyb ? 1 : 0;
    }
  }
  __syncthreads();

  // ---- state: S[m][n] rows 4 lg + e of tile m, columns 16 n + l; Z[m] z ----
  f32x4 S[NT][4], Z[NT];
#pragma unroll
  for (int m = 0; m < NT; ++m) {
    Z[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) S[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // packed (library) row of internal feature row f = 16 m + row (-1: none)
  auto abi_row = [](int m, int row) __attribute__((always_inline)) -> long {
    if (m < 4) return 1 + 16 * m + row;
    if (m < 8) return abi_index(D, 16 * (m - 4) + row, 16 * (m - 4) + row);
    return row == 0 ? 0 : -1;
  };
  if (OUT && p.state_in != nullptr) {
    const float* si = p.state_in + (long)bh * SF;
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long af = abi_row(m, 4 * lg + e);
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) S[m][n][e] = si[af * DV + 16 * n + l];
        Z[m][e] = si[PF * DV + af];
      }
  }
  if (OUT && seg > 0) {
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) S[m][n] = S[m][n] + P[m][n];
#pragma unroll
    for (int m = 0; m < NT; ++m) Z[m] = Z[m] + PZ[m];
    if (lg == 0)
#pragma unroll
      for (int n = 0; n < 4; ++n) S[8][n][0] += P8[n];
  }

  // ---- chunk rows ----
  const int off16 = 16 * lane;
  auto fetch = [&](int c, Pre& r) __attribute__((always_inline)) {
    const long r0 = rowbase + (long)c * C;
    const int left = N - c * C;
    const auto rk = buf_rsrc(p.k + r0 * D, left * D * 2);
    const auto rv = buf_rsrc(p.v + r0 * DV, left * DV * 2);
    if (OUT) {
      const auto rq = buf_rsrc(p.q + r0 * D, left * D * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) r.q[u] = buf_load16(rq, off16 + 1024 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) r.k[u] = buf_load16(rk, off16 + 1024 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) r.v[u] = buf_load16(rv, off16 + 1024 * u);
  };
  // LayerNorm + affine of one 16-byte piece (dims 8 (lane % 8) ..) of a row
  // whose other pieces sit in the seven neighbouring lanes, in fp32
  auto premap_vals = [&](uint4 w, const float* gm, const float* bt, float (&x)[8]) __attribute__((always_inline)) {
    unpack4(make_uint2(w.x, w.y), *reinterpret_cast<float(*)[4]>(&x[0]));
    unpack4(make_uint2(w.z, w.w), *reinterpret_cast<float(*)[4]>(&x[4]));
    float s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s1 += x[i];
    const float mu = sum8(s1) * (1.f / D);
    float s2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] -= mu;
      s2 += x[i] * x[i];
    }
    const float rstd = __builtin_amdgcn_rsqf(sum8(s2) * (1.f / D) + p.ln_eps);
    const int d0 = 8 * (lane & 7);
    const float4 g0 = lds_f4(gm + d0), g1 = lds_f4(gm + d0 + 4);
    const float4 b0 = lds_f4(bt + d0), b1 = lds_f4(bt + d0 + 4);
    const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const float bb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = fmaf(x[i] * rstd, gg[i], bb[i]);
  };
  auto pack8 = [](const float (&x)[8]) __attribute__((always_inline)) {
    return make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
  };
  auto commit = [&](int c, const Pre& r) __attribute__((always_inline)) {
    const int nvalid = min(C, N - c * C);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = lane + 64 * u, row = idx / 8;
      const int off = row * D + 8 * ((idx & 7) ^ vswz16(row));
      float x[8];
      if (PREMAP) {
        premap_vals(r.k[u], sh.gk, sh.bk, x);
      } else {
        unpack4(make_uint2(r.k[u].x, r.k[u].y), *reinterpret_cast<float(*)[4]>(&x[0]));
        unpack4(make_uint2(r.k[u].z, r.k[u].w), *reinterpret_cast<float(*)[4]>(&x[4]));
      }
      float x2[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x2[i] = x[i] * x[i];
      uint4 kw = PREMAP ? pack8(x) : r.k[u], kw2 = pack8(x2);
      if (PREMAP && row >= nvalid) {  // the mapped zero row is beta, not zero
        kw = make_uint4(0, 0, 0, 0);
        kw2 = kw;
      }
      *reinterpret_cast<uint4*>(&sh.k[off]) = kw;
      *reinterpret_cast<uint4*>(&sh.k2[off]) = kw2;
      if (OUT) {
        uint4 qw = r.q[u];
        if (PREMAP) {
          float xq[8];
          premap_vals(qw, sh.gq, sh.bq, xq);
          qw = pack8(xq);
        }
        *reinterpret_cast<uint4*>(&sh.q[off]) = qw;
      }
      *reinterpret_cast<uint4*>(&sh.v[off]) = r.v[u];
    }
  };

  // transposing reads (rows 4 lg .. 4 lg + 3 and 16 + 4 lg ..) of column
  // 16 c0 + l: the update's operands, keys in the order of the score tiles
  int tro[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 4 * lg + l / 4, cc = 16 * n + 4 * (l % 4);
    tro[n] = r * D + 8 * ((cc >> 3) ^ vswz16(r)) + (cc & 7);
  }
  auto tr8 = [&](const uint16_t* tile, int n) __attribute__((always_inline)) {
    const uint2 lo = v_rows4_at(tile, tro[n]), hi = v_rows4_at(tile + 16 * D, tro[n]);
    return u4_frag(lo.x, lo.y, hi.x, hi.y);
  };
  const bf16x8 ones = kOnes;
  // the constant feature (tile 8, row 0): as an update operand (feature row
  // l, eight tokens) ones in lanes l == 0; in the token layout (K-block 4,
  // position 8 lg + j) a one at lg == 0, j == 0
  const bf16x8 cst_rows = l == 0 ? ones : u4_frag(0, 0, 0, 0);
  const bf16x8 cst_tok = lg == 0 ? u4_frag(0x3f80u, 0, 0, 0) : u4_frag(0, 0, 0, 0);

  // ---- per-token features of row t of a tile, K-block kb: dims (kb & 1) 32
  // + 4 lg + j and + 16 (linear, kb < 2; squares, kb 2, 3); kb 4: the constant ----
  auto row_lin = [&](const uint16_t* tile, int t, int kb) __attribute__((always_inline)) {
    const uint2 x0 = lds_u2(tile + piece4_offset(t, 8 * kb + lg));
    const uint2 x1 = lds_u2(tile + piece4_offset(t, 8 * kb + 4 + lg));
    return make_uint4(x0.x, x0.y, x1.x, x1.y);
  };
  auto sq_frag = [&](uint4 w, const float* cf) __attribute__((always_inline)) {
    float x[8];
    unpack4(make_uint2(w.x, w.y), *reinterpret_cast<float(*)[4]>(&x[0]));
    unpack4(make_uint2(w.z, w.w), *reinterpret_cast<float(*)[4]>(&x[4]));
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = cf ? x[j] * x[j] * cf[j] : x[j] * x[j];
    return frag8(x);
  };
  auto lin_frag = [&](uint4 w, const float* cf) __attribute__((always_inline)) {
    float x[8];
    unpack4(make_uint2(w.x, w.y), *reinterpret_cast<float(*)[4]>(&x[0]));
    unpack4(make_uint2(w.z, w.w), *reinterpret_cast<float(*)[4]>(&x[4]));
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] *= cf[j];
    return frag8(x);
  };

  // ---- the state before a chunk as bf16 operands (H and z), K-block kb:
  // tiles 2 kb and 2 kb + 1 (tile 9 is zero) ----
  bf16x8 As[NKBW][4], Az[NKBW];
  auto convert = [&](auto KC) __attribute__((always_inline)) {
    constexpr int kb = decltype(KC)::value;
    auto frag = [&](const f32x4& x0, const f32x4* x1) __attribute__((always_inline)) {
      return u4_frag(pack_bf16(x0[0], x0[1]), pack_bf16(x0[2], x0[3]), x1 ? pack_bf16((*x1)[0], (*x1)[1]) : 0u,
                     x1 ? pack_bf16((*x1)[2], (*x1)[3]) : 0u);
    };
#pragma unroll
    for (int n = 0; n < 4; ++n) As[kb][n] = frag(S[2 * kb][n], 2 * kb + 1 < NT ? &S[2 * kb + 1][n] : nullptr);
    Az[kb] = frag(Z[2 * kb], 2 * kb + 1 < NT ? &Z[2 * kb + 1] : nullptr);
  };
  auto convert_all = [&]() __attribute__((always_inline)) {
    convert(std::integral_constant<int, 0>{});
    convert(std::integral_constant<int, 1>{});
    convert(std::integral_constant<int, 2>{});
    convert(std::integral_constant<int, 3>{});
    convert(std::integral_constant<int, 4>{});
  };

  // ---- state update with the chunk ----
  auto update_chunk = [&]() __attribute__((always_inline)) {
    bf16x8 Vf[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) Vf[n] = tr8(sh.v, n);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // linear tile m (dims 16 m + l) and its squares (tile m + 4)
      const bf16x8 A = tr8(sh.k, m), A2 = tr8(sh.k2, m);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        S[m][n] = mma32(A, Vf[n], S[m][n]);
        S[m + 4][n] = mma32(A2, Vf[n], S[m + 4][n]);
      }
      Z[m] = mma32(A, ones, Z[m]);
      Z[m + 4] = mma32(A2, ones, Z[m + 4]);
    }
#pragma unroll
    for (int n = 0; n < 4; ++n) S[8][n] = mma32(cst_rows, Vf[n], S[8][n]);
    Z[8] = mma32(cst_rows, ones, Z[8]);
  };

  // the state stays in the accumulator registers across chunks (without
  // this the compiler parks part of it in VGPRs and copies it every chunk)
  auto pin_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < NT; ++m) {
#pragma unroll
      for (int n = 0; n < 4; ++n) asm volatile("" : "+a"(S[m][n]));
      asm volatile("" : "+a"(Z[m]));
    }
  };
  if (!OUT) {
    Pre pa, pb;
    fetch(c_begin, pa);
    if (c_begin + 1 < c_end) fetch(c_begin + 1, pb);
    for (int c = c_begin; c < c_end; c += 2) {
      pin_state();
      commit(c, pa);
      if (c + 2 < c_end) fetch(c + 2, pa);
      update_chunk();
      pin_state();
      if (c + 1 < c_end) {
        commit(c + 1, pb);
        if (c + 3 < c_end) fetch(c + 3, pb);
        update_chunk();
      }
    }
  }

  Pre pre;
  if (OUT) {
    fetch(c_begin, pre);
    convert_all();
  }
  const float a_cf = sh.a;
  const bool badh = sh.bad != 0;
  for (int c = c_begin; OUT && c < c_end; ++c) {
    pin_state();
    commit(c, pre);
    if (c + 1 < c_end) fetch(c + 1, pre);
    const int nvalid = min(C, N - c * C);
    // key features of a key tile (token layout: row = key l), K-blocks 0..3
    // (K-block 4 is the constant, cst_tok); key tile 0 serves both query tiles
    auto key_feats = [&](int kt, bf16x8 (&Kf)[4]) __attribute__((always_inline)) {
      Kf[0] = __builtin_bit_cast(bf16x8, row_lin(sh.k, 16 * kt + l, 0));
      Kf[1] = __builtin_bit_cast(bf16x8, row_lin(sh.k, 16 * kt + l, 1));
      Kf[2] = __builtin_bit_cast(bf16x8, row_lin(sh.k2, 16 * kt + l, 0));
      Kf[3] = __builtin_bit_cast(bf16x8, row_lin(sh.k2, 16 * kt + l, 1));
    };
    bf16x8 Kf0[4];
    key_feats(0, Kf0);
    auto tile = [&](auto TC) __attribute__((always_inline)) {
      constexpr int T = decltype(TC)::value;
      if (16 * T >= nvalid) return;
      // query features times their coefficients: B operand of the readout
      // and of the within-chunk scores
      bf16x8 Bq[NKBW];
      {
        const uint4 w0 = row_lin(sh.q, 16 * T + l, 0), w1 = row_lin(sh.q, 16 * T + l, 1);
        float cf[4][8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float4 c0 = lds_f4(&sh.coef[kb][4 * lg]), c1 = lds_f4(&sh.coef[kb][16 + 4 * lg]);
          cf[kb][0] = c0.x; cf[kb][1] = c0.y; cf[kb][2] = c0.z; cf[kb][3] = c0.w;
          cf[kb][4] = c1.x; cf[kb][5] = c1.y; cf[kb][6] = c1.z; cf[kb][7] = c1.w;
        }
        Bq[0] = lin_frag(w0, cf[0]);
        Bq[1] = lin_frag(w1, cf[1]);
        Bq[2] = sq_frag(w0, cf[2]);
        Bq[3] = sq_frag(w1, cf[3]);
        const float ca8[8] = {lg == 0 ? a_cf : 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        Bq[4] = frag8(ca8);
      }
      f32x4 Y[4], Dn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < 4; ++n) Y[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < NKBW; ++kb) {
#pragma unroll
        for (int n = 0; n < 4; ++n) Y[n] = mma32(As[kb][n], Bq[kb], Y[n]);
        Dn = mma32(Az[kb], Bq[kb], Dn);
      }
      // within-chunk scores kappa(q, k) of key tiles 0 .. T (rows: keys 4 lg
      // + e, columns: queries l), the causal mask on the diagonal tile
      float pk[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if (kt > T) {
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[kt][e] = 0.f;
          continue;
        }
        bf16x8 Kf1[4];
        if (kt == 1) key_feats(1, Kf1);
        const bf16x8(&Kf)[4] = kt == 0 ? Kf0 : Kf1;
        f32x4 sc = mma32(cst_tok, Bq[4], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sc = mma32(Kf[kb], Bq[kb], sc);
#pragma unroll
        for (int e = 0; e < 4; ++e) pk[kt][e] = (kt < T || 4 * lg + e <= l) ? sc[e] : 0.f;
      }
      const float x8[8] = {pk[0][0], pk[0][1], pk[0][2], pk[0][3], pk[1][0], pk[1][1], pk[1][2], pk[1][3]};
      const bf16x8 Pf = frag8(x8);
#pragma unroll
      for (int n = 0; n < 4; ++n) Y[n] = mma32(tr8(sh.v, n), Pf, Y[n]);
      Dn = mma32(ones, Pf, Dn);
      {
        const float rinv = badh ? __builtin_nanf("") : __builtin_amdgcn_rcpf(Dn[0]);
        const auto ry = buf_rsrc(p.y + (rowbase + (long)c * C + 16 * T) * DV, (nvalid - 16 * T) * DV * 2);
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = Y[n][e] * rinv;
          buf_store8(ry, l * DV * 2 + 8 * lg + 32 * n, make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])));
        }
      }
    };
    tile(std::integral_constant<int, 0>{});
    tile(std::integral_constant<int, 1>{});
    update_chunk();
    convert_all();
  }
  // the constant feature counted 1 for every row of the last chunk, also past
  // the end of the sequence (the mapped key rows there are zero)
  if (c_end == nchunks && lg == 0) Z[8][0] -= (float)(nchunks * C - N);

  if (!OUT) {
    float4* bs = reinterpret_cast<float4*>(p.blocksum) + ((long)seg * BH + bh) * NBS * kWave + lane;
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) bs[(4 * m + n) * kWave] = make_float4(S[m][n][0], S[m][n][1], S[m][n][2], S[m][n][3]);
    // z is the same in every column: lane (lg, m) keeps tile m's
    f32x4 zsel = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NT; ++m)
      if (l == m) zsel = Z[m];
    bs[32 * kWave] = make_float4(zsel[0], zsel[1], zsel[2], zsel[3]);
    bs[33 * kWave] = lg == 0 ? make_float4(S[8][0][0], S[8][1][0], S[8][2][0], S[8][3][0]) : make_float4(0.f, 0.f, 0.f, 0.f);
  } else if (c_end == nchunks && p.state_out != nullptr) {
    float* so = p.state_out + (long)bh * SF;
#pragma unroll
    for (int m = 0; m < NT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const long af = abi_row(m, 4 * lg + e);
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) so[af * DV + 16 * n + l] = S[m][n][e];
        if (l == 0) so[PF * DV + af] = Z[m][e];
      }
  }
}

struct PlanD {
  int nseg, seg_chunks;
};

size_t segsum_bytes_d(int BH, int nseg) { return (size_t)(nseg - 1) * BH * dw::NBS * kWave * sizeof(float4); }

PlanD pland(int BH, int nchunks, size_t workspace_bytes) {
  if (nchunks <= 1) return PlanD{1, 1};
  int nseg = std::min({std::max(1, (dw::kSegTarget + BH - 1) / BH), dw::kSegMax, nchunks});
  for (;; --nseg) {
    PlanD pl{};
    pl.seg_chunks = (nchunks + nseg - 1) / nseg;
    pl.nseg = std::max(1, (nchunks + pl.seg_chunks - 1) / pl.seg_chunks);
    if (pl.nseg <= 1) return PlanD{1, nchunks};
    if (segsum_bytes_d(BH, pl.nseg) <= workspace_bytes) return pl;
  }
}

}  // namespace

bool dimw_supported(int d_h, int dtype, bool diagonal, int Hq, int Hkv) {
  return d_h == 64 && dtype == 1 && diagonal && Hq == Hkv;
}

size_t dimw_workspace_bytes(int B, int Hkv, int N) {
  const int BH = B * Hkv;
  const PlanD pl = pland(BH, (N + dw::C - 1) / dw::C, (size_t)-1);
  return pl.nseg > 1 ? segsum_bytes_d(BH, pl.nseg) : 0;
}

hipError_t launch_dimw(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + dw::C - 1) / dw::C;
  const PlanD pl = pland(BH, nchunks, a.workspace ? workspace_bytes : 0);
  Args16 p{};
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.k = reinterpret_cast<const uint16_t*>(a.k);
  p.v = reinterpret_cast<const uint16_t*>(a.v);
  p.group_of_dim = a.group_of_dim;
  p.ca = a.ca; p.cb = a.cb; p.cc = a.cc; p.G = a.G;
  p.gamma_q = a.gamma_q; p.beta_q = a.beta_q; p.gamma_k = a.gamma_k; p.beta_k = a.beta_k;
  p.ln_eps = a.ln_eps;
  p.state_in = a.state_in; p.state_out = a.state_out;
  p.blocksum = reinterpret_cast<float*>(a.workspace);
  p.y = reinterpret_cast<uint16_t*>(a.y);
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.seg_chunks = pl.seg_chunks; p.blk_chunks = pl.seg_chunks; p.nblk = pl.nseg - 1;
  const long per_slot = (long)BH * dw::NBS * kWave;
#define OAL_DIMW(PM)                                                                                          \
  do {                                                                                                        \
    if (pl.nseg > 1)                                                                                          \
      hipLaunchKernelGGL((dimw_kernel<false, PM>), dim3(pl.nseg - 1, BH), dim3(kWave), 0, stream, p);         \
    if (pl.nseg > 2)                                                                                          \
      hipLaunchKernelGGL(segment_prefix_scan_kernel, dim3((unsigned)((per_slot + 255) / 256)), dim3(256), 0,   \
                         stream, reinterpret_cast<float4*>(a.workspace), pl.nseg - 1, per_slot);              \
    hipLaunchKernelGGL((dimw_kernel<true, PM>), dim3(pl.nseg, BH), dim3(kWave), 0, stream, p);                \
  } while (0)
  if (a.premap) {
    OAL_DIMW(true);
  } else {
    OAL_DIMW(false);
  }
#undef OAL_DIMW
  return hipGetLastError();
}

}  // namespace oal
