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
// Segments.  The outputs of segment s start from the initial state plus the
// sums phi_K^T [V | 1] over segments 0 .. s - 1.  With four or more segments
// per sequence one launch does it all: a workgroup of four waves takes four
// consecutive segments; each wave first sums its segment (the last segment
// of the sequence needs no sum), the waves hand their sums to the later
// waves of the group through LDS, and with two groups per sequence wave 3 of
// the first group publishes the group's total for the second group (device-
// scope stores and a flag, polled with a bound); then every wave produces
// its segment's outputs.  With two or three segments a first kernel writes
// the segment sums, a scan turns them into prefix sums and the outputs
// kernel reads them.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <atomic>
#include <chrono>
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

constexpr int NQF = 5 * NT;    // accumulator quads per lane (S[m][0..3], then z[m])

// kernel modes
constexpr int kSums = 0;     // sums of phi_K^T [V | 1] over a segment
constexpr int kOutputs = 1;  // outputs of a segment from the scanned sums
constexpr int kChained = 2;  // both, four segments per workgroup, prefixes formed in the launch

struct __align__(16) Tiles {  // one wave's chunk
  uint16_t q[C * D];   // mapped query rows [32][64] bf16, 16-byte pieces permuted (vswz16)
  uint16_t k[C * D];   // mapped key rows, same layout; rows past the end zero
  uint16_t k2[C * D];  // their elementwise squares (rounded once from fp32), same layout
  uint16_t v[C * DV];  // value rows, same layout
};
struct __align__(16) Tables {  // per head
  float coef[4][32];   // query-side coefficient of K-block kb's row p (kb 0, 1: linear; 2, 3: squares)
  float gq[D], bq[D], gk[D], bk[D];  // pre-map affine of the head
  float a;             // constant coefficient
  int bad;             // a group id outside [0, G), or a chained prefix that never arrived
};
struct __align__(16) LdsOne {
  Tiles t[1];
  Tables tb;
};
// The four waves' chunk tiles, and between the two loops (when no tile is in
// use) the segment sums of waves 0..2 handed to the later waves, in register
// order (quad 5 m + n: S[m][n], 5 m + 4: z[m]).
constexpr int kXchBytes = 3 * NQF * kWave * 16;
struct __align__(16) LdsChained {
  union {
    Tiles t[4];
    unsigned char xch[kXchBytes];
  };
  Tables tb;
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


template <int MODE, bool PREMAP>
__global__ __launch_bounds__(MODE == dw::kChained ? 4 * kWave : kWave, 1) void dimw_kernel(const Args16 p) {
  using namespace dw;
  constexpr bool OUT = MODE != kSums;
  constexpr bool SUMS = MODE != kOutputs;
  typedef std::conditional_t<MODE == kChained, LdsChained, LdsOne> L;
  __shared__ L sh;
  const int lane = threadIdx.x % kWave, lg = lane / 16, l = lane % 16;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  Tiles& tl = sh.t[MODE == kChained ? wv : 0];
  Tables& tb = sh.tb;
  // (sequence x head, segment).  Chained launches run at most two groups of
  // four segments per sequence, group-major: the first groups never wait,
  // and the second groups that wait (one workgroup per compute unit) are
  // fewer than the compute units (the planner checks), so some first group
  // always finds a compute unit whatever the dispatch order.
  int seg, bh, grp = 0;
  if constexpr (MODE == kChained) {
    bh = blockIdx.x % p.BH;
    grp = blockIdx.x / p.BH;
    seg = 4 * grp + wv;
  } else {
    seg = blockIdx.x;
    bh = blockIdx.y;
  }
  const int BH = MODE == kChained ? p.BH : gridDim.y;
  const int N = seq_len_of(p.seq_lens, bh / p.Hkv, p.N);  // rows of this sequence (row stride p.N)
  const int nchunks = (N + C - 1) / C;
  const int c_begin = seg * p.seg_chunks, c_end = min(c_begin + p.seg_chunks, nchunks);
  const bool live = c_begin < c_end;          // empty segments past the end
  // the segment that ends the sequence (of an empty sequence: segment 0,
  // which then only writes the final state)
  const bool last = nchunks == 0 ? seg == 0 : live && c_end == nchunks;
  const long rowbase = (long)bh * p.N;
  const int h = bh % p.Hq;  // query head = KV head
  constexpr long SF = PF * (DV + 1);

  // ---- prefix of the earlier segments (segment sums in the compact layout:
  // rows 4 m + n: S[m][n] of tiles 0..7; row 32, lane (lg, m): z of tile m,
  // rows 4 lg ..; row 33, lane (0, l): row 0 of tile 8 at columns 16 n + l).
  // Issued first so that the loads overlap the table set-up. ----
  f32x4 P[8][4], PZ[NT], P8;
  if (MODE == kOutputs && seg > 0) {
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

  // ---- per-head tables, spread over the workgroup's threads ----
  {
    const float rs = 0.125f, rd = 1.f / 64.f;  // 1/sqrt(d), 1/d at d = 64
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int i = tid; i < 128; i += nth) {
      const int kb = i / 32, pr = i % 32;
      const int r = (kb & 1) * 32 + pr;
      const int g = min(max(p.group_of_dim[h * D + r], 0), p.G - 1);
      tb.coef[kb][pr] = kb < 2 ? p.cb[h * p.G + g] * rs : p.cc[(h * p.G + g) * p.G + g] * rd;
    }
    if (PREMAP) {
      const int nw = nth / kWave;  // four arrays over the waves
      for (int j = wv; j < 4; j += nw) {
        const float* src = j == 0 ? p.gamma_q : j == 1 ? p.beta_q : j == 2 ? p.gamma_k : p.beta_k;
        float* dst = j == 0 ? tb.gq : j == 1 ? tb.bq : j == 2 ? tb.gk : tb.bk;
        dst[lane] = src[h * D + lane];
      }
    }
    if (wv == 0) {
      const int g = p.group_of_dim[h * D + lane];
      const bool anyb = __ballot(g < 0 || g >= p.G) != 0;
      if (lane == 0) {
        tb.a = p.ca[h];
        tb.bad = anyb ? 1 : 0;
      }
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
  auto load_state_in = [&]() __attribute__((always_inline)) {
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
  };
  // the sums of the chained launch start segment 0 from the initial state, so
  // that every later prefix includes it
  if (p.state_in != nullptr && (MODE == kOutputs || (MODE == kChained && seg == 0))) load_state_in();
  if (MODE == kOutputs && seg > 0) {
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
  auto fetch = [&](int c, Pre& r, bool wq) __attribute__((always_inline)) {
    const long r0 = rowbase + (long)c * C;
    const int left = N - c * C;
    const auto rk = buf_rsrc(p.k + r0 * D, left * D * 2);
    const auto rv = buf_rsrc(p.v + r0 * DV, left * DV * 2);
    if (wq) {
      const auto rq = buf_rsrc(p.q + r0 * D, left * D * 2);
#pragma unroll
      for (int u = 0; u < 4; ++u) r.q[u] = buf_load16(rq, off16 + 1024 * u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) r.k[u] = buf_load16(rk, off16 + 1024 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) r.v[u] = buf_load16(rv, off16 + 1024 * u);
  };
  // Pre-map (LayerNorm or unit l2 norm, then the affine) of one 16-byte piece (dims 8 (lane % 8) ..) of a row
  // whose other pieces sit in the seven neighbouring lanes, in fp32
  auto premap_vals = [&](uint4 w, const float* gm, const float* bt, float (&x)[8]) __attribute__((always_inline)) {
    unpack4(make_uint2(w.x, w.y), *reinterpret_cast<float(*)[4]>(&x[0]));
    unpack4(make_uint2(w.z, w.w), *reinterpret_cast<float(*)[4]>(&x[4]));
    float s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s1 += x[i];
    const float mu = sum8(s1) * p.pn.mean_w;
    float s2 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[i] -= mu;
      s2 += x[i] * x[i];
    }
    const float rstd = __builtin_amdgcn_rsqf(sum8(s2) * p.pn.var_w + p.ln_eps);
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
  auto commit = [&](int c, const Pre& r, bool wq) __attribute__((always_inline)) {
    const int nvalid = min(C, N - c * C);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int idx = lane + 64 * u, row = idx / 8;
      const int off = row * D + 8 * ((idx & 7) ^ vswz16(row));
      float x[8];
      if (PREMAP) {
        premap_vals(r.k[u], tb.gk, tb.bk, x);
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
      *reinterpret_cast<uint4*>(&tl.k[off]) = kw;
      *reinterpret_cast<uint4*>(&tl.k2[off]) = kw2;
      if (wq) {
        uint4 qw = r.q[u];
        if (PREMAP) {
          float xq[8];
          premap_vals(qw, tb.gq, tb.bq, xq);
          qw = pack8(xq);
        }
        *reinterpret_cast<uint4*>(&tl.q[off]) = qw;
      }
      *reinterpret_cast<uint4*>(&tl.v[off]) = r.v[u];
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
    for (int n = 0; n < 4; ++n) Vf[n] = tr8(tl.v, n);
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // linear tile m (dims 16 m + l) and its squares (tile m + 4)
      const bf16x8 A = tr8(tl.k, m), A2 = tr8(tl.k2, m);
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
  // ---- segment sum (the segment that ends the sequence needs none) ----
  if (SUMS && live && !last) {
    Pre pa, pb;
    fetch(c_begin, pa, false);
    if (c_begin + 1 < c_end) fetch(c_begin + 1, pb, false);
    for (int c = c_begin; c < c_end; c += 2) {
      pin_state();
      commit(c, pa, false);
      if (c + 2 < c_end) fetch(c + 2, pa, false);
      update_chunk();
      pin_state();
      if (c + 1 < c_end) {
        commit(c + 1, pb, false);
        if (c + 3 < c_end) fetch(c + 3, pb, false);
        update_chunk();
      }
    }
  }

  Pre pre;
  if (OUT && live) fetch(c_begin, pre, true);
  bool lost = false;  // a chained prefix that never arrived
  if constexpr (MODE == kChained) {
    // ---- exclusive prefix of the segment: the sums of the earlier waves of
    // the group through LDS, plus the published total of the earlier group of
    // the sequence.  Wave 3 of a group that has a successor publishes the
    // group's inclusive total. ----
    float4* xch = reinterpret_cast<float4*>(sh.xch);
    auto quad = [&](int q) __attribute__((always_inline)) -> f32x4& { return q % 5 < 4 ? S[q / 5][q % 5] : Z[q / 5]; };
    auto slot = [&](int j, int q) __attribute__((always_inline)) {
      return __builtin_bit_cast(f32x4, xch[(j * NQF + q) * kWave + lane]);
    };
    __syncthreads();  // every wave is done with its tiles
    if (wv < 3)
#pragma unroll
      for (int q = 0; q < NQF; ++q) {
        const f32x4 x = quad(q);
        xch[(wv * NQF + q) * kWave + lane] = make_float4(x[0], x[1], x[2], x[3]);
      }
    __syncthreads();
    const auto rpub = buf_rsrc(p.pub + (long)bh * NQF * kWave, NQF * kWave * 16);
    // wave w: the sums of waves 0 .. w - 1 (wave 3 of a first group with a
    // successor also publishes them plus its own), one pass over the quads
    auto prefix_from_slots = [&](auto WC, bool publish) __attribute__((always_inline)) {
      constexpr int W = decltype(WC)::value, QB = 9;  // quads per batch of LDS reads in flight
#pragma unroll
      for (int q0 = 0; q0 < NQF; q0 += QB) {
        f32x4 x[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < W; ++j) {
          f32x4 r[QB];
#pragma unroll
          for (int i = 0; i < QB; ++i) r[i] = slot(j, q0 + i);
#pragma unroll
          for (int i = 0; i < QB; ++i) x[i] = x[i] + r[i];
        }
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          if (publish) store_coherent(rpub, 16 * ((q0 + i) * kWave + lane), x[i] + quad(q0 + i));
          quad(q0 + i) = x[i];
        }
      }
    };
    switch (wv) {
      case 0: prefix_from_slots(std::integral_constant<int, 0>{}, false); break;
      case 1: prefix_from_slots(std::integral_constant<int, 1>{}, false); break;
      case 2: prefix_from_slots(std::integral_constant<int, 2>{}, false); break;
      default:
        if (grp == 0 && p.nwg > 1) {
          prefix_from_slots(std::integral_constant<int, 3>{}, true);
          if (lane == 0) publish_flag(p.ctl + bh, p.tag);
        } else {
          prefix_from_slots(std::integral_constant<int, 3>{}, false);
        }
    }
    if (grp > 0) {
      lost = !wait_published(p.ctl + bh, p.tag);
      f32x4 t[NQF];
#pragma unroll
      for (int q = 0; q < NQF; ++q) t[q] = load_coherent(rpub, 16 * (q * kWave + lane));
#pragma unroll
      for (int q = 0; q < NQF; ++q) quad(q) = quad(q) + t[q];
    }
    if (seg == 0 && p.state_in != nullptr) load_state_in();
    __syncthreads();  // the hand-over slots are read before the tiles reuse them
  }
  if (OUT && live) convert_all();
  const float a_cf = tb.a;
  const bool badh = tb.bad != 0 || lost;
  for (int c = c_begin; OUT && c < c_end; ++c) {
    pin_state();
    commit(c, pre, true);
    if (c + 1 < c_end) fetch(c + 1, pre, true);
    const int nvalid = min(C, N - c * C);
    // key features of a key tile (token layout: row = key l), K-blocks 0..3
    // (K-block 4 is the constant, cst_tok); key tile 0 serves both query tiles
    auto key_feats = [&](int kt, bf16x8 (&Kf)[4]) __attribute__((always_inline)) {
      Kf[0] = __builtin_bit_cast(bf16x8, row_lin(tl.k, 16 * kt + l, 0));
      Kf[1] = __builtin_bit_cast(bf16x8, row_lin(tl.k, 16 * kt + l, 1));
      Kf[2] = __builtin_bit_cast(bf16x8, row_lin(tl.k2, 16 * kt + l, 0));
      Kf[3] = __builtin_bit_cast(bf16x8, row_lin(tl.k2, 16 * kt + l, 1));
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
        const uint4 w0 = row_lin(tl.q, 16 * T + l, 0), w1 = row_lin(tl.q, 16 * T + l, 1);
        float cf[4][8];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float4 c0 = lds_f4(&tb.coef[kb][4 * lg]), c1 = lds_f4(&tb.coef[kb][16 + 4 * lg]);
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
      for (int n = 0; n < 4; ++n) Y[n] = mma32(tr8(tl.v, n), Pf, Y[n]);
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
  if (OUT && last && lg == 0) Z[8][0] -= (float)(nchunks * C - N);

  if (MODE == kSums) {
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
  } else if (OUT && last && p.state_out != nullptr) {
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
  int nwg;  // chained launch with nwg groups of four segments; 0: three-kernel path
};

size_t segsum_bytes_d(int BH, int nseg) { return (size_t)(nseg - 1) * BH * dw::NBS * kWave * sizeof(float4); }
// chained launch: ticket and flags, then the published group totals
// chained launch with two groups: a flag per sequence, then the first
// groups' published totals
size_t ctl_bytes_d(int BH) { return ((size_t)BH * sizeof(uint64_t) + 255) / 256 * 256; }
size_t chained_bytes_d(int BH, int nwg) {
  return nwg > 1 ? ctl_bytes_d(BH) + (size_t)BH * dw::NQF * kWave * sizeof(float4) : 0;
}

// About kSegTarget waves: with four or more segments per sequence, groups of
// four segments chained in one launch (two groups when the workspace holds
// the published totals and the waiting groups are fewer than the compute
// units, else one); below that the block sums, the scan and the outputs as
// three launches.
PlanD pland(int BH, int nchunks, size_t workspace_bytes, int cus) {
  if (nchunks <= 1) return PlanD{1, 1, 0};
  const int target = std::min({std::max(1, (dw::kSegTarget + BH - 1) / BH), dw::kSegMax, nchunks});
  if (target >= 4) {
    int nwg = target / 4;  // 1 or 2 (kSegMax = 8)
    if (chained_bytes_d(BH, nwg) > workspace_bytes || BH >= cus) nwg = 1;
    PlanD pl{};
    pl.nwg = nwg;
    pl.nseg = 4 * nwg;
    pl.seg_chunks = (nchunks + pl.nseg - 1) / pl.nseg;
    return pl;
  }
  for (int nseg = target;; --nseg) {
    PlanD pl{};
    pl.seg_chunks = (nchunks + nseg - 1) / nseg;
    pl.nseg = std::max(1, (nchunks + pl.seg_chunks - 1) / pl.seg_chunks);
    if (pl.nseg <= 1) return PlanD{1, nchunks, 0};
    if (segsum_bytes_d(BH, pl.nseg) <= workspace_bytes) return pl;
  }
}

}  // namespace

// A 64-bit tag unique to each chained launch in the process: a counter from
// a start that mixes the clock and an address
uint64_t chained_launch_tag() {
  static std::atomic<uint64_t> next{0x9e3779b97f4a7c15ull ^
                                    (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count() ^
                                    ((uint64_t)(uintptr_t)&next << 17)};
  return next.fetch_add(1, std::memory_order_relaxed);
}

// compute units of the current device (cached per device)
int device_cus() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool dimw_supported(int d_h, int dtype, bool diagonal, int Hq, int Hkv) {
  return d_h == 64 && dtype == 1 && diagonal && Hq == Hkv;
}

size_t dimw_workspace_bytes(int B, int Hkv, int N) {
  const int BH = B * Hkv;
  const PlanD pl = pland(BH, (N + dw::C - 1) / dw::C, (size_t)-1, 1 << 30);
  if (pl.nwg > 0) return chained_bytes_d(BH, pl.nwg);
  return pl.nseg > 1 ? segsum_bytes_d(BH, pl.nseg) : 0;
}

hipError_t launch_dimw(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + dw::C - 1) / dw::C;
  const PlanD pl = pland(BH, nchunks, a.workspace ? workspace_bytes : 0, device_cus());
  Args16 p{};
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.k = reinterpret_cast<const uint16_t*>(a.k);
  p.v = reinterpret_cast<const uint16_t*>(a.v);
  p.group_of_dim = a.group_of_dim;
  p.ca = a.ca; p.cb = a.cb; p.cc = a.cc; p.G = a.G;
  p.gamma_q = a.gamma_q; p.beta_q = a.beta_q; p.gamma_k = a.gamma_k; p.beta_k = a.beta_k;
  p.ln_eps = a.ln_eps;
  p.pn = premap_norm(a.premap_kind, dw::D);
  p.state_in = a.state_in; p.state_out = a.state_out;
  p.blocksum = reinterpret_cast<float*>(a.workspace);
  p.y = reinterpret_cast<uint16_t*>(a.y);
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.seq_lens = a.seq_lens;
  p.seg_chunks = pl.seg_chunks; p.blk_chunks = pl.seg_chunks; p.nblk = pl.nseg - 1;
  p.nwg = pl.nwg; p.nseg = pl.nseg; p.BH = BH;
  if (pl.nwg > 1) {
    p.ctl = reinterpret_cast<uint64_t*>(a.workspace);
    p.pub = reinterpret_cast<float4*>(reinterpret_cast<char*>(a.workspace) + ctl_bytes_d(BH));
    p.tag = chained_launch_tag();
  }
  const long per_slot = (long)BH * dw::NBS * kWave;
#define OAL_DIMW(PM)                                                                                          \
  do {                                                                                                        \
    if (pl.nwg > 0) {                                                                                         \
      hipLaunchKernelGGL((dimw_kernel<dw::kChained, PM>), dim3(BH * pl.nwg), dim3(4 * kWave), 0, stream, p);  \
      break;                                                                                                  \
    }                                                                                                         \
    if (pl.nseg > 1)                                                                                          \
      hipLaunchKernelGGL((dimw_kernel<dw::kSums, PM>), dim3(pl.nseg - 1, BH), dim3(kWave), 0, stream, p);     \
    if (pl.nseg > 2)                                                                                          \
      hipLaunchKernelGGL(segment_prefix_scan_kernel, dim3((unsigned)((per_slot + 255) / 256)), dim3(256), 0,   \
                         stream, reinterpret_cast<float4*>(a.workspace), pl.nseg - 1, per_slot);              \
    hipLaunchKernelGGL((dimw_kernel<dw::kOutputs, PM>), dim3(pl.nseg, BH), dim3(kWave), 0, stream, p);        \
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
