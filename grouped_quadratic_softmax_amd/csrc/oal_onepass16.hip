// One-pass causal prefill at d_h = 16 with bfloat16 activations (the Based
// Taylor workload's shape and any grouped kernel of up to eight groups at
// that head dimension).
//
// The prefix state of the OAL paper's Eq. (5) at d_h = 16 has 153 packed
// features (App. D) times d_v + 1 = 65 columns: 40 KB in fp32.  It stays in
// MFMA accumulators for the whole pass; only q, k, v and y move through HBM.
//
// Feature order.  The 153 features are held as ten tiles m of sixteen rows l
// (160 rows, seven of them zero), chosen so that both MFMA layouts can build
// their operand from registers:
//   m = 0..7   the pair (l, (l - m) mod 16)   (m = 0: the square of dim l)
//   m = 8      l < 8: the pair (l, l + 8);  l >= 8: the linear term of dim l
//   m = 9      l < 8: the linear term of dim l;  l = 8: the constant;  else 0
// Every unordered pair r <= t appears exactly once (a pair with index
// difference 8 only in rows l < 8 of tile 8).
//
// State update S += phi_K(K_c)^T [V_c | 1]: the A operand of the
// 16x16x32 MFMA holds feature row l of a tile for eight tokens; a lane holds
// k_l of its eight tokens, and the partner value k_{(l-m) mod 16} of every
// tile comes from the lane (l - m) mod 16 of the same sixteen-lane row by a
// DPP row rotation, so the key features are built without any LDS traffic.
// The accumulator of tile m holds rows 4 lg + e of the tile for the wave's
// sixteen value columns; accumulator tiles 2b and 2b + 1 converted to bf16
// form, unchanged, the B operand of the readout for K-block b (positions
// 8 lg + e and 8 lg + 4 + e), so the state is never copied through LDS.
//
// Readout phi_Q(Q_c) [H | z] with the state before the chunk: a lane holds
// the query features of one token for K-block positions 8 lg + j, i.e. rows
// 4 lg + (j % 4) of tiles 2b + j / 4.  The lane keeps its token's q row
// rotated by 4 lg (dims 4 lg, 4 lg + 1, ... mod 16), so that the partner
// index (4 lg + j - m) mod 16 is the same register for every lane.  Each
// query feature carries its coefficient: a for the constant, b_g(r)/sqrt(d)
// for a linear term, and for a pair the symmetric c of the two groups / d,
// twice off the diagonal (Eq. (6)).  The normaliser column z stays in fp32
// (VALU sums of the fp32 key features), and so does the denominator.
//
// Within-chunk pairs: per group a masked 16x16x16 MFMA gives the partial
// dot products of the group for a 16 x 16 tile of (key, query) pairs
// (sec. 4.2), the polynomial a + sum b_g s_g + sum c_gh s_g s_h and the
// causal mask (j <= i) are applied in registers, and P [V | 1] runs on the
// 16x16x32 MFMA with the scores, unchanged, as its A operand.
//
// Work split: a CTA of four waves serves one (sequence, KV head) and one
// segment of whole 64-token chunks; wave w owns value columns 16 w .. 16 w +
// 15 (its share of the state is ten accumulator tiles).  A first kernel sums
// phi_K^T [V | 1] over blocks of chunks before the last segment into the
// workspace; the second starts every segment from the initial state plus the
// earlier blocks' sums.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cstddef>
#include <type_traits>

#include "oal_device.h"
#include "oal_internal.h"
#include "oal_onepass16.h"

namespace oal {

namespace {

#ifndef OP16_OCC
#define OP16_OCC 1
#endif

// Barrier for the LDS tiles that leaves outstanding global loads in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xf | (7 << 4) | (3 << 14));  // lgkmcnt 0 only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Pre-map (LayerNorm or unit l2 norm, then the affine) of four dims of a token row spread over four consecutive
// lanes, with this lane's gamma and beta values.
__device__ __forceinline__ void premap4(float (&x)[4], const float (&gamma)[4], const float (&beta)[4], float eps,
                                        PremapNorm pn) {
  float s = x[0] + x[1] + x[2] + x[3];
  s = quad_sum(s);
  const float mu = s * pn.mean_w;
  float v2 = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) v2 += (x[i] - mu) * (x[i] - mu);
  v2 = quad_sum(v2);
  const float inv = 1.f / sqrtf(v2 * pn.var_w + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = gamma[i] * (x[i] - mu) * inv + beta[i];
}

// LDS of one CTA (dynamic).  The block-sum kernel uses only raw and kt.
struct __align__(16) Lds16 {
  uint16_t raw[2][CK * (2 * DH + DV)];  // two slots of raw chunk rows (q, k, v bf16); the 16-byte pieces
                                        // of a v row are permuted (vswz)
  float kt[DH][CK + 4];          // keys transposed (after the pre-map)
  uint4 sb[NKB][5][kWave];       // state before the chunk times the query coefficients, as readout B
                                 // fragments (K-block, column tile 0..3 of H / tile 4: z in every column, lane)
  float qd[CK][DH];              // query rows (after the pre-map)
  float kr[CK][DH];              // key rows (after the pre-map)
  uint16_t ys[4][16][DV + 8];    // output rows, one 16-row tile per wave
  float coefq[RMAX][FT];         // query-side coefficient of every feature row, per head
  float poly[RMAX][1 + 8 + 64];  // a, b_g / sqrt(d), sym(c)_gh / d per head
  int gid[RMAX][DH];             // group of every dimension, per head (clamped)
  int bad[RMAX];                 // a group id outside [0, G)
};
constexpr size_t kLdsSums = offsetof(Lds16, sb);  // what the block-sum kernel uses

constexpr size_t kLdsOut = sizeof(Lds16);

// OUT = false: block sums (first kernel); OUT = true: outputs (second
// kernel).  NG: group count rounded up to 1, 2, 4 or 8 (groups past G have
// no dimensions and zero coefficients).
//
// Wave w owns the state rows of tiles m = w, w + 4, w + 8 (< 10) for all 64
// value columns (the update builds only those key features), and reads out
// the 16 query rows 16 w .. 16 w + 15 of the chunk (their query features,
// within-chunk pairs and denominators), against the whole state shared
// through LDS as bf16 fragments.
template <bool PREMAP, bool OUT, int NG, bool MULTI>
__global__ __launch_bounds__(256, OP16_OCC) void onepass16_kernel(const Args16 p) {
  extern __shared__ __align__(16) unsigned char lds_raw[];
  Lds16& sh = *reinterpret_cast<Lds16*>(lds_raw);
  const int seg = blockIdx.x, bh = blockIdx.y;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv, R = MULTI ? p.Hq / p.Hkv : 1;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave index, uniform
  const int lg = lane / 16, l = lane % 16;
  const int N = p.N;
  const int nchunks = (N + CK - 1) / CK;
  const int span = OUT ? p.seg_chunks : p.blk_chunks;
  const int c_begin = seg * span, c_end = min(c_begin + span, nchunks);
  const long kvbase = (long)bh * N;
  constexpr long SF = D16 * (DV + 1);
  const int ntile = w < 2 ? 3 : 2;  // state tiles of this wave

  // ---- per-head tables (outputs kernel) ----
  if (OUT) {
    const float rs = 0.25f, rd = 1.f / 16.f;  // 1/sqrt(d), 1/d at d = 16
    for (int i = tid; i < R * FT; i += 256) {
      const int hh = i / FT, f = i % FT, h = kvh * R + hh;
      int r = 0, t = 0;
      op_feature(f / 16, f % 16, r, t);
      float cf = 0.f;
      if (r == DH) {
        cf = p.ca[h];
      } else if (r >= 0) {
        const int g1 = min(max(p.group_of_dim[h * DH + r], 0), p.G - 1);
        if (t == DH) {
          cf = p.cb[h * p.G + g1] * rs;
        } else {
          const int g2 = min(max(p.group_of_dim[h * DH + t], 0), p.G - 1);
          cf = 0.5f * (p.cc[(h * p.G + g1) * p.G + g2] + p.cc[(h * p.G + g2) * p.G + g1]) * rd;
          if (r != t) cf *= 2.f;
        }
      }
      sh.coefq[hh][f] = cf;
    }
    for (int i = tid; i < R * 73; i += 256) {
      const int hh = i / 73, j = i % 73, h = kvh * R + hh;
      float x = 0.f;
      if (j == 0) {
        x = p.ca[h];
      } else if (j < 9) {
        if (j - 1 < p.G) x = p.cb[h * p.G + j - 1] * rs;
      } else {
        const int g1 = (j - 9) / 8, g2 = (j - 9) % 8;
        if (g1 < p.G && g2 < p.G)
          x = 0.5f * (p.cc[(h * p.G + g1) * p.G + g2] + p.cc[(h * p.G + g2) * p.G + g1]) * rd;
      }
      sh.poly[hh][j] = x;
    }
    if (w == 0) {
      for (int hh = 0; hh < R; ++hh) {
        const int h = kvh * R + hh;
        bool badg = false;
        if (lane < DH) {
          const int g = p.group_of_dim[h * DH + lane];
          badg = g < 0 || g >= p.G;
          sh.gid[hh][lane] = min(max(g, 0), p.G - 1);
        }
        const bool anyb = __ballot(badg) != 0;
        if (lane == 0) sh.bad[hh] = anyb ? 1 : 0;
      }
    }
  }

  // ---- state: acc[i][n] holds rows 16 m + 4 lg + e (m = w + 4 i) of
  // columns 16 n + l; accz[i] the same rows of z, in every column (the
  // update multiplies the key features by a ones operand) ----
  f32x4 acc[3][4], accz[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    accz[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (OUT) {
    const int nblk_before = seg * (p.seg_chunks / p.blk_chunks);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= ntile) continue;
      const int m = w + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = 16 * m + 4 * lg + e;
        const int af = abi_map_dev.f[f];
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          float x = 0.f;
          if (af >= 0 && p.state_in != nullptr) x = p.state_in[(long)bh * SF + (long)af * DV + 16 * n + l];
          for (int s = 0; s < nblk_before; ++s)
            x += p.blocksum[(((long)s * gridDim.y + bh) * FT + f) * (DV + 1) + 16 * n + l];
          acc[i][n][e] = x;
        }
        float x = 0.f;
        if (af >= 0 && p.state_in != nullptr) x = p.state_in[(long)bh * SF + D16 * DV + af];
        for (int s = 0; s < nblk_before; ++s)
          x += p.blocksum[(((long)s * gridDim.y + bh) * FT + f) * (DV + 1) + DV];
        accz[i][e] = x;
      }
    }
  }

  // ---- chunk loads: three 16-byte pieces per thread, loaded into registers
  // one chunk ahead and written into the raw slot of their chunk at the end
  // of the chunk before.  Thread t < 128 takes piece t of the q rows (outputs
  // kernel; nothing in the block-sum kernel), thread t >= 128 piece t - 128
  // of the k rows, and every thread pieces t and t + 256 of the v rows (row
  // piece / 8, columns 8 (piece % 8) ..).  Rows past the end load row N - 1
  // (in bounds) and are zeroed when staged (v rows past the end only ever
  // meet zero key features and masked scores).  Slot layout: q [64][16],
  // k [64][16], v [64][64] bf16, row-major. ----
  constexpr int RQ = 0, RK = CK * DH, RV = 2 * CK * DH;  // slot offsets (elements)
  const uint16_t* vtile = &sh.raw[0][0] + RV;           // v rows of the chunk being processed
  struct Raw3 {
    uint4 a, v0, v1;
  };
  const int qk_piece = tid & 127;
  const bool isk = tid >= 128;
  auto fetch = [&](int c) __attribute__((always_inline)) {
    Raw3 r;
    const int cc = min(c, nchunks - 1);
    const int arow = min(cc * CK + qk_piece / 2, N - 1);
    if (isk) r.a = *reinterpret_cast<const uint4*>(p.k + (kvbase + arow) * DH + 8 * (qk_piece & 1));
    else if (OUT) r.a = *reinterpret_cast<const uint4*>(p.q + (((long)b * p.Hq + kvh * R) * N + arow) * DH + 8 * (qk_piece & 1));
    const int vr0 = min(cc * CK + tid / 8, N - 1), vr1 = min(cc * CK + 32 + tid / 8, N - 1);
    r.v0 = *reinterpret_cast<const uint4*>(p.v + (kvbase + vr0) * DV + 8 * (tid & 7));
    r.v1 = *reinterpret_cast<const uint4*>(p.v + (kvbase + vr1) * DV + 8 * (tid & 7));
    return r;
  };
  auto commit = [&](int c, const Raw3& r) __attribute__((always_inline)) {
    uint16_t* slot = &sh.raw[c & 1][0];
    if (isk || OUT) *reinterpret_cast<uint4*>(slot + (isk ? RK : RQ) + 8 * qk_piece) = r.a;
    const int lr0 = tid / 8, lr1 = 32 + tid / 8;
    *reinterpret_cast<uint4*>(slot + RV + lr0 * DV + 8 * ((tid & 7) ^ vswz(lr0))) = r.v0;
    *reinterpret_cast<uint4*>(slot + RV + lr1 * DV + 8 * ((tid & 7) ^ vswz(lr1))) = r.v1;
  };
  const int srow = tid / 4, sq = tid % 4;
  // offsets (in the v tile) of the transposed fragment reads: the update's
  // (key step ks, half h, column tile n) and the within-chunk products'
  // (key step ks, key tile half, column tile n), fixed per lane
  int uoff[2][2][4], poff[2][2][4];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        uoff[ks][h][n] = v_rows4_offset(32 * ks + 8 * lg + 4 * h, 16 * n, l);
        poff[ks][h][n] = v_rows4_offset(32 * ks + 16 * h + 4 * lg, 16 * n, l);
      }
  // pre-map parameters of this thread's four dims (keys; queries of the
  // current head), loaded outside the chunk loop
  float gk[4] = {1.f, 1.f, 1.f, 1.f}, bk[4] = {0.f, 0.f, 0.f, 0.f};
  float gq[4] = {1.f, 1.f, 1.f, 1.f}, bq[4] = {0.f, 0.f, 0.f, 0.f};
  auto load_premap_q = [&](int hh) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gq[i] = p.gamma_q[(kvh * R + hh) * DH + 4 * sq + i];
      bq[i] = p.beta_q[(kvh * R + hh) * DH + 4 * sq + i];
    }
  };
  if (PREMAP) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      gk[i] = p.gamma_k[kvh * DH + 4 * sq + i];
      bk[i] = p.beta_k[kvh * DH + 4 * sq + i];
    }
    if (OUT) load_premap_q(0);
  }
  auto stage_q_vals = [&](float (&x)[4], int c, int hh) __attribute__((always_inline)) {
    (void)hh;
    const bool ok = c * CK + srow < N;
    if (PREMAP) premap4(x, gq, bq, p.ln_eps, p.pn);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = ok ? x[i] : 0.f;
    lds_st_f4(&sh.qd[srow][4 * sq], x[0], x[1], x[2], x[3]);
  };
  auto stage_q = [&](uint2 qw, int c, int hh) __attribute__((always_inline)) {
    float x[4];
    unpack4(qw, x);
    stage_q_vals(x, c, hh);
  };
  auto stage = [&](int c) __attribute__((always_inline)) {
    const uint16_t* slot = &sh.raw[c & 1][0];
    const bool ok = c * CK + srow < N;
    float x[4];
    unpack4(lds_u2(slot + RK + srow * DH + 4 * sq), x);
    if (PREMAP) premap4(x, gk, bk, p.ln_eps, p.pn);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = ok ? x[i] : 0.f;
      sh.kt[4 * sq + i][srow] = x[i];
    }
    if (OUT) lds_st_f4(&sh.kr[srow][4 * sq], x[0], x[1], x[2], x[3]);
    // (v rows stay in the ring as copied; rows past the end hold row N - 1,
    // which meets only zero key features and masked scores)
    if (OUT) {
      float xq[4];
      unpack4(lds_u2(slot + RQ + srow * DH + 4 * sq), xq);
      stage_q_vals(xq, c, 0);
    }
  };

  // ---- state update with chunk c (reads kt, vt): this wave's tiles ----
  auto update = [&](auto WC, int c) __attribute__((always_inline)) {
    constexpr int W = decltype(WC)::value;
    const int nvalid = min(CK, N - c * CK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int t0 = 32 * ks + 8 * lg;
      float kv[8];
      const float4 k0 = lds_f4(&sh.kt[l][t0]);
      const float4 k1 = lds_f4(&sh.kt[l][t0 + 4]);
      kv[0] = k0.x; kv[1] = k0.y; kv[2] = k0.z; kv[3] = k0.w;
      kv[4] = k1.x; kv[5] = k1.y; kv[6] = k1.z; kv[7] = k1.w;
      bf16x8 Bv[4];
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint2 lo = v_rows4_at(vtile, uoff[ks][0][n]), hi = v_rows4_at(vtile, uoff[ks][1][n]);
        Bv[n] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
      auto tile = [&](auto MC, int i) __attribute__((always_inline)) {
        constexpr int M = decltype(MC)::value;
        float f[8];
        key_features<M>(kv, l, t0, nvalid, f);
        const bf16x8 A = frag8(f);
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[i][n] = mma32(A, Bv[n], acc[i][n]);
        accz[i] = mma32(A, kOnes, accz[i]);
      };
      tile(std::integral_constant<int, W>{}, 0);
      tile(std::integral_constant<int, W + 4>{}, 1);
      if constexpr (W + 8 < MT) tile(std::integral_constant<int, W + 8>{}, 2);
    }
  };
  auto update_any = [&](int c) __attribute__((always_inline)) {
    switch (w) {
      case 0: update(std::integral_constant<int, 0>{}, c); break;
      case 1: update(std::integral_constant<int, 1>{}, c); break;
      case 2: update(std::integral_constant<int, 2>{}, c); break;
      default: update(std::integral_constant<int, 3>{}, c); break;
    }
  };

  // ---- share the state before the chunk, each feature row times its
  // query-side coefficient for head hh (so the query features stay plain
  // monomials), as bf16 readout fragments: rows 16 m + 4 lg + e of tile m go
  // to K-block m / 2, positions 8 lg + 4 (m % 2) + e; z likewise into
  // column tile 4 ----
  float cf[3][4];  // coefficients of this wave's state rows for the current head
  auto load_coef = [&](int hh) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      const int m = min(w + 4 * i, MT - 1);
      const float4 c0 = lds_f4(&sh.coefq[hh][16 * m + 4 * lg]);
      cf[i][0] = c0.x; cf[i][1] = c0.y; cf[i][2] = c0.z; cf[i][3] = c0.w;
    }
  };
  auto share_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= ntile) continue;
      const int m = w + 4 * i;
      unsigned char* base = reinterpret_cast<unsigned char*>(&sh.sb[m >> 1][0][lane]) + 8 * (m & 1);
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        const f32x4& a = n < 4 ? acc[i][n] : accz[i];
        const uint2 v2 = make_uint2(pack_bf16(a[0] * cf[i][0], a[1] * cf[i][1]),
                                    pack_bf16(a[2] * cf[i][2], a[3] * cf[i][3]));
        lds_st_u2(base + n * kWave * sizeof(uint4), v2);
      }
    }
  };

  // ---- within-chunk pairs of this wave's query tile QT (keys of tiles
  // 0..QT), added into Y and into the denominator tile Dn ----
  auto intra = [&](auto QC, int hh, f32x4 (&Y)[4], f32x4& Dn) __attribute__((always_inline)) {
    constexpr int QT = decltype(QC)::value;
    const float* pl = sh.poly[hh];
    int gd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) gd[i] = sh.gid[hh][4 * lg + i];
    const float4 qv = lds_f4(&sh.qd[16 * QT + l][4 * lg]);
    const bf16x4s Bq = __builtin_bit_cast(bf16x4s, make_uint2(pack_bf16(qv.x, qv.y), pack_bf16(qv.z, qv.w)));
    float pk[QT + 1][4];
#pragma unroll
    for (int kt = 0; kt <= QT; ++kt) {
      const float4 kv4 = lds_f4(&sh.kr[16 * kt + l][4 * lg]);
      const float kx[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
      f32x4 sg[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        float mk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) mk[i] = (NG == 1 || gd[i] == g) ? kx[i] : 0.f;
        const bf16x4s Ak = __builtin_bit_cast(bf16x4s, make_uint2(pack_bf16(mk[0], mk[1]), pack_bf16(mk[2], mk[3])));
        sg[g] = mma16(Ak, Bq, f32x4{0.f, 0.f, 0.f, 0.f});
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // kappa = a + sum_g s_g (b_g + sum_{h >= g} c'_gh s_h), c'_gh = 2 sym(c)_gh off the diagonal
        float kap = pl[0];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          float inner = pl[1 + g];
#pragma unroll
          for (int h2 = g; h2 < NG; ++h2) inner += (h2 == g ? 1.f : 2.f) * pl[9 + 8 * g + h2] * sg[h2][e];
          kap += sg[g][e] * inner;
        }
        if (kt == QT) kap = 4 * lg + e <= l ? kap : 0.f;  // causal mask inside the diagonal tile
        pk[kt][e] = kap;
      }
    }
    // P [V] over key steps of two key tiles (32 keys), every column tile
#pragma unroll
    for (int ks = 0; 2 * ks <= QT; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[e] = pk[2 * ks][e];
        x[4 + e] = 2 * ks + 1 <= QT ? pk[2 * ks + 1 < QT + 1 ? 2 * ks + 1 : QT][e] : 0.f;
      }
      const bf16x8 A = frag8(x);
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        const uint2 va = v_rows4_at(vtile, poff[ks][0][n]);
        const uint2 vb = v_rows4_at(vtile, poff[ks][1][n]);
        Y[n] = mma32(A, __builtin_bit_cast(bf16x8, make_uint4(va.x, va.y, vb.x, vb.y)), Y[n]);
      }
      Dn = mma32(A, kOnes, Dn);
    }
  };

  // ---- readout of query tile w for head hh, normalise, store ----
  auto readout = [&](int c, int hh) __attribute__((always_inline)) {
    const int nvalid = min(CK, N - c * CK);
    f32x4 Y[4], Dn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) Y[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float Qr[16];
    // dims 4 lg, 4 lg + 1, ... (mod 16): the row's float4 groups in rotated order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 x = lds_f4(&sh.qd[16 * w + l][4 * ((lg + i) & 3)]);
      Qr[4 * i] = x.x; Qr[4 * i + 1] = x.y; Qr[4 * i + 2] = x.z; Qr[4 * i + 3] = x.w;
    }
    // tile 8: pair (l, l + 8) in rows l < 8 (lane rows 0, 1), linear term above;
    // tile 9: linear term in rows l < 8, the constant and zeros above
    float p8[4], b9[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      p8[jj] = lg < 2 ? Qr[jj + 8] : 1.f;
      b9[jj] = lg < 2 ? Qr[jj] : 1.f;
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int m = 2 * kb + j / 4, jj = j % 4;
        if (m < 8) f[j] = Qr[jj] * Qr[(jj - m + 16) & 15];
        else if (m == 8) f[j] = Qr[jj] * p8[jj];
        else f[j] = b9[jj];
      }
      const bf16x8 A = frag8(f);
#pragma unroll
      for (int n = 0; n < 4; ++n) Y[n] = mma32(A, __builtin_bit_cast(bf16x8, lds_u4(&sh.sb[kb][n][lane])), Y[n]);
      Dn = mma32(A, __builtin_bit_cast(bf16x8, lds_u4(&sh.sb[kb][4][lane])), Dn);
    }
    switch (w) {
      case 0: intra(std::integral_constant<int, 0>{}, hh, Y, Dn); break;
      case 1: intra(std::integral_constant<int, 1>{}, hh, Y, Dn); break;
      case 2: intra(std::integral_constant<int, 2>{}, hh, Y, Dn); break;
      default: intra(std::integral_constant<int, 3>{}, hh, Y, Dn); break;
    }
    // Dn holds the denominator of row 4 lg + e in every column
    float rinv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) rinv[e] = __builtin_amdgcn_rcpf(Dn[e]);
    const bool badh = sh.bad[hh] != 0;
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float y0 = badh ? __builtin_nanf("") : Y[n][e] * rinv[e];
        const float y1 = badh ? __builtin_nanf("") : Y[n][e + 1] * rinv[e + 1];
        const uint32_t pr = pack_bf16(y0, y1);
        sh.ys[w][4 * lg + e][16 * n + l] = (uint16_t)(pr & 0xffffu);
        sh.ys[w][4 * lg + e + 1][16 * n + l] = (uint16_t)(pr >> 16);
      }
    // this wave's 16 rows x 128 bytes: two 16-byte stores per lane (its own
    // rows of ys: no barrier needed)
    uint16_t* yp = p.y + (((long)b * p.Hq + kvh * R + hh) * N + (long)c * CK + 16 * w) * DV;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int vi = lane + 64 * u, row = vi / 8, cv = vi % 8;
      if (16 * w + row < nvalid)
        *reinterpret_cast<uint4*>(yp + (long)row * DV + 8 * cv) = lds_u4(&sh.ys[w][row][8 * cv]);
    }
  };

  {
    const Raw3 r0 = fetch(c_begin);
    commit(c_begin, r0);
  }
  Raw3 rnext = fetch(c_begin + 1);
  __syncthreads();  // tables and the first chunk's rows
  if (OUT) load_coef(0);

  for (int c = c_begin; c < c_end; ++c) {
    vtile = &sh.raw[c & 1][0] + RV;
    stage(c);
    if (OUT) share_state();
    // the next chunk's rows into the other slot (last read during chunk
    // c - 1, which every wave has finished), then the loads of the chunk
    // after it: issued before this chunk's output stores, so that waiting
    // for them never waits for those stores
    if (c + 1 < c_end) commit(c + 1, rnext);
    if (c + 2 < c_end) rnext = fetch(c + 2);
    lds_barrier();
    if (OUT && !MULTI) readout(c, 0);
    if (OUT && MULTI) {
      for (int hh = 0; hh < R; ++hh) {
        if (hh > 0) {
          const long qb = ((long)b * p.Hq + kvh * R + hh) * N;
          const int row = min(c * CK + srow, N - 1);
          const uint2 qw = *reinterpret_cast<const uint2*>(p.q + (qb + row) * DH + 4 * sq);
          if (PREMAP) load_premap_q(hh);
          lds_barrier();  // every wave done with the previous head's query rows and fragments
          stage_q(qw, c, hh);
          load_coef(hh);
          share_state();
          lds_barrier();
        }
        readout(c, hh);
      }
      if (R > 1) {
        load_coef(0);
        if (PREMAP) load_premap_q(0);
      }
    }
    update_any(c);
    lds_barrier();
  }

  // ---- results (z: every column of accz holds it; lane column 0 writes) ----
  if (!OUT) {
    // block sum of this CTA: [blk][bh][FT][DV + 1]
    float* bs = p.blocksum + ((long)seg * gridDim.y + bh) * FT * (DV + 1);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= ntile) continue;
      const int m = w + 4 * i;
#pragma unroll
      for (int n = 0; n < 4; ++n)
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[(16 * m + 4 * lg + e) * (DV + 1) + 16 * n + l] = acc[i][n][e];
      if (l == 0)
#pragma unroll
        for (int e = 0; e < 4; ++e) bs[(16 * m + 4 * lg + e) * (DV + 1) + DV] = accz[i][e];
    }
  } else if (seg == (int)gridDim.x - 1 && p.state_out != nullptr) {
    float* so = p.state_out + (long)bh * SF;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      if (i >= ntile) continue;
      const int m = w + 4 * i;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int af = abi_map_dev.f[16 * m + 4 * lg + e];
#pragma unroll
        for (int n = 0; n < 4; ++n)
          if (af >= 0) so[(long)af * DV + 16 * n + l] = acc[i][n][e];
        if (af >= 0 && l == 0) so[D16 * DV + af] = accz[i][e];
      }
    }
  }
}

// Segment plan: about one CTA per compute unit for the outputs kernel, the
// summed blocks sized so that the first kernel also fills the chip, both
// limited by the workspace.
struct Plan16 {
  int nseg, seg_chunks, blk_chunks, nblk;
};

Plan16 plan16(int BH, int nchunks, size_t workspace_bytes) {
  const size_t blk_bytes = (size_t)FT * (DV + 1) * sizeof(float) * BH;
  Plan16 pl{};
  if (nchunks <= 1) return Plan16{1, 1, 1, 0};
#ifndef OP16_CTAS
#define OP16_CTAS 256
#endif
  int nseg = std::max(1, std::min((OP16_CTAS + BH - 1) / BH, nchunks / 4));
  for (;; --nseg) {
    pl.nseg = nseg;
    pl.seg_chunks = (nchunks + nseg - 1) / nseg;
    pl.nseg = (nchunks + pl.seg_chunks - 1) / pl.seg_chunks;
    if (pl.nseg <= 1) {
      pl = Plan16{1, nchunks, std::max(nchunks, 1), 0};
      return pl;
    }
    // split each segment into f blocks so that the first kernel has about
    // 512 CTAs
    int f = std::max(1, 512 / (BH * (pl.nseg - 1)));
    while (f > 1 && pl.seg_chunks % f != 0) --f;
    pl.blk_chunks = pl.seg_chunks / f;
    pl.nblk = (pl.nseg - 1) * f;
    if ((size_t)pl.nblk * blk_bytes <= workspace_bytes) return pl;
    // fewer blocks per segment, then fewer segments
    pl.blk_chunks = pl.seg_chunks;
    pl.nblk = pl.nseg - 1;
    if ((size_t)pl.nblk * blk_bytes <= workspace_bytes) return pl;
  }
}

}  // namespace

// Up to eight groups in either build; more (up to one per dimension, the
// dimension-aware kernel with any symmetric c) in the one-wave build only.
bool onepass16_supported(int d_h, int dtype, bool diagonal, int G, int Hq, int Hkv, bool premap) {
  if (d_h != 16 || dtype != 1 || diagonal || G < 1 || Hq / Hkv > RMAX) return false;
  return G <= 8 || (G <= DH && onepass16w_supported(Hq, Hkv, premap));
}

// The workspace that lets either build run at full parallelism (the
// pre-map, which picks the CTA build, is not known when it is sized).
size_t onepass16_workspace_bytes(int B, int Hq, int Hkv, int N) {
  const int BH = B * Hkv;
  const int nchunks = (N + CK - 1) / CK;
  const Plan16 pl = plan16(BH, nchunks, (size_t)-1);
  const size_t cta = (size_t)pl.nblk * BH * FT * (DV + 1) * sizeof(float);
  return onepass16w_supported(Hq, Hkv, false) ? std::max(cta, onepass16w_workspace_bytes(B, Hkv, N)) : cta;
}

hipError_t launch_onepass16(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  if (onepass16w_supported(a.Hq, a.Hkv, a.premap)) return launch_onepass16w(a, workspace_bytes, stream);
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + CK - 1) / CK;
  const Plan16 pl = plan16(BH, nchunks, a.workspace ? workspace_bytes : 0);
  Args16 p{};
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.k = reinterpret_cast<const uint16_t*>(a.k);
  p.v = reinterpret_cast<const uint16_t*>(a.v);
  p.group_of_dim = a.group_of_dim;
  p.ca = a.ca; p.cb = a.cb; p.cc = a.cc; p.G = a.G;
  p.gamma_q = a.gamma_q; p.beta_q = a.beta_q; p.gamma_k = a.gamma_k; p.beta_k = a.beta_k;
  p.ln_eps = a.ln_eps;
  p.pn = premap_norm(a.premap_kind, DH);
  p.state_in = a.state_in; p.state_out = a.state_out;
  p.blocksum = reinterpret_cast<float*>(a.workspace);
  p.y = reinterpret_cast<uint16_t*>(a.y);
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N;
  p.seg_chunks = pl.seg_chunks; p.blk_chunks = pl.blk_chunks; p.nblk = pl.nblk;
  const int NG = a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : 8;
#define OAL_OP16(PM, G_)                                                                                     \
  do {                                                                                                       \
    auto ks = onepass16_kernel<PM, false, 1, false>;                                                         \
    auto ko = a.Hq == a.Hkv ? onepass16_kernel<PM, true, G_, false> : onepass16_kernel<PM, true, G_, true>;   \
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(ko), hipFuncAttributeMaxDynamicSharedMemorySize,   \
                            (int)kLdsOut) != hipSuccess)                                                     \
      return hipErrorInvalidValue;                                                                           \
    if (pl.nblk > 0) hipLaunchKernelGGL(ks, dim3(pl.nblk, BH), dim3(256), kLdsSums, stream, p);              \
    hipLaunchKernelGGL(ko, dim3(pl.nseg, BH), dim3(256), kLdsOut, stream, p);                                \
  } while (0)
#define OAL_OP16_G(PM)          \
  switch (NG) {                 \
    case 1: OAL_OP16(PM, 1); break; \
    case 2: OAL_OP16(PM, 2); break; \
    case 4: OAL_OP16(PM, 4); break; \
    default: OAL_OP16(PM, 8); break; \
  }
  if (a.premap) {
    OAL_OP16_G(true)
  } else {
    OAL_OP16_G(false)
  }
#undef OAL_OP16_G
#undef OAL_OP16
  return hipGetLastError();
}

}  // namespace oal
