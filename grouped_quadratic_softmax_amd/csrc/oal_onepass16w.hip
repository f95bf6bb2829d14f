// Causal prefill at d_h = 16 with bfloat16 activations for heads with their
// own keys and values (as many query heads as KV heads), one wavefront per
// (sequence x head, segment of the sequence).
//
// The wave holds the whole prefix state of the OAL paper's Eq. (5) for its
// head -- the 153 packed features (App. D) in ten accumulator tiles of
// sixteen rows, times the 64 value columns and the normaliser column z -- in
// its own MFMA accumulators for the whole segment.  Nothing is shared with
// other waves: no barrier, no state traffic through LDS.  Per 64-token chunk:
//
//  1. the chunk's q, k, v rows (loaded into registers one chunk ahead) are
//     written to the wave's LDS tile;
//  2. the state before the chunk is rounded once to bf16 MFMA operands (the
//     accumulator tiles 2b and 2b + 1 form, unchanged, the operand of
//     K-block b);
//  3. every 16-token query tile is read out, phi_Q(q_i)^T [H | z] (Eq. (6)),
//     as H^T phi_Q^T so that the result holds whole output rows per lane;
//     the query features carry the coefficients (a, b_g / sqrt(d), the
//     symmetric c / d), so the state stays coefficient-free;
//  4. the within-chunk pairs of the tile: per group a masked 16x16x16 MFMA
//     gives the group's partial dot products for 16 x 16 (key, query) pairs
//     (sec. 4.2), the polynomial and the causal mask are applied in
//     registers, and V^T P^T runs on the 16x16x32 MFMA with the scores,
//     unchanged, as its B operand and the value fragments of the update as
//     its A operand;
//  5. the state update S += phi_K(K_c)^T [V_c | 1] with key features built
//     in registers by DPP row rotations.
//
// Segments.  The outputs of segment s start from the initial state plus the
// sums phi_K^T [V | 1] over segments 0 .. s - 1.  With four or more segments
// per sequence one launch does it all: a workgroup of four waves takes four
// consecutive segments; each wave first sums its segment (the last segment
// of the sequence needs no sum), the waves hand their sums to the later
// waves of the group through LDS, and with two groups per sequence wave 3 of
// the first group publishes the group's total for the second group (device-
// scope stores and a flag, polled with a bound); then every wave produces
// its segment's outputs.  With two or three segments a first kernel of the
// same shape writes the segment sums, a scan turns them into prefix sums,
// and the outputs kernel reads them.
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

constexpr int kQuads = 5 * MT;  // accumulator quads per lane: (tile m, column tile 0..3 of H, 4: z)
constexpr int kWaveSegTarget = 1024;  // waves that fill the chip once (one per SIMD)
constexpr int kWaveSegMax = 8;

// kernel modes
constexpr int kSumsW = 0;     // sums of phi_K^T [V | 1] over a segment
constexpr int kOutputsW = 1;  // outputs of a segment from the scanned sums
constexpr int kChainedW = 2;  // both, four segments per workgroup, prefixes formed in the launch

struct __align__(16) TilesW {  // one wave's chunk
  uint16_t q[CK * DH];     // query rows [64][16]
  uint16_t k[CK * DH];     // key rows [64][16] (rows past the end zero)
  uint16_t v[CK * DV];     // value rows [64][64], 16-byte pieces permuted (vswz16); rows past the end zero
};
struct __align__(16) TablesW {  // per head
  float coefq[FT];         // query-side coefficient of every feature row
  float poly[1 + 8 + 64];  // a, b_g / sqrt(d), sym(c)_gh / d
  uint2 gmask[8][4];       // [group][lg]: bf16 lane masks of dims 4 lg .. 4 lg + 3 in the group
  int bad;                 // a group id outside [0, G), or a chained prefix that never arrived
};
struct __align__(16) LdsOneW {
  TilesW t[1];
  TablesW tb;
};
// The four waves' chunk tiles, and between the two loops (when no tile is in
// use) the segment sums of waves 0..2 handed to the later waves, in register
// order (quad 5 m + n: S[m][n], 5 m + 4: z[m]).
constexpr int kXchBytesW = 3 * kQuads * kWave * 16;
struct __align__(16) LdsChainedW {
  union {
    TilesW t[4];
    unsigned char xch[kXchBytesW];
  };
  TablesW tb;
};

// Prefetched chunk rows of one lane: q and k, two 16-byte pieces each
// (pieces lane and lane + 64 of the 128 in a [64][16] tile); v, eight
// pieces (lane + 64 u of the 512 in a [64][64] tile).
struct PreW {
  uint4 q[2], k[2], v[8];
};

template <int MODE, int NG>
__global__ __launch_bounds__(MODE == kChainedW ? 4 * kWave : kWave, 1) void onepass16w_kernel(const Args16 p) {
  constexpr bool OUT = MODE != kSumsW;
  constexpr bool SUMS = MODE != kOutputsW;
  typedef std::conditional_t<MODE == kChainedW, LdsChainedW, LdsOneW> L;
  __shared__ L shm;
  const int lane = threadIdx.x % kWave, lg = lane / 16, l = lane % 16;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // wave-uniform
  TilesW& sh = shm.t[MODE == kChainedW ? wv : 0];
  TablesW& tb = shm.tb;
  // (sequence x head, segment).  Chained launches run at most two groups of
  // four segments per sequence, group-major: the first groups never wait,
  // and the second groups that wait (one workgroup per compute unit) are
  // fewer than the compute units (the planner checks), so some first group
  // always finds a compute unit whatever the dispatch order.
  int seg, bh, grp = 0;
  if constexpr (MODE == kChainedW) {
    bh = blockIdx.x % p.BH;
    grp = blockIdx.x / p.BH;
    seg = 4 * grp + wv;
  } else {
    seg = blockIdx.x;
    bh = blockIdx.y;
  }
  const int BH = MODE == kChainedW ? p.BH : gridDim.y;
  const int N = seq_len_of(p.seq_lens, bh / p.Hkv, p.N);  // rows of this sequence (row stride p.N)
  const int nchunks = (N + CK - 1) / CK;
  const int c_begin = seg * p.seg_chunks, c_end = min(c_begin + p.seg_chunks, nchunks);
  const bool live = c_begin < c_end;          // empty segments past the end
  // the segment that ends the sequence (of an empty sequence: segment 0,
  // which then only writes the final state)
  const bool last = nchunks == 0 ? seg == 0 : live && c_end == nchunks;
  const long rowbase = (long)bh * p.N;  // rows of q, k, v and y of this (sequence, head)
  constexpr long SF = D16 * (DV + 1);

  // ---- per-head tables (outputs), spread over the workgroup's threads ----
  if (OUT) {
    const int h = bh % p.Hq;
    const float rs = 0.25f, rd = 1.f / 16.f;  // 1/sqrt(d), 1/d at d = 16
    const int tid = threadIdx.x, nth = blockDim.x;
    for (int f = tid; f < FT; f += nth) {
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
      tb.coefq[f] = cf;
    }
    for (int j = tid; j < 73; j += nth) {
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
      tb.poly[j] = x;
    }
    int g = 0;
    bool badg = false;
    if (wv == 0 && lane < DH) {
      g = p.group_of_dim[h * DH + lane];
      badg = g < 0 || g >= p.G;
      g = min(max(g, 0), p.G - 1);
    }
    const bool anyb = __ballot(badg) != 0;
    if (wv == 0 && lane == 0) tb.bad = anyb ? 1 : 0;
    if (wv == 0 && lane < 32) {  // lane = 4 group + lg: masks of dims 4 lg .. 4 lg + 3
      const int gg = lane / 4, lgg = lane % 4;
      uint32_t m0 = 0, m1 = 0;
      for (int i = 0; i < 4; ++i) {
        const int gi = __shfl(g, 4 * lgg + i);
        if (gi == gg) (i < 2 ? m0 : m1) |= 0xffffu << (16 * (i & 1));
      }
      tb.gmask[gg][lgg] = make_uint2(m0, m1);
    }
  }

  // ---- state: S[m][n] holds rows 4 lg + e of tile m, columns 16 n + l;
  // Z[m] the same rows of z in every column ----
  f32x4 S[MT][4], Z[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    Z[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) S[m][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto load_state_in = [&]() __attribute__((always_inline)) {
    const float* si = p.state_in + (long)bh * SF;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int af = abi_map_dev.f[16 * m + 4 * lg + e];
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) S[m][n][e] = si[(long)af * DV + 16 * n + l];
        Z[m][e] = si[D16 * DV + af];
      }
  };
  // the sums of the chained launch start segment 0 from the initial state, so
  // that every later prefix includes it
  if (p.state_in != nullptr && (MODE == kOutputsW || (MODE == kChainedW && seg == 0))) load_state_in();
  if (MODE == kOutputsW && seg > 0) {
    // the sum over the earlier segments, slot seg - 1 of the prefix-summed
    // segment sums ([slot][bh][quad][lane] float4)
    const auto rb = buf_rsrc(reinterpret_cast<const float4*>(p.blocksum) + ((long)(seg - 1) * BH + bh) * kQuads * kWave,
                             kQuads * kWave * 16);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        const f32x4 x = __builtin_bit_cast(f32x4, buf_load16(rb, 16 * lane + (5 * m + n) * kWave * 16));
        f32x4& a = n < 4 ? S[m][n] : Z[m];
        a = p.state_in != nullptr ? a + x : x;
      }
    }
  }

  // ---- chunk rows: loaded one chunk ahead into registers through buffer
  // descriptors that end at the end of the sequence, so rows past it read as
  // zero; lane i takes the 16-byte pieces i + 64 u of each row-major tile ----
  const int off16 = 16 * lane;
  auto fetch = [&](int c, PreW& r, bool wq) __attribute__((always_inline)) {
    const long r0 = rowbase + (long)c * CK;
    const int left = N - c * CK;
    const auto rk = buf_rsrc(p.k + r0 * DH, left * DH * 2);
    const auto rv = buf_rsrc(p.v + r0 * DV, left * DV * 2);
    if (wq) {
      const auto rq = buf_rsrc(p.q + r0 * DH, left * DH * 2);
#pragma unroll
      for (int u = 0; u < 2; ++u) r.q[u] = buf_load16(rq, off16 + 1024 * u);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) r.k[u] = buf_load16(rk, off16 + 1024 * u);
#pragma unroll
    for (int u = 0; u < 8; ++u) r.v[u] = buf_load16(rv, off16 + 1024 * u);
  };
  auto commit = [&](const PreW& r, bool wq) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int idx = lane + 64 * u;
      if (wq) *reinterpret_cast<uint4*>(&sh.q[8 * idx]) = r.q[u];
      *reinterpret_cast<uint4*>(&sh.k[8 * idx]) = r.k[u];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int idx = lane + 64 * u, row = idx / 8;
      *reinterpret_cast<uint4*>(&sh.v[row * DV + 8 * ((idx & 7) ^ vswz16(row))]) = r.v[u];
    }
  };

  // Token order of a 32-token key step ks: operand position 8 lg + j holds
  // token 32 ks + 4 lg + j (j < 4) or 32 ks + 16 + 4 lg + j - 4 (j >= 4), the
  // rows of the score tiles 2 ks and 2 ks + 1 as the 16x16x16 MFMA leaves
  // them.  The transposing reads of rows 4 lg .. 4 lg + 3 (value tile, column
  // tile n; key tile) sit at these lane offsets; the other row quads of the
  // step are 16 and 32 rows further on.
  int vo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 4 * lg + l / 4, cc = 16 * n + 4 * (l % 4);
    vo[n] = r * DV + 8 * ((cc >> 3) ^ vswz16(r)) + (cc & 7);
  }
  const int ko = (4 * lg + l / 4) * DH + 4 * (l % 4);
  // value fragment of key step ks, column tile n: B operand of the update,
  // A operand of the within-chunk products
  auto vfrag = [&](int ks, int n) __attribute__((always_inline)) {
    const uint2 lo = v_rows4_at(sh.v + 32 * ks * DV, vo[n]);
    const uint2 hi = v_rows4_at(sh.v + (32 * ks + 16) * DV, vo[n]);
    return u4_frag(lo.x, lo.y, hi.x, hi.y);
  };

  // ---- the state before a chunk as bf16 operands, each feature row times
  // its query-side coefficient (so that the query features stay plain
  // monomials).  K-block kb is rounded as soon as its two tiles hold the
  // state (during the update of the chunk before), so the rounding overlaps
  // the update's MFMAs. ----
  bf16x8 As[NKB][4], Az[NKB];
  auto convert = [&](auto KC) __attribute__((always_inline)) {
    constexpr int kb = decltype(KC)::value;
    const float4 c0 = lds_f4(&tb.coefq[32 * kb + 4 * lg]), c1 = lds_f4(&tb.coefq[32 * kb + 16 + 4 * lg]);
    auto frag = [&](const f32x4& x0, const f32x4& x1) __attribute__((always_inline)) {
      return u4_frag(pack_bf16(x0[0] * c0.x, x0[1] * c0.y), pack_bf16(x0[2] * c0.z, x0[3] * c0.w),
                     pack_bf16(x1[0] * c1.x, x1[1] * c1.y), pack_bf16(x1[2] * c1.z, x1[3] * c1.w));
    };
#pragma unroll
    for (int n = 0; n < 4; ++n) As[kb][n] = frag(S[2 * kb][n], S[2 * kb + 1][n]);
    Az[kb] = frag(Z[2 * kb], Z[2 * kb + 1]);
  };
  const bf16x8 ones = kOnes;  // B operand that sums the rows of A (z, denominators)
  auto update_chunk = [&](auto CONV) __attribute__((always_inline)) {
      constexpr bool conv = decltype(CONV)::value;  // round the next chunk's operands
      // ---- state update with the chunk: both key steps of a tile back to
      // back, so that each accumulator is updated in place ----
      {
        float kv[2][8];
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float x[4];
          unpack4(k_rows4_at(sh.k + 32 * ks * DH, ko), x);
          kv[ks][0] = x[0]; kv[ks][1] = x[1]; kv[ks][2] = x[2]; kv[ks][3] = x[3];
          unpack4(k_rows4_at(sh.k + (32 * ks + 16) * DH, ko), x);
          kv[ks][4] = x[0]; kv[ks][5] = x[1]; kv[ks][6] = x[2]; kv[ks][7] = x[3];
        }
        bf16x8 Vf[2][4];
  #pragma unroll
        for (int ks = 0; ks < 2; ++ks)
  #pragma unroll
          for (int n = 0; n < 4; ++n) Vf[ks][n] = vfrag(ks, n);
        auto mtile = [&](auto MC) __attribute__((always_inline)) {
          constexpr int M = decltype(MC)::value;
          float f0[8], f1[8];
          key_features<M>(kv[0], l, 0, CK, f0);  // the constant is 1 for every token (fixed up below)
          key_features<M>(kv[1], l, 0, CK, f1);
          const bf16x8 A0 = frag8(f0), A1 = frag8(f1);
  #pragma unroll
          for (int n = 0; n < 4; ++n) S[M][n] = mma32(A1, Vf[1][n], mma32(A0, Vf[0][n], S[M][n]));
          Z[M] = mma32(A1, ones, mma32(A0, ones, Z[M]));
        };
        // the next chunk's operands of K-block kb are rounded one tile after
        // tiles 2 kb and 2 kb + 1 were updated
        mtile(std::integral_constant<int, 0>{});
        mtile(std::integral_constant<int, 1>{});
        mtile(std::integral_constant<int, 2>{});
        if (conv) convert(std::integral_constant<int, 0>{});
        mtile(std::integral_constant<int, 3>{});
        mtile(std::integral_constant<int, 4>{});
        if (conv) convert(std::integral_constant<int, 1>{});
        mtile(std::integral_constant<int, 5>{});
        mtile(std::integral_constant<int, 6>{});
        if (conv) convert(std::integral_constant<int, 2>{});
        mtile(std::integral_constant<int, 7>{});
        mtile(std::integral_constant<int, 8>{});
        if (conv) convert(std::integral_constant<int, 3>{});
        mtile(std::integral_constant<int, 9>{});
        if (conv) convert(std::integral_constant<int, 4>{});
      }
  };

  // keep the state in accumulation registers across the loops (an empty
  // statement that only constrains register allocation; without it the
  // loop-carried tiles are allocated to ordinary VGPRs and copied around
  // every MFMA)
  auto pin_state = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
      for (int n = 0; n < 4; ++n) asm volatile("" : "+a"(S[m][n]));
      asm volatile("" : "+a"(Z[m]));
    }
  };
  // ---- segment sum (the segment that ends the sequence needs none): the
  // chunk rows two chunks ahead are in flight (the update alone is too short
  // to cover one chunk's load latency) ----
  if (SUMS && live && !last) {
    PreW pa, pb;
    fetch(c_begin, pa, false);
    if (c_begin + 1 < c_end) fetch(c_begin + 1, pb, false);
    for (int c = c_begin; c < c_end; c += 2) {
      pin_state();
      commit(pa, false);
      if (c + 2 < c_end) fetch(c + 2, pa, false);
      update_chunk(std::false_type{});
      pin_state();
      if (c + 1 < c_end) {
        commit(pb, false);
        if (c + 3 < c_end) fetch(c + 3, pb, false);
        update_chunk(std::false_type{});
      }
    }
  }

  PreW pre;
  if (OUT && live) fetch(c_begin, pre, true);
  bool lost = false;  // a chained prefix that never arrived
  if constexpr (MODE == kChainedW) {
    // ---- exclusive prefix of the segment: the sums of the earlier waves of
    // the group through LDS, plus the published total of the first group of
    // the sequence.  Wave 3 of a first group with a successor publishes the
    // group's total. ----
    float4* xch = reinterpret_cast<float4*>(shm.xch);
    auto quad = [&](int q) __attribute__((always_inline)) -> f32x4& { return q % 5 < 4 ? S[q / 5][q % 5] : Z[q / 5]; };
    auto slot = [&](int j, int q) __attribute__((always_inline)) {
      return __builtin_bit_cast(f32x4, xch[(j * kQuads + q) * kWave + lane]);
    };
    __syncthreads();  // every wave is done with its tiles
    if (wv < 3)
#pragma unroll
      for (int q = 0; q < kQuads; ++q) {
        const f32x4 x = quad(q);
        xch[(wv * kQuads + q) * kWave + lane] = make_float4(x[0], x[1], x[2], x[3]);
      }
    __syncthreads();
    const auto rpub = buf_rsrc(p.pub + (long)bh * kQuads * kWave, kQuads * kWave * 16);
    // wave w: the sums of waves 0 .. w - 1 (wave 3 of a first group with a
    // successor also publishes them plus its own), one pass over the quads
    auto prefix_from_slots = [&](auto WC, bool publish) __attribute__((always_inline)) {
      constexpr int W = decltype(WC)::value, QB = 10;  // quads per batch of LDS reads in flight
#pragma unroll
      for (int q0 = 0; q0 < kQuads; q0 += QB) {
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
      f32x4 t[kQuads];
#pragma unroll
      for (int q = 0; q < kQuads; ++q) t[q] = load_coherent(rpub, 16 * (q * kWave + lane));
#pragma unroll
      for (int q = 0; q < kQuads; ++q) quad(q) = quad(q) + t[q];
    }
    if (seg == 0 && p.state_in != nullptr) load_state_in();
  }
  __syncthreads();  // tables; in a chained group also: the hand-over slots are read before the tiles reuse them
  if (OUT && live) {
    convert(std::integral_constant<int, 0>{});
    convert(std::integral_constant<int, 1>{});
    convert(std::integral_constant<int, 2>{});
    convert(std::integral_constant<int, 3>{});
    convert(std::integral_constant<int, 4>{});
  }

  for (int c = c_begin; OUT && c < c_end; ++c) {
    pin_state();
    commit(pre, true);
    // The next chunk's loads are issued part-way through the readout, so
    // that their registers are not live while the whole bf16 state is.
    // Every wait on the memory counter also waits for them: nothing in the
    // chunk may spill.
    {
      const int nvalid = min(CK, N - c * CK);
      const bool badh = tb.bad != 0 || lost;
      auto tile = [&](auto TC, auto FC) __attribute__((always_inline)) {
        constexpr int T = decltype(TC)::value;
        constexpr bool full = decltype(FC)::value;  // a whole chunk: no row test
        if (!full && 16 * T >= nvalid) return;
        // row 16 t + l of a tile (q or k), dims rotated by 4 lg, and the
        // monomials of its features in K-block kb, rows 4 lg + j % 4 of tiles
        // 2 kb + j / 4 (tile 8: pair (l, l + 8) in rows l < 8 (lane rows 0,
        // 1), linear term above; tile 9: linear term in rows l < 8, the
        // constant and zero rows above)
        auto load_row = [&](const uint16_t* tile, int t, float (&R)[16], uint2 (&w)[4]) __attribute__((always_inline)) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            w[i] = lds_u2(&tile[(16 * t + l) * DH + 4 * ((lg + i) & 3)]);
            float x[4];
            unpack4(w[i], x);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) R[4 * i + jj] = x[jj];
          }
        };
        auto monomials = [&](const float (&R)[16], int kb, float (&f)[8]) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int m = 2 * kb + j / 4, jj = j % 4;
            const float p8 = lg < 2 ? R[jj + 8] : 1.f, b9 = lg < 2 ? R[jj] : 1.f;
            if (m < 8) f[j] = R[jj] * R[(jj - m + 16) & 15];
            else if (m == 8) f[j] = R[jj] * p8;
            else f[j] = b9;
          }
        };
        uint2 qw[4];
        float Qr[16];
        load_row(sh.q, T, Qr, qw);
        f32x4 Y[4], Dn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int n = 0; n < 4; ++n) Y[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          float f[8];
          monomials(Qr, kb, f);
          const bf16x8 Bq = frag8(f);
#pragma unroll
          for (int n = 0; n < 4; ++n) Y[n] = mma32(As[kb][n], Bq, Y[n]);
          Dn = mma32(Az[kb], Bq, Dn);
        }
        // within-chunk pairs: key tiles 0 .. T against query tile T
        const bf16x4s Bqs = __builtin_bit_cast(bf16x4s, qw[0]);  // dims 4 lg .. 4 lg + 3 of the query
        float pk[T + 1][4];
#pragma unroll
        for (int kt = 0; kt <= T && NG > 8; ++kt) {
          // more than eight groups (up to one per dimension, with any
          // symmetric c): kappa = sum_f coef_f phi_f(k) phi_f(q) over the
          // packed features, coefficient-weighted key features against the
          // query features, five K-blocks on MFMA
          float Kr[16];
          uint2 kw4[4];
          load_row(sh.k, kt, Kr, kw4);
          f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) {
            const float4 c0 = lds_f4(&tb.coefq[32 * kb + 4 * lg]), c1 = lds_f4(&tb.coefq[32 * kb + 16 + 4 * lg]);
            const float cf[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
            float fk[8], fq[8];
            monomials(Kr, kb, fk);
            monomials(Qr, kb, fq);
#pragma unroll
            for (int j = 0; j < 8; ++j) fk[j] *= cf[j];
            sc = mma32(frag8(fk), frag8(fq), sc);
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) pk[kt][e] = (kt < T || 4 * lg + e <= l) ? sc[e] : 0.f;  // causal mask
        }
#pragma unroll
        for (int kt = 0; kt <= T && NG <= 8; ++kt) {
          const uint2 kw = lds_u2(&sh.k[(16 * kt + l) * DH + 4 * lg]);
          constexpr int NGG = NG <= 8 ? NG : 1;
          f32x4 sg[NGG];
#pragma unroll
          for (int g = 0; g < NGG; ++g) {
            uint2 km = kw;
            if (NGG > 1) {
              const uint2 mk = tb.gmask[g][lg];
              km = make_uint2(kw.x & mk.x, kw.y & mk.y);
            }
            sg[g] = mma16(__builtin_bit_cast(bf16x4s, km), Bqs, f32x4{0.f, 0.f, 0.f, 0.f});
          }
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // kappa = a + sum_g s_g (b_g + sum_{h >= g} c'_gh s_h), c'_gh = 2 sym(c)_gh off the diagonal
            float kap = tb.poly[0];
#pragma unroll
            for (int g = 0; g < NGG; ++g) {
              float inner = tb.poly[1 + g];
#pragma unroll
              for (int h2 = g; h2 < NGG; ++h2) inner += (h2 == g ? 1.f : 2.f) * tb.poly[9 + 8 * g + h2] * sg[h2][e];
              kap += sg[g][e] * inner;
            }
            if (kt == T) kap = 4 * lg + e <= l ? kap : 0.f;  // causal mask inside the diagonal tile
            pk[kt][e] = kap;
          }
        }
#pragma unroll
        for (int ks = 0; 2 * ks <= T; ++ks) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[e] = pk[2 * ks][e];
            x[4 + e] = 2 * ks + 1 <= T ? pk[2 * ks + 1 < T + 1 ? 2 * ks + 1 : T][e] : 0.f;
          }
          const bf16x8 Pf = frag8(x);
#pragma unroll
          for (int n = 0; n < 4; ++n) Y[n] = mma32(vfrag(ks, n), Pf, Y[n]);
          Dn = mma32(ones, Pf, Dn);
        }
        // Y[n][e]: column 16 n + 4 lg + e of query row 16 T + l; Dn: its
        // denominator in every element.  Rows past the end of the sequence
        // fall outside the descriptor and are not written.
        {
          // a bad group id makes the head's outputs NaN (NaN times anything)
          const float rinv = badh ? __builtin_nanf("") : __builtin_amdgcn_rcpf(Dn[0]);
          const auto ry = buf_rsrc(p.y + (rowbase + (long)c * CK + 16 * T) * DV, (nvalid - 16 * T) * DV * 2);
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            float y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = Y[n][e] * rinv;
            buf_store8(ry, l * DV * 2 + 8 * lg + 32 * n, make_uint2(pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])));
          }
        }
      };
      // the chunk after this one (the last chunk reloads itself, unused)
      const int cn = c + 1 < c_end ? c + 1 : c;
      if (nvalid == CK) {
        tile(std::integral_constant<int, 0>{}, std::true_type{});
        tile(std::integral_constant<int, 1>{}, std::true_type{});
        fetch(cn, pre, true);
        tile(std::integral_constant<int, 2>{}, std::true_type{});
        tile(std::integral_constant<int, 3>{}, std::true_type{});
      } else {
        tile(std::integral_constant<int, 0>{}, std::false_type{});
        tile(std::integral_constant<int, 1>{}, std::false_type{});
        fetch(cn, pre, true);
        tile(std::integral_constant<int, 2>{}, std::false_type{});
        tile(std::integral_constant<int, 3>{}, std::false_type{});
      }
    }

    update_chunk(std::true_type{});
  }
  // The constant feature (tile 9, row 8: lane row 2, element 0) counted 1 for
  // every row of the last chunk, also past the end of the sequence; the key
  // rows there are zero, so only z's constant row needs the fix.
  if (OUT && last && lg == 2) Z[9][0] -= (float)(nchunks * CK - N);

  // ---- results ----
  if (MODE == kSumsW) {
    float4* bs = reinterpret_cast<float4*>(p.blocksum) + ((long)seg * BH + bh) * kQuads * kWave + lane;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int n = 0; n < 5; ++n) {
        const f32x4& a = n < 4 ? S[m][n] : Z[m];
        bs[(5 * m + n) * kWave] = make_float4(a[0], a[1], a[2], a[3]);
      }
  } else if (OUT && last && p.state_out != nullptr) {
    float* so = p.state_out + (long)bh * SF;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int af = abi_map_dev.f[16 * m + 4 * lg + e];
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) so[(long)af * DV + 16 * n + l] = S[m][n][e];
        if (l == 0) so[D16 * DV + af] = Z[m][e];
      }
  }
}

struct PlanW {
  int nseg, seg_chunks;
  int nwg;  // chained launch with nwg groups of four segments; 0: three-kernel path
};

size_t blocksum_bytes_w(int BH, int nseg) { return (size_t)(nseg - 1) * BH * kQuads * kWave * sizeof(float4); }
// chained launch with two groups: a flag per sequence, then the first
// groups' published totals
size_t ctl_bytes_w(int BH) { return ((size_t)BH * sizeof(uint64_t) + 255) / 256 * 256; }
size_t chained_bytes_w(int BH, int nwg) {
  return nwg > 1 ? ctl_bytes_w(BH) + (size_t)BH * kQuads * kWave * sizeof(float4) : 0;
}

// About one wave per SIMD, at most eight segments.  With four or more
// segments per sequence, groups of four segments chained in one launch (two
// groups when the workspace holds the published totals and the waiting
// groups are fewer than the compute units, else one); below that the block
// sums, the scan and the outputs as three launches, fewer segments if the
// workspace is short.
PlanW planw(int BH, int nchunks, size_t workspace_bytes, int cus) {
  if (nchunks <= 1) return PlanW{1, 1, 0};
  const int target = std::min({std::max(1, (kWaveSegTarget + BH - 1) / BH), kWaveSegMax, std::max(nchunks, 1)});
  if (target >= 4) {
    int nwg = target / 4;  // 1 or 2 (kWaveSegMax = 8)
    if (chained_bytes_w(BH, nwg) > workspace_bytes || BH >= cus) nwg = 1;
    PlanW pl{};
    pl.nwg = nwg;
    pl.nseg = 4 * nwg;
    pl.seg_chunks = (nchunks + pl.nseg - 1) / pl.nseg;
    return pl;
  }
  for (int nseg = target;; --nseg) {
    PlanW pl{};
    pl.seg_chunks = (nchunks + nseg - 1) / nseg;
    pl.nseg = std::max(1, (nchunks + pl.seg_chunks - 1) / pl.seg_chunks);
    if (pl.nseg <= 1 || blocksum_bytes_w(BH, pl.nseg) <= workspace_bytes) {
      if (pl.nseg <= 1) pl = PlanW{1, std::max(nchunks, 1), 0};
      return pl;
    }
  }
}

}  // namespace

bool onepass16w_supported(int Hq, int Hkv, bool premap) { return Hq == Hkv && !premap; }

size_t onepass16w_workspace_bytes(int B, int Hkv, int N) {
  const int BH = B * Hkv;
  const PlanW pl = planw(BH, (N + CK - 1) / CK, (size_t)-1, 1 << 30);
  if (pl.nwg > 0) return chained_bytes_w(BH, pl.nwg);
  return pl.nseg > 1 ? blocksum_bytes_w(BH, pl.nseg) : 0;
}

hipError_t launch_onepass16w(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + CK - 1) / CK;
  const PlanW pl = planw(BH, nchunks, a.workspace ? workspace_bytes : 0, device_cus());
  Args16 p{};
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.k = reinterpret_cast<const uint16_t*>(a.k);
  p.v = reinterpret_cast<const uint16_t*>(a.v);
  p.group_of_dim = a.group_of_dim;
  p.ca = a.ca; p.cb = a.cb; p.cc = a.cc; p.G = a.G;
  p.state_in = a.state_in; p.state_out = a.state_out;
  p.blocksum = reinterpret_cast<float*>(a.workspace);
  p.y = reinterpret_cast<uint16_t*>(a.y);
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.seq_lens = a.seq_lens;
  p.seg_chunks = pl.seg_chunks; p.blk_chunks = pl.seg_chunks; p.nblk = pl.nseg - 1;
  p.nwg = pl.nwg; p.nseg = pl.nseg; p.BH = BH;
  if (pl.nwg > 1) {
    p.ctl = reinterpret_cast<uint64_t*>(a.workspace);
    p.pub = reinterpret_cast<float4*>(reinterpret_cast<char*>(a.workspace) + ctl_bytes_w(BH));
    p.tag = chained_launch_tag();
  }
  const int NG = a.G <= 1 ? 1 : a.G <= 2 ? 2 : a.G <= 4 ? 4 : a.G <= 8 ? 8 : 16;
  const long per_slot = (long)BH * kQuads * kWave;  // float4 per slot of segment sums
#define OAL_OP16W(G_)                                                                                  \
  do {                                                                                                 \
    if (pl.nwg > 0) {                                                                                  \
      hipLaunchKernelGGL((onepass16w_kernel<kChainedW, G_>), dim3(BH * pl.nwg), dim3(4 * kWave), 0, stream, p); \
      break;                                                                                           \
    }                                                                                                  \
    if (pl.nseg > 1)                                                                                   \
      hipLaunchKernelGGL((onepass16w_kernel<kSumsW, 1>), dim3(pl.nseg - 1, BH), dim3(kWave), 0, stream, p); \
    if (pl.nseg > 2)                                                                                   \
      hipLaunchKernelGGL(segment_prefix_scan_kernel, dim3((unsigned)((per_slot + 255) / 256)), dim3(256), 0, stream, \
                         reinterpret_cast<float4*>(a.workspace), pl.nseg - 1, per_slot);             \
    hipLaunchKernelGGL((onepass16w_kernel<kOutputsW, G_>), dim3(pl.nseg, BH), dim3(kWave), 0, stream, p); \
  } while (0)
  switch (NG) {
    case 1: OAL_OP16W(1); break;
    case 2: OAL_OP16W(2); break;
    case 4: OAL_OP16W(4); break;
    case 8: OAL_OP16W(8); break;
    default: OAL_OP16W(16); break;
  }
#undef OAL_OP16W
  return hipGetLastError();
}

}  // namespace oal
