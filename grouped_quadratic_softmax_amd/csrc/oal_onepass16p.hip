// Causal prefill at d_h = 16 with bfloat16 activations for heads with their
// own keys and values, two waves per (sequence x head, segment of the
// sequence): the state of the OAL paper's Eq. (5) -- 153 packed features
// (App. D) in ten accumulator tiles of sixteen rows, times the 64 value
// columns and the normaliser column z -- is split by feature tiles, tiles
// 0..4 in one wave, 5..9 in the other.  Each wave holds half the state
// (100 registers), so two waves fit on every SIMD and the
// matrix cores run one wave's products while the other wave builds features.
//
// Per 64-token chunk (the chunk's q, k and v rows land in LDS straight from
// HBM one chunk ahead, shared by the two waves of the segment):
//  1. readout phi_Q(q_i)^T [H | z] (Eq. (6)) over the wave's own features
//     for every 16-token query tile; the query features carry the
//     coefficients (a, b_g / sqrt(d), the symmetric c / d) through the
//     state operands, so the state stays coefficient-free.  A wave owns two
//     query tiles (0 and 3, or 1 and 2: five within-chunk tiles each) and
//     hands its partial readout of the other two to its partner through LDS;
//  2. for an owned query tile, the within-chunk pairs (sec. 4.2): per group
//     a masked 16x16x16 MFMA gives the group's partial dot products, the
//     polynomial and the causal mask are applied in registers, and V^T P^T
//     runs on the 16x16x32 MFMA; the partner's partial is added and the row
//     is normalised;
//  3. the state update S += phi_K(K_c)^T [V_c | 1] over the wave's own
//     feature tiles, key features from DPP row rotations.
//
// Segments.  A workgroup of eight waves takes four consecutive segments of
// one (sequence x head) (two workgroups per sequence at most); each wave
// first sums its half of its segment (the last segment of the sequence needs
// no sum), the sums go to the later segments of the group through LDS, and
// with two groups the last segment of the first group publishes the group's
// total per half (device-scope stores and a flag, polled with a bound); then
// every wave produces its part of its segment's outputs.
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

constexpr int kHT = MT / 2;      // feature tiles per wave
constexpr int kQP = 5 * kHT;     // accumulator quads per wave: (tile, column tile 0..3 of H, 4: z)
constexpr int kPW = 8;           // waves per workgroup: four segments x two halves
constexpr int kWaveTargetP = 2048;  // waves that fill the chip twice (two per SIMD)
constexpr int kSegMaxP = 8;

struct __align__(16) TileP {  // one segment's chunk rows, shared by its two waves
  uint16_t q[CK * DH];        // [64][16]
  uint16_t k[CK * DH];        // [64][16]
  uint16_t v[CK * DV];        // [64][64], 16-byte pieces permuted (vswz16)
};
struct __align__(16) XchP {   // a partial readout of one query tile handed to the partner
  float4 y[4][kWave];         // [column tile][lane]
  float dn[kWave];
};
struct __align__(16) WorkP {
  TileP t[2][4];              // [buffer][segment of the workgroup]
  XchP x[kPW];                // [wave]
};
constexpr int kSlotBytesP = 3 * 2 * kQP * kWave * 16;  // segment sums of segments 0..2, both halves
struct __align__(16) TablesP {
  float coefq[FT];            // query-side coefficient of every feature row
  float poly[1 + 8 + 64];     // a, b_g / sqrt(d), sym(c)_gh / d
  uint2 gmask[8][4];          // [group][lg]: bf16 lane masks of dims 4 lg .. 4 lg + 3 in the group
  int bad;                    // a group id outside [0, G)
};
struct __align__(16) LdsP {
  union {
    WorkP w;
    unsigned char slots[kSlotBytesP];
  };
  TablesP tb;
};
static_assert(sizeof(LdsP) <= 160 * 1024, "LDS budget");

typedef __attribute__((address_space(3))) void lds_void;
typedef unsigned int u32x4w __attribute__((ext_vector_type(4)));
// Raw buffer descriptor words (gfx9 family) over `bytes` bytes from `base`.
__device__ __forceinline__ u32x4w rsrc_words(const void* base, int bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4w{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, (unsigned)max(bytes, 0), 0x00020000u};
}
// 64 lanes x 16 bytes from the buffer (at voff + soff) straight into LDS:
// lane i's bytes land at lds + 16 i; bytes past the descriptor's end read
// as zero.  Written out so that the compiler, which cannot tell the two chunk
// buffers apart, does not wait for the transfer before every LDS read: the
// chunk loops wait for their own transfers (vmcnt) and meet at a barrier
// before the data is read.  The instruction has no register results.  M0
// (the LDS address) is not declared clobbered: the compiler reserves it and
// these kernels use it for nothing else.
__device__ __forceinline__ void lds_dma16(const u32x4w& r, void* lds, int voff, int soff) {
  const unsigned m0v = (unsigned)(uintptr_t)(lds_void*)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
               : "memory");
}
// Workgroup barrier for LDS data only: the wave's LDS writes are complete,
// and the compiler keeps memory accesses on their side of it.  (A full
// __syncthreads() also waits for every outstanding HBM transfer, including
// the next chunk's.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ void wait_transfers() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int NG, int HF>
__device__ __forceinline__ void pair_body(const Args16& p, LdsP& shm) {
  constexpr int M0 = kHT * HF;  // first feature tile of this wave
  const int lane = threadIdx.x % kWave, lg = lane / 16, l = lane % 16;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int sl = wv & 3;         // segment within the workgroup
  const int partner = wv ^ 4;
  TablesP& tb = shm.tb;
  const int bh = blockIdx.x % p.BH, grp = blockIdx.x / p.BH, seg = 4 * grp + sl;
  const int N = seq_len_of(p.seq_lens, bh / p.Hkv, p.N);
  const int nchunks = (N + CK - 1) / CK;
  const int c_begin = seg * p.seg_chunks, c_end = min(c_begin + p.seg_chunks, nchunks);
  const bool live = c_begin < c_end;
  const bool last = nchunks == 0 ? seg == 0 : live && c_end == nchunks;
  const long rowbase = (long)bh * p.N;
  constexpr long SF = D16 * (DV + 1);

  // ---- per-head tables, spread over the workgroup's threads ----
  {
    const int h = bh % p.Hq;
    const float rs = 0.25f, rd = 1.f / 16.f;  // 1/sqrt(d), 1/d at d = 16
    const int tid = threadIdx.x, nth = kPW * kWave;
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

  // ---- this wave's half of the state: S[i][n] holds rows 4 lg + e of tile
  // M0 + i, columns 16 n + l; Z[i] the same rows of z in every column ----
  f32x4 S[kHT][4], Z[kHT];
#pragma unroll
  for (int i = 0; i < kHT; ++i) {
    Z[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int n = 0; n < 4; ++n) S[i][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto load_state_in = [&]() __attribute__((always_inline)) {
    const float* si = p.state_in + (long)bh * SF;
#pragma unroll
    for (int i = 0; i < kHT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int af = abi_map_dev.f[16 * (M0 + i) + 4 * lg + e];
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) S[i][n][e] = si[(long)af * DV + 16 * n + l];
        Z[i][e] = si[D16 * DV + af];
      }
  };
  // segment 0's sum starts from the initial state, so that every later
  // prefix includes it
  if (p.state_in != nullptr && seg == 0) load_state_in();

  // ---- chunk rows into LDS: wave half 0 brings q, k and value rows 0..15,
  // half 1 value rows 16..63 (six 1 KB transfers each; q only for outputs).
  // The descriptors end at the end of the sequence.  Transfer u covers the
  // 64 pieces 64 u .. 64 u + 63 (eight value rows); the value pieces' lane
  // offsets depend only on the parity of u, the rest is a scalar offset. ----
  auto v_voff = [&](int u) __attribute__((always_inline)) {
    const int idx = 64 * u + lane, row = idx >> 3;
    return row * (DV * 2) + 16 * ((idx & 7) ^ vswz16(row));
  };
  auto dma = [&](int c, int buf, bool wq) __attribute__((always_inline)) {
    TileP& T = shm.w.t[buf][sl];
    const long r0 = rowbase + (long)c * CK;
    const int left = N - c * CK;
    int ln = lane;
    asm volatile("" : "+v"(ln));  // recomputed here, not held in registers across the chunk
    const int o16 = 16 * ln;
    const int ov0 = (ln >> 3) * (DV * 2) + 16 * ((ln & 7) ^ vswz16(ln >> 3));
    const int ov1 = (ln >> 3) * (DV * 2) + 16 * ((ln & 7) ^ vswz16(8 + (ln >> 3)));
    const u32x4w rv = rsrc_words(p.v + r0 * DV, left * DV * 2);
    if (HF == 0) {
      const u32x4w rk = rsrc_words(p.k + r0 * DH, left * DH * 2);
      if (wq) {
        const u32x4w rq = rsrc_words(p.q + r0 * DH, left * DH * 2);
#pragma unroll
        for (int u = 0; u < 2; ++u) lds_dma16(rq, T.q + 512 * u, o16, 1024 * u);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_dma16(rk, T.k + 512 * u, o16, 1024 * u);
#pragma unroll
      for (int u = 0; u < 2; ++u) lds_dma16(rv, T.v + 512 * u, u & 1 ? ov1 : ov0, 1024 * u);
    } else {
#pragma unroll
      for (int u = 2; u < 8; ++u) lds_dma16(rv, T.v + 512 * u, u & 1 ? ov1 : ov0, 1024 * u);
    }
  };
  // rows past the end of the sequence as zeros (whatever the transfers left
  // there), each half over the rows it brings
  auto zero_tail = [&](int c, int buf, bool wq) __attribute__((always_inline)) {
    TileP& T = shm.w.t[buf][sl];
    const int left = N - c * CK;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    if (HF == 0) {
      for (int idx = lane; idx < 128; idx += kWave)
        if (idx / 2 >= left) {
          if (wq) *reinterpret_cast<uint4*>(&T.q[8 * idx]) = z;
          *reinterpret_cast<uint4*>(&T.k[8 * idx]) = z;
        }
      for (int idx = lane; idx < 128; idx += kWave)
        if (idx / 8 >= left) *reinterpret_cast<uint4*>(&T.v[8 * idx]) = z;
    } else {
      for (int idx = 128 + lane; idx < 512; idx += kWave)
        if (idx / 8 >= left) *reinterpret_cast<uint4*>(&T.v[8 * idx]) = z;
    }
  };

  // Token order of a 32-token key step ks: operand position 8 lg + j holds
  // token 32 ks + 4 lg + j (j < 4) or 32 ks + 16 + 4 lg + j - 4 (j >= 4), the
  // rows of the score tiles 2 ks and 2 ks + 1 as the 16x16x16 MFMA leaves
  // them.
  int vo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int r = 4 * lg + l / 4, cc = 16 * n + 4 * (l % 4);
    vo[n] = r * DV + 8 * ((cc >> 3) ^ vswz16(r)) + (cc & 7);
  }
  const int ko = (4 * lg + l / 4) * DH + 4 * (l % 4);
  auto vfrag = [&](const TileP& T, int ks, int n) __attribute__((always_inline)) {
    const uint2 lo = v_rows4_at(T.v + 32 * ks * DV, vo[n]);
    const uint2 hi = v_rows4_at(T.v + (32 * ks + 16) * DV, vo[n]);
    return u4_frag(lo.x, lo.y, hi.x, hi.y);
  };

  // ---- the state before a chunk as bf16 operands times the query-side
  // coefficients: two-tile K-blocks for the 16x16x32 MFMA, and the one tile
  // left over (tile 4 in half 0, tile 5 in half 1) for the 16x16x16 MFMA ----
  constexpr int kSingle = HF == 0 ? 4 : 0;     // local index of the lone tile
  constexpr int kPair0 = HF == 0 ? 0 : 1;      // local index of the first tile of K-block 0
  bf16x8 Ap[2][4], Apz[2];
  bf16x4s A1[4], A1z;
  auto convert_pair = [&](auto KC) __attribute__((always_inline)) {
    constexpr int kb = decltype(KC)::value, i0 = kPair0 + 2 * kb, m = M0 + i0;
    const float4 c0 = lds_f4(&tb.coefq[16 * m + 4 * lg]), c1 = lds_f4(&tb.coefq[16 * (m + 1) + 4 * lg]);
    auto frag = [&](const f32x4& x0, const f32x4& x1) __attribute__((always_inline)) {
      return u4_frag(pack_bf16(x0[0] * c0.x, x0[1] * c0.y), pack_bf16(x0[2] * c0.z, x0[3] * c0.w),
                     pack_bf16(x1[0] * c1.x, x1[1] * c1.y), pack_bf16(x1[2] * c1.z, x1[3] * c1.w));
    };
#pragma unroll
    for (int n = 0; n < 4; ++n) Ap[kb][n] = frag(S[i0][n], S[i0 + 1][n]);
    Apz[kb] = frag(Z[i0], Z[i0 + 1]);
  };
  auto convert_single = [&]() __attribute__((always_inline)) {
    constexpr int m = M0 + kSingle;
    const float4 c0 = lds_f4(&tb.coefq[16 * m + 4 * lg]);
    auto frag = [&](const f32x4& x) __attribute__((always_inline)) {
      return __builtin_bit_cast(bf16x4s, make_uint2(pack_bf16(x[0] * c0.x, x[1] * c0.y),
                                                    pack_bf16(x[2] * c0.z, x[3] * c0.w)));
    };
#pragma unroll
    for (int n = 0; n < 4; ++n) A1[n] = frag(S[kSingle][n]);
    A1z = frag(Z[kSingle]);
  };
  const bf16x8 ones = kOnes;

  // state update with a chunk over this wave's tiles; with CONV the next
  // chunk's operands are rounded as soon as their tiles hold the state
  auto update_chunk = [&](const TileP& T, auto CONV) __attribute__((always_inline)) {
    constexpr bool conv = decltype(CONV)::value;
    float kv[2][8];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float x[4];
      unpack4(k_rows4_at(T.k + 32 * ks * DH, ko), x);
      kv[ks][0] = x[0]; kv[ks][1] = x[1]; kv[ks][2] = x[2]; kv[ks][3] = x[3];
      unpack4(k_rows4_at(T.k + (32 * ks + 16) * DH, ko), x);
      kv[ks][4] = x[0]; kv[ks][5] = x[1]; kv[ks][6] = x[2]; kv[ks][7] = x[3];
    }
    bf16x8 Vf[2][4];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int n = 0; n < 4; ++n) Vf[ks][n] = vfrag(T, ks, n);
    auto mtile = [&](auto IC) __attribute__((always_inline)) {
      constexpr int i = decltype(IC)::value;
      float f0[8], f1[8];
      key_features<M0 + i>(kv[0], l, 0, CK, f0);  // the constant is 1 for every token (fixed up at the end)
      key_features<M0 + i>(kv[1], l, 0, CK, f1);
      const bf16x8 K0 = frag8(f0), K1 = frag8(f1);
#pragma unroll
      for (int n = 0; n < 4; ++n) S[i][n] = mma32(K1, Vf[1][n], mma32(K0, Vf[0][n], S[i][n]));
      Z[i] = mma32(K1, ones, mma32(K0, ones, Z[i]));
    };
    mtile(std::integral_constant<int, 0>{});
    if (conv && HF == 1) convert_single();
    mtile(std::integral_constant<int, 1>{});
    if (conv && HF == 0) convert_pair(std::integral_constant<int, 0>{});
    mtile(std::integral_constant<int, 2>{});
    if (conv && HF == 1) convert_pair(std::integral_constant<int, 0>{});
    mtile(std::integral_constant<int, 3>{});
    if (conv && HF == 0) convert_pair(std::integral_constant<int, 1>{});
    mtile(std::integral_constant<int, 4>{});
    if (conv && HF == 0) convert_single();
    if (conv && HF == 1) convert_pair(std::integral_constant<int, 1>{});
  };

  // ---- segment sums (the segment that ends the sequence needs none); all
  // eight waves step through the same number of chunks and barriers ----
  const bool sums = live && !last;
  if (sums) dma(c_begin, 0, false);
  for (int j = 0; j < p.seg_chunks; ++j) {
    const int c = c_begin + j;
    const bool act = sums && c < c_end;
    wait_transfers();
    if (act && N - c * CK < CK) zero_tail(c, j & 1, false);
    lds_barrier();  // the chunk is in LDS; everyone is done with the other buffer
    if (act && c + 1 < c_end) dma(c + 1, (j + 1) & 1, false);
    if (act) update_chunk(shm.w.t[j & 1][sl], std::false_type{});
  }

  // ---- the first output chunk's rows, in registers until the hand-over
  // slots (which share the LDS) are read ----
  uint4 pre[6];
  const bool outs = live;
  if (outs) {
    const long r0 = rowbase + (long)c_begin * CK;
    const int left = N - c_begin * CK;
    const auto rv = buf_rsrc(p.v + r0 * DV, left * DV * 2);
    if (HF == 0) {
      const auto rq = buf_rsrc(p.q + r0 * DH, left * DH * 2);
      const auto rk = buf_rsrc(p.k + r0 * DH, left * DH * 2);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        pre[u] = buf_load16(rq, 16 * (64 * u + lane));
        pre[2 + u] = buf_load16(rk, 16 * (64 * u + lane));
        pre[4 + u] = buf_load16(rv, v_voff(u));
      }
    } else {
#pragma unroll
      for (int u = 0; u < 6; ++u) pre[u] = buf_load16(rv, v_voff(2 + u));
    }
  }

  // ---- exclusive prefix of the segment, per half: the sums of the earlier
  // segments of the group through LDS, plus the published total of the
  // first group of the sequence ----
  bool lost = false;
  {
    float4* slots = reinterpret_cast<float4*>(shm.slots);
    auto quad = [&](int q) __attribute__((always_inline)) -> f32x4& { return q % 5 < 4 ? S[q / 5][q % 5] : Z[q / 5]; };
    auto slot_at = [&](int j, int q) __attribute__((always_inline)) { return ((j * 2 + HF) * kQP + q) * kWave + lane; };
    lds_barrier();  // every wave is done with the chunk tiles
    if (sl < 3)
#pragma unroll
      for (int q = 0; q < kQP; ++q) {
        const f32x4 x = quad(q);
        slots[slot_at(sl, q)] = make_float4(x[0], x[1], x[2], x[3]);
      }
    lds_barrier();
    uint64_t* flag = p.ctl + 2 * bh + HF;
    const auto rpub = buf_rsrc(p.pub + ((long)bh * 2 + HF) * kQP * kWave, kQP * kWave * 16);
    auto prefix_from_slots = [&](auto WC, bool publish) __attribute__((always_inline)) {
      constexpr int W = decltype(WC)::value, QB = 5;
#pragma unroll
      for (int q0 = 0; q0 < kQP; q0 += QB) {
        f32x4 x[QB];
#pragma unroll
        for (int i = 0; i < QB; ++i) x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < W; ++j) {
#pragma unroll
          for (int i = 0; i < QB; ++i) x[i] = x[i] + __builtin_bit_cast(f32x4, slots[slot_at(j, q0 + i)]);
        }
#pragma unroll
        for (int i = 0; i < QB; ++i) {
          if (publish) store_coherent(rpub, 16 * ((q0 + i) * kWave + lane), x[i] + quad(q0 + i));
          quad(q0 + i) = x[i];
        }
      }
    };
    switch (sl) {
      case 0: prefix_from_slots(std::integral_constant<int, 0>{}, false); break;
      case 1: prefix_from_slots(std::integral_constant<int, 1>{}, false); break;
      case 2: prefix_from_slots(std::integral_constant<int, 2>{}, false); break;
      default:
        if (grp == 0 && p.nwg > 1) {
          prefix_from_slots(std::integral_constant<int, 3>{}, true);
          if (lane == 0) publish_flag(flag, p.tag);
        } else {
          prefix_from_slots(std::integral_constant<int, 3>{}, false);
        }
    }
    if (grp > 0) {
      lost = !wait_published(flag, p.tag);
      f32x4 t[kQP];
#pragma unroll
      for (int q = 0; q < kQP; ++q) t[q] = load_coherent(rpub, 16 * (q * kWave + lane));
#pragma unroll
      for (int q = 0; q < kQP; ++q) quad(q) = quad(q) + t[q];
    }
    if (seg == 0 && p.state_in != nullptr) load_state_in();
  }
  lds_barrier();  // the slots are read before the chunk tiles reuse the LDS
  if (outs) {
    TileP& T = shm.w.t[0][sl];
    if (HF == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        *reinterpret_cast<uint4*>(T.q + 512 * u + 8 * lane) = pre[u];
        *reinterpret_cast<uint4*>(T.k + 512 * u + 8 * lane) = pre[2 + u];
        *reinterpret_cast<uint4*>(T.v + 512 * u + 8 * lane) = pre[4 + u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < 6; ++u) *reinterpret_cast<uint4*>(T.v + 512 * (2 + u) + 8 * lane) = pre[u];
    }
    convert_pair(std::integral_constant<int, 0>{});
    convert_pair(std::integral_constant<int, 1>{});
    convert_single();
  }

  // ---- outputs ----
  const bool badh = tb.bad != 0 || lost;  // tb is read after the barriers above
  XchP& mine = shm.w.x[wv];
  const XchP& theirs = shm.w.x[partner];
  // query tile T of the chunk in T_: partial readout over this wave's
  // features (Y[n][e]: column 16 n + 4 lg + e of query row 16 T + l; Dn: its
  // denominator part in every element)
  auto readout = [&](const TileP& Tl, auto TC, f32x4 (&Y)[4], f32x4& Dn, uint2 (&qw)[4], float (&Qr)[16])
      __attribute__((always_inline)) {
    constexpr int T = decltype(TC)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qw[i] = lds_u2(&Tl.q[(16 * T + l) * DH + 4 * ((lg + i) & 3)]);
      float x[4];
      unpack4(qw[i], x);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) Qr[4 * i + jj] = x[jj];
    }
    // monomial of feature row 4 lg + jj of tile m for this lane's query row
    auto mono = [&](int m, int jj) __attribute__((always_inline)) {
      const float p8 = lg < 2 ? Qr[jj + 8] : 1.f, b9 = lg < 2 ? Qr[jj] : 1.f;
      if (m < 8) return Qr[jj] * Qr[(jj - m + 16) & 15];
      if (m == 8) return Qr[jj] * p8;
      return b9;
    };
#pragma unroll
    for (int n = 0; n < 4; ++n) Y[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    Dn = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int m = M0 + kPair0 + 2 * kb;
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = mono(m + j / 4, j % 4);
      const bf16x8 Bq = frag8(f);
#pragma unroll
      for (int n = 0; n < 4; ++n) Y[n] = mma32(Ap[kb][n], Bq, Y[n]);
      Dn = mma32(Apz[kb], Bq, Dn);
    }
    {
      constexpr int m = M0 + kSingle;
      const bf16x4s Bq = __builtin_bit_cast(
          bf16x4s, make_uint2(pack_bf16(mono(m, 0), mono(m, 1)), pack_bf16(mono(m, 2), mono(m, 3))));
#pragma unroll
      for (int n = 0; n < 4; ++n) Y[n] = mma16(A1[n], Bq, Y[n]);
      Dn = mma16(A1z, Bq, Dn);
    }
  };
  auto hand_over = [&](const TileP& Tl, auto TC, int nvalid) __attribute__((always_inline)) {
    constexpr int T = decltype(TC)::value;
    if (16 * T >= nvalid) return;
    f32x4 Y[4], Dn;
    uint2 qw[4];
    float Qr[16];
    readout(Tl, TC, Y, Dn, qw, Qr);
#pragma unroll
    for (int n = 0; n < 4; ++n) mine.y[n][lane] = make_float4(Y[n][0], Y[n][1], Y[n][2], Y[n][3]);
    mine.dn[lane] = Dn[0];
  };
  auto own = [&](const TileP& Tl, auto TC, long crow, int nvalid) __attribute__((always_inline)) {
    constexpr int T = decltype(TC)::value;
    if (16 * T >= nvalid) return;
    f32x4 Y[4], Dn;
    uint2 qw[4];
    float Qr[16];
    readout(Tl, TC, Y, Dn, qw, Qr);
    // within-chunk pairs: key tiles 0 .. T against query tile T
    const bf16x4s Bqs = __builtin_bit_cast(bf16x4s, qw[0]);  // dims 4 lg .. 4 lg + 3 of the query
    float pk[T + 1][4];
#pragma unroll
    for (int kt = 0; kt <= T; ++kt) {
      const uint2 kw = lds_u2(&Tl.k[(16 * kt + l) * DH + 4 * lg]);
      f32x4 sg[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        uint2 km = kw;
        if (NG > 1) {
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
        for (int g = 0; g < NG; ++g) {
          float inner = tb.poly[1 + g];
#pragma unroll
          for (int h2 = g; h2 < NG; ++h2) inner += (h2 == g ? 1.f : 2.f) * tb.poly[9 + 8 * g + h2] * sg[h2][e];
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
      for (int n = 0; n < 4; ++n) Y[n] = mma32(vfrag(Tl, ks, n), Pf, Y[n]);
      Dn = mma32(ones, Pf, Dn);
    }
    // the partner's part of the readout
    const float den = Dn[0] + theirs.dn[lane];
    const float rinv = badh ? __builtin_nanf("") : __builtin_amdgcn_rcpf(den);
    const auto ry = buf_rsrc(p.y + (crow + 16 * T) * DV, (nvalid - 16 * T) * DV * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const float4 o = theirs.y[n][lane];
      const float y0 = (Y[n][0] + o.x) * rinv, y1 = (Y[n][1] + o.y) * rinv;
      const float y2 = (Y[n][2] + o.z) * rinv, y3 = (Y[n][3] + o.w) * rinv;
      buf_store8(ry, l * DV * 2 + 8 * lg + 32 * n, make_uint2(pack_bf16(y0, y1), pack_bf16(y2, y3)));
    }
  };

  for (int j = 0; j < p.seg_chunks; ++j) {
    const int c = c_begin + j;
    const bool act = outs && c < c_end;
    const int nvalid = min(CK, N - c * CK);
    const TileP& Tl = shm.w.t[j & 1][sl];
    const long crow = rowbase + (long)c * CK;
    wait_transfers();
    if (act && j > 0 && nvalid < CK) zero_tail(c, j & 1, true);
    lds_barrier();  // the chunk is in LDS; everyone is done with the other buffer
    if (act && c + 1 < c_end) dma(c + 1, (j + 1) & 1, true);
    if (act) {
      if (HF == 0) hand_over(Tl, std::integral_constant<int, 1>{}, nvalid);
      else hand_over(Tl, std::integral_constant<int, 0>{}, nvalid);
    }
    lds_barrier();
    if (act) {
      if (HF == 0) own(Tl, std::integral_constant<int, 0>{}, crow, nvalid);
      else own(Tl, std::integral_constant<int, 1>{}, crow, nvalid);
    }
    lds_barrier();  // the partner has read this wave's slot
    if (act) {
      if (HF == 0) hand_over(Tl, std::integral_constant<int, 2>{}, nvalid);
      else hand_over(Tl, std::integral_constant<int, 3>{}, nvalid);
    }
    lds_barrier();
    if (act) {
      if (HF == 0) own(Tl, std::integral_constant<int, 3>{}, crow, nvalid);
      else own(Tl, std::integral_constant<int, 2>{}, crow, nvalid);
      update_chunk(Tl, std::true_type{});
    }
  }
  // The constant feature (tile 9, row 8: half 1, local tile 4, lane row 2,
  // element 0) counted 1 for every row of the last chunk, also past the end
  // of the sequence; the key rows there are zero, so only z's constant row
  // needs the fix.
  if (HF == 1 && last && lg == 2) Z[4][0] -= (float)(nchunks * CK - N);

  if (last && p.state_out != nullptr) {
    float* so = p.state_out + (long)bh * SF;
#pragma unroll
    for (int i = 0; i < kHT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int af = abi_map_dev.f[16 * (M0 + i) + 4 * lg + e];
        if (af < 0) continue;
#pragma unroll
        for (int n = 0; n < 4; ++n) so[(long)af * DV + 16 * n + l] = S[i][n][e];
        if (l == 0) so[D16 * DV + af] = Z[i][e];
      }
  }
}

template <int NG>
__global__ __launch_bounds__(kPW * kWave, 1) void onepass16p_kernel(const Args16 p) {
  __shared__ LdsP shm;
  const int hf = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave) >> 2;
  if (hf == 0) pair_body<NG, 0>(p, shm);
  else pair_body<NG, 1>(p, shm);
}

struct PlanP {
  int nseg, seg_chunks, nwg;
};
size_t ctl_bytes_p(int BH) { return ((size_t)BH * 2 * sizeof(uint64_t) + 255) / 256 * 256; }
size_t chained_bytes_p(int BH, int nwg) {
  return nwg > 1 ? ctl_bytes_p(BH) + (size_t)BH * 2 * kQP * kWave * sizeof(float4) : 0;
}
// Two waves per segment, about two waves per SIMD, four or eight segments:
// one group of four per sequence, or two when the workspace holds the
// published totals and the waiting groups are fewer than the compute units.
// nseg = 0: fewer than four segments would do, which this build does not.
PlanP planp(int BH, int nchunks, size_t workspace_bytes, int cus) {
  const int target = std::min({std::max(1, (kWaveTargetP / 2 + BH - 1) / BH), kSegMaxP, std::max(nchunks, 1)});
  if (target < 4) return PlanP{0, 0, 0};
  int nwg = target / 4;
  if (chained_bytes_p(BH, nwg) > workspace_bytes || BH >= cus) nwg = 1;
  PlanP pl{};
  pl.nwg = nwg;
  pl.nseg = 4 * nwg;
  pl.seg_chunks = (nchunks + pl.nseg - 1) / pl.nseg;
  return pl;
}

}  // namespace

bool onepass16p_supported(const FwdLaunch& a, size_t workspace_bytes) {
  // up to two groups: with more, the within-chunk group products do not fit
  // the registers of two waves per SIMD
  if (a.Hq != a.Hkv || a.premap || a.G < 1 || a.G > 2) return false;
  const int BH = a.B * a.Hkv;
  return planp(BH, (a.N + CK - 1) / CK, a.workspace ? workspace_bytes : 0, device_cus()).nseg >= 4;
}

size_t onepass16p_workspace_bytes(int B, int Hkv, int N) {
  const int BH = B * Hkv;
  const PlanP pl = planp(BH, (N + CK - 1) / CK, (size_t)-1, 1 << 30);
  return pl.nseg >= 4 ? chained_bytes_p(BH, pl.nwg) : 0;
}

hipError_t launch_onepass16p(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream) {
  const int BH = a.B * a.Hkv;
  const int nchunks = (a.N + CK - 1) / CK;
  const PlanP pl = planp(BH, nchunks, a.workspace ? workspace_bytes : 0, device_cus());
  if (pl.nseg < 4) return hipErrorInvalidValue;
  Args16 p{};
  p.q = reinterpret_cast<const uint16_t*>(a.q);
  p.k = reinterpret_cast<const uint16_t*>(a.k);
  p.v = reinterpret_cast<const uint16_t*>(a.v);
  p.group_of_dim = a.group_of_dim;
  p.ca = a.ca; p.cb = a.cb; p.cc = a.cc; p.G = a.G;
  p.state_in = a.state_in; p.state_out = a.state_out;
  p.y = reinterpret_cast<uint16_t*>(a.y);
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.N = a.N; p.seq_lens = a.seq_lens;
  p.seg_chunks = pl.seg_chunks; p.blk_chunks = pl.seg_chunks; p.nblk = 0;
  p.nwg = pl.nwg; p.nseg = pl.nseg; p.BH = BH;
  if (pl.nwg > 1) {
    p.ctl = reinterpret_cast<uint64_t*>(a.workspace);
    p.pub = reinterpret_cast<float4*>(reinterpret_cast<char*>(a.workspace) + ctl_bytes_p(BH));
    p.tag = chained_launch_tag();
  }
  const dim3 grid(BH * pl.nwg), block(kPW * kWave);
  if (a.G <= 1) hipLaunchKernelGGL((onepass16p_kernel<1>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((onepass16p_kernel<2>), grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace oal
