// Shared pieces of the d_h = 16 bf16 prefill kernels: the feature order of
// the packed state held as MFMA accumulator tiles, the key features built
// from DPP row rotations, bf16 fragment packing, the transposing LDS reads
// of the value tile, and the argument block.
//
// Feature order (the OAL paper's App. D counts 153 packed features at
// d_h = 16).  They are held as ten tiles m of sixteen rows l (160 rows,
// seven of them zero):
//   m = 0..7   the pair (l, (l - m) mod 16)   (m = 0: the square of dim l)
//   m = 8      l < 8: the pair (l, l + 8);  l >= 8: the linear term of dim l
//   m = 9      l < 8: the linear term of dim l;  l = 8: the constant;  else 0
// Every unordered pair r <= t appears exactly once (a pair with index
// difference 8 only in rows l < 8 of tile 8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oal_device.h"

namespace oal {
namespace {

constexpr int DH = 16;
constexpr int DV = 64;
constexpr int CK = 64;        // tokens per chunk
constexpr int MT = 10;        // feature tiles of sixteen rows
constexpr int FT = MT * 16;   // 160 feature rows (153 used)
constexpr int NKB = MT / 2;   // K-blocks of 32 features
constexpr int RMAX = 8;       // query heads per KV head
constexpr long D16 = 153;     // packed feature count at d_h = 16

typedef short bf16x4s __attribute__((ext_vector_type(4)));

// (r, t) of internal feature (m, l): t == DH is the linear term of r,
// (DH, DH) the constant, r < 0 a zero row.
__host__ __device__ constexpr void op_feature(int m, int l, int& r, int& t) {
  if (m < 8) {
    r = l;
    t = (l - m + 16) & 15;
  } else if (m == 8) {
    r = l;
    t = l < 8 ? l + 8 : DH;
  } else if (l < 8) {
    r = l;
    t = DH;
  } else if (l == 8) {
    r = DH;
    t = DH;
  } else {
    r = -1;
    t = -1;
  }
}

// Packed (library) index of internal feature row f = 16 m + l, -1 for zero rows.
struct AbiMap {
  short f[FT];
};
constexpr AbiMap make_abi_map() {
  AbiMap a{};
  for (int m = 0; m < MT; ++m)
    for (int l = 0; l < 16; ++l) {
      int r = 0, t = 0;
      op_feature(m, l, r, t);
      short v = -1;
      if (r == DH) {
        v = 0;
      } else if (r >= 0 && t == DH) {
        v = (short)(1 + r);
      } else if (r >= 0) {
        const int lo = r < t ? r : t, hi = r < t ? t : r;
        v = (short)(1 + DH + lo * DH - lo * (lo - 1) / 2 + (hi - lo));
      }
      a.f[16 * m + l] = v;
    }
  return a;
}
__device__ constexpr AbiMap abi_map_dev = make_abi_map();


template <int CTRL>
__device__ __forceinline__ float dppf(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
// value of lane (l - m) mod 16 of the same sixteen-lane row (DPP row rotate right by m)
__device__ __forceinline__ float row_ror(float x, int m) {
  switch (m) {
    case 1: return dppf<0x121>(x);
    case 2: return dppf<0x122>(x);
    case 3: return dppf<0x123>(x);
    case 4: return dppf<0x124>(x);
    case 5: return dppf<0x125>(x);
    case 6: return dppf<0x126>(x);
    case 7: return dppf<0x127>(x);
    case 8: return dppf<0x128>(x);
    default: return x;
  }
}

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const f32x2v x = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2v));
}
__device__ __forceinline__ bf16x8 frag8(const float (&x)[8]) {
  const uint4 w = make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                             pack_bf16(x[6], x[7]));
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ f32x4 mma32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// bf16 ones: the B operand that sums the A operand's rows
constexpr uint4 kOnesBits = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};
#define kOnes (__builtin_bit_cast(bf16x8, kOnesBits))
__device__ __forceinline__ f32x4 mma16(const bf16x4s& a, const bf16x4s& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16-, 8- and 32-byte LDS accesses
__device__ __forceinline__ uint4 lds_u4(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 lds_u2(const void* p) { return *reinterpret_cast<const uint2*>(p); }
__device__ __forceinline__ float4 lds_f4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void lds_st_f4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void lds_st_u2(void* p, uint2 v) { *reinterpret_cast<uint2*>(p) = v; }

__device__ __forceinline__ void unpack4(uint2 w, float (&x)[4]) {
  x[0] = __uint_as_float(w.x << 16);
  x[1] = __uint_as_float(w.x & 0xffff0000u);
  x[2] = __uint_as_float(w.y << 16);
  x[3] = __uint_as_float(w.y & 0xffff0000u);
}

struct Args16 {
  const uint16_t *q, *k, *v;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  int G;
  const float *gamma_q, *beta_q, *gamma_k, *beta_k;
  float ln_eps;
  PremapNorm pn;    // the pre-map's normalisation (LayerNorm or unit l2 norm)
  const float* state_in;
  float* state_out;
  float* blocksum;  // [nblk][BH][FT][DV + 1] fp32: sums of phi_K^T [V | 1] over blocks of chunks
  uint16_t* y;
  int Hq, Hkv, N;
  int seg_chunks;   // chunks per segment (outputs kernel)
  int blk_chunks;   // chunks per summed block (divides seg_chunks)
  int nblk;         // blocks summed by the first kernel per (sequence, KV head)
  // one-launch segment chaining (workgroups of four segment waves)
  uint64_t* ctl;    // [BH]: == tag once the first group's total is published
  float4* pub;      // [BH][quads x 64 lanes]: the first groups' totals
  uint64_t tag;     // unique to the launch
  int nwg, nseg, BH;
  const int32_t* seq_lens;  // [B] lengths within the padded N (null: all N)
};

// Key features of tile M for the eight tokens t0 .. t0 + 7 whose k_l this
// lane holds (kv); lane row l.  Partners come from lane (l - M) mod 16 of the
// same row.  Tile 9 row 8 is the constant (1 for tokens inside the
// sequence); its rows 9..15 are zero.
template <int M>
__device__ __forceinline__ void key_features(const float (&kv)[8], int l, int t0, int nvalid, float (&f)[8]) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if constexpr (M == 0) {
      f[j] = kv[j] * kv[j];
    } else if constexpr (M < 8) {
      f[j] = kv[j] * row_ror(kv[j], M);
    } else if constexpr (M == 8) {
      const float pr = row_ror(kv[j], 8);
      f[j] = kv[j] * (l < 8 ? pr : 1.f);
    } else {
      f[j] = l < 8 ? kv[j] : (l == 8 && t0 + j < nvalid ? 1.f : 0.f);
    }
  }
}

// Piece permutation of the v rows in LDS: row r keeps its 16-byte piece p
// (columns 8 p .. 8 p + 7) at position p ^ vswz(r), which spreads the
// transposed fragment reads below over the LDS banks (two accesses per bank,
// the minimum for 64 lanes x 8 bytes).
__device__ __forceinline__ int vswz(int r) { return ((r >> 1) ^ (r >> 3)) & 7; }

typedef short v4s16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s16 lds_v4s16;
// Four consecutive rows of one value column from the row-major v tile, by the
// transposing LDS read: within each 16-lane group, lane i receives element
// i % 4 of the 8-byte chunk read by lane 4 e + i / 4 (e = 0..3).  Lane s of
// the group therefore reads row r0 + s / 4, columns c0 + 4 (s % 4) .. + 3, and
// lane i ends up with rows r0 .. r0 + 3 of column c0 + i.
__device__ __forceinline__ int v_rows4_offset(int r0, int c0, int s) {
  const int r = r0 + s / 4, c = c0 + 4 * (s % 4);
  return r * DV + 8 * ((c >> 3) ^ vswz(r)) + (c & 7);
}
__device__ __forceinline__ uint2 v_rows4_at(const uint16_t* vtile, int off) {
  const v4s16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(vtile + off));
  return __builtin_bit_cast(uint2, x);
}


// Raw buffer descriptor (gfx9 family) over `bytes` bytes from `base`: loads
// past the end read zero, stores past the end are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, max(bytes, 0), 0x00020000);
}
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, int voff, uint2 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2v, x), r, voff, 0, 0);
}

__device__ __forceinline__ uint2 k_rows4_at(const uint16_t* ktile, int off) {
  const v4s16 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s16*)(ktile + off));
  return __builtin_bit_cast(uint2, x);
}

// Piece permutation of the value rows in LDS, periodic in 16 rows: row r
// keeps its 16-byte piece p at p ^ vswz16(r).  Over any 16 consecutive rows
// the eight even (odd) rows send their 32-byte column pairs to each bank
// quarter exactly twice, so the transposing reads below (16 rows x 32
// bytes) take the minimal two passes; being periodic, the offsets of rows
// 16 and 32 further on differ by constants.
__device__ __forceinline__ int vswz16(int r) { return (((r & 15) >> 1) ^ ((r & 15) >> 3)) & 7; }
__device__ __forceinline__ bf16x8 u4_frag(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  return __builtin_bit_cast(bf16x8, make_uint4(a, b, c, d));
}

// Hand-over of a group total between workgroups on any XCD.  The data and
// the flag go through device-scope accesses (cache policy SC1: they bypass
// the non-coherent L2 of each XCD), and the writer waits for its data stores
// to complete before it sets the flag.  This avoids the whole-L2 write-back
// and invalidation that release and acquire fences cost.
constexpr int kDeviceScope = 16;  // SC1 in the buffer instructions' cache-policy operand
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, int voff, const f32x4& x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, x), r, voff, 0, kDeviceScope);
}
__device__ __forceinline__ f32x4 load_coherent(__amdgpu_buffer_rsrc_t r, int voff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kDeviceScope));
}
// The flag holds a 64-bit tag unique to the launch (a process-wide counter
// from a random start), so whatever the workspace held before cannot pass
// for it and the flags need no clearing between launches.
__device__ __forceinline__ void publish_flag(uint64_t* flag, uint64_t tag) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the data stores are complete
  __hip_atomic_store(flag, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until another workgroup has published a group total.  Bounded: false
// after about 2^20 polls.
__device__ __forceinline__ bool wait_published(const uint64_t* flag, uint64_t tag) {
  for (int i = 0; i < (1 << 20); ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == tag) {
      asm volatile("" ::: "memory");
      return true;
    }
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Segment sums -> inclusive prefix sums over segments, in place: slot s
// becomes the sum of the segment sums 0 .. s (float4 per thread).
__global__ __launch_bounds__(256) void segment_prefix_scan_kernel(float4* __restrict__ bs, int nblk, long per_slot) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= per_slot) return;
  float4 acc = bs[i];
  for (int s = 1; s < nblk; ++s) {
    const float4 x = bs[s * per_slot + i];
    acc = make_float4(acc.x + x.x, acc.y + x.y, acc.z + x.z, acc.w + x.w);
    bs[s * per_slot + i] = acc;
  }
}

}  // namespace
}  // namespace oal
