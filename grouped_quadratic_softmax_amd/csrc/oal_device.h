// Device helpers shared by the OAL HIP kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oal_layout.h"

namespace oal {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---- element access: activations are float or bfloat16 bit patterns ----
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  __bf16 h = (__bf16)x;  // round to nearest even (v_cvt_pk_bf16_f32)
  return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ void store_elem(float* p, float x) { *p = x; }
__device__ __forceinline__ void store_elem(uint16_t* p, float x) { *p = bf16_bits(x); }

template <typename T>
struct IsBf16 {
  static constexpr bool value = false;
};
template <>
struct IsBf16<uint16_t> {
  static constexpr bool value = true;
};

// ---- MFMA operand fragments: 8 elements per lane ----
// bf16 path: one v_mfma_f32_16x16x32_bf16 per fragment pair.
// fp32 path: eight v_mfma_f32_16x16x4_f32, element e of lane group lg being
// the same K index in A and B, so the contraction covers the same 32 indices.
template <bool BF16>
struct Frag;
template <>
struct Frag<true> {
  bf16x8 v;
};
template <>
struct Frag<false> {
  float v[8];
};

template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_from(const float (&x)[8]);
template <>
__device__ __forceinline__ Frag<true> frag_from<true>(const float (&x)[8]) {
  Frag<true> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = (__bf16)x[e];
  return f;
}
template <>
__device__ __forceinline__ Frag<false> frag_from<false>(const float (&x)[8]) {
  Frag<false> f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f.v[e] = x[e];
  return f;
}

template <bool BF16>
__device__ __forceinline__ Frag<BF16> frag_zero() {
  float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  return frag_from<BF16>(z);
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<true>& a, const Frag<true>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma(f32x4& acc, const Frag<false>& a, const Frag<false>& b) {
#pragma unroll
  for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// Fragment loads from memory holding the fragment's element type
// (bf16 bits or float), 8 consecutive elements.
__device__ __forceinline__ Frag<true> frag_load(const uint16_t* p) {
  Frag<true> f;
  f.v = *reinterpret_cast<const bf16x8*>(p);
  return f;
}
__device__ __forceinline__ Frag<false> frag_load(const float* p) {
  Frag<false> f;
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
  return f;
}

// Storage type of snapshot / fragment memory for an activation type.
template <typename T>
struct FragStore {
  typedef float type;
};
template <>
struct FragStore<uint16_t> {
  typedef uint16_t type;
};

__device__ __forceinline__ void store4(uint16_t* p, const f32x4& x) {
  uint2 w;
  w.x = (uint32_t)bf16_bits(x[0]) | ((uint32_t)bf16_bits(x[1]) << 16);
  w.y = (uint32_t)bf16_bits(x[2]) | ((uint32_t)bf16_bits(x[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, const f32x4& x) {
  *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
}

// ---- cross-lane reductions on DPP (no LDS round trip) ----
// DPP control codes: quad_perm patterns and shifts within a row of 16 lanes.
constexpr int kDppXor1 = 0xb1;   // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4e;   // quad_perm [2, 3, 0, 1]
constexpr int kDppShr1 = 0x111;  // row_shr:1
constexpr int kDppShr2 = 0x112;
constexpr int kDppShr4 = 0x114;
constexpr int kDppShr8 = 0x118;

// x of the lane selected by CTRL; a lane whose source lies outside its row
// receives `fill`.
template <int CTRL>
__device__ __forceinline__ float dpp(float x, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                               __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float lane_value(float x, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), lane));
}
// sum / max over aligned groups of 4 lanes, in every lane of the group
// Length of sequence b: its entry of seq_lens clamped to [0, N], or N
// (padded layout: rows past a sequence's length are not part of it).
__device__ __forceinline__ int seq_len_of(const int32_t* seq_lens, int b, int N) {
  return seq_lens == nullptr ? N : min(max(seq_lens[b], 0), N);
}

// Normalisation of the pre-map gamma * norm(x) + beta over d_h:
//   mu = mean_w * sum_r x_r,  norm(x) = (x - mu) / sqrt(var_w * sum_r (x_r - mu)^2 + eps)
// LayerNorm (kind 0): mean_w = var_w = 1 / d_h; unit l2 norm (kind 1):
// mean_w = 0, var_w = 1.
struct PremapNorm {
  float mean_w, var_w;
};
__host__ __device__ inline PremapNorm premap_norm(int kind, int dh) {
  return kind == 1 ? PremapNorm{0.f, 1.f} : PremapNorm{1.f / (float)dh, 1.f / (float)dh};
}

__device__ __forceinline__ float quad_sum(float x) {
  x += dpp<kDppXor1>(x, 0.f);
  return x + dpp<kDppXor2>(x, 0.f);
}
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x, x));
  return fmaxf(x, dpp<kDppXor2>(x, x));
}
// sum / max over each row of 16 lanes, valid in the row's last lane
__device__ __forceinline__ float row_sum_last(float x) {
  x += dpp<kDppShr1>(x, 0.f);
  x += dpp<kDppShr2>(x, 0.f);
  x += dpp<kDppShr4>(x, 0.f);
  return x + dpp<kDppShr8>(x, 0.f);
}
__device__ __forceinline__ float row_max_last(float x) {
  x = fmaxf(x, dpp<kDppShr1>(x, x));
  x = fmaxf(x, dpp<kDppShr2>(x, x));
  x = fmaxf(x, dpp<kDppShr4>(x, x));
  return fmaxf(x, dpp<kDppShr8>(x, x));
}
// over the whole wave, returned (uniform) in every lane
__device__ __forceinline__ float wave_sum(float x) {
  x = row_sum_last(x);
  return (lane_value(x, 15) + lane_value(x, 31)) + (lane_value(x, 47) + lane_value(x, 63));
}
__device__ __forceinline__ float wave_max(float x) {
  x = row_max_last(x);
  return fmaxf(fmaxf(lane_value(x, 15), lane_value(x, 31)), fmaxf(lane_value(x, 47), lane_value(x, 63)));
}

}  // namespace oal
