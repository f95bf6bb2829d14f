// Two machine-ceiling probes that put the roofline fractions of the attention
// kernels on measured rather than only published peaks.  Neither is part of
// the attention method.
//
//  * An in-place streaming update x <- a x + b over a large fp32 buffer: every
//    byte is read once and written once, the access pattern of a kernel whose
//    reads and writes are of the same size (the decode step's state
//    read-modify-write).  16-byte accesses, four in flight per thread,
//    consecutive lanes on consecutive addresses.
//  * A register-only chain of bf16 MFMAs (v_mfma_f32_16x16x32_bf16, the
//    instruction of the prefill kernels): eight independent accumulators per
//    wave so that the matrix pipe never waits on a result, no memory traffic
//    inside the loop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/oal.h"
#include "../../include/oal_ceilings.h"

namespace oal {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 4;

__global__ __launch_bounds__(kStreamThreads) void stream_rw_kernel(float4* __restrict__ x, size_t n4, float a,
                                                                    float b) {
  const size_t per_block = (size_t)kStreamThreads * kStreamUnroll;
  for (size_t base = (size_t)blockIdx.x * per_block; base < n4; base += (size_t)gridDim.x * per_block) {
    float4 r[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads + threadIdx.x;
      if (i < n4) r[u] = x[i];
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const size_t i = base + (size_t)u * kStreamThreads + threadIdx.x;
      if (i < n4) x[i] = make_float4(a * r[u].x + b, a * r[u].y + b, a * r[u].z + b, a * r[u].w + b);
    }
  }
}

constexpr int kMfmaChains = 8;
constexpr int kMfmaUnroll = 16;

__global__ __launch_bounds__(256) void mfma_chain_kernel(float* __restrict__ out, int iters, float seed) {
  // operands depend on the thread and on a runtime seed, so nothing folds
  bf16x8 av, bv[kMfmaChains];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    av[j] = (__bf16)(seed * (float)(threadIdx.x + j));
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) bv[c][j] = (__bf16)(seed * (float)(j + c - (int)threadIdx.x));
  }
  f32x4 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  // sixteen rounds per trip, so that register moves the compiler may add at
  // the back edge are spread over many MFMAs
  for (int it = 0; it < iters; it += kMfmaUnroll) {
#pragma unroll
    for (int u = 0; u < kMfmaUnroll; ++u) {
#pragma unroll
      for (int c = 0; c < kMfmaChains; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[c], acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace oal

extern "C" {

int oal_ceiling_stream_rw(float* buf, size_t n_floats, void* stream) {
  if (buf == nullptr || n_floats == 0 || n_floats % 4 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return OAL_ERR_INVALID_ARG;
  const size_t n4 = n_floats / 4;
  const size_t per_block = (size_t)oal::kStreamThreads * oal::kStreamUnroll;
  const size_t blocks = std::min<size_t>((n4 + per_block - 1) / per_block, 256 * 16);
  hipLaunchKernelGGL(oal::stream_rw_kernel, dim3((unsigned)blocks), dim3(oal::kStreamThreads), 0,
                     (hipStream_t)stream, reinterpret_cast<float4*>(buf), n4, 0.999f, 1e-3f);
  return hipGetLastError() == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

double oal_ceiling_mfma_flops(int n_workgroups, int iters) {
  // 256 threads = four waves per workgroup; 2 * 16 * 16 * 32 flops per MFMA
  return (double)n_workgroups * 4.0 * iters * oal::kMfmaChains * 2.0 * 16 * 16 * 32;
}

int oal_ceiling_mfma(float* out, int n_workgroups, int iters, void* stream) {
  if (out == nullptr || n_workgroups <= 0 || iters <= 0 || iters % oal::kMfmaUnroll != 0)
    return OAL_ERR_INVALID_ARG;
  hipLaunchKernelGGL(oal::mfma_chain_kernel, dim3(n_workgroups), dim3(256), 0, (hipStream_t)stream, out, iters,
                     1.0f / 1024.0f);
  return hipGetLastError() == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

}  // extern "C"
