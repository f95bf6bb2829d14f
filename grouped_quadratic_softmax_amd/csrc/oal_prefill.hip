// Prefill dispatch: head dimension -> kernels, plus the empty-sequence
// state pass-through.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "oal_internal.h"

namespace oal {

hipError_t launch_fwd_d16(const FwdLaunch& a, int stages, hipStream_t stream);
hipError_t launch_fwd_d32(const FwdLaunch& a, int stages, hipStream_t stream);
hipError_t launch_fwd_d64(const FwdLaunch& a, int stages, hipStream_t stream);
size_t fwd_workspace_bytes_d16(int B, int Hq, int Hkv, int N, int dtype);
size_t fwd_workspace_bytes_d32(int B, int Hq, int Hkv, int N, int dtype);
size_t fwd_workspace_bytes_d64(int B, int Hq, int Hkv, int N, int dtype);

// state_out <- state_in (or zeros) for an empty sequence; a plain kernel so
// that callers may capture it in a graph.
__global__ void state_passthrough_kernel(const float* __restrict__ src, float* __restrict__ dst, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    dst[i] = src ? src[i] : 0.f;
}

hipError_t launch_state_passthrough(const float* src, float* dst, long n, hipStream_t stream) {
  const long blocks = (n + 255) / 256;
  hipLaunchKernelGGL(state_passthrough_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)), dim3(256), 0,
                     stream, src, dst, n);
  return hipGetLastError();
}

size_t fwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d_h, int dtype) {
  switch (d_h) {
    case 16: return fwd_workspace_bytes_d16(B, Hq, Hkv, N, dtype);
    case 32: return fwd_workspace_bytes_d32(B, Hq, Hkv, N, dtype);
    default: return fwd_workspace_bytes_d64(B, Hq, Hkv, N, dtype);
  }
}

hipError_t launch_fwd(const FwdLaunch& a, int stages, hipStream_t stream) {
  switch (a.d_h) {
    case 16: return launch_fwd_d16(a, stages, stream);
    case 32: return launch_fwd_d32(a, stages, stream);
    default: return launch_fwd_d64(a, stages, stream);
  }
}

}  // namespace oal
