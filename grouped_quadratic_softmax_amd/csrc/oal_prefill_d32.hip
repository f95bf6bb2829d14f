// Prefill kernels for d_h = 32 (bf16 and fp32 activations).
#include "oal_prefill.h"

namespace oal {

hipError_t launch_fwd_d32(const FwdLaunch& a, int stages, hipStream_t stream) {
  return a.dtype == 1 ? launch_fwd_t<uint16_t, 32>(a, stages, stream) : launch_fwd_t<float, 32>(a, stages, stream);
}

size_t fwd_workspace_bytes_d32(int B, int Hq, int Hkv, int N, int dtype) {
  return dtype == 1 ? (size_t)fwd_ws<uint16_t, 32>(B, Hq, Hkv, N).total : (size_t)fwd_ws<float, 32>(B, Hq, Hkv, N).total;
}

}  // namespace oal
