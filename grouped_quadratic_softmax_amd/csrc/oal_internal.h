// Launch descriptors shared by the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace oal {

// Tokens per prefill chunk.
constexpr int kChunk = 64;

struct FwdLaunch {
  int B, Hq, Hkv, N, d_h, G, dtype;
  const void *q, *k, *v;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  bool diagonal;
  bool premap;
  const float *gamma_q, *beta_q, *gamma_k, *beta_k;
  float ln_eps;
  int premap_kind = 0;  // OAL_PREMAP_LAYERNORM or OAL_PREMAP_L2
  const int32_t* seq_lens = nullptr;  // [B] device lengths within the padded N (null: all N)
  const float* state_in;
  float* state_out;
  void* y;
  void* workspace;
};

struct DecodeLaunch {
  int B, Hq, Hkv, d_h, G, dtype;
  const void *q, *k, *v;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  bool diagonal;
  bool premap;
  const float *gamma_q, *beta_q, *gamma_k, *beta_k;
  float ln_eps;
  int premap_kind = 0;  // OAL_PREMAP_LAYERNORM or OAL_PREMAP_L2
  float* state;
  void* y;
  void* workspace;
};

struct ContribLaunch {
  int P, Hq, Hkv, N, d_h, dtype;
  const void *q, *k;
  const int32_t* seq_lens;
  float* chi_per_prompt;
  float* chi_mean;
  void* workspace;
};

size_t fwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d_h, int dtype);
// stages: bit 0 = chunk states (scan), bit 1 = outputs (readout)
hipError_t launch_fwd(const FwdLaunch& a, int stages, hipStream_t stream);
// Small feature spaces (the dimension-wise form, or the full space at
// d_h = 16): state kept in one CTA, sequences cut into segments that use the
// workspace for their sums (one segment without a workspace).
bool small_path_supported(int d_h, bool diagonal, int Hq, int Hkv);
size_t small_segment_bytes(int d_h, bool diagonal);
// workspace that lets the small path use its full number of segments
size_t small_workspace_bytes(int B, int Hkv, int N, int d_h, bool diagonal, int dtype);
size_t small_workspace_bytes_for(int B, int Hq, int Hkv, int N, int d_h, bool diagonal, int dtype);
hipError_t launch_fwd_small(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream);
// One-pass prefill at d_h = 16 with bf16 activations: the state stays in MFMA
// accumulators; sequences are cut into segments whose starting states come
// from block sums in the workspace (one segment without a workspace).  Up
// to eight groups, or up to d_h groups for heads with their own keys and no
// pre-map.
bool onepass16_supported(int d_h, int dtype, bool diagonal, int G, int Hq, int Hkv, bool premap);
size_t onepass16_workspace_bytes(int B, int Hq, int Hkv, int N);
hipError_t launch_onepass16(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream);
// dimension-wise form at d_h = 64, bf16, heads with their own keys: one wave
// per (sequence x head, segment)
bool dimw_supported(int d_h, int dtype, bool diagonal, int Hq, int Hkv);
size_t dimw_workspace_bytes(int B, int Hkv, int N);
hipError_t launch_dimw(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream);
// one wave per (sequence x head, segment): heads with their own keys, no pre-map
// Chained one-launch prefills: a tag unique to the launch for the flags of
// their hand-over, and the compute units of the current device.
uint64_t chained_launch_tag();
int device_cus();

bool onepass16w_supported(int Hq, int Hkv, bool premap);
size_t onepass16w_workspace_bytes(int B, int Hkv, int N);
hipError_t launch_onepass16w(const FwdLaunch& a, size_t workspace_bytes, hipStream_t stream);
hipError_t launch_state_passthrough(const float* src, float* dst, long n, hipStream_t stream);
void decode_slicing(int d_h, long states, int& rows, int& nslice, bool diagonal);
size_t decode_workspace_bytes(int B, int Hq, int Hkv, int d_h);
hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream);
// the decode step's scratch array of the current device (see oal_decode_step_noalloc)
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_scratch(void** ptr);
// Backward pass at d_h = 16, d_v = 64, heads with their own keys, no pre-map
struct BwdLaunch {
  int B, H, N, G, dtype;
  const void *q, *k, *v, *dy;
  const int32_t* group_of_dim;
  const float *ca, *cb, *cc;
  float *dq, *dk, *dv, *da, *db, *dc;
  void* workspace;
};
bool bwd16_supported(int d_h, int d_v, int dtype, bool diagonal, int G, int Hq, int Hkv);
size_t bwd16_workspace_bytes(int B, int H, int N);
hipError_t launch_bwd16(const BwdLaunch& a, hipStream_t stream);
size_t contrib_workspace_bytes(int P, int Hq, int Hkv, int N, int d_h);
hipError_t launch_contrib(const ContribLaunch& a, hipStream_t stream);

}  // namespace oal
