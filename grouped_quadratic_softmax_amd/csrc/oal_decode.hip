// Recurrent single-token decode for OAL attention on gfx950.
//
// Per (sequence, KV head) the fp32 state S = [H | z] of the OAL paper's
// Eq. (5) (packed as in App. D) is streamed once from HBM: each row f gets the
// rank-1 update H[f] += phi_k(k)_f v and z[f] += phi_k(k)_f, is written back,
// and is read by every query head of the group, num_h += phi_q,h(q_h)_f H[f]
// and den_h += phi_q,h(q_h)_f z[f] (Eq. (6)); y_h = num_h / den_h.  The new
// token therefore belongs to its own causal prefix.
//
// The D feature rows of a state are cut into `nslice` slices so that even a
// handful of sequences fills the chip.  Kernel 1 runs one 256-thread CTA per
// (slice, sequence x KV head): it computes the feature values phi_k and
// phi_q,h of its rows into LDS, streams the rows with 16 threads per 256-byte
// row (float4 loads and stores, fully coalesced, four rows in flight per
// thread) and writes the partial (num_h, den_h) of the slice.  Kernel 2 adds
// the slices in a fixed order and divides.  With a single slice kernel 1
// divides and stores y itself.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

namespace {
constexpr int DV = 64;
constexpr int NC = DV + 1;

template <int DH>
__device__ __forceinline__ void premap_vec(float* x, const float* __restrict__ gamma,
                                           const float* __restrict__ beta, float eps, PremapNorm pn) {
  float mu = 0.f;
  for (int c = 0; c < DH; ++c) mu += x[c];
  mu *= pn.mean_w;
  float var = 0.f;
  for (int c = 0; c < DH; ++c) {
    const float t = x[c] - mu;
    var += t * t;
  }
  var *= pn.var_w;
  const float inv = 1.f / sqrtf(var + eps);
  for (int c = 0; c < DH; ++c) x[c] = gamma[c] * (x[c] - mu) * inv + beta[c];
}

// Packed feature f -> (r, t) over the augmented key [k_0 .. k_{d-1}, 1]:
// f = 0 is (d, d), f = 1 + r is (r, d), and the pairs r <= t follow in
// row-major upper-triangle order.
template <int DH>
__device__ __forceinline__ void feature_pair(int f, int& r, int& t) {
  if (f == 0) {
    r = DH;
    t = DH;
    return;
  }
  if (f <= DH) {
    r = f - 1;
    t = DH;
    return;
  }
  const int p = f - 1 - DH;
  // first pair of row r sits at r*DH - r(r-1)/2; solve for r, then fix up
  const float b = 2.f * DH + 1.f;
  int rr = (int)((b - sqrtf(b * b - 8.f * (float)p)) * 0.5f);
  rr = max(0, min(rr, DH - 1));
  while (rr > 0 && rr * DH - rr * (rr - 1) / 2 > p) --rr;
  while (rr + 1 < DH && (rr + 1) * DH - (rr + 1) * rr / 2 <= p) ++rr;
  r = rr;
  t = rr + (p - (rr * DH - rr * (rr - 1) / 2));
}
}  // namespace

// Rows per slice (a multiple of 16) and slice count for `states` states.
void decode_slicing(int d_h, long states, int& rows, int& nslice, bool diagonal) {
  const int D = diagonal ? 1 + 2 * d_h : (int)packed_features(d_h);
  // about 512 CTAs (two per compute unit): with 32-128 states, more and
  // smaller slices only add per-CTA set-up; from 256 states on, up to eight
  // slices while that keeps >= 2048 CTAs (three slices of 720 rows stream
  // worse than eight of 272 there)
  long want = (512 + states - 1) / states;
  if (states >= 256) {
    const long a2048 = (2048 + states - 1) / states;
    const long floor8 = a2048 < 8 ? a2048 : 8;
    if (want < floor8) want = floor8;
  }
  want = want < 1 ? 1 : want;
  // up to 256 feature rows (d_h = 16, or the dimension-wise form) one slice
  // per state writes the outputs itself: the second launch that adds the
  // slices costs more than the parallelism gains (8 x 16 states: 8.8 ->
  // 6.8 us; 64 x 16: 19.3 -> 15.3 us)
  if (D <= 256) want = 1;
  const long min_slices = (D + 1023) / 1024;           // at most 1024 rows per CTA
  if (want < min_slices) want = min_slices;
  const long max_slices = (D + 63) / 64;               // at least 64 rows per CTA
  if (want > max_slices) want = max_slices;
  rows = (int)(((D + want - 1) / want + 15) / 16 * 16);
  nslice = (D + rows - 1) / rows;
}

template <typename T, int DH, int RMAX, bool PREMAP>
__global__ __launch_bounds__(256) void decode_partial_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int32_t* __restrict__ group_of_dim, const float* __restrict__ ca,
    const float* __restrict__ cb, const float* __restrict__ cc, int G,
    const float* __restrict__ gamma_q, const float* __restrict__ beta_q,
    const float* __restrict__ gamma_k, const float* __restrict__ beta_k, float ln_eps, PremapNorm pn,
    float* __restrict__ state, float* __restrict__ part, T* __restrict__ y, int Hq, int Hkv, int rows,
    int diagonal) {
  constexpr int D = (int)packed_features(DH);
  // rows of the state this step touches: all D features, or in the
  // dimension-wise form the constant, linear and squared ones (1 + 2 d_h)
  const int DN = diagonal ? 1 + 2 * DH : D;
  auto row_of = [&](int u) __attribute__((always_inline)) {
    return (diagonal && u > DH) ? (int)abi_index(DH, u - 1 - DH, u - 1 - DH) : u;
  };
  extern __shared__ float smem[];
  float* phik = smem;                 // [rows]
  float* phiq = smem + rows;          // [RMAX][rows]
  __shared__ float khat[DH + 1];
  __shared__ float qhat[RMAX][DH + 1];
  __shared__ float vv[DV];
  __shared__ float red[16][RMAX][DV];
  __shared__ float dred[RMAX][256 / kWave];
  __shared__ int bad;
  __shared__ int gmap[RMAX][DH];  // group of each dimension (clamped; `bad` flags ids out of range)

  const int slice = blockIdx.x, nslice = gridDim.x;
  const int bh = blockIdx.y;
  const int b = bh / Hkv, kvh = bh % Hkv;
  const int R = Hq / Hkv;
  const int tid = threadIdx.x;
  const int f0 = slice * rows, f1 = min(f0 + rows, DN);

  if (tid == 0) bad = 0;
  if (tid < DH) khat[tid] = to_f32(k[(long)bh * DH + tid]);
  if (tid == DH) khat[DH] = 1.f;
  if (tid < DV) vv[tid] = to_f32(v[(long)bh * DV + tid]);
  for (int idx = tid; idx < R * (DH + 1); idx += blockDim.x) {
    const int hh = idx / (DH + 1), r = idx % (DH + 1);
    qhat[hh][r] = r < DH ? to_f32(q[((long)b * Hq + kvh * R + hh) * DH + r]) : 1.f;
  }
  __syncthreads();
  if (PREMAP) {
    if (tid == 0) premap_vec<DH>(khat, gamma_k + kvh * DH, beta_k + kvh * DH, ln_eps, pn);
    if (tid >= 64 && tid - 64 < R) {
      const int hh = tid - 64, h = kvh * R + hh;
      premap_vec<DH>(qhat[hh], gamma_q + h * DH, beta_q + h * DH, ln_eps, pn);
    }
  }
  for (int idx = tid; idx < R * DH; idx += blockDim.x) {
    const int g = group_of_dim[(kvh * R + idx / DH) * DH + idx % DH];
    if (g < 0 || g >= G) atomicOr(&bad, 1);
    gmap[idx / DH][idx % DH] = min(max(g, 0), G - 1);
  }
  __syncthreads();

  // feature values of the slice rows: const, linear r, pairs r <= t; the
  // coefficient of (r, t) is the symmetric c of the two groups (read from
  // global memory, cached) times 2 off the diagonal
  const float inv_sqrt_d = 1.f / sqrtf((float)DH);
  for (int f = f0 + tid; f < f1; f += blockDim.x) {
    int r, t;
    feature_pair<DH>(row_of(f), r, t);
    phik[f - f0] = khat[r] * khat[t];
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh) {
      if (hh >= R) break;
      const int h = kvh * R + hh;
      float cf;
      if (r == DH) {
        cf = ca[h];
      } else if (t == DH) {
        cf = cb[h * G + gmap[hh][r]] * inv_sqrt_d;
      } else if (diagonal) {
        const int g1 = gmap[hh][r];
        cf = r == t ? cc[(h * G + g1) * G + g1] / DH : 0.f;
      } else {
        const int g1 = gmap[hh][r], g2 = gmap[hh][t];
        const float m = r == t ? 1.f : 2.f;
        cf = m * 0.5f * (cc[(h * G + g1) * G + g2] + cc[(h * G + g2) * G + g1]) / DH;
      }
      phiq[hh * rows + (f - f0)] = cf * qhat[hh][r] * qhat[hh][t];
    }
  }
  __syncthreads();

  // ---- stream the slice's H rows: 16 threads per row, float4 each ----
  float* sp = state + (long)bh * D * NC;
  const int c4 = tid % 16, rg = tid / 16;
  const float4 v4 = make_float4(vv[4 * c4], vv[4 * c4 + 1], vv[4 * c4 + 2], vv[4 * c4 + 3]);
  float acc[RMAX][4];
#pragma unroll
  for (int hh = 0; hh < RMAX; ++hh) acc[hh][0] = acc[hh][1] = acc[hh][2] = acc[hh][3] = 0.f;

  constexpr int U = 8;
  for (int fb = f0 + rg; fb < f1; fb += 16 * U) {
    float4 hv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = fb + 16 * u;
      if (f < f1) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(&sp[(long)row_of(f) * DV + 4 * c4]);
        hv[u] = make_float4(w[0], w[1], w[2], w[3]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int f = fb + 16 * u;
      if (f >= f1) continue;
      const float pk = phik[f - f0];
      float4 x = hv[u];
      x.x += pk * v4.x;
      x.y += pk * v4.y;
      x.z += pk * v4.z;
      x.w += pk * v4.w;
      *reinterpret_cast<f32x4*>(&sp[(long)row_of(f) * DV + 4 * c4]) = f32x4{x.x, x.y, x.z, x.w};
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh) {
        if (hh < R) {
          const float pq = phiq[hh * rows + (f - f0)];
          acc[hh][0] += pq * x.x;
          acc[hh][1] += pq * x.y;
          acc[hh][2] += pq * x.z;
          acc[hh][3] += pq * x.w;
        }
      }
    }
  }
  // ---- the slice's z entries ----
  float dacc[RMAX];
#pragma unroll
  for (int hh = 0; hh < RMAX; ++hh) dacc[hh] = 0.f;
  float* zp = sp + (long)D * DV;
  for (int f = f0 + tid; f < f1; f += blockDim.x) {
    const int fr = row_of(f);
    const float zn = zp[fr] + phik[f - f0];
    zp[fr] = zn;
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh)
      if (hh < R) dacc[hh] += phiq[hh * rows + (f - f0)] * zn;
  }

  // ---- reductions (fixed order) ----
#pragma unroll
  for (int hh = 0; hh < RMAX; ++hh) {
    if (hh >= R) break;
#pragma unroll
    for (int e = 0; e < 4; ++e) red[rg][hh][4 * c4 + e] = acc[hh][e];
    const float dsum = wave_sum(dacc[hh]);
    if (tid % kWave == 0) dred[hh][tid / kWave] = dsum;
  }
  __syncthreads();
  const float nanv = __builtin_nanf("");
  for (int idx = tid; idx < R * NC; idx += blockDim.x) {
    const int hh = idx / NC, n = idx % NC;
    float val;
    if (n < DV) {
      val = 0.f;
      for (int g = 0; g < 16; ++g) val += red[g][hh][n];
    } else {
      val = dred[hh][0] + dred[hh][1] + dred[hh][2] + dred[hh][3];
    }
    if (nslice == 1) {
      if (n < DV) {
        const float den = dred[hh][0] + dred[hh][1] + dred[hh][2] + dred[hh][3];
        store_elem(&y[((long)b * Hq + kvh * R + hh) * DV + n], bad ? nanv : val / den);
      }
    } else {
      part[(((long)bh * nslice + slice) * R + hh) * NC + n] = (bad && n == DV) ? nanv : val;
    }
  }
}

// y[b, h, :] = sum over slices of num / sum over slices of den, slices added
// in index order.  One thread per output element.
template <typename T>
__global__ __launch_bounds__(256) void decode_finish_kernel(const float* __restrict__ part, T* __restrict__ y,
                                                            int B, int Hq, int Hkv, int nslice) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long total = (long)B * Hq * DV;
  if (idx >= total) return;
  const int n = (int)(idx % DV);
  const long bhq = idx / DV;
  const int h = (int)(bhq % Hq), b = (int)(bhq / Hq);
  const int R = Hq / Hkv, kvh = h / R, hh = h % R;
  const long bh = (long)b * Hkv + kvh;
  float num = 0.f, den = 0.f;
#pragma unroll 8
  for (int s = 0; s < nslice; ++s) {
    const float* x = part + ((bh * nslice + s) * R + hh) * NC;
    num += x[n];
    den += x[DV];
  }
  store_elem(&y[idx], num / den);
}

size_t decode_workspace_bytes(int B, int Hq, int Hkv, int d_h) {
  int rows, nslice;
  decode_slicing(d_h, (long)B * Hkv, rows, nslice, false);  // bounds the dimension-wise form too
  if (nslice == 1) return 0;
  return (size_t)B * Hkv * nslice * (Hq / Hkv) * NC * sizeof(float);
}

template <typename T, int DH, int RMAX>
static hipError_t launch_decode_r(const DecodeLaunch& a, hipStream_t stream) {
  int rows, nslice;
  decode_slicing(DH, (long)a.B * a.Hkv, rows, nslice, a.diagonal);
  const size_t shm = (size_t)(1 + RMAX) * rows * sizeof(float);
  dim3 grid(nslice, a.B * a.Hkv);
  const T* qq = reinterpret_cast<const T*>(a.q);
  const T* kk = reinterpret_cast<const T*>(a.k);
  const T* vv = reinterpret_cast<const T*>(a.v);
  T* yy = reinterpret_cast<T*>(a.y);
  float* part = reinterpret_cast<float*>(a.workspace);
  if (a.premap)
    hipLaunchKernelGGL((decode_partial_kernel<T, DH, RMAX, true>), grid, dim3(256), shm, stream, qq, kk, vv,
                       a.group_of_dim, a.ca, a.cb, a.cc, a.G, a.gamma_q, a.beta_q, a.gamma_k, a.beta_k,
                       a.ln_eps, premap_norm(a.premap_kind, DH), a.state, part, yy, a.Hq, a.Hkv, rows,
                       (int)a.diagonal);
  else
    hipLaunchKernelGGL((decode_partial_kernel<T, DH, RMAX, false>), grid, dim3(256), shm, stream, qq, kk, vv,
                       a.group_of_dim, a.ca, a.cb, a.cc, a.G, nullptr, nullptr, nullptr, nullptr, 0.f,
                       premap_norm(0, DH), a.state, part, yy, a.Hq, a.Hkv, rows, (int)a.diagonal);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || nslice == 1) return err;
  const long total = (long)a.B * a.Hq * DV;
  hipLaunchKernelGGL((decode_finish_kernel<T>), dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     part, yy, a.B, a.Hq, a.Hkv, nslice);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_decode_d(const DecodeLaunch& a, hipStream_t stream) {
  const int R = a.Hq / a.Hkv;
  if (R <= 1) return launch_decode_r<T, DH, 1>(a, stream);
  if (R <= 2) return launch_decode_r<T, DH, 2>(a, stream);
  if (R <= 4) return launch_decode_r<T, DH, 4>(a, stream);
  return launch_decode_r<T, DH, 8>(a, stream);
}

hipError_t launch_decode(const DecodeLaunch& a, hipStream_t stream) {
  if (a.dtype == 1) {
    switch (a.d_h) {
      case 16: return launch_decode_d<uint16_t, 16>(a, stream);
      case 32: return launch_decode_d<uint16_t, 32>(a, stream);
      default: return launch_decode_d<uint16_t, 64>(a, stream);
    }
  }
  switch (a.d_h) {
    case 16: return launch_decode_d<float, 16>(a, stream);
    case 32: return launch_decode_d<float, 32>(a, stream);
    default: return launch_decode_d<float, 64>(a, stream);
  }
}

// ---- scratch for the decode step of callers that cannot allocate ----
// One array per device that loads the library, held until the process ends.
// In host code `scratch` names a host-side stand-in, not the device array:
// the device address comes from hipGetSymbolAddress, once per device with
// that device current, and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

}  // namespace oal
