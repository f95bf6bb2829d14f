// Per-dimension contribution score chi (the OAL paper's Eq. (2)) on gfx950.
//
//   chi_{p,r} = (1 / |Omega_p|) sum_{j <= i < N_p} |q_ir k_jr| / sqrt(d_h)
//             = sum_i |q_ir| * (sum_{j<=i} |k_jr|) / (sqrt(d_h) N_p (N_p+1) / 2)
//
// A token segment is summarised per dimension by the triple
//   A = sum |q|,  B = sum_i |q_i| * (prefix of |k| inside the segment),  K = sum |k|
// and two adjacent segments L, R combine in order as
//   (A_L + A_R, B_L + B_R + K_L A_R, K_L + K_R).
// Lanes of a wave are (token slot, dimension); each lane scans its slot's
// tokens sequentially (coalesced rows), the slots of a wave are combined with
// wavefront shuffles, the four waves of a CTA through LDS, and the CTAs of a
// prompt by a second, sequential kernel.  All terms are non-negative, so fp32
// accumulation has no cancellation; the result is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

constexpr int kContribTB = 1024;  // tokens per CTA (256 per wave)

template <typename T, int DH, int RMAX>
__global__ __launch_bounds__(256) void contrib_partial_kernel(const T* __restrict__ q,
                                                              const T* __restrict__ k,
                                                              const int32_t* __restrict__ seq_lens,
                                                              float* __restrict__ part, int Hq,
                                                              int Hkv, int N, int nblk) {
  constexpr int S = kWave / DH;          // token slots per wave
  constexpr int TW = kContribTB / 4;     // tokens per wave
  constexpr int TS = TW / S;             // tokens per slot
  constexpr int NV = 2 * RMAX + 1;       // A[R], B[R], K
  __shared__ float xs[4][NV][DH];

  const int blk = blockIdx.x, kvh = blockIdx.y, p = blockIdx.z;
  const int R = Hq / Hkv;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int slot = lane / DH, r = lane % DH;
  int n = seq_lens ? seq_lens[p] : N;
  const bool badlen = n < 1 || n > N;
  if (badlen) n = 0;

  float A[RMAX], Bs[RMAX], K = 0.f;
#pragma unroll
  for (int hh = 0; hh < RMAX; ++hh) A[hh] = Bs[hh] = 0.f;

  const int t0 = blk * kContribTB + wave * TW + slot * TS;
  const int t1 = min(t0 + TS, n);
  const T* kp = k + ((long)(p * Hkv + kvh) * N) * DH + r;
  const T* qp = q + ((long)(p * Hq + kvh * R) * N) * DH + r;
  for (int t = t0; t < t1; ++t) {
    K += fabsf(to_f32(kp[(long)t * DH]));
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh) {
      if (hh < R) {
        const float qa = fabsf(to_f32(qp[((long)hh * N + t) * DH]));
        A[hh] += qa;
        Bs[hh] += qa * K;
      }
    }
  }

  // ordered combine of the slots of this wave (slot s holds tokens after s-1)
#pragma unroll
  for (int off = DH; off < kWave; off <<= 1) {
    const float Kr = __shfl_down(K, off);
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh) {
      const float Ar = __shfl_down(A[hh], off);
      const float Br = __shfl_down(Bs[hh], off);
      Bs[hh] += Br + K * Ar;
      A[hh] += Ar;
    }
    K += Kr;
  }
  // lanes of slot 0 now hold the wave's triple for dimension r
  if (slot == 0) {
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh) {
      xs[wave][hh][r] = A[hh];
      xs[wave][RMAX + hh][r] = Bs[hh];
    }
    xs[wave][2 * RMAX][r] = K;
  }
  __syncthreads();
  if (threadIdx.x < DH) {
    const int rr = threadIdx.x;
    float cA[RMAX], cB[RMAX], cK = 0.f;
#pragma unroll
    for (int hh = 0; hh < RMAX; ++hh) cA[hh] = cB[hh] = 0.f;
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh) {
        const float Ar = xs[w][hh][rr], Br = xs[w][RMAX + hh][rr];
        cB[hh] += Br + cK * Ar;
        cA[hh] += Ar;
      }
      cK += xs[w][2 * RMAX][rr];
    }
    float* out = part + (((long)p * Hkv + kvh) * nblk + blk) * (2 * R + 1) * DH;
    for (int hh = 0; hh < R && hh < RMAX; ++hh) {
      out[hh * DH + rr] = cA[hh];
      out[(R + hh) * DH + rr] = cB[hh];
    }
    out[2 * R * DH + rr] = badlen ? __builtin_nanf("") : cK;
  }
}

// One CTA per query head; thread r combines the CTA triples of every prompt in
// token order, then averages over prompts with equal weights.
template <int DH>
__global__ __launch_bounds__(64) void contrib_combine_kernel(const float* __restrict__ part,
                                                             const int32_t* __restrict__ seq_lens,
                                                             float* __restrict__ chi_per_prompt,
                                                             float* __restrict__ chi_mean, int P,
                                                             int Hq, int Hkv, int N, int nblk) {
  const int h = blockIdx.x, r = threadIdx.x;
  if (r >= DH) return;
  const int R = Hq / Hkv, kvh = h / R, hh = h % R;
  const float inv_sqrt_d = 1.f / sqrtf((float)DH);
  float mean = 0.f;
  for (int p = 0; p < P; ++p) {
    const int n = seq_lens ? seq_lens[p] : N;
    const float* base = part + ((long)p * Hkv + kvh) * nblk * (2 * R + 1) * DH;
    float tot = 0.f, kc = 0.f;
    const int nb_used = n >= 1 && n <= N ? (n + kContribTB - 1) / kContribTB : nblk;
    for (int blk = 0; blk < nb_used; ++blk) {
      const float* x = base + (long)blk * (2 * R + 1) * DH;
      tot += x[(R + hh) * DH + r] + kc * x[hh * DH + r];
      kc += x[2 * R * DH + r];
    }
    const float pairs = 0.5f * (float)n * (float)(n + 1);
    const bool badlen = n < 1 || n > N;
    const float chi = badlen ? __builtin_nanf("") : tot * inv_sqrt_d / pairs;
    if (chi_per_prompt) chi_per_prompt[((long)p * Hq + h) * DH + r] = chi;
    mean += chi;
  }
  chi_mean[(long)h * DH + r] = mean / (float)P;
}

size_t contrib_workspace_bytes(int P, int Hq, int Hkv, int N, int d_h) {
  const long nblk = (N + kContribTB - 1) / kContribTB;
  const int R = Hq / Hkv;
  return (size_t)P * Hkv * nblk * (2 * R + 1) * d_h * sizeof(float);
}

template <typename T, int DH, int RMAX>
static hipError_t launch_contrib_r(const ContribLaunch& a, hipStream_t stream) {
  const int nblk = (a.N + kContribTB - 1) / kContribTB;
  float* part = reinterpret_cast<float*>(a.workspace);
  hipLaunchKernelGGL((contrib_partial_kernel<T, DH, RMAX>), dim3(nblk, a.Hkv, a.P), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(a.q), reinterpret_cast<const T*>(a.k), a.seq_lens, part,
                     a.Hq, a.Hkv, a.N, nblk);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((contrib_combine_kernel<DH>), dim3(a.Hq), dim3(64), 0, stream, part, a.seq_lens,
                     a.chi_per_prompt, a.chi_mean, a.P, a.Hq, a.Hkv, a.N, nblk);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_contrib_d(const ContribLaunch& a, hipStream_t stream) {
  const int R = a.Hq / a.Hkv;
  if (R <= 1) return launch_contrib_r<T, DH, 1>(a, stream);
  if (R <= 2) return launch_contrib_r<T, DH, 2>(a, stream);
  if (R <= 4) return launch_contrib_r<T, DH, 4>(a, stream);
  if (R <= 8) return launch_contrib_r<T, DH, 8>(a, stream);
  return launch_contrib_r<T, DH, 16>(a, stream);
}

hipError_t launch_contrib(const ContribLaunch& a, hipStream_t stream) {
  if (a.dtype == 1) {
    switch (a.d_h) {
      case 16: return launch_contrib_d<uint16_t, 16>(a, stream);
      case 32: return launch_contrib_d<uint16_t, 32>(a, stream);
      default: return launch_contrib_d<uint16_t, 64>(a, stream);
    }
  }
  switch (a.d_h) {
    case 16: return launch_contrib_d<float, 16>(a, stream);
    case 32: return launch_contrib_d<float, 32>(a, stream);
    default: return launch_contrib_d<float, 64>(a, stream);
  }
}

}  // namespace oal
