// Per-dimension contribution score chi (the OAL paper's Eq. (2)) on gfx950.
//
//   chi_{p,r} = (1 / |Omega_p|) sum_{j <= i < N_p} |q_ir k_jr| / sqrt(d_h)
//             = sum_i |q_ir| * (sum_{j<=i} |k_jr|) / (sqrt(d_h) N_p (N_p+1) / 2)
//
// A token segment is summarised per dimension by the triple
//   A = sum |q|,  B = sum_i |q_i| * (prefix of |k| inside the segment),  K = sum |k|
// and two adjacent segments L, R combine in order as
//   (A_L + A_R, B_L + B_R + K_L A_R, K_L + K_R).
//
// Kernel 1 (partial): one CTA per (token block, KV head and pair of its
// query heads, prompt).  Its 256 threads are (d_h / 8) dimension octets x
// token slots; slot s scans a contiguous run of the block's tokens with
// 16-byte loads (every load of four tokens issued before their arithmetic),
// the slots of a wave are combined in order with wavefront shuffles, the four
// waves through LDS, and the block triples go to the workspace.
// Kernel 2 (combine): one CTA per query head folds the block triples of each
// prompt in token order (one thread per (prompt, dimension)), normalises,
// and averages over prompts with equal weights, in prompt order.
// All terms are non-negative, so fp32 accumulation has no cancellation; the
// result is deterministic.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "oal_device.h"
#include "oal_internal.h"

namespace oal {

namespace {

// Eight consecutive activations kept as raw 16-byte (bf16) or 32-byte (fp32)
// vectors until they are needed as floats.
template <typename T>
struct Octet;
template <>
struct Octet<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(ws[j] << 16);
      x[2 * j + 1] = __uint_as_float(ws[j] & 0xffff0000u);
    }
  }
};
template <>
struct Octet<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void get(float (&x)[8]) const {
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
};

}  // namespace

// Tokens per partial block: a power of two of at least 128 (measured best on
// gfx950 for 2k-token prompts: fewer block triples to fold).  Each token slot
// of a CTA (256 threads over d_h / 8 dimension octets) should scan a run of
// at least eight tokens, so that its loads and sums outweigh the ordered
// combine, as long as the grid keeps about 1024 CTAs (`ctas_per_block` CTAs
// per token block); and the blocks per prompt stay at or below 64.
static int contrib_block_tokens(int N, int d_h, long ctas_per_block) {
  const int slots = 256 / (d_h / 8);
  int tb = 128;
  while (tb < 8 * slots) tb *= 2;
  while (tb > 128 && (long)((N + tb - 1) / tb) * ctas_per_block < 1024) tb /= 2;
  while ((long)tb * 64 < (long)N) tb *= 2;
  return tb;
}
static long contrib_ctas_per_block(int P, int Hq, int Hkv) {
  const int R = Hq / Hkv, rmax = R <= 1 ? 1 : 2;  // query heads per CTA (launch_contrib_d)
  return (long)P * Hkv * ((R + rmax - 1) / rmax);
}

template <typename T, int DH, int RMAX>
__global__ __launch_bounds__(256) void contrib_partial_kernel(const T* __restrict__ q,
                                                              const T* __restrict__ k,
                                                              const int32_t* __restrict__ seq_lens,
                                                              float* __restrict__ part, int Hq,
                                                              int Hkv, int N, int nblk, int TB) {
  constexpr int NO = DH / 8;                   // dimension octets per row (16-byte loads)
  constexpr int TPQ = 256 / NO;                // token slots per CTA
  constexpr int SPW = kWave / NO;              // token slots per wave
  constexpr int NV = 2 * RMAX + 1;             // A[R], B[R], K
  __shared__ float xs[4][NV][DH];

  // blockIdx.y = KV head x head group: this CTA serves query heads
  // hg*RMAX .. of the KV head (local index hh = hg*RMAX + j)
  const int R = Hq / Hkv, NHG = (R + RMAX - 1) / RMAX;
  const int blk = blockIdx.x, kvh = blockIdx.y / NHG, hg = blockIdx.y % NHG, p = blockIdx.z;
  const int h0 = hg * RMAX, RH = min(RMAX, R - h0);  // heads of this CTA
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int oct = lane % NO, wslot = lane / NO;
  const int slot = wave * SPW + wslot;
  int n = seq_lens ? seq_lens[p] : N;
  const bool badlen = n < 1 || n > N;
  if (badlen) n = 0;

  float A[RMAX][8], Bs[RMAX][8], K[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) K[e] = 0.f;
#pragma unroll
  for (int hh = 0; hh < RMAX; ++hh)
#pragma unroll
    for (int e = 0; e < 8; ++e) A[hh][e] = Bs[hh][e] = 0.f;

  const int per = TB / TPQ;  // tokens per slot (a contiguous run)
  const int t0 = blk * TB + slot * per;
  const int t1 = min(t0 + per, n);
  const T* kp = k + ((long)(p * Hkv + kvh) * N) * DH + 8 * oct;
  const T* qp = q + ((long)(p * Hq + kvh * R + h0) * N) * DH + 8 * oct;
  // TU tokens per step: every load of the step is issued (raw 16-byte
  // vectors) before any arithmetic, which then runs in token order
  constexpr int TU = 4;
  for (int t = t0; t < t1; t += TU) {
    Octet<T> kr[TU], qr[TU][RMAX];
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      const int tt = min(t + u, t1 - 1);  // in range; a dead token is skipped below
      kr[u].load(kp + (long)tt * DH);
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh)
        if (hh < RH) qr[u][hh].load(qp + ((long)hh * N + tt) * DH);
    }
#pragma unroll
    for (int u = 0; u < TU; ++u) {
      if (t + u >= t1) break;
      float kx[8];
      kr[u].get(kx);
#pragma unroll
      for (int e = 0; e < 8; ++e) K[e] += fabsf(kx[e]);
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh) {
        if (hh < RH) {
          float qx[8];
          qr[u][hh].get(qx);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float qa = fabsf(qx[e]);
            A[hh][e] += qa;
            Bs[hh][e] += qa * K[e];
          }
        }
      }
    }
  }

  // ordered combine of the slots of this wave: slot s absorbs slot s + 1,
  // then the pair at s + 2, ... (the lane of slot s is always the left part)
#pragma unroll
  for (int off = NO; off < kWave; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float Kr = __shfl_down(K[e], off);
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh) {
        if (hh < RH) {
          const float Ar = __shfl_down(A[hh][e], off);
          const float Br = __shfl_down(Bs[hh][e], off);
          Bs[hh][e] += Br + K[e] * Ar;
          A[hh][e] += Ar;
        }
      }
      K[e] += Kr;
    }
  }
  if (wslot == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int r = 8 * oct + e;
#pragma unroll
      for (int hh = 0; hh < RMAX; ++hh) {
        if (hh < RH) {
          xs[wave][hh][r] = A[hh][e];
          xs[wave][RMAX + hh][r] = Bs[hh][e];
        }
      }
      xs[wave][2 * RMAX][r] = K[e];
    }
  }
  __syncthreads();
  // ordered combine of the four waves: one thread per (head, dimension)
  float* out = part + (((long)p * Hkv + kvh) * nblk + blk) * (2 * R + 1) * DH;
  for (int idx = threadIdx.x; idx < RH * DH; idx += blockDim.x) {
    const int hh = idx / DH, r = idx % DH;
    float cA = 0.f, cB = 0.f, cK = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float Ar = xs[w][hh][r];
      cB += xs[w][RMAX + hh][r] + cK * Ar;
      cA += Ar;
      cK += xs[w][2 * RMAX][r];
    }
    out[(h0 + hh) * DH + r] = cA;
    out[(R + h0 + hh) * DH + r] = cB;
    if (hg == 0 && hh == 0) out[2 * R * DH + r] = badlen ? __builtin_nanf("") : cK;
  }
}

// One CTA per query head, 4 x DH threads: thread (w, r) takes prompts
// w, w + 4, ... and folds all block triples of its prompt in token order
// (sixteen blocks' loads in flight at a time); the prompt means are then
// added in prompt order.
template <int DH>
__global__ __launch_bounds__(4 * DH) void contrib_combine_kernel(const float* __restrict__ part,
                                                                 const int32_t* __restrict__ seq_lens,
                                                                 float* __restrict__ chi_per_prompt,
                                                                 float* __restrict__ chi_mean, int P,
                                                                 int Hq, int Hkv, int N, int nblk, int TB) {
  __shared__ float red[4][DH];
  const int h = blockIdx.x;
  const int r = threadIdx.x % DH, w = threadIdx.x / DH;
  const int R = Hq / Hkv, kvh = h / R, hh = h % R;
  const float inv_sqrt_d = 1.f / sqrtf((float)DH);
  const long stride = (long)(2 * R + 1) * DH;
  constexpr int U = 16;
  float mean = 0.f;
  for (int p0 = 0; p0 < P; p0 += 4) {
    const int p = p0 + w;
    float chi = 0.f;
    if (p < P) {
      const int n = seq_lens ? seq_lens[p] : N;
      const bool badlen = n < 1 || n > N;
      const int nb_used = badlen ? nblk : (n + TB - 1) / TB;
      const float* base = part + ((long)p * Hkv + kvh) * nblk * stride;
      float tA = 0.f, tB = 0.f, tK = 0.f;
      for (int bb = 0; bb < nb_used; bb += U) {
        float xa[U], xb[U], xk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float* x = base + (long)min(bb + u, nb_used - 1) * stride;
          xa[u] = x[hh * DH + r];
          xb[u] = x[(R + hh) * DH + r];
          xk[u] = x[2 * R * DH + r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (bb + u < nb_used) {
            tB += xb[u] + tK * xa[u];
            tA += xa[u];
            tK += xk[u];
          }
        }
      }
      const float pairs = 0.5f * (float)n * (float)(n + 1);
      chi = (badlen || tK != tK) ? __builtin_nanf("") : tB * inv_sqrt_d / pairs;
      if (chi_per_prompt) chi_per_prompt[((long)p * Hq + h) * DH + r] = chi;
    }
    __syncthreads();  // previous group's means consumed
    red[w][r] = chi;
    __syncthreads();
    if (w == 0)
      for (int i = 0; i < 4 && p0 + i < P; ++i) mean += red[i][r];
  }
  if (w == 0) chi_mean[(long)h * DH + r] = mean / (float)P;
}

size_t contrib_workspace_bytes(int P, int Hq, int Hkv, int N, int d_h) {
  const int TB = contrib_block_tokens(N, d_h, contrib_ctas_per_block(P, Hq, Hkv));
  const long nblk = (N + TB - 1) / TB;
  const int R = Hq / Hkv;
  return (size_t)P * Hkv * nblk * (2 * R + 1) * d_h * sizeof(float);
}

template <typename T, int DH, int RMAX>
static hipError_t launch_contrib_r(const ContribLaunch& a, hipStream_t stream) {
  const int TB = contrib_block_tokens(a.N, a.d_h, contrib_ctas_per_block(a.P, a.Hq, a.Hkv));
  const int nblk = (a.N + TB - 1) / TB;
  float* part = reinterpret_cast<float*>(a.workspace);
  const int nhg = (a.Hq / a.Hkv + RMAX - 1) / RMAX;
  hipLaunchKernelGGL((contrib_partial_kernel<T, DH, RMAX>), dim3(nblk, a.Hkv * nhg, a.P), dim3(256), 0, stream,
                     reinterpret_cast<const T*>(a.q), reinterpret_cast<const T*>(a.k), a.seq_lens, part,
                     a.Hq, a.Hkv, a.N, nblk, TB);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((contrib_combine_kernel<DH>), dim3(a.Hq), dim3(4 * DH), 0, stream, part, a.seq_lens,
                     a.chi_per_prompt, a.chi_mean, a.P, a.Hq, a.Hkv, a.N, nblk, TB);
  return hipGetLastError();
}

template <typename T, int DH>
static hipError_t launch_contrib_d(const ContribLaunch& a, hipStream_t stream) {
  // at most two query heads per CTA: more CTAs in flight, fewer live
  // accumulators per thread (the keys are re-read per head pair)
  const int R = a.Hq / a.Hkv;
  if (R <= 1) return launch_contrib_r<T, DH, 1>(a, stream);
  return launch_contrib_r<T, DH, 2>(a, stream);
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
