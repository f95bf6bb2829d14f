// Output-matching calibration of the kernel factors: the procedure of the
// OAL paper's App. B (Eq. (20), the squared error between the normalised OAL
// outputs and the softmax outputs, and its coefficient-calibration settings:
// Adam, gradient-norm clipping, one training sequence and a set of causal
// query positions per update, periodic validation, early stopping, the best
// checkpoint per head over several initialisation candidates).
//
// Device work: the softmax targets of every training and validation
// sequence (once per call), and per update the forward pass (oal_fwd) of
// the sampled sequence, the loss and dL/dy at the sampled positions, and the
// backward pass (oal_bwd) for the coefficient gradients; per validation the
// forward pass of the validation sequences and their squared errors.  Host
// work: the factor -> coefficient map and its gradient, and the optimiser
// on the (G + 1)(G + 2) / 2 factor entries of each head, in fp32 as the
// settings state.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "../../include/oal.h"
#include "oal_device.h"
#include "oal_internal.h"

namespace oal {
namespace {
namespace cal {

constexpr int DV = 64;
constexpr int RB = 32;  // query rows per workgroup of the softmax kernel
constexpr int KB = 64;  // keys per LDS block

template <bool BF16>
__device__ __forceinline__ float act(const void* p, long i) {
  if (BF16) return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  return reinterpret_cast<const float*>(p)[i];
}

template <bool BF16>
__device__ __forceinline__ void put(void* p, long i, float x) {
  if (BF16) reinterpret_cast<uint16_t*>(p)[i] = bf16_bits(x);
  else reinterpret_cast<float*>(p)[i] = x;
}

// Causal softmax attention of every row, the calibration target:
// y_i = sum_{j<=i} exp(q_i . k_j / sqrt(d) - m_i) v_j / sum_{j<=i} exp(...),
// by blocks of 64 keys with a running maximum.  Grid: (row blocks of 32,
// B * Hq); thread (row r = tid / 8, columns 8 (tid % 8) ..).
template <bool BF16>
__global__ __launch_bounds__(256) void softmax_rows_kernel(const void* q, const void* k, const void* v, float* y,
                                                           int Hq, int Hkv, int N, int d) {
  __shared__ float qs[RB][65];
  __shared__ float ks[KB][65];
  __shared__ float vs[KB][DV + 4];
  __shared__ float sc[RB][KB + 1];
  const int bhq = blockIdx.y, b = bhq / Hq, h = bhq % Hq, kh = h / (Hq / Hkv);
  const int i0 = blockIdx.x * RB, tid = threadIdx.x, r = tid >> 3, cg = tid & 7;
  const long qbase = ((long)b * Hq + h) * N, kbase = ((long)b * Hkv + kh) * N;
  const float scale = 1.f / sqrtf((float)d);
  for (int e = tid; e < RB * d; e += 256) {
    const int rr = e / d, dd = e % d;
    qs[rr][dd] = i0 + rr < N ? act<BF16>(q, (qbase + i0 + rr) * d + dd) : 0.f;
  }
  const int i = i0 + r;
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.f;
  const int jend = min(N, i0 + RB);  // keys up to the block's last row
  for (int j0 = 0; j0 < jend; j0 += KB) {
    __syncthreads();  // the previous block is done (and the query rows are staged)
    for (int e = tid; e < KB * d; e += 256) {
      const int jj = e / d, dd = e % d;
      ks[jj][dd] = j0 + jj < N ? act<BF16>(k, (kbase + j0 + jj) * d + dd) : 0.f;
    }
    for (int e = tid; e < KB * DV; e += 256) {
      const int jj = e / DV, cc = e % DV;
      vs[jj][cc] = j0 + jj < N ? act<BF16>(v, (kbase + j0 + jj) * DV + cc) : 0.f;
    }
    __syncthreads();
    // scores of row r for keys 8 t + cg of the block (masked past i)
    for (int t = 0; t < KB / 8; ++t) {
      const int jj = 8 * t + cg, j = j0 + jj;
      float s = 0.f;
      for (int dd = 0; dd < d; ++dd) s = fmaf(qs[r][dd], ks[jj][dd], s);
      sc[r][jj] = j <= i && j < N ? s * scale : -INFINITY;
    }
    __syncthreads();
    float mb = -INFINITY;
    for (int jj = 0; jj < KB; ++jj) mb = fmaxf(mb, sc[r][jj]);
    const float mn = fmaxf(m, mb);
    if (mn == -INFINITY) continue;  // no key of this block (or before) is causal for the row
    const float corr = __expf(m - mn);
    l *= corr;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] *= corr;
    for (int jj = 0; jj < KB; ++jj) {
      const float pj = __expf(sc[r][jj] - mn);
      l += pj;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(pj, vs[jj][8 * cg + c], acc[c]);
    }
    m = mn;
  }
  if (i < N) {
    const float rl = 1.f / l;
#pragma unroll
    for (int c = 0; c < 8; ++c) y[(qbase + i) * DV + 8 * cg + c] = acc[c] * rl;
  }
}

// n elements of an activation buffer to zero
template <bool BF16>
__global__ __launch_bounds__(256) void zero_kernel(void* x, long n) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) put<BF16>(x, i, 0.f);
}

// dL/dy rows of the previous update back to zero: grid (P, H), 64 threads
template <bool BF16>
__global__ __launch_bounds__(64) void clear_rows_kernel(void* dy, int N, const int32_t* pos) {
  const int h = blockIdx.y, row = pos[blockIdx.x];
  put<BF16>(dy, ((long)h * N + row) * DV + threadIdx.x, 0.f);
}

// dL/dy of the update's objective (1/P) sum_p ||yhat_ip - y_ip||^2 at its
// positions, 2 (yhat_ip - y_ip) / P; one workgroup per head.
template <bool BF16>
__global__ __launch_bounds__(256) void loss_rows_kernel(const void* yhat, const float* ysm, void* dy, int N,
                                                        const int32_t* pos, int P) {
  const int h = blockIdx.x;
  for (int e = threadIdx.x; e < P * DV; e += 256) {
    const int pp = e / DV, cc = e % DV;
    const long idx = ((long)h * N + pos[pp]) * DV + cc;
    put<BF16>(dy, idx, 2.f * (act<BF16>(yhat, idx) - ysm[idx]) / (float)P);
  }
}

// Squared error and target energy of whole sequences, one workgroup per
// (sequence, head): out[2 bh] = ||yhat - y||_F^2, out[2 bh + 1] = ||y||_F^2.
template <bool BF16>
__global__ __launch_bounds__(256) void seq_errors_kernel(const void* yhat, const float* ysm, double* out, int N) {
  __shared__ double r0[256], r1[256];
  const long base = (long)blockIdx.x * N * DV;
  double se = 0.0, en = 0.0;
  for (long e = threadIdx.x; e < (long)N * DV; e += 256) {
    const float t = ysm[base + e];
    const double err = (double)act<BF16>(yhat, base + e) - (double)t;
    se += err * err;
    en += (double)t * t;
  }
  r0[threadIdx.x] = se;
  r1[threadIdx.x] = en;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) {
      r0[threadIdx.x] += r0[threadIdx.x + w];
      r1[threadIdx.x] += r1[threadIdx.x + w];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    out[2 * blockIdx.x] = r0[0];
    out[2 * blockIdx.x + 1] = r1[0];
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace layout of one calibration call.
struct CalibLayout {
  size_t ysm_train, ysm_val, yhat, yval, dy, dq, dk, dv, coef, dcoef, pos, errs, fwd_ws, fwd_val_ws, bwd_ws;
  size_t total;
};

CalibLayout calib_layout(const oal_dims* d, int n_val, const oal_coeffs* cs) {
  CalibLayout L{};
  const size_t T = d->batch, H = d->n_q_heads, N = d->seq_len, dh = d->d_h, G = d->n_groups;
  const size_t es = d->dtype == OAL_BF16 ? 2 : 4;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.ysm_train = take(T * H * N * DV * 4);
  L.ysm_val = take((size_t)n_val * H * N * DV * 4);
  L.yhat = take(H * N * DV * es);
  L.yval = take((size_t)n_val * H * N * DV * es);
  L.dy = take(H * N * DV * es);
  L.dq = take(H * N * dh * 4);
  L.dk = take(H * N * dh * 4);
  L.dv = take(H * N * DV * 4);
  L.coef = take(H * (1 + G + G * G) * 4);
  L.dcoef = take(H * (1 + G + G * G) * 4);
  L.pos = take(2 * (size_t)N * 4);
  L.errs = take((size_t)n_val * H * 2 * 8);
  oal_dims one = *d;
  one.batch = 1;
  oal_dims val = *d;
  val.batch = n_val;
  L.fwd_ws = take(oal_fwd_workspace_bytes_for(&one, cs));
  L.fwd_val_ws = take(oal_fwd_workspace_bytes_for(&val, cs));
  L.bwd_ws = take(oal_bwd_workspace_bytes(&one));
  L.total = off;
  return L;
}

// (a, b, c) of one head from its factor (M = L L^T; a = eps + M_00,
// b_g = 2 M_0g, c_gh = M_gh), as oal_coeffs_from_factor computes them
void coeffs_of(const float* Lh, int G, double eps, float* a, float* b, float* c) {
  const int n = G + 1;
  auto M = [&](int i, int j) {
    double s = 0.0;
    for (int t = 0; t <= std::min(i, j); ++t) s += (double)Lh[i * n + t] * Lh[j * n + t];
    return s;
  };
  *a = (float)(eps + M(0, 0));
  for (int g = 0; g < G; ++g) b[g] = (float)(2.0 * M(0, g + 1));
  for (int g = 0; g < G; ++g)
    for (int hh = 0; hh < G; ++hh) c[g * G + hh] = (float)M(g + 1, hh + 1);
}

// gradient on the lower triangle of L from (da, db, dc): with Mbar the
// entries of M the map reads ([[da, 2 db^T], [0, dc]]), dL = (Mbar + Mbar^T) L
void factor_grad_of(const float* Lh, int G, float da, const float* db, const float* dc, double* gL) {
  const int n = G + 1;
  std::vector<double> Mb(n * n, 0.0);
  Mb[0] = da;
  for (int g = 0; g < G; ++g) Mb[g + 1] = 2.0 * db[g];
  for (int g = 0; g < G; ++g)
    for (int hh = 0; hh < G; ++hh) Mb[(g + 1) * n + hh + 1] = dc[g * G + hh];
  for (int i = 0; i < n; ++i)
    for (int j = 0; j <= i; ++j) {
      double s = 0.0;
      for (int t = j; t < n; ++t) s += (Mb[i * n + t] + Mb[t * n + i]) * Lh[t * n + j];
      gL[i * n + j] = s;
    }
}

}  // namespace cal
}  // namespace
}  // namespace oal

extern "C" {

size_t oal_calibrate_workspace_bytes(const oal_dims* dims, int32_t n_val, const int32_t* group_of_dim) {
  if (dims == nullptr || n_val < 1 || dims->batch < 1 || dims->seq_len < 1) return 0;
  oal_dims one = *dims;
  one.batch = 1;
  if (oal_bwd_workspace_bytes(&one) == 0) return 0;
  oal_coeffs probe{};
  probe.group_of_dim = group_of_dim;
  return oal::cal::calib_layout(dims, n_val, &probe).total;
}

int oal_calibrate(const oal_dims* dims, const void* q_train, const void* k_train, const void* v_train, int32_t n_val,
                  const void* q_val, const void* k_val, const void* v_val, const int32_t* group_of_dim,
                  int32_t n_init, const double* inits, int32_t n_updates, const int32_t* plan,
                  const oal_calib_params* prm, double* L_out, double* mse_out, double* relmse_out,
                  int32_t* init_out, double* cand_mse_out, int32_t* updates_out, void* workspace,
                  size_t workspace_bytes, void* stream) {
  using namespace oal::cal;
  if (dims == nullptr || prm == nullptr || inits == nullptr || L_out == nullptr || mse_out == nullptr ||
      relmse_out == nullptr || init_out == nullptr || group_of_dim == nullptr)
    return OAL_ERR_INVALID_ARG;
  const int T = dims->batch, H = dims->n_q_heads, N = dims->seq_len, dh = dims->d_h, G = dims->n_groups;
  const int P = prm->n_positions;
  if (T < 1 || N < 1 || n_val < 1 || n_init < 1 || n_updates < 0 || (n_updates > 0 && plan == nullptr))
    return OAL_ERR_INVALID_ARG;
  if (P < 1 || P > N || prm->validate_every < 1 || prm->patience < 1 || !(prm->lr >= 0.0) || !(prm->clip > 0.0) ||
      !(prm->eps >= 0.0))
    return OAL_ERR_INVALID_ARG;
  if (q_train == nullptr || k_train == nullptr || v_train == nullptr || q_val == nullptr || k_val == nullptr ||
      v_val == nullptr)
    return OAL_ERR_INVALID_ARG;
  if (dims->n_kv_heads != H || dims->d_v != DV || G < 1 || G > dh) return OAL_ERR_UNSUPPORTED;
  oal_dims one = *dims;
  one.batch = 1;
  if (oal_bwd_workspace_bytes(&one) == 0) return OAL_ERR_UNSUPPORTED;
  // the plan: sequence in [0, T), P distinct positions in [0, N)
  std::vector<char> seen(N);
  for (int u = 0; u < n_updates; ++u) {
    const int32_t* row = plan + (size_t)u * (1 + P);
    if (row[0] < 0 || row[0] >= T) return OAL_ERR_INVALID_ARG;
    std::fill(seen.begin(), seen.end(), 0);
    for (int p = 0; p < P; ++p) {
      if (row[1 + p] < 0 || row[1 + p] >= N || seen[row[1 + p]]) return OAL_ERR_INVALID_ARG;
      seen[row[1 + p]] = 1;
    }
  }
  const bool bf16 = dims->dtype == OAL_BF16;
  const int n = G + 1, nco = 1 + G + G * G;
  char* ws = reinterpret_cast<char*>(workspace);
  oal_coeffs cs{};
  cs.group_of_dim = group_of_dim;
  CalibLayout lay{};
  {
    // sizes need a coefficient struct only for the forward path choice
    oal_coeffs probe{};
    probe.group_of_dim = group_of_dim;
    lay = calib_layout(dims, n_val, &probe);
  }
  if (ws == nullptr || workspace_bytes < lay.total) return OAL_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  float* coef = reinterpret_cast<float*>(ws + lay.coef);
  cs.a = coef;
  cs.b = coef + H;
  cs.c = coef + H + (size_t)H * G;
  cs.diagonal = 0;
  float* dco = reinterpret_cast<float*>(ws + lay.dcoef);
  float *ysm_t = reinterpret_cast<float*>(ws + lay.ysm_train), *ysm_v = reinterpret_cast<float*>(ws + lay.ysm_val);
  void *yhat = ws + lay.yhat, *yval = ws + lay.yval, *dy = ws + lay.dy;
  int32_t* pos = reinterpret_cast<int32_t*>(ws + lay.pos);  // [2][N]: this update's positions, the previous
  double* errs = reinterpret_cast<double*>(ws + lay.errs);
  const size_t es = bf16 ? 2 : 4;
  const size_t seq_qk = (size_t)H * N * dh * es, seq_v = (size_t)H * N * DV * es;

  // targets, and dL/dy starting at zero
  {
    const dim3 blk(256);
    if (bf16) {
      hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3((N + RB - 1) / RB, T * H), blk, 0, st, q_train, k_train,
                         v_train, ysm_t, H, H, N, dh);
      hipLaunchKernelGGL(softmax_rows_kernel<true>, dim3((N + RB - 1) / RB, n_val * H), blk, 0, st, q_val, k_val,
                         v_val, ysm_v, H, H, N, dh);
    } else {
      hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3((N + RB - 1) / RB, T * H), blk, 0, st, q_train, k_train,
                         v_train, ysm_t, H, H, N, dh);
      hipLaunchKernelGGL(softmax_rows_kernel<false>, dim3((N + RB - 1) / RB, n_val * H), blk, 0, st, q_val, k_val,
                         v_val, ysm_v, H, H, N, dh);
    }
    const long ndy = (long)H * N * DV;
    if (bf16)
      hipLaunchKernelGGL(zero_kernel<true>, dim3((unsigned)((ndy + 255) / 256)), dim3(256), 0, st, dy, ndy);
    else
      hipLaunchKernelGGL(zero_kernel<false>, dim3((unsigned)((ndy + 255) / 256)), dim3(256), 0, st, dy, ndy);
    if (hipGetLastError() != hipSuccess) return OAL_ERR_HIP;
  }
  oal_dims vd = *dims;
  vd.batch = n_val;
  std::vector<float> hco(nco * H), hdco(nco * H);
  std::vector<double> herr((size_t)n_val * H * 2);
  auto upload_coeffs = [&](const std::vector<float>& Lf) -> int {
    for (int h = 0; h < H; ++h)
      coeffs_of(&Lf[(size_t)h * n * n], G, prm->eps, &hco[h], &hco[H + (size_t)h * G], &hco[H + (size_t)H * G + (size_t)h * G * G]);
    return hipMemcpyAsync(coef, hco.data(), hco.size() * 4, hipMemcpyHostToDevice, st) == hipSuccess ? OAL_OK
                                                                                                     : OAL_ERR_HIP;
  };
  // validation MSE and RelMSE of every head
  auto validate = [&](const std::vector<float>& Lf, std::vector<double>& mse, std::vector<double>& rel) -> int {
    int s = upload_coeffs(Lf);
    if (s != OAL_OK) return s;
    s = oal_fwd(&vd, q_val, k_val, v_val, &cs, nullptr, nullptr, nullptr, yval, ws + lay.fwd_val_ws,
                lay.bwd_ws - lay.fwd_val_ws, stream);
    if (s != OAL_OK) return s;
    if (bf16)
      hipLaunchKernelGGL(seq_errors_kernel<true>, dim3(n_val * H), dim3(256), 0, st, yval, ysm_v, errs, N);
    else
      hipLaunchKernelGGL(seq_errors_kernel<false>, dim3(n_val * H), dim3(256), 0, st, yval, ysm_v, errs, N);
    if (hipGetLastError() != hipSuccess) return OAL_ERR_HIP;
    if (hipMemcpyAsync(herr.data(), errs, herr.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return OAL_ERR_HIP;
    for (int h = 0; h < H; ++h) {
      double sm = 0.0, sr = 0.0;
      for (int b = 0; b < n_val; ++b) {
        const double se = herr[((size_t)b * H + h) * 2], en = herr[((size_t)b * H + h) * 2 + 1];
        sm += se / ((double)N * DV);
        sr += se / en;
      }
      mse[h] = sm / n_val;
      rel[h] = sr / n_val;
    }
    return OAL_OK;
  };

  const int ntri = n * (n + 1) / 2;
  std::vector<double> best_mse_all((size_t)n_init * H), best_rel_all((size_t)n_init * H);
  std::vector<float> best_L_all((size_t)n_init * H * n * n);
  std::vector<int32_t> upd_all((size_t)n_init * H);
  std::vector<int32_t> hpos(P);
  for (int ci = 0; ci < n_init; ++ci) {
    std::vector<float> Lf((size_t)H * n * n, 0.f);
    for (int h = 0; h < H; ++h)
      for (int i = 0; i < n; ++i)
        for (int j = 0; j <= i; ++j)
          Lf[((size_t)h * n + i) * n + j] = (float)inits[(((size_t)ci * H + h) * n + i) * n + j];
    std::vector<float> m((size_t)H * ntri, 0.f), v((size_t)H * ntri, 0.f);
    std::vector<double> best(H), brel(H), cur(H), crel(H);
    int s = validate(Lf, best, brel);
    if (s != OAL_OK) return s;
    std::vector<float> bestL = Lf;
    std::vector<int> last(H, 0), done(H, 0);
    std::vector<char> active(H, 1);
    int prevP = 0, prev_slot = 0;
    for (int u = 1; u <= n_updates; ++u) {
      if (std::none_of(active.begin(), active.end(), [](char a) { return a != 0; })) break;
      const int32_t* row = plan + (size_t)(u - 1) * (1 + P);
      const int seq = row[0];
      for (int p = 0; p < P; ++p) hpos[p] = row[1 + p];
      if ((s = upload_coeffs(Lf)) != OAL_OK) return s;
      // positions of this update (slot u % 2), the previous update's rows cleared
      int32_t* cur_pos = pos + (size_t)(u & 1) * N;
      int32_t* old_pos = pos + (size_t)((u - 1) & 1) * N;
      if (hipMemcpyAsync(cur_pos, hpos.data(), P * 4, hipMemcpyHostToDevice, st) != hipSuccess) return OAL_ERR_HIP;
      const char* qs = reinterpret_cast<const char*>(q_train) + (size_t)seq * seq_qk;
      const char* ks = reinterpret_cast<const char*>(k_train) + (size_t)seq * seq_qk;
      const char* vs = reinterpret_cast<const char*>(v_train) + (size_t)seq * seq_v;
      s = oal_fwd(&one, qs, ks, vs, &cs, nullptr, nullptr, nullptr, yhat, ws + lay.fwd_ws, lay.fwd_val_ws - lay.fwd_ws,
                  stream);
      if (s != OAL_OK) return s;
      const float* yt = ysm_t + (size_t)seq * H * N * DV;
      if (bf16) {
        if (prevP > 0) hipLaunchKernelGGL(clear_rows_kernel<true>, dim3(prevP, H), dim3(64), 0, st, dy, N, old_pos);
        hipLaunchKernelGGL(loss_rows_kernel<true>, dim3(H), dim3(256), 0, st, yhat, yt, dy, N, cur_pos, P);
      } else {
        if (prevP > 0) hipLaunchKernelGGL(clear_rows_kernel<false>, dim3(prevP, H), dim3(64), 0, st, dy, N, old_pos);
        hipLaunchKernelGGL(loss_rows_kernel<false>, dim3(H), dim3(256), 0, st, yhat, yt, dy, N, cur_pos, P);
      }
      if (hipGetLastError() != hipSuccess) return OAL_ERR_HIP;
      prevP = P;
      prev_slot = u & 1;
      float* da = dco;
      float* db = dco + H;
      float* dc = dco + H + (size_t)H * G;
      s = oal_bwd(&one, qs, ks, vs, dy, &cs, reinterpret_cast<float*>(ws + lay.dq), reinterpret_cast<float*>(ws + lay.dk),
                  reinterpret_cast<float*>(ws + lay.dv), da, db, dc, ws + lay.bwd_ws, lay.total - lay.bwd_ws, stream);
      if (s != OAL_OK) return s;
      if (hipMemcpyAsync(hdco.data(), dco, hdco.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
          hipStreamSynchronize(st) != hipSuccess)
        return OAL_ERR_HIP;
      // Adam on the lower triangle of each active head's factor, its
      // gradient norm clipped at clip
      const float b1 = 0.9f, b2 = 0.999f, aeps = 1e-8f, lr = (float)prm->lr;
      const float c1 = 1.f - powf(b1, (float)u), c2 = 1.f - powf(b2, (float)u);
      std::vector<double> gL(n * n);
      for (int h = 0; h < H; ++h) {
        if (!active[h]) continue;
        float* Lh = &Lf[(size_t)h * n * n];
        factor_grad_of(Lh, G, hdco[h], &hdco[H + (size_t)h * G], &hdco[H + (size_t)H * G + (size_t)h * G * G], gL.data());
        double nrm = 0.0;
        for (int i = 0; i < n; ++i)
          for (int j = 0; j <= i; ++j) nrm += gL[i * n + j] * gL[i * n + j];
        nrm = sqrt(nrm);
        const double sc = nrm > prm->clip ? prm->clip / (nrm + 1e-6) : 1.0;
        int e = 0;
        for (int i = 0; i < n; ++i)
          for (int j = 0; j <= i; ++j, ++e) {
            const float g = (float)(gL[i * n + j] * sc);
            float& mm = m[(size_t)h * ntri + e];
            float& vv = v[(size_t)h * ntri + e];
            mm = b1 * mm + (1.f - b1) * g;
            vv = b2 * vv + (1.f - b2) * g * g;
            Lh[i * n + j] -= lr * (mm / c1) / (sqrtf(vv / c2) + aeps);
          }
        done[h] = u;
      }
      if (u % prm->validate_every == 0) {
        if ((s = validate(Lf, cur, crel)) != OAL_OK) return s;
        for (int h = 0; h < H; ++h) {
          if (!active[h]) continue;
          if (cur[h] < best[h]) {
            best[h] = cur[h];
            brel[h] = crel[h];
            last[h] = u;
            std::copy(&Lf[(size_t)h * n * n], &Lf[(size_t)(h + 1) * n * n], &bestL[(size_t)h * n * n]);
          } else if (u - last[h] >= prm->patience) {
            active[h] = 0;
          }
        }
      }
    }
    // dL/dy back to zero for the next candidate
    if (prevP > 0) {
      if (bf16)
        hipLaunchKernelGGL(clear_rows_kernel<true>, dim3(prevP, H), dim3(64), 0, st, dy, N, pos + (size_t)prev_slot * N);
      else
        hipLaunchKernelGGL(clear_rows_kernel<false>, dim3(prevP, H), dim3(64), 0, st, dy, N, pos + (size_t)prev_slot * N);
      if (hipGetLastError() != hipSuccess) return OAL_ERR_HIP;
    }
    for (int h = 0; h < H; ++h) {
      best_mse_all[(size_t)ci * H + h] = best[h];
      best_rel_all[(size_t)ci * H + h] = brel[h];
      upd_all[(size_t)ci * H + h] = done[h];
    }
    std::copy(bestL.begin(), bestL.end(), &best_L_all[(size_t)ci * H * n * n]);
  }
  // the best candidate of every head
  for (int h = 0; h < H; ++h) {
    int pick = 0;
    for (int ci = 1; ci < n_init; ++ci)
      if (best_mse_all[(size_t)ci * H + h] < best_mse_all[(size_t)pick * H + h]) pick = ci;
    init_out[h] = pick;
    mse_out[h] = best_mse_all[(size_t)pick * H + h];
    relmse_out[h] = best_rel_all[(size_t)pick * H + h];
    for (int e = 0; e < n * n; ++e) L_out[(size_t)h * n * n + e] = best_L_all[((size_t)pick * H + h) * n * n + e];
  }
  if (cand_mse_out != nullptr) std::copy(best_mse_all.begin(), best_mse_all.end(), cand_mse_out);
  if (updates_out != nullptr) std::copy(upd_all.begin(), upd_all.end(), updates_out);
  return OAL_OK;
}

}  // extern "C"
