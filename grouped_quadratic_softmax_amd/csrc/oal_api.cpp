// C ABI of the OAL library: argument validation on the host, workspace
// sizing and dispatch to the HIP kernels.  Nothing here allocates, frees or
// synchronises.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <initializer_list>

#include "../../include/oal.h"
#include "oal_internal.h"
#include "oal_layout.h"

namespace {

bool supported_dh(int d) { return d == 16 || d == 32 || d == 64; }

// Activations, states and workspaces are read and written with 16-byte
// vector accesses; a null pointer passes (nullness is checked separately).
bool all_aligned16(std::initializer_list<const void*> ps) {
  for (const void* p : ps)
    if (((uintptr_t)p & 15) != 0) return false;
  return true;
}

// Common shape checks.  `need_seq` is false for decode.
int check_dims(const oal_dims* d, bool need_seq) {
  if (d == nullptr) return OAL_ERR_INVALID_ARG;
  if (d->batch < 0 || d->n_q_heads < 1 || d->n_kv_heads < 1) return OAL_ERR_INVALID_ARG;
  if (d->n_q_heads % d->n_kv_heads != 0) return OAL_ERR_INVALID_ARG;
  if (need_seq && d->seq_len < 0) return OAL_ERR_INVALID_ARG;
  if (d->d_h < 1 || d->d_v < 1) return OAL_ERR_INVALID_ARG;
  if (d->dtype != OAL_F32 && d->dtype != OAL_BF16) return OAL_ERR_INVALID_ARG;
  if (!supported_dh(d->d_h) || d->d_v != 64) return OAL_ERR_UNSUPPORTED;
  return OAL_OK;
}

int check_coeff_dims(const oal_dims* d) {
  if (d->n_groups < 1 || d->n_groups > d->d_h) return OAL_ERR_INVALID_ARG;
  return OAL_OK;
}

int check_coeff_ptrs(const oal_coeffs* c) {
  if (c == nullptr || c->group_of_dim == nullptr || c->a == nullptr || c->b == nullptr || c->c == nullptr)
    return OAL_ERR_INVALID_ARG;
  return OAL_OK;
}

int check_prep(const oal_prep* p) {
  if (p == nullptr) return OAL_OK;
  if (p->gamma_q == nullptr || p->beta_q == nullptr || p->gamma_k == nullptr || p->beta_k == nullptr)
    return OAL_ERR_INVALID_ARG;
  if (!(p->ln_eps >= 0.f) || !isfinite(p->ln_eps)) return OAL_ERR_INVALID_ARG;
  if (p->kind != OAL_PREMAP_LAYERNORM && p->kind != OAL_PREMAP_L2) return OAL_ERR_INVALID_ARG;
  return OAL_OK;
}

// Which prefill build serves a call: the one-call small-space path (the
// dimension-wise form), the one-call path at d_h = 16, or the chunk path.
// Calls with per-sequence lengths take the one-launch builds only (heads
// with their own keys), else the chunk path.
struct FwdPath {
  bool small = false, onepass = false;
};
FwdPath fwd_path(const oal_dims* dims, bool diagonal, bool premap, bool varlen) {
  FwdPath p;
  const int d = dims->d_h, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads;
  p.small = oal::small_path_supported(d, diagonal, Hq, Hkv) &&
            (!varlen || oal::dimw_supported(d, dims->dtype, diagonal, Hq, Hkv));
  p.onepass = oal::onepass16_supported(d, dims->dtype, diagonal, dims->n_groups, Hq, Hkv, premap) &&
              (!varlen || oal::onepass16w_supported(Hq, Hkv, premap));
  return p;
}

}  // namespace

extern "C" {

const char* oal_version(void) { return "oal-mi355x 0.1.0 (gfx950)"; }

const char* oal_status_str(int status) {
  switch (status) {
    case OAL_OK: return "OAL_OK";
    case OAL_ERR_INVALID_ARG: return "OAL_ERR_INVALID_ARG";
    case OAL_ERR_UNSUPPORTED: return "OAL_ERR_UNSUPPORTED";
    case OAL_ERR_WORKSPACE: return "OAL_ERR_WORKSPACE";
    case OAL_ERR_HIP: return "OAL_ERR_HIP";
    default: return "OAL_ERR_UNKNOWN";
  }
}

int64_t oal_feature_count(int32_t d_h) {
  if (d_h < 1) return 0;
  return oal::packed_features(d_h);
}

int64_t oal_state_floats(int32_t d_h, int32_t d_v) {
  if (d_h < 1 || d_v < 1) return 0;
  return oal::packed_features(d_h) * (int64_t)(d_v + 1);
}

int oal_coeffs_from_factor(int32_t n_heads, int32_t n_groups, double eps, const double* L, float* a,
                           float* b, float* c) {
  if (n_heads < 0 || n_groups < 1 || L == nullptr || a == nullptr || b == nullptr || c == nullptr)
    return OAL_ERR_INVALID_ARG;
  const int n = n_groups + 1;
  for (int h = 0; h < n_heads; ++h) {
    const double* Lh = L + (size_t)h * n * n;
    // M = L L^T over the lower triangle of L
    auto M = [&](int i, int j) {
      double s = 0.0;
      const int m = i < j ? i : j;
      for (int t = 0; t <= m; ++t) s += Lh[i * n + t] * Lh[j * n + t];
      return s;
    };
    a[h] = (float)(eps + M(0, 0));
    for (int g = 0; g < n_groups; ++g) b[(size_t)h * n_groups + g] = (float)(2.0 * M(0, g + 1));
    for (int g = 0; g < n_groups; ++g)
      for (int hh = 0; hh < n_groups; ++hh)
        c[((size_t)h * n_groups + g) * n_groups + hh] = (float)M(g + 1, hh + 1);
  }
  return OAL_OK;
}

int oal_check_coeffs(const oal_dims* dims, const int32_t* group_of_dim_host, const float* c_host) {
  if (dims == nullptr || group_of_dim_host == nullptr) return OAL_ERR_INVALID_ARG;
  const int G = dims->n_groups;
  if (dims->n_q_heads < 1 || dims->d_h < 1 || G < 1 || G > dims->d_h) return OAL_ERR_INVALID_ARG;
  const size_t nmap = (size_t)dims->n_q_heads * dims->d_h;
  for (size_t i = 0; i < nmap; ++i)
    if (group_of_dim_host[i] < 0 || group_of_dim_host[i] >= G) return OAL_ERR_INVALID_ARG;
  if (c_host != nullptr) {
    const size_t nc = (size_t)dims->n_q_heads * G * G;
    for (size_t i = 0; i < nc; ++i)
      if (!isfinite(c_host[i])) return OAL_ERR_INVALID_ARG;
  }
  return OAL_OK;
}

size_t oal_fwd_workspace_bytes(const oal_dims* dims) {
  if (check_dims(dims, true) != OAL_OK) return 0;
  return oal::fwd_workspace_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->seq_len, dims->d_h,
                                 dims->dtype);
}

namespace {
size_t workspace_for_path(const oal_dims* dims, const oal_coeffs* coeffs, bool varlen) {
  if (coeffs == nullptr || check_dims(dims, true) != OAL_OK) return 0;
  const bool diagonal = coeffs->diagonal != 0;
  const FwdPath path = fwd_path(dims, diagonal, false, varlen);
  if (path.onepass)
    return oal::onepass16_workspace_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->seq_len);
  if (!path.small)
    return diagonal ? 0 : oal_fwd_workspace_bytes(dims);
  return oal::small_workspace_bytes_for(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->seq_len, dims->d_h,
                                       diagonal, dims->dtype);
}
}  // namespace

size_t oal_fwd_workspace_bytes_for(const oal_dims* dims, const oal_coeffs* coeffs) {
  return workspace_for_path(dims, coeffs, false);
}

size_t oal_fwd_varlen_workspace_bytes_for(const oal_dims* dims, const oal_coeffs* coeffs) {
  return workspace_for_path(dims, coeffs, true);
}

namespace {

// Shared validation and dispatch of oal_fwd and its two stages.
// stages: bit 0 = chunk states, bit 1 = outputs.
int fwd_stages(const oal_dims* dims, const void* q, const void* k, const void* v, const oal_coeffs* coeffs,
               const oal_prep* prep, const float* state_in, float* state_out, void* y, void* workspace,
               size_t workspace_bytes, void* stream, int stages, const int32_t* seq_lens = nullptr) {
  const bool want_states = stages & 1, want_out = stages & 2;
  int st = check_dims(dims, true);
  if (st != OAL_OK) return st;
  bool diagonal = false, small = false, onepass = false;
  if (want_out) {
    if ((st = check_coeff_dims(dims)) != OAL_OK) return st;
    if ((st = check_coeff_ptrs(coeffs)) != OAL_OK) return st;
    diagonal = coeffs->diagonal != 0;
    const FwdPath path = fwd_path(dims, diagonal, prep != nullptr, seq_lens != nullptr);
    small = want_states && path.small;
    onepass = want_states && path.onepass;
    if (diagonal && !small) return OAL_ERR_UNSUPPORTED;  // no separate stages for this form
    if (!small && !onepass && dims->n_groups > 8) return OAL_ERR_UNSUPPORTED;
  }
  if ((st = check_prep(prep)) != OAL_OK) return st;
  if (dims->batch == 0) return OAL_OK;
  if (dims->seq_len == 0) {
    // nothing to attend to; the state passes through unchanged
    if (want_states && state_out != nullptr) {
      const long n = (long)dims->batch * dims->n_kv_heads * oal_state_floats(dims->d_h, dims->d_v);
      if (oal::launch_state_passthrough(state_in, state_out, n, (hipStream_t)stream) != hipSuccess)
        return OAL_ERR_HIP;
    }
    return OAL_OK;
  }
  if (k == nullptr || v == nullptr) return OAL_ERR_INVALID_ARG;
  if (want_out && (q == nullptr || y == nullptr)) return OAL_ERR_INVALID_ARG;
  if (want_states && state_out != nullptr && state_out == state_in) return OAL_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, v, y, state_in, state_out, workspace})) return OAL_ERR_INVALID_ARG;
  if (!small && !onepass) {  // the one-pass paths take any workspace
    const size_t need = oal_fwd_workspace_bytes(dims);
    if (workspace == nullptr || workspace_bytes < need) return OAL_ERR_WORKSPACE;
  }

  oal::FwdLaunch a{};
  a.B = dims->batch; a.Hq = dims->n_q_heads; a.Hkv = dims->n_kv_heads; a.N = dims->seq_len;
  a.d_h = dims->d_h; a.G = dims->n_groups; a.dtype = dims->dtype;
  a.q = q; a.k = k; a.v = v;
  if (want_out) {
    a.group_of_dim = coeffs->group_of_dim; a.ca = coeffs->a; a.cb = coeffs->b; a.cc = coeffs->c;
  }
  a.premap = prep != nullptr;
  if (prep) {
    a.gamma_q = prep->gamma_q; a.beta_q = prep->beta_q; a.gamma_k = prep->gamma_k; a.beta_k = prep->beta_k;
    a.ln_eps = prep->ln_eps;
    a.premap_kind = prep->kind;
  }
  a.state_in = state_in; a.state_out = state_out; a.y = y; a.workspace = workspace;
  a.diagonal = diagonal;
  a.seq_lens = seq_lens;
  if (onepass)
    return oal::launch_onepass16(a, workspace ? workspace_bytes : 0, (hipStream_t)stream) == hipSuccess
               ? OAL_OK
               : OAL_ERR_HIP;
  if (small)
    return oal::launch_fwd_small(a, workspace ? workspace_bytes : 0, (hipStream_t)stream) == hipSuccess
               ? OAL_OK
               : OAL_ERR_HIP;
  return oal::launch_fwd(a, stages, (hipStream_t)stream) == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

}  // namespace

int oal_fwd(const oal_dims* dims, const void* q, const void* k, const void* v, const oal_coeffs* coeffs,
            const oal_prep* prep, const float* state_in, float* state_out, void* y, void* workspace,
            size_t workspace_bytes, void* stream) {
  return fwd_stages(dims, q, k, v, coeffs, prep, state_in, state_out, y, workspace, workspace_bytes, stream, 3);
}

int oal_fwd_varlen(const oal_dims* dims, const int32_t* seq_lens, const void* q, const void* k, const void* v,
                   const oal_coeffs* coeffs, const oal_prep* prep, const float* state_in, float* state_out,
                   void* y, void* workspace, size_t workspace_bytes, void* stream) {
  if (seq_lens == nullptr) return OAL_ERR_INVALID_ARG;
  return fwd_stages(dims, q, k, v, coeffs, prep, state_in, state_out, y, workspace, workspace_bytes, stream, 3,
                    seq_lens);
}

int oal_fwd_states(const oal_dims* dims, const void* k, const void* v, const oal_prep* prep,
                   const float* state_in, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream) {
  return fwd_stages(dims, nullptr, k, v, nullptr, prep, state_in, state_out, nullptr, workspace,
                    workspace_bytes, stream, 1);
}

int oal_fwd_outputs(const oal_dims* dims, const void* q, const void* k, const void* v,
                    const oal_coeffs* coeffs, const oal_prep* prep, const float* state_in, void* y,
                    void* workspace, size_t workspace_bytes, void* stream) {
  // state_in only tells the first chunk whether there is an initial state to read
  return fwd_stages(dims, q, k, v, coeffs, prep, state_in, nullptr, y, workspace, workspace_bytes, stream, 2);
}

size_t oal_decode_workspace_bytes(const oal_dims* dims) {
  if (check_dims(dims, false) != OAL_OK) return 0;
  if (dims->n_q_heads / dims->n_kv_heads > 8) return 0;
  return oal::decode_workspace_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->d_h);
}

int oal_decode_step(const oal_dims* dims, const void* q, const void* k, const void* v,
                    const oal_coeffs* coeffs, const oal_prep* prep, float* state, void* y, void* workspace,
                    size_t workspace_bytes, void* stream) {
  int st = check_dims(dims, false);
  if (st != OAL_OK) return st;
  if ((st = check_coeff_dims(dims)) != OAL_OK) return st;
  if ((st = check_coeff_ptrs(coeffs)) != OAL_OK) return st;
  if ((st = check_prep(prep)) != OAL_OK) return st;
  if (dims->n_q_heads / dims->n_kv_heads > 8) return OAL_ERR_UNSUPPORTED;
  if (dims->batch == 0) return OAL_OK;
  if (q == nullptr || k == nullptr || v == nullptr || state == nullptr || y == nullptr)
    return OAL_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, v, y, state, workspace})) return OAL_ERR_INVALID_ARG;
  const size_t need = oal_decode_workspace_bytes(dims);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return OAL_ERR_WORKSPACE;
  oal::DecodeLaunch a{};
  a.B = dims->batch; a.Hq = dims->n_q_heads; a.Hkv = dims->n_kv_heads; a.d_h = dims->d_h;
  a.G = dims->n_groups; a.dtype = dims->dtype;
  a.q = q; a.k = k; a.v = v;
  a.group_of_dim = coeffs->group_of_dim; a.ca = coeffs->a; a.cb = coeffs->b; a.cc = coeffs->c;
  a.diagonal = coeffs->diagonal != 0;
  a.premap = prep != nullptr;
  if (prep) {
    a.gamma_q = prep->gamma_q; a.beta_q = prep->beta_q; a.gamma_k = prep->gamma_k; a.beta_k = prep->beta_k;
    a.ln_eps = prep->ln_eps;
    a.premap_kind = prep->kind;
  }
  a.state = state; a.y = y; a.workspace = workspace;
  return oal::launch_decode(a, (hipStream_t)stream) == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

int oal_decode_step_noalloc(const oal_dims* dims, const void* q, const void* k, const void* v,
                            const oal_coeffs* coeffs, const oal_prep* prep, float* state, void* y, void* stream) {
  const size_t need = oal_decode_workspace_bytes(dims);
  void* ws = nullptr;
  if (need > 0) {
    if (need > oal::kDecodeScratchBytes) return OAL_ERR_WORKSPACE;
    if (oal::decode_scratch(&ws) != hipSuccess) return OAL_ERR_HIP;
  }
  return oal_decode_step(dims, q, k, v, coeffs, prep, state, y, ws, need, stream);
}

size_t oal_contrib_workspace_bytes(const oal_dims* dims) {
  if (check_dims(dims, true) != OAL_OK) return 0;
  if (dims->n_q_heads / dims->n_kv_heads > 16) return 0;
  return oal::contrib_workspace_bytes(dims->batch, dims->n_q_heads, dims->n_kv_heads, dims->seq_len,
                                      dims->d_h);
}

int oal_contrib(const oal_dims* dims, const void* q, const void* k, const int32_t* seq_lens,
                float* chi_per_prompt, float* chi_mean, void* workspace, size_t workspace_bytes,
                void* stream) {
  int st = check_dims(dims, true);
  if (st != OAL_OK) return st;
  if (dims->n_q_heads / dims->n_kv_heads > 16) return OAL_ERR_UNSUPPORTED;
  if (dims->batch < 1 || dims->seq_len < 1) return OAL_ERR_INVALID_ARG;
  if (q == nullptr || k == nullptr || chi_mean == nullptr) return OAL_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, workspace})) return OAL_ERR_INVALID_ARG;
  const size_t need = oal_contrib_workspace_bytes(dims);
  if (workspace == nullptr || workspace_bytes < need) return OAL_ERR_WORKSPACE;
  oal::ContribLaunch a{};
  a.P = dims->batch; a.Hq = dims->n_q_heads; a.Hkv = dims->n_kv_heads; a.N = dims->seq_len;
  a.d_h = dims->d_h; a.dtype = dims->dtype;
  a.q = q; a.k = k; a.seq_lens = seq_lens; a.chi_per_prompt = chi_per_prompt; a.chi_mean = chi_mean;
  a.workspace = workspace;
  return oal::launch_contrib(a, (hipStream_t)stream) == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

size_t oal_bwd_workspace_bytes(const oal_dims* dims) {
  if (check_dims(dims, true) != OAL_OK || check_coeff_dims(dims) != OAL_OK) return 0;
  if (!oal::bwd16_supported(dims->d_h, dims->d_v, dims->dtype, false, dims->n_groups, dims->n_q_heads,
                            dims->n_kv_heads))
    return 0;
  return oal::bwd16_workspace_bytes(dims->batch, dims->n_q_heads, dims->seq_len);
}

int oal_bwd(const oal_dims* dims, const void* q, const void* k, const void* v, const void* dy,
            const oal_coeffs* coeffs, float* dq, float* dk, float* dv, float* da, float* db, float* dc,
            void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_dims(dims, true);
  if (st != OAL_OK) return st;
  if ((st = check_coeff_dims(dims)) != OAL_OK) return st;
  if ((st = check_coeff_ptrs(coeffs)) != OAL_OK) return st;
  if (!oal::bwd16_supported(dims->d_h, dims->d_v, dims->dtype, coeffs->diagonal != 0, dims->n_groups,
                            dims->n_q_heads, dims->n_kv_heads))
    return OAL_ERR_UNSUPPORTED;
  if (da == nullptr || db == nullptr || dc == nullptr) return OAL_ERR_INVALID_ARG;
  const bool work = dims->batch > 0 && dims->seq_len > 0;
  if (work && (q == nullptr || k == nullptr || v == nullptr || dy == nullptr || dq == nullptr ||
               dk == nullptr || dv == nullptr))
    return OAL_ERR_INVALID_ARG;
  if (!all_aligned16({q, k, v, dy, dq, dk, dv, workspace})) return OAL_ERR_INVALID_ARG;
  const size_t need = oal_bwd_workspace_bytes(dims);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return OAL_ERR_WORKSPACE;
  oal::BwdLaunch a{};
  a.B = dims->batch; a.H = dims->n_q_heads; a.N = dims->seq_len; a.G = dims->n_groups; a.dtype = dims->dtype;
  a.q = q; a.k = k; a.v = v; a.dy = dy;
  a.group_of_dim = coeffs->group_of_dim; a.ca = coeffs->a; a.cb = coeffs->b; a.cc = coeffs->c;
  a.dq = dq; a.dk = dk; a.dv = dv; a.da = da; a.db = db; a.dc = dc;
  a.workspace = workspace;
  return oal::launch_bwd16(a, (hipStream_t)stream) == hipSuccess ? OAL_OK : OAL_ERR_HIP;
}

}  // extern "C"
