// Host-side dimension grouping of the OAL paper ("Not All Dimensions Are
// Equal: Outlier-Aware Attention Linearization with Grouped Quadratic
// Kernels", App. B): the outlier-aware procedure with bootstrap support, and
// the fixed-budget rule of the group-budget diagnostic.  Plain C++ on the
// host, fp64 throughout, with every sum taken in a fixed order so that a
// reference implementation that follows the same steps reaches the same
// decisions bit for bit.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <vector>

#include "../../include/oal.h"

namespace {

bool finite_nonneg(float x) { return isfinite(x) && x >= 0.f; }

// dimension indices by ascending score, equal scores in index order
std::vector<int> stable_order(const std::vector<double>& chi) {
  std::vector<int> pi(chi.size());
  for (size_t i = 0; i < pi.size(); ++i) pi[i] = (int)i;
  std::stable_sort(pi.begin(), pi.end(), [&](int a, int b) { return chi[a] < chi[b]; });
  return pi;
}

// group g holds the sorted positions between the g-th and (g+1)-th cut
void assign_groups(const std::vector<int>& pi, std::vector<int> cuts, int32_t* group_of_dim) {
  std::sort(cuts.begin(), cuts.end());
  const int d = (int)pi.size();
  int g = 0;
  size_t next = 0;
  for (int pos = 0; pos < d; ++pos) {
    while (next < cuts.size() && pos >= cuts[next]) {
      ++g;
      ++next;
    }
    group_of_dim[pi[pos]] = g;
  }
}

// adjacent contribution gap at cut k (1 <= k < d): score at sorted position
// k + 1 over the guarded score at position k (1-based positions)
double gap_ratio(const std::vector<double>& chi, const std::vector<int>& pi, int k, double eps) {
  return chi[pi[k]] / std::max(chi[pi[k - 1]], eps);
}

}  // namespace

extern "C" {

int oal_group_dims(int32_t d_h, int32_t P, const float* chi_pp, int32_t B, const int32_t* boot,
                   const oal_group_params* prm, int32_t* group_of_dim, double* rho, double* support) {
  if (d_h < 2 || P < 1 || B < 1 || chi_pp == nullptr || boot == nullptr || prm == nullptr ||
      group_of_dim == nullptr)
    return OAL_ERR_INVALID_ARG;
  if (!(prm->alpha > 0.0 && prm->alpha <= 1.0) || !(prm->gamma >= 0.0 && prm->gamma <= 1.0) ||
      !(prm->tau > 0.0) || !isfinite(prm->tau) || !(prm->eps > 0.0) || !isfinite(prm->eps) || prm->g_min < 1 ||
      prm->g_min > d_h)
    return OAL_ERR_INVALID_ARG;
  const long n = (long)P * d_h;
  for (long i = 0; i < n; ++i)
    if (!finite_nonneg(chi_pp[i])) return OAL_ERR_INVALID_ARG;
  for (long i = 0; i < (long)B * P; ++i)
    if (boot[i] < 0 || boot[i] >= P) return OAL_ERR_INVALID_ARG;
  const int d = d_h;
  const double eps = prm->eps, tau = prm->tau;

  // full-sample scores and their stable ascending order
  std::vector<double> chi(d);
  for (int r = 0; r < d; ++r) {
    double tot = 0.0;
    for (int p = 0; p < P; ++p) tot += (double)chi_pp[(long)p * d + r];
    chi[r] = tot / P;
  }
  const std::vector<int> pi = stable_order(chi);

  // candidate cuts: the top ceil(alpha d) tail and the cut just before it
  const int m = (int)ceil(prm->alpha * d);
  const int k0 = std::max(1, d - m);
  const int nc = d - k0;
  std::vector<double> rk(nc), sk(nc);
  for (int c = 0; c < nc; ++c) rk[c] = gap_ratio(chi, pi, k0 + c, eps);

  // bootstrap support: replicate scores with pi fixed, then for every cut
  // the smallest upper-side score over the largest lower-side score
  std::vector<long> count(nc, 0);
  std::vector<double> chib(d), lo_max(d), up_min(d);
  for (int b = 0; b < B; ++b) {
    const int32_t* idx = boot + (long)b * P;
    for (int r = 0; r < d; ++r) {
      double tot = 0.0;
      for (int i = 0; i < P; ++i) tot += (double)chi_pp[(long)idx[i] * d + r];
      chib[r] = tot / P;
    }
    for (int pos = 0; pos < d; ++pos) lo_max[pos] = pos == 0 ? chib[pi[0]] : std::max(lo_max[pos - 1], chib[pi[pos]]);
    for (int pos = d - 1; pos >= 0; --pos)
      up_min[pos] = pos == d - 1 ? chib[pi[d - 1]] : std::min(up_min[pos + 1], chib[pi[pos]]);
    for (int c = 0; c < nc; ++c) {
      const int k = k0 + c;  // lower side: positions 0..k-1, upper: k..d-1
      if (up_min[k] / std::max(lo_max[k - 1], eps) >= tau) ++count[c];
    }
  }
  for (int c = 0; c < nc; ++c) sk[c] = (double)count[c] / B;

  // natural cuts, then the fallback up to g_min groups
  std::vector<int> cuts;
  std::vector<int> rest;
  for (int c = 0; c < nc; ++c) {
    if (rk[c] >= tau && sk[c] >= prm->gamma) cuts.push_back(k0 + c);
    else rest.push_back(c);
  }
  if ((int)cuts.size() + 1 < prm->g_min) {
    std::stable_sort(rest.begin(), rest.end(), [&](int a, int b) {
      return sk[a] > sk[b] || (sk[a] == sk[b] && rk[a] > rk[b]);
    });
    for (int c : rest) {
      if ((int)cuts.size() + 1 >= prm->g_min) break;
      cuts.push_back(k0 + c);
    }
  }
  assign_groups(pi, cuts, group_of_dim);
  if (rho != nullptr || support != nullptr) {
    for (int k = 0; k < d; ++k) {
      const bool cand = k >= k0;
      if (rho) rho[k] = cand ? rk[k - k0] : NAN;
      if (support) support[k] = cand ? sk[k - k0] : NAN;
    }
  }
  return (int)cuts.size() + 1;
}

int oal_group_dims_budget(int32_t d_h, const float* chi_in, int32_t n_groups, double eps, int32_t* group_of_dim) {
  if (d_h < 1 || chi_in == nullptr || group_of_dim == nullptr || n_groups < 1 || n_groups > d_h ||
      !(eps > 0.0) || !isfinite(eps))
    return OAL_ERR_INVALID_ARG;
  for (int r = 0; r < d_h; ++r)
    if (!finite_nonneg(chi_in[r])) return OAL_ERR_INVALID_ARG;
  const int d = d_h;
  std::vector<double> chi(d);
  for (int r = 0; r < d; ++r) chi[r] = (double)chi_in[r];
  const std::vector<int> pi = stable_order(chi);
  std::vector<int> ks;
  std::vector<double> rk(d, 0.0);
  for (int k = 1; k < d; ++k) {
    rk[k] = gap_ratio(chi, pi, k, eps);
    ks.push_back(k);
  }
  std::stable_sort(ks.begin(), ks.end(), [&](int a, int b) { return rk[a] > rk[b]; });
  ks.resize(n_groups - 1);
  assign_groups(pi, ks, group_of_dim);
  return n_groups;
}

}  // extern "C"
