// Internal feature layout of the prefill kernels (host and device).
//
// The prefix state of the OAL paper's Eq. (5) is a linear map over features
// phi(k) = [1, k_r, k_r k_t] (raw second moments, App. D packs r <= t).  The
// prefill kernels keep it in an MFMA-friendly order, blocked in groups of 32
// features (the K depth of one v_mfma_f32_16x16x32_bf16):
//
//  * quadratic part: the d_h dimensions form nb = d_h/4 blocks of four.  The
//    block pairs (rb <= tb) are listed tb-major [(0,0), (0,1), (1,1), (0,2),
//    ...] and padded with an empty pair to an even count; K-block kb < NQ
//    holds pairs 2kb (slot 0) and 2kb+1 (slot 1).  Inside slot s the feature
//    (r, t) = (4rb + rho, 4tb + tau) has K index 16s + 4rho + tau.  A
//    diagonal pair (rb == tb) is stored as the full 4x4 square, so both (r, t)
//    and (t, r) appear, each with multiplicity one; an off-diagonal pair holds
//    r < t only and carries multiplicity two on the query side.
//  * linear part: NL = ceil((d_h+1)/32) K-blocks hold u = 32j + k, where
//    u < d_h is the linear feature k_u, u == d_h the constant and larger u are
//    zero.
//
// MFMA lane view (16x16x32): lane l belongs to lane group lg = l / 16 and
// owns K indices [8lg, 8lg+8).  For a quadratic K-block that is slot lg/2,
// rows rho in {2(lg%2), 2(lg%2)+1} and tau = 0..3: two query coordinates times
// four, which keeps feature construction at one multiply per feature.
#pragma once

namespace oal {

__host__ __device__ constexpr int nb_blocks(int d) { return d / 4; }
__host__ __device__ constexpr int n_pairs(int d) { return nb_blocks(d) * (nb_blocks(d) + 1) / 2; }
__host__ __device__ constexpr int nq_kblocks(int d) { return (n_pairs(d) + 1) / 2; }
__host__ __device__ constexpr int nl_kblocks(int d) { return (d + 1 + 31) / 32; }
__host__ __device__ constexpr int n_kblocks(int d) { return nq_kblocks(d) + nl_kblocks(d); }
__host__ __device__ constexpr long packed_features(int d) { return 1L + d + (long)d * (d + 1) / 2; }

// Snapshot of one state in the internal layout: [KB][DV+1][32] elements
// (value columns 0..DV-1, then the normaliser column z).
__host__ __device__ constexpr long snap_elems(int d, int dv) { return (long)n_kblocks(d) * (dv + 1) * 32; }

// Block pair p (tb-major) -> (rb, tb); p beyond the real pairs -> (-1, -1).
__host__ __device__ inline void pair_of(int d, int p, int& rb, int& tb) {
  if (p >= n_pairs(d)) {
    rb = -1;
    tb = -1;
    return;
  }
  int t = 0;
  while ((t + 1) * (t + 2) / 2 <= p) ++t;
  tb = t;
  rb = p - t * (t + 1) / 2;
}

// Index of the packed (library ABI) feature for internal feature (kb, k);
// -1 for padding.  `canonical` is set when the internal feature is the r <= t
// representative (used when writing a state back: each ABI entry once).
__host__ __device__ inline long abi_feature(int d, int kb, int k, bool& canonical) {
  canonical = true;
  if (kb < nq_kblocks(d)) {
    int rb, tb;
    pair_of(d, 2 * kb + k / 16, rb, tb);
    if (rb < 0) return -1;
    int m = k % 16;
    int r = 4 * rb + m / 4, t = 4 * tb + m % 4;
    if (r > t) {
      canonical = false;
      int x = r;
      r = t;
      t = x;
    }
    // row-major upper triangle: pairs before row r, then offset t - r
    long before = (long)r * d - (long)r * (r - 1) / 2;
    return 1 + d + before + (t - r);
  }
  int u = 32 * (kb - nq_kblocks(d)) + k;
  if (u < d) return 1 + u;
  if (u == d) return 0;
  return -1;
}

}  // namespace oal
