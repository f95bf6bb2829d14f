// Internal feature layout of the prefill kernels (host and device).
//
// The prefix state of the OAL paper's Eq. (5) is a linear map over the key
// features phi(k) = [1, k_r, k_r k_t] (App. D packs the pairs r <= t).  The
// prefill kernels keep it in an MFMA-friendly order, blocked in K-blocks of
// 32 features (the K depth of one 16x16x32 MFMA):
//
//  * quadratic part: the d_h dimensions form nb = d_h/4 blocks of four.  The
//    block pairs (rb <= tb) are listed tb-major [(0,0), (0,1), (1,1), (0,2),
//    ...] and padded with an empty pair to an even count; K-block kb < NQ
//    holds pairs 2kb (slot 0) and 2kb+1 (slot 1).  Position k of the K-block
//    belongs to MFMA lane group lg = k / 8: slot s = lg / 2, query rows
//    rho in {2(lg%2), 2(lg%2)+1} and tau = 0..3, i.e. position
//    k = 8 lg + 4 (rho % 2) + tau holds (r, t) = (4 rb + rho, 4 tb + tau).
//    A lane therefore builds its eight features from two r values times four
//    t values.  A diagonal pair (rb == tb) is stored as the full 4x4 square,
//    so both (r, t) and (t, r) appear, each with multiplicity one; an
//    off-diagonal pair holds r < t only and carries multiplicity two on the
//    query side.
//  * linear part: NL = ceil(d_h / 32) K-blocks; position k of K-block
//    NQ + j is the linear feature u = 32 j + k (padding when u >= d_h).
//  * the constant feature is kept outside the K-blocks (its row of the
//    state is [sum_j v_j, n]).
//
// Snapshot of a state (one per chunk start): [KB][NCOL][32] elements, value
// columns 0..d_v-1 then the normaliser column z, each column holding the 32
// features of the K-block contiguously, so that MFMA lane group lg loads its
// eight features as one 16-byte vector.  The scan kernel's accumulator tiles
// map onto the same order: accumulator row rho (0..15) of M-tile m (0, 1)
// is position 8 (rho / 4) + 4 m + (rho % 4).
#pragma once

namespace oal {

__host__ __device__ constexpr int nb_blocks(int d) { return d / 4; }
__host__ __device__ constexpr int n_pairs(int d) { return nb_blocks(d) * (nb_blocks(d) + 1) / 2; }
__host__ __device__ constexpr int nq_kblocks(int d) { return (n_pairs(d) + 1) / 2; }
__host__ __device__ constexpr int nl_kblocks(int d) { return (d + 31) / 32; }
__host__ __device__ constexpr int n_kblocks(int d) { return nq_kblocks(d) + nl_kblocks(d); }
__host__ __device__ constexpr long packed_features(int d) { return 1L + d + (long)d * (d + 1) / 2; }

// Block pair p (tb-major) -> (rb, tb); p beyond the real pairs -> (-1, -1).
__host__ __device__ constexpr void pair_of(int d, int p, int& rb, int& tb) {
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

// Feature at position k of K-block kb.  Returns false for padding.  On
// success r is the first dimension, t the second (t == d for a linear
// feature) and mult the query-side multiplicity (1 or 2).
__host__ __device__ constexpr bool kfeature(int d, int kb, int k, int& r, int& t, int& mult) {
  if (kb < nq_kblocks(d)) {
    const int lg = k / 8;
    int rb = 0, tb = 0;
    pair_of(d, 2 * kb + lg / 2, rb, tb);
    if (rb < 0) return false;
    r = 4 * rb + 2 * (lg % 2) + (k % 8) / 4;
    t = 4 * tb + k % 4;
    mult = rb == tb ? 1 : 2;
    return true;
  }
  const int u = 32 * (kb - nq_kblocks(d)) + k;
  if (u >= d) return false;
  r = u;
  t = d;
  mult = 1;
  return true;
}

// Packed (library ABI) feature index of (r, t): t == d is the linear term r;
// otherwise the pair min(r,t) <= max(r,t) in row-major upper-triangle order.
__host__ __device__ inline long abi_index(int d, int r, int t) {
  if (t == d) return 1 + r;
  if (r > t) {
    const int x = r;
    r = t;
    t = x;
  }
  const long before = (long)r * d - (long)r * (r - 1) / 2;
  return 1 + d + before + (t - r);
}

// Compile-time table of kfeature over all K-block positions:
// r | t << 7 | mult << 14, or kPadFeature for padding.
constexpr unsigned short kPadFeature = 0xffff;
template <int D>
struct KPosTable {
  unsigned short e[n_kblocks(D) * 32];
};
template <int D>
constexpr KPosTable<D> make_kpos_table() {
  KPosTable<D> tab{};
  for (int kb = 0; kb < n_kblocks(D); ++kb)
    for (int k = 0; k < 32; ++k) {
      int r = 0, t = 0, m = 0;
      tab.e[kb * 32 + k] =
          kfeature(D, kb, k, r, t, m) ? (unsigned short)(r | (t << 7) | (m << 14)) : kPadFeature;
    }
  return tab;
}

// Accumulator row rho (0..15) of scan M-tile m (0, 1) -> K-block position.
__host__ __device__ constexpr int acc_position(int m, int rho) { return 8 * (rho / 4) + 4 * m + rho % 4; }

}  // namespace oal
