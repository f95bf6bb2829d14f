/*
 * oal.h -- C ABI of the MI355X (gfx950) library for causal OAL attention.
 *
 * OAL ("Not All Dimensions Are Equal: Outlier-Aware Attention Linearization
 * with Grouped Quadratic Kernels", arXiv 2610.13674) replaces the softmax
 * kernel by a grouped quadratic kernel.  For a query q and key k of dimension
 * d_h, with x_r = q_r k_r / sqrt(d_h) (paper, sec. 4.1) and the group sums
 * s_g = sum_{r in group g} x_r (sec. 4.2):
 *
 *     kappa(q, k) = a + sum_g b_g s_g + sum_{g,h} c_gh s_g s_h
 *
 * (the dimension-aware kernel of the paper's Eq. (3) with b_r = b_g(r) and
 * C_rt = c_g(r)g(t), the coefficient sharing of the discussion slides'
 * "A squared quadratic form guarantees positive weights").  The causal output
 * is y_i = sum_{j<=i} kappa(q_i,k_j) v_j / sum_{j<=i} kappa(q_i,k_j) (paper,
 * sec. 2, linear attention; the causal pair set of Eq. (2) includes j = i),
 * evaluated in linear time through the prefix states of Eq. (5) and the
 * readout of Eq. (6).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a caller-owned DEVICE pointer unless stated
 *    otherwise.  The library never allocates, frees or synchronises (the one
 *    exception, oal_calibrate, synchronises its stream and says so), keeps no
 *    global mutable state and is safe to call from several host threads.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *    and is complete when that stream is synchronised.
 *  - Activations are contiguous row-major: q [B, Hq, N, d_h], k [B, Hkv, N,
 *    d_h], v [B, Hkv, N, d_v], y [B, Hq, N, d_v].  q, k, v and y share the
 *    element type `dtype` (OAL_F32: float; OAL_BF16: bfloat16 bits).
 *    Activations, states and workspaces start on a 16-byte boundary
 *    (OAL_ERR_INVALID_ARG otherwise): the kernels move them in 16-byte
 *    vectors.
 *    Coefficients, pre-map parameters and states are always float32.
 *  - Query head h reads KV head h / (Hq / Hkv) (GQA with consecutive query
 *    heads per KV head; the paper's App. B uses the model's native map).
 *  - Coefficients (device): group_of_dim [Hq, d_h] int32 in [0, G);
 *    a [Hq]; b [Hq, G]; c [Hq, G, G].  Only the symmetric part of c enters
 *    the kernel, exactly as in the sum over ordered pairs (g, h).  A group id
 *    outside [0, G) cannot be detected on the host from device memory: the
 *    kernels then write NaN to every output of that query head.  Callers that
 *    hold host copies can check them first with oal_check_coeffs().
 *  - State layout (per (batch, KV head), float32, `oal_state_floats` floats):
 *    H [D][d_v] followed by z [D], with D = 1 + d_h + d_h(d_h+1)/2 features in
 *    the order: 0 = constant, 1 + r = linear term r, then the pairs r <= t in
 *    row-major upper-triangle order.  Entries are the raw moments of Eq. (5):
 *    H[f][l] = sum_j phi_f(k_j) v_jl and z[f] = sum_j phi_f(k_j), with
 *    phi = [1, k_r, k_r k_t]; the packed count is the one of the paper's
 *    App. D (139,425 floats at d_h = d_v = 64).  The dimension-wise form
 *    (oal_coeffs.diagonal) has the features [1, k_r, k_r^2] only: its calls
 *    read and write the rows of those (constant, linear terms, squares) and
 *    leave the rows of the pairs r < t as the buffer holds them.
 *  - Supported shapes: d_h in {16, 32, 64}; d_v = 64; prefill: 1 <= G <= 8
 *    with any group map, or any G <= d_h in the dimension-wise form
 *    (oal_coeffs.diagonal); decode and chi: any G <= d_h.  Others return
 *    OAL_ERR_UNSUPPORTED.
 *  - Every call returns a status; no exception or abort crosses the ABI.
 *    Arguments are validated on the host before anything is enqueued.  A
 *    zero-length batch or sequence is valid and enqueues nothing.
 *  - A denominator <= 0 (possible only when [[a, b^T/2], [b/2, c]] is not
 *    positive semidefinite) is not trapped: it yields +-Inf or NaN outputs.
 */
#ifndef OAL_H
#define OAL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OAL_OK = 0,
  OAL_ERR_INVALID_ARG = -1, /* bad dimension, null pointer, Hq % Hkv != 0 ... */
  OAL_ERR_UNSUPPORTED = -2, /* valid but not implemented (d_h, d_v, G) */
  OAL_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  OAL_ERR_HIP = -4          /* a HIP launch failed */
};

enum { OAL_F32 = 0, OAL_BF16 = 1 };

typedef struct oal_dims {
  int32_t batch;      /* B (prefill, decode: sequences; contrib: prompts P) */
  int32_t n_q_heads;  /* Hq */
  int32_t n_kv_heads; /* Hkv, divides Hq */
  int32_t seq_len;    /* N (prefill and contrib; ignored by decode) */
  int32_t d_h;        /* query/key head dimension */
  int32_t d_v;        /* value head dimension */
  int32_t n_groups;   /* G */
  int32_t dtype;      /* OAL_F32 or OAL_BF16 */
} oal_dims;

/* Grouped kernel coefficients, all device pointers (see conventions).
 *
 * diagonal != 0 selects the dimension-wise form
 *     kappa = a + sum_r b_g(r) x_r + sum_r c_g(r)g(r) x_r^2,
 * which is the grouped kernel when every group holds one dimension and c is
 * diagonal (the ReBased feature map read as an elementwise square, "Linear
 * Transformers with Learnable Kernel Functions", section on the learnable
 * parabola); off-diagonal entries of c are then ignored and any G <= d_h is
 * accepted.  Its features are [1, k_r, k_r^2] (1 + 2 d_h of them); oal_fwd
 * and oal_decode_step read and write only the constant, linear and
 * squared-dimension entries of a state (the other entries of state_out are
 * not written).  Prefill of this form needs Hq / Hkv <= 8 and runs as one
 * oal_fwd call; the two-stage calls oal_fwd_states / oal_fwd_outputs do not
 * support it. */
typedef struct oal_coeffs {
  const int32_t* group_of_dim; /* [Hq, d_h] */
  const float* a;              /* [Hq] */
  const float* b;              /* [Hq, G] */
  const float* c;              /* [Hq, G, G] */
  int32_t diagonal;            /* 0: grouped kernel; nonzero: dimension-wise form */
} oal_coeffs;

/* Optional pre-map x -> gamma * norm(x) + beta applied to q and k before
 * the kernel, per head over d_h.  norm is chosen by `kind`:
 *  OAL_PREMAP_LAYERNORM (0): LayerNorm with the mean and biased variance and
 *    no affine of its own, eps added to the variance -- the ReBased map
 *    ("Linear Transformers with Learnable Kernel Functions", section on
 *    letting training place the parabola);
 *  OAL_PREMAP_L2 (1): x / sqrt(sum_r x_r^2 + eps), the unit vector -- the
 *    TaylorShift-style map ("Not All Dimensions Are Equal...", App. F.1,
 *    the TaylorShift baseline: with gamma = tau sqrt(d_h) on queries,
 *    gamma = 1 on keys, beta = 0 and a = 1, b = 1, c = 1/2 the kernel is
 *    1 + s + s^2/2 of s = tau qhat . khat).
 * Device pointers; pass NULL for the whole struct to disable.  Any other
 * kind: OAL_ERR_INVALID_ARG. */
#define OAL_PREMAP_LAYERNORM 0
#define OAL_PREMAP_L2 1
typedef struct oal_prep {
  const float* gamma_q; /* [Hq, d_h] */
  const float* beta_q;  /* [Hq, d_h] */
  const float* gamma_k; /* [Hkv, d_h] */
  const float* beta_k;  /* [Hkv, d_h] */
  float ln_eps;         /* added inside the root, e.g. 1e-5 */
  int32_t kind;         /* OAL_PREMAP_LAYERNORM or OAL_PREMAP_L2 */
} oal_prep;

/* Library version string. */
const char* oal_version(void);

/* Human-readable name of a status code. */
const char* oal_status_str(int status);

/* Packed feature count D = 1 + d_h + d_h(d_h+1)/2 (paper, App. D). */
int64_t oal_feature_count(int32_t d_h);

/* Floats per state block: D * (d_v + 1). */
int64_t oal_state_floats(int32_t d_h, int32_t d_v);

/* Host helper: maps the factor of the positive group-aware kernel to its
 * coefficients (paper, sec. 4.3, Eq. (7): kappa = eps + sbar^T L L^T sbar with
 * sbar = [1, s_1..s_G]; mapping of the discussion slides: with M = L L^T,
 * a = eps + M_00, b_g = 2 M_0g, c_gh = M_gh).  HOST pointers: L [H, G+1, G+1]
 * row-major (only the lower triangle is read); outputs a [H], b [H, G],
 * c [H, G, G].  Computed in double, stored as float. */
int oal_coeffs_from_factor(int32_t n_heads, int32_t n_groups, double eps, const double* L,
                           float* a, float* b, float* c);

/* Host helper: checks HOST copies of a group map [Hq, d_h] (every id in
 * [0, G)) and, when c is non-NULL, that c [Hq, G, G] is finite.  Returns
 * OAL_OK or OAL_ERR_INVALID_ARG. */
int oal_check_coeffs(const oal_dims* dims, const int32_t* group_of_dim_host, const float* c_host);

/* Bytes of device workspace oal_fwd needs for `dims` (0 if invalid), for
 * any coefficients; also what oal_fwd_states / oal_fwd_outputs need. */
size_t oal_fwd_workspace_bytes(const oal_dims* dims);

/* Bytes of device workspace that let oal_fwd run at full parallelism with
 * coefficients of this kind (only coeffs->diagonal is read; the pointers in
 * *coeffs are not touched).  0 if invalid, or if none is needed.
 *
 * The small feature space of the dimension-wise form (1 + 2 d_h features,
 * Hq / Hkv <= 8) is prefilled by oal_fwd in one pass that keeps each prefix
 * state on chip and cuts every sequence into segments; the workspace holds
 * per-segment sums (an F x 65 fp32 block per segment and batch x KV head).
 * There oal_fwd accepts any workspace, including none: a smaller one only
 * means fewer segments (the results are the same up to fp32 rounding
 * order).
 *
 * The grouped form at d_h = 16 with bf16 activations (G <= 8, Hq / Hkv <= 8)
 * is prefilled the same way, with the whole state (153 packed features x
 * (d_v + 1), App. D) held in MFMA accumulators; its workspace holds the
 * per-block sums (a 160 x 65 fp32 block per block of chunks and batch x KV
 * head) and again may be of any size, including none.  For every other case
 * the figure is oal_fwd_workspace_bytes(dims). */
size_t oal_fwd_workspace_bytes_for(const oal_dims* dims, const oal_coeffs* coeffs);

/* Causal prefill (paper, Eqs. (5)-(6), evaluated chunk by chunk).
 *   q, k, v, y: activations (see conventions); y is written for all N rows.
 *   coeffs:     device coefficients; prep: NULL or the ReBased pre-map.
 *   state_in:   NULL (start from zero) or [B, Hkv, oal_state_floats] initial
 *               states, so that a call continues an earlier prefix.
 *   state_out:  NULL or [B, Hkv, oal_state_floats]; receives the states after
 *               the last token (may not alias state_in).
 *   workspace:  device scratch of at least oal_fwd_workspace_bytes(dims)
 *               (for the dimension-wise form and the grouped form at
 *               d_h = 16 in bf16, any size: see oal_fwd_workspace_bytes_for);
 *               undefined after the call.
 * Calls that share a workspace must be ordered on one stream. */
int oal_fwd(const oal_dims* dims, const void* q, const void* k, const void* v,
            const oal_coeffs* coeffs, const oal_prep* prep, const float* state_in, float* state_out,
            void* y, void* workspace, size_t workspace_bytes, void* stream);

/* Causal prefill of sequences of different lengths in the padded layout
 * ("Not All Dimensions Are Equal...", sec. 3.1, Eq. (2): prompts of length
 * N_p; here the prefill of such a batch): sequence b of q, k, v, y holds
 * seq_lens[b] valid rows (device int32 [batch]; values are clamped to
 * [0, seq_len]) at the start of its seq_len-row slot.
 *   y:         rows below seq_lens[b] as oal_fwd would write them for a
 *              sequence of that length; the other rows are not written.
 *   state_out: the states after seq_lens[b] tokens (state_in, or zero, for
 *              an empty sequence).
 * Heads with their own keys take the one-launch builds (d_h = 16 bf16 and
 * the dimension-wise form at d_h = 64 bf16); the other grouped forms take
 * the chunk path, whose workspace is oal_fwd_workspace_bytes(dims); the
 * dimension-wise form with grouped-query heads returns OAL_ERR_UNSUPPORTED.
 * Workspace: oal_fwd_varlen_workspace_bytes_for(dims, coeffs).  Other
 * arguments and errors as for oal_fwd; seq_lens == NULL:
 * OAL_ERR_INVALID_ARG. */
size_t oal_fwd_varlen_workspace_bytes_for(const oal_dims* dims, const oal_coeffs* coeffs);
int oal_fwd_varlen(const oal_dims* dims, const int32_t* seq_lens, const void* q, const void* k, const void* v,
                   const oal_coeffs* coeffs, const oal_prep* prep, const float* state_in, float* state_out,
                   void* y, void* workspace, size_t workspace_bytes, void* stream);

/* The two stages of oal_fwd, for callers that schedule or time them
 * separately.  oal_fwd(...) is exactly oal_fwd_states(...) followed by
 * oal_fwd_outputs(...) on the same stream with the same workspace (the
 * dimension-wise form has no separate stages).
 *   oal_fwd_states:  the prefix states of Eq. (5) at every chunk start, kept
 *                    in the workspace (and the final state in state_out).
 *   oal_fwd_outputs: the Eq. (6) readout against those states plus the
 *                    within-chunk pairs, normalised into y.  The workspace
 *                    must hold the states of a preceding oal_fwd_states call
 *                    with the same dims, k, v, prep and state_in.  Its
 *                    state_in must be that call's pointer: only whether it
 *                    is null is read (the first chunk then skips the read of
 *                    the initial state), not the memory behind it.
 * Arguments and errors as for oal_fwd. */
int oal_fwd_states(const oal_dims* dims, const void* k, const void* v, const oal_prep* prep,
                   const float* state_in, float* state_out, void* workspace, size_t workspace_bytes,
                   void* stream);
int oal_fwd_outputs(const oal_dims* dims, const void* q, const void* k, const void* v,
                    const oal_coeffs* coeffs, const oal_prep* prep, const float* state_in, void* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of device workspace oal_decode_step needs for `dims` (0 when none
 * is needed or `dims` is invalid). */
size_t oal_decode_workspace_bytes(const oal_dims* dims);

/* One recurrent decode step for `dims->batch` independent sequences (paper,
 * Eqs. (5)-(6) for a single token): state <- state + phi(k) [v, 1]^T, then
 * y = (phi_q(q)^T state)[:d_v] / (phi_q(q)^T state)[d_v].  The new token is
 * part of its own causal prefix.
 *   q [B, Hq, d_h], k [B, Hkv, d_h], v [B, Hkv, d_v], y [B, Hq, d_v];
 *   state [B, Hkv, oal_state_floats], updated in place;
 *   workspace: device scratch of at least oal_decode_workspace_bytes(dims)
 *              (may be NULL when that is 0); contents undefined afterwards.
 * Supports Hq / Hkv <= 8.  Calls that share a workspace or a state must be
 * ordered on one stream. */
int oal_decode_step(const oal_dims* dims, const void* q, const void* k, const void* v,
                    const oal_coeffs* coeffs, const oal_prep* prep, float* state, void* y,
                    void* workspace, size_t workspace_bytes, void* stream);

/* oal_decode_step for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, results and errors as oal_decode_step, without the
 * workspace: its scratch is a 32 MiB device array of the library (one per
 * device that loads it, held until the process ends; its address is looked
 * up once per device, on the first call with that device current).  Nothing
 * is allocated.  Returns OAL_ERR_WORKSPACE when oal_decode_workspace_bytes(dims)
 * exceeds 32 MiB.  Every call on a device uses that device's array, so calls
 * that may overlap on one device (on different streams without ordering,
 * or from several threads) race and must not be made. */
int oal_decode_step_noalloc(const oal_dims* dims, const void* q, const void* k, const void* v,
                            const oal_coeffs* coeffs, const oal_prep* prep, float* state, void* y, void* stream);

/* Bytes of device workspace oal_contrib needs for `dims` (0 if invalid). */
size_t oal_contrib_workspace_bytes(const oal_dims* dims);

/* Per-dimension contribution score (paper, sec. 3.1, Eq. (2)):
 *   chi_{p,r} = mean over causal pairs j <= i < N_p of |q_ir k_jr| / sqrt(d_h),
 *   chi_r     = equal-weight mean of chi_{p,r} over the P = dims->batch prompts.
 *   q [P, Hq, N, d_h], k [P, Hkv, N, d_h] (raw, no pre-map); query head h
 *   pairs with KV head h / (Hq / Hkv).
 *   seq_lens:       NULL (every prompt has N tokens) or DEVICE int32 [P] with
 *                   1 <= N_p <= N; rows at and beyond N_p are ignored.  A
 *                   length outside that range makes the prompt's scores NaN.
 *   chi_per_prompt: NULL or float [P, Hq, d_h].
 *   chi_mean:       float [Hq, d_h].
 * Uses float accumulation of non-negative terms; deterministic. */
int oal_contrib(const oal_dims* dims, const void* q, const void* k, const int32_t* seq_lens,
                float* chi_per_prompt, float* chi_mean, void* workspace, size_t workspace_bytes,
                void* stream);

/* Bytes of device workspace oal_bwd needs for `dims` (0 if invalid or
 * unsupported). */
size_t oal_bwd_workspace_bytes(const oal_dims* dims);

/* Backward pass of the causal attention of oal_fwd (no pre-map, no initial
 * state): the gradients of L = sum(dy * y) with respect to q, k, v and the
 * coefficients, which the output-matching calibration of the paper (App. B,
 * Eq. (20)) and the joint adaptation of the coefficients (App. F.2) take.
 * With y_i = num_i / den_i (num_i = sum_{j<=i} kappa_ij v_j, den_i =
 * sum_{j<=i} kappa_ij), dkappa_ij = (dy_i . v_j - dy_i . y_i) / den_i for
 * j <= i, and the chain rule through kappa (header comment) gives
 *   dq_i = sum_j dkappa_ij dkappa/dq_i,  dk_j = sum_i dkappa_ij dkappa/dk_j,
 *   dv_j = sum_{i>=j} kappa_ij dy_i / den_i,
 *   da = sum dkappa,  db_g = sum dkappa s_g,  dc_gh = sum dkappa s_g s_h.
 *   q, k [B, H, N, d_h], v, dy [B, H, N, d_v] in `dtype` (the same for all
 *   four); dq, dk [B, H, N, d_h], dv [B, H, N, d_v] float32, overwritten;
 *   da [H], db [H, G], dc [H, G, G] float32, summed over the batch and
 *   overwritten (zeros when B or N is 0: the one case where a zero-length
 *   call still enqueues work).
 *   workspace: at least oal_bwd_workspace_bytes(dims) (the recomputed
 *              dL/d[num, den] rows and per-sequence coefficient sums);
 *              contents undefined afterwards.
 * Supports d_h = 16, d_v = 64, heads with their own keys (Hq == Hkv), any
 * G <= 16, the grouped kernel (coeffs->diagonal == 0); others return
 * OAL_ERR_UNSUPPORTED.  Recomputes the forward pass in float32; the result is
 * deterministic.  Calls that share a workspace must be ordered on one
 * stream. */
int oal_bwd(const oal_dims* dims, const void* q, const void* k, const void* v, const void* dy,
            const oal_coeffs* coeffs, float* dq, float* dk, float* dv, float* da, float* db, float* dc,
            void* workspace, size_t workspace_bytes, void* stream);

/* Settings of the output-matching calibration (paper, App. B,
 * "Coefficient-calibration settings": Adam at lr 0.02, gradient norm clipped
 * at 10, 32 causal query positions per update, validation every 100 updates,
 * early stop after 400 updates without improvement). */
typedef struct oal_calib_params {
  double lr;              /* Adam learning rate (betas 0.9, 0.999, epsilon 1e-8) */
  double clip;            /* per-head gradient norm bound (> 0) */
  double eps;             /* the kernel's epsilon of Eq. (7): a = eps + M_00 */
  int32_t n_positions;    /* P: sampled query positions per update (1..N) */
  int32_t validate_every; /* updates between validations (>= 1) */
  int32_t patience;       /* a head stops after this many updates without improvement (>= 1) */
} oal_calib_params;

/* Bytes of device workspace oal_calibrate needs (0 if invalid or
 * unsupported); group_of_dim: the device group map the call will use. */
size_t oal_calibrate_workspace_bytes(const oal_dims* dims, int32_t n_val, const int32_t* group_of_dim);

/* Output-matching calibration of the factors L of every head (paper, App. B,
 * Eq. (20): L* minimises the squared error between the normalised OAL
 * outputs and the causal softmax outputs, kappa = eps + sbar^T L L^T sbar as
 * in oal_coeffs_from_factor), by the coefficient-calibration settings.
 * For each initialisation candidate c: starting from inits[c], for update
 * u = 1 .. n_updates the plan row u - 1 names a training sequence s and P
 * distinct positions i_1 .. i_P; each head takes one Adam step on the lower
 * triangle of its factor against the gradient of
 *     (1/P) sum_p || yhat_{i_p}(L; s) - y^softmax_{i_p}(s) ||^2,
 * its norm first scaled down to clip when larger.  Validation (whole
 * sequences, before the first update and every validate_every updates)
 * gives each head's MSE = mean over validation sequences of
 * ||Yhat_b - Y_b||_F^2 / n_b (n_b = N d_v scalar outputs) and RelMSE = mean
 * of ||Yhat_b - Y_b||_F^2 / ||Y_b||_F^2; a head keeps its lowest-MSE
 * checkpoint and stops updating once that is patience updates old.  Finally
 * every head takes the candidate with the lowest checkpoint MSE.  Heads are
 * independent problems (their own clipping, stopping and selection).
 *   dims:     batch = T training sequences of seq_len N; heads with their own
 *             keys; d_h, d_v, G, dtype as oal_bwd supports them (d_h = 16,
 *             d_v = 64, G <= 16; otherwise OAL_ERR_UNSUPPORTED).
 *   q/k/v_train [T, H, N, d], q/k/v_val [n_val, H, N, d]: device, dtype.
 *   group_of_dim: device [H, d_h] (ids in [0, G)).
 *   inits:    HOST double [n_init, H, G+1, G+1] (lower triangles read).
 *   plan:     HOST int32 [n_updates, 1 + P]: sequence in [0, T), then P
 *             distinct positions in [0, N) (OAL_ERR_INVALID_ARG otherwise).
 *   outputs (HOST): L_out [H, G+1, G+1] (upper triangle zero), mse_out and
 *             relmse_out [H] of the chosen checkpoints, init_out [H] the
 *             chosen candidates; optional (NULL to skip) cand_mse_out
 *             [n_init, H] and updates_out [n_init, H] (updates each head
 *             ran).
 *   workspace: oal_calibrate_workspace_bytes(dims, n_val, group_of_dim).
 * The optimiser runs on the host in fp32; the targets, forward and backward
 * passes on the device.  Unlike the other entry points this call is
 * synchronous: it synchronises `stream` after every update and validation
 * (its next step depends on the gradients), and returns when it is done. */
int oal_calibrate(const oal_dims* dims, const void* q_train, const void* k_train, const void* v_train, int32_t n_val,
                  const void* q_val, const void* k_val, const void* v_val, const int32_t* group_of_dim,
                  int32_t n_init, const double* inits, int32_t n_updates, const int32_t* plan,
                  const oal_calib_params* params, double* L_out, double* mse_out, double* relmse_out,
                  int32_t* init_out, double* cand_mse_out, int32_t* updates_out, void* workspace,
                  size_t workspace_bytes, void* stream);

/* ---- dimension grouping (host functions; every pointer below is HOST) ---- */

/* Settings of the outlier-aware grouping (paper, App. B, "Grouping
 * settings"): tail fraction alpha, minimum bootstrap support gamma, gap
 * threshold tau (1.5 in the paper), division guard eps (> 0), and the
 * minimum group count g_min (2 in the paper). */
typedef struct oal_group_params {
  double alpha;
  double gamma;
  double tau;
  double eps;
  int32_t g_min;
} oal_group_params;

/* Outlier-aware grouping of one query head's dimensions (paper, App. B,
 * "Dimension grouping"; the bootstrap separation R_k^(b) as defined on the
 * discussion deck's backup slide on bootstrap support).
 *   chi_pp [P, d_h]: per-prompt contribution scores chi_{p,r} (>= 0, finite),
 *                    e.g. one head's rows of oal_contrib's chi_per_prompt.
 *   boot [B, P]:     prompt indices in [0, P) of B >= 1 bootstrap replicates,
 *                    drawn by the caller with replacement (repeats count).
 *   group_of_dim [d_h] (out): group ids 0..G-1; group 0 is the
 *                    low-contribution bulk, higher ids refine the tail.
 *   rho, support [d_h] (out, each may be NULL): for every candidate cut k
 *                    (entry k), the gap ratio rho_k and the bootstrap
 *                    support S_k; NaN at positions that are not candidates.
 * Steps: chi_r = mean over prompts; stable ascending order pi; candidate
 * cuts k = max(1, d_h - ceil(alpha d_h)) .. d_h - 1 (a cut at k separates
 * sorted positions 1..k from k+1..d_h); rho_k = chi_{pi_{k+1}} /
 * max(chi_{pi_k}, eps); S_k = fraction of replicates whose bootstrap scores
 * (mean over the sampled prompts, pi fixed) keep min(upper) / max(max(lower),
 * eps) >= tau; natural cuts have rho_k >= tau and S_k >= gamma; below g_min
 * groups, unused candidates are added by descending (S_k, rho_k), ties in
 * candidate order.  All arithmetic is fp64 in a fixed order.
 * Returns G >= 1, or OAL_ERR_INVALID_ARG. */
int oal_group_dims(int32_t d_h, int32_t P, const float* chi_pp, int32_t B, const int32_t* boot,
                   const oal_group_params* params, int32_t* group_of_dim, double* rho, double* support);

/* Fixed-budget grouping (paper, App. B, "Group-budget diagnostic"): the
 * n_groups - 1 largest adjacent gaps rho_k (k = 1..d_h-1, as above) of the
 * stably sorted profile chi [d_h] become the boundaries; equal gaps are taken
 * in cut order.  group_of_dim [d_h] (out) as above; 1 <= n_groups <= d_h.
 * Returns n_groups, or OAL_ERR_INVALID_ARG. */
int oal_group_dims_budget(int32_t d_h, const float* chi, int32_t n_groups, double eps, int32_t* group_of_dim);

#ifdef __cplusplus
}
#endif

#endif /* OAL_H */
