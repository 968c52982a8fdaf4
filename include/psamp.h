/*
 * psamp.h -- C ABI of libpsamp: proportional (prioritized-replay) sampling
 * on AMD Instinct MI355X (gfx950).
 *
 * Every array argument is a DEVICE pointer owned by the caller.  Every call
 * validates its arguments on the host, enqueues its kernels on `stream` (a
 * hipStream_t passed as void*; NULL means the null stream) and returns
 * without synchronising.  On a validation error nothing is enqueued and no
 * output is touched.  No call allocates, frees or memsets device memory, or
 * changes the current device: scratch space ("workspace") comes from the
 * caller, sized by the matching *_workspace_size() query, and must be
 * zero-filled once after it is allocated; after that the library keeps it
 * consistent by itself (no per-call reset).  A workspace must not be used by
 * two calls that can run at the same time.
 *
 * Preconditions that cannot be checked without a device sync (priorities
 * finite and >= 0 with at least one > 0, indices in range, threshold
 * fractions in [0, 1)) are the caller's; breaking them yields unspecified
 * values but never an out-of-bounds access or a hang: every index is clamped
 * and every cross-workgroup wait is bounded (a timed-out wait sets a bit that
 * psamp_workspace_errors() reports).
 *
 * Sources (page title, then section):
 *   [PR615] "trainer: parallel build_cdf scan + tiled (bitwise-identical)
 *           mingru backward" -- "1. Parallel build_cdf".
 *   [SEGT]  "GPU Segment Tree for PER Sampling" -- "Tree Layout",
 *           "Operations", "CUDA Kernels", "Memory", "Integration with
 *           GpuReplayBuffer", "Non-Goals".
 *   [PF]    POPCORNBENCH particle-filter trace (Kimi-K2.6, l2_p48) -- the
 *           reference model's resampling step.
 *   [PER]   prioritized experience replay as named in [SEGT] "Non-Goals":
 *           P(i) = p_i^alpha / sum_j p_j^alpha, IS_i = (N P(i))^-beta / max.
 */
#ifndef PSAMP_H
#define PSAMP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PSAMP_OK = 0,
    PSAMP_E_NULL = 1,        /* a required pointer is NULL                  */
    PSAMP_E_SIZE = 2,        /* a size is out of range                      */
    PSAMP_E_DTYPE = 3,       /* unsupported dtype or dtype pair             */
    PSAMP_E_PARAM = 4,       /* alpha / beta / flags out of range           */
    PSAMP_E_WORKSPACE = 5,   /* workspace missing or too small              */
    PSAMP_E_ALIGN = 6,       /* pointer not aligned to its element size     */
    PSAMP_E_LAUNCH = 7,      /* the HIP runtime rejected a kernel launch    */
    PSAMP_E_UNSUPPORTED = 8  /* valid request this build does not support   */
} psamp_status;

typedef enum {
    PSAMP_F32 = 0,
    PSAMP_F64 = 1,
    PSAMP_U32 = 2,
    PSAMP_U64 = 3,
    PSAMP_I32 = 4
} psamp_dtype;

/* Human-readable name of a status code (static string, never NULL). */
const char* psamp_status_string(psamp_status s);
/* Version of this ABI; bumped on any incompatible change. */
int psamp_abi_version(void);

/* ------------------------------------------------------------------------
 * (1) p^alpha and the inclusive CDF.  [PR615] "1. Parallel build_cdf": the
 * CDF of the B priorities, C_i = sum_{j<=i} w_j, one pass per update; [PER]
 * w_i = p_i^alpha.  Single pass over the input (no size limit beyond n).
 *
 *   prio   : n priorities, PSAMP_F32 (fp mode) or PSAMP_U32 (integer mode).
 *   alpha  : exponent (fp mode, finite, > 0); ignored in integer mode, where
 *            w_i = q_i so that every sum is exact.
 *   cdf    : n outputs.  fp mode: PSAMP_F64 (weights and sums in double) or
 *            PSAMP_F32 (same double arithmetic, stored as float).  Integer
 *            mode: PSAMP_U64, exact.
 *   total  : 1 element of cdf_t, receives C_{n-1} (bit-equal to it).  Stays
 *            on the device; psamp_sample reads it there.
 *   n      : 1 <= n <= 2^31 - 1 (integer mode: n <= 2^31 - 1 keeps T < 2^63).
 *   ws     : workspace of psamp_build_cdf_workspace_size(n_max) bytes, where
 *            n_max is the largest n ever used with it; pass the same ws_bytes
 *            on every call that shares it (256 B + 4 KiB per 65536 elements).
 * fp mode is deterministic run to run (fixed association); integer mode is
 * exact.  Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM, E_WORKSPACE, E_ALIGN
 * (prio 4-byte, cdf/total element-aligned), E_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t psamp_build_cdf_workspace_size(int64_t n);
psamp_status psamp_build_cdf(const void* prio, psamp_dtype prio_t, int64_t n,
                             double alpha, void* cdf, psamp_dtype cdf_t,
                             void* total, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * (2a) Thresholds and search.  Sample i gets the threshold
 *   stratified: t_i = ((i + U_i) / k) * T        (fp64: one rounding each
 *                                                  for / and *)
 *   iid:        t_i = U_i * T
 * and the index idx_i = min(first j with C_j >= t_i, n - 1) -- [PF]
 * searchsorted with right=False, then clamp to n-1.
 *   cdf, total : from psamp_build_cdf (PSAMP_F64, PSAMP_F32 or PSAMP_U64),
 *                or any non-decreasing CDF with total = its last value
 *                (device memory; for a CDF that decreases somewhere every
 *                index is still written, in [0, n), but unspecified).
 *   u          : k fractions.  fp CDF: PSAMP_F32 values in [0,1).  Integer
 *                CDF: PSAMP_U32 values r_i (U_i = r_i / 2^32), and
 *                  stratified: t_i = floor(((i 2^32 + r_i) T) / (k 2^32)) + 1
 *                  iid:        t_i = floor((r_i T) / 2^32) + 1
 *                computed exactly, so integer mode is bit-exact.
 *   out_idx    : k int32 indices (non-decreasing in i when stratified).
 *   k          : 0 <= k <= 2^31 - 1 (0 is a no-op).
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM (stratified not 0/1), E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
psamp_status psamp_sample(const void* cdf, psamp_dtype cdf_t, int64_t n,
                          const void* total, const void* u, psamp_dtype u_t,
                          int64_t k, int stratified, int32_t* out_idx, void* stream);

/* ------------------------------------------------------------------------
 * (2c) Fused CDF scan + stratified sample: psamp_build_cdf followed by
 * psamp_sample(stratified = 1), with the same CDF, T and indices bit for bit,
 * in two passes that never read the CDF back: a pass of tile sums gives
 * every tile its prefix and T up front, and each tile of the scan then draws
 * its own samples (stratified thresholds are non-decreasing, and tile j owns
 * exactly those in (C at the end of tile j-1, C at its own end]).
 * [PR615] "1. Parallel build_cdf" with [PF] searchsorted.
 *   Arguments as psamp_build_cdf and psamp_sample; ws as psamp_build_cdf
 *   (the same workspace may serve both).  cdf_t PSAMP_F64 or PSAMP_U64 is
 *   fused up to n = 2^20 and, above, when the draws are sparse (64 k < n);
 *   above 2^20 with dense draws the call runs the two kernels of the two
 *   calls (the scan, then the sampler that reads the CDF once from its
 *   side), which is faster there than drawing inside the scan's tiles.
 *   PSAMP_F32 (whose rounding breaks the tiles' ownership of the
 *   thresholds) and k = 0 also run the two calls.  The results are the
 *   same bits on every path.
 * Errors: those of psamp_build_cdf and psamp_sample.
 * ---------------------------------------------------------------------- */
psamp_status psamp_build_cdf_sample(const void* prio, psamp_dtype prio_t, int64_t n,
                                    double alpha, const void* u, psamp_dtype u_t, int64_t k,
                                    void* cdf, psamp_dtype cdf_t, void* total,
                                    int32_t* out_idx, void* ws, size_t ws_bytes,
                                    void* stream);

/* ------------------------------------------------------------------------
 * (2b) Importance-sampling weights.  [PER]: P_i = w_{idx_i} / T,
 * v_i = (N P_i)^-beta, IS_i = v_i / max_j v_j over the k sampled entries.
 * N and T cancel, so the kernel evaluates the equal closed form
 * IS_i = (w_min / w_i)^beta = (p_min / p_i)^(alpha beta) (fp mode) or
 * (q_min / q_i)^beta (integer mode), with w_min the smallest sampled weight.
 *   prio   : the n priorities the CDF was built from (F32 or U32).
 *   idx    : k indices from psamp_sample (clamped into [0, n) on use).
 *   out_w  : k float weights in (0, 1]; the largest is exactly 1.  Must not
 *            overlap prio (the gathered priorities are parked there).
 *   ws     : psamp_is_weights_workspace_size(k) bytes (256 B up to 8192
 *            samples; above, 8448 B plus 4 B per 4096 samples; 0 for
 *            k = 0), zero-filled once after allocation; the calls keep it
 *            consistent, whatever sizes share it.  One ws must not serve two
 *            calls that may run at the same time.  One kernel whose blocks
 *            wait for one another's minima serves up to 8192 samples (at
 *            most 8 blocks of 1024) and, above, as long as its blocks of
 *            4096 samples (at most 1024) can all be resident on the device
 *            at once; larger batches take two kernels.  A wait that does not
 *            end within about a second (blocks kept from running by other
 *            work on the device) sets bit 0 of the workspace errors
 *            (psamp_workspace_errors) instead of hanging.
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM (beta < 0 or not finite,
 * alpha <= 0), E_WORKSPACE, E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
size_t psamp_is_weights_workspace_size(int64_t k);
psamp_status psamp_is_weights(const void* prio, psamp_dtype prio_t, int64_t n,
                              double alpha, const int32_t* idx, int64_t k,
                              double beta, float* out_w, void* ws, size_t ws_bytes,
                              void* stream);

/* ------------------------------------------------------------------------
 * (3) Sum tree, in the flat layout of [SEGT] "Tree Layout": an array of
 * 2*cap_pow2 nodes, index 0 unused, root at 1, children of j at 2j and
 * 2j+1, leaf i at cap_pow2 + i; every internal node is the sum of its two
 * children, recomputed as fl(left + right) ([SEGT] "Operations -- Update").
 * tree_t is PSAMP_F32 (leaves p^alpha rounded to float, sums in float, as
 * on the page) or PSAMP_U64 (leaves q from U32 priorities, exact sums).
 * Leaves n_valid .. cap_pow2-1 are 0.  Memory: 2 * cap_pow2 * sizeof(node);
 * the tree pointer must be 16-byte aligned (E_ALIGN otherwise), priorities
 * and index arrays 4-byte aligned.
 * ---------------------------------------------------------------------- */
/* Capacity rounded up to a power of two ([SEGT] "Tree Layout"); 0 if
 * capacity < 1 or the result would exceed 2^30. */
int64_t psamp_segtree_cap_pow2(int64_t capacity);

/* Build every node from n_valid priorities (0 < n_valid <= cap_pow2 <= 2^30).
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM, E_ALIGN, E_LAUNCH. */
psamp_status psamp_segtree_build(void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                 const void* prio, psamp_dtype prio_t, int64_t n_valid,
                                 double alpha, void* stream);

/* Batched update ([SEGT] "Operations -- Update"): leaf idx_j <- prio_j^alpha
 * for j = 0..m-1; when an index repeats, the entry with the largest j wins
 * (as if the updates were applied one by one in batch order); every
 * ancestor of a changed leaf is recomputed exactly once, after both of its
 * children are final, so the tree stays bit-equal to a fresh build of its
 * leaves.  Entries with idx_j outside [0, cap_pow2) are ignored.  An
 * entry in [n_valid, cap_pow2) -- n_valid being the count later passed to
 * psamp_segtree_sample -- writes a padding leaf: its mass stays in every
 * sum above it, and a descent that ends on it is clamped to n_valid - 1, so
 * callers keep idx_j below n_valid.  0 <= m <= 2^31 - 1 (m = 0 is a no-op
 * and may pass NULL pointers); the batch is processed in order, in chunks
 * of 1024 entries, so later entries still win over earlier ones.  Each
 * chunk runs as 64 workgroups, one per subtree below the top 6 levels;
 * each publishes its subtree's root in ws and workgroup 0 recomputes those
 * levels from them (its wait is bounded, about a second: should other work
 * keep the other workgroups from starting that long, the top levels are
 * left wrong and ws is not left zero).
 * ws: psamp_segtree_update_workspace_size(cap_pow2, m) bytes (512), 8-byte
 *   aligned, zero-filled once after allocation (every call leaves it zero
 *   again); one ws must not serve two updates that may run at the same time.
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM, E_WORKSPACE, E_ALIGN, E_LAUNCH. */
size_t psamp_segtree_update_workspace_size(int64_t cap_pow2, int64_t m);
psamp_status psamp_segtree_update(void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                  const int32_t* idx, const void* prio,
                                  psamp_dtype prio_t, int64_t m, double alpha,
                                  void* ws, size_t ws_bytes, void* stream);

/* Root-to-leaf descent ([SEGT] "Operations -- Sample"): at each node go left
 * if t <= left sum (or if the right sum is 0), else t -= left sum and go
 * right; the result is clamped to n_valid - 1.  Thresholds: F32 tree --
 * iid t = U_i * root (float), stratified t = (float)(((i + U_i) / k) * root)
 * (double); U64 tree -- the integer formulas of psamp_sample with U32 r_i.
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM, E_ALIGN, E_LAUNCH. */
psamp_status psamp_segtree_sample(const void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                  int64_t n_valid, const void* u, psamp_dtype u_t,
                                  int64_t k, int stratified, int32_t* out_idx, void* stream);

/* ------------------------------------------------------------------------
 * (3b) Replay priorities on the sum tree ([SEGT] "Integration with
 * GpuReplayBuffer": insert_batch writes the new priorities and updates the
 * tree at the inserted slots, update_priorities is the tree's batched
 * update, sample_proportional is the descent, total_priority is the root).
 * A ring of `capacity` slots: insert writes slots cursor, cursor+1, ...
 * (mod capacity) in batch order; the filled slots are [0, size).  The tree
 * is F32 (leaf = p^alpha rounded to float), 2 * cap_pow2 floats of device
 * memory, zero-filled by the caller before psamp_replay_init.  The struct is
 * host memory owned by the caller; insert advances cursor and size when it
 * enqueues.  ws: psamp_replay_workspace_size(capacity, largest batch) bytes
 * of device memory, zero-filled once: the tree update's workspace, then the
 * IS weights'.
 * Calls are stream-ordered like the rest of the library; two streams must
 * not use one psamp_replay at the same time.
 * ---------------------------------------------------------------------- */
typedef struct {
    int64_t capacity;   /* slots in the ring                              */
    int64_t cap_pow2;   /* psamp_segtree_cap_pow2(capacity)               */
    int64_t cursor;     /* next slot an insert writes, in [0, capacity)   */
    int64_t size;       /* filled slots, in [0, capacity]                 */
    double alpha;       /* leaf = p^alpha                                 */
    float* tree;        /* device, 2 * cap_pow2 floats                    */
    void* ws;           /* device workspace                               */
    size_t ws_bytes;
} psamp_replay;

size_t psamp_replay_workspace_size(int64_t capacity, int64_t max_batch);
/* Fills *rb for an empty ring.  Errors: E_NULL, E_SIZE (capacity < 1 or
 * over 2^30), E_PARAM (alpha <= 0 or not finite), E_ALIGN (tree not 16-byte aligned). */
psamp_status psamp_replay_init(psamp_replay* rb, int64_t capacity, double alpha, float* tree,
                               void* ws, size_t ws_bytes);
/* insert_batch: out_slots[i] = (cursor + i) mod capacity, leaf of that slot
 * <- prio[i]^alpha (a slot written twice in one batch keeps the later
 * value), then cursor += m (mod capacity), size = min(size + m, capacity).
 * prio: m floats >= 0.  out_slots: m int32 (device), required: the caller
 * stores its items there.  Errors: E_NULL, E_SIZE, E_PARAM (bad *rb),
 * E_ALIGN, E_WORKSPACE, E_LAUNCH. */
psamp_status psamp_replay_insert(psamp_replay* rb, const float* prio, int64_t m,
                                 int32_t* out_slots, void* stream);
/* update_priorities: leaf of slots[j] <- prio[j]^alpha, later j winning on
 * repeats.  Slots must be filled ones ([0, size)); others are ignored when
 * outside [0, cap_pow2).  Errors: as insert. */
psamp_status psamp_replay_update(psamp_replay* rb, const int32_t* slots, const float* prio,
                                 int64_t m, void* stream);
/* sample_proportional: k descents over the filled slots with the thresholds
 * of psamp_segtree_sample (F32 tree; stratified 0 or 1), and, when out_w is
 * not NULL, the IS weights of psamp_is_weights on the leaves:
 * (L_min / L_i)^beta = (N P_i)^-beta / max over the batch.
 * Errors: E_NULL, E_SIZE (empty ring), E_PARAM, E_WORKSPACE, E_LAUNCH. */
psamp_status psamp_replay_sample(const psamp_replay* rb, const float* u, int64_t k,
                                 int stratified, double beta, int32_t* out_slots, float* out_w,
                                 void* stream);
/* total_priority: the device address of the root (the sum of all leaves);
 * NULL if rb or its tree is NULL. */
const float* psamp_replay_total(const psamp_replay* rb);

/* ------------------------------------------------------------------------
 * (4) Row-batched systematic resampling ([PF], the reference model's
 * resampling step).  Per row b of P float log-weights:
 *   lse  = m + log(sum_j exp(lw_j - m)),  m = max_j lw_j
 *   W_j  = exp(lw_j - lse),  C = inclusive cumsum of W   (double)
 *   u_k  = (k + u_row[b]) / P                           (float arithmetic)
 *   anc_k = min(first j with C_j >= u_k, P - 1)
 *   logw   : rows x P floats, row stride ld_in elements (>= P).
 *   u_row  : rows floats in [0, 1).
 *   out_anc: rows x P int32, row stride ld_out elements (>= P).
 *   1 <= P <= 8192, 1 <= rows <= 2^31 - 1.
 *   A -inf log-weight weighs 0.  A NaN or +inf one breaks the precondition
 *   (PSAMP_CHECK_LOGWEIGHT when checks are on); the ancestors are then
 *   still written and in [0, P), with no other guarantee.
 * Errors: E_NULL, E_SIZE, E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
psamp_status psamp_resample_rows(const float* logw, int64_t rows, int64_t P,
                                 int64_t ld_in, const float* u_row, int32_t* out_anc,
                                 int64_t ld_out, void* stream);

/* ------------------------------------------------------------------------
 * (4b) One particle-filter step, fused ([PF], the reference model's forward
 * pass around its resampling step).  Per filter b of P particles in D
 * dimensions with O observed values:
 *   pred_j  = A x_j + sigma_p eps_j
 *   ll_j    = -0.5 * sum_o (obs_o - (C pred_j)_o)^2 / sigma_o^2
 *   lw'_j   = logw_j + ll_j
 *   anc     = psamp_resample_rows(lw', u_row[b])        (same rule, same bits)
 *   x_out_k = pred_{anc_k},  logw_out_k = (float)(-log P)
 * Up to lw' all arithmetic is float32: each dot product summed in increasing
 * index from +0, the noise term added last, ll = (-0.5 * S) / (sigma_o *
 * sigma_o) with a correctly rounded division.
 *   x, eps, x_out : rows x P x D floats (particle-major, contiguous),
 *                   16-byte aligned.  eps holds standard normal draws.
 *   logw, logw_out: rows x P floats.  obs: rows x O floats.
 *   A: D x D, C: O x D floats, row-major, in device memory.
 *   u_row: rows floats in [0, 1).  anc_out: rows x P int32 or NULL.
 *   x_out may be x and logw_out may be logw (in-place update).
 *   1 <= P <= 8192, D in {1, 2, 4, 8}, P * D <= 16384, 1 <= O <= 8,
 *   1 <= rows <= 2^31 - 1.  sigma_o > 0 and finite, sigma_p finite.
 * Errors: E_NULL, E_SIZE, E_PARAM, E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
psamp_status psamp_pf_step(const float* x, const float* logw, const float* obs,
                           const float* A, const float* C, const float* eps, float sigma_p,
                           float sigma_o, const float* u_row, int64_t rows, int64_t P,
                           int64_t D, int64_t O, float* x_out, float* logw_out,
                           int32_t* anc_out, void* stream);

/* ------------------------------------------------------------------------
 * Priority rewrite (the scatter of [SEGT] "Integration" --
 * update_priorities_gpu): prio[idx_j] = vals_j for j = 0..m-1, the largest
 * j winning on repeated indices; indices outside [0, n) are ignored.
 * prio_t / vals: PSAMP_F32 or PSAMP_U32 (same dtype for both).
 * flags: 0, or PSAMP_SCATTER_GROUPED when equal indices are adjacent in idx
 *   (true of the non-decreasing output of stratified psamp_sample): then one
 *   atomic-free kernel runs and ws may be NULL.  A false promise gives
 *   unspecified (but in-bounds) results.
 * ws: psamp_scatter_workspace_size(n, m) bytes (one uint32 per item, zeroed
 *   once; every call leaves it zeroed again), unless GROUPED.
 * Errors: E_NULL, E_SIZE, E_DTYPE, E_PARAM (unknown flag), E_WORKSPACE,
 * E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
#define PSAMP_SCATTER_GROUPED 1
size_t psamp_scatter_workspace_size(int64_t n, int64_t m);
psamp_status psamp_scatter_lww(void* prio, psamp_dtype prio_t, int64_t n,
                               const int32_t* idx, const void* vals, int64_t m, int flags,
                               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * One prioritized-replay minibatch update, fused: exactly
 *   psamp_build_cdf(prio F32 -> cdf F64, total)
 *   psamp_sample(stratified, u -> out_idx)
 *   psamp_is_weights(-> out_w)
 *   psamp_scatter_lww(prio[out_idx] = new_prio, PSAMP_SCATTER_GROUPED)
 * (the per-update hot loop of the PER trainers on the pages: [PR615] runs
 * the CDF rebuild 32-128 times per train call; [SEGT] "Problem" samples
 * from the rebuilt prefix sum every step).  Same results, bit for bit, as
 * the four calls; in one kernel when one workgroup per 1024 (or 8192)
 * priorities can be resident at once, else in three kernels (tile sums;
 * scan, draws, drawn priorities and rewrite; IS weights).
 *   prio     : n float priorities, read, then rewritten at the drawn indices
 *              with new_prio (skipped when new_prio is NULL).
 *   u        : k float fractions in [0,1) (stratified thresholds).
 *   out_idx, out_w : k draws and their IS weights.
 *   cdf, total : n + 1 doubles of output (the CDF before the rewrite).
 *   ws       : psamp_per_round_workspace_size(n, k) bytes, 256-byte aligned.
 * Errors: as the four calls.
 * ---------------------------------------------------------------------- */
size_t psamp_per_round_workspace_size(int64_t n, int64_t k);
psamp_status psamp_per_round(void* prio, int64_t n, double alpha, double beta,
                             const float* u, int64_t k, const float* new_prio,
                             int32_t* out_idx, float* out_w, double* cdf, double* total,
                             void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * psamp_per_round without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments (less ws, ws_bytes), same
 * kernels and the same results bit for bit as psamp_per_round; the
 * workspace is a library-owned device array of 256 B + 4 KiB per 65536
 * priorities up to PSAMP_NOALLOC_MAX_N (4 MiB + 256 B), one per GPU, kept
 * until the process ends.  No call allocates or frees anything.
 *   n : 1 <= n <= PSAMP_NOALLOC_MAX_N (E_SIZE above).
 * The array is shared by every call on one GPU and keeps the last call's
 * state (it stays consistent, as a caller's workspace does): two calls that
 * may overlap on one GPU -- on different streams, or from different host
 * threads -- race and give unspecified results.  A bounded wait that gives
 * up sets a bit in that array, which no call reports.  The first call on
 * each device finds the array's address and, unless its stream is being
 * captured, clears it with a kernel on that stream.
 * Errors: those of psamp_per_round (E_WORKSPACE never), E_LAUNCH if the
 * array's address cannot be found.
 * ---------------------------------------------------------------------- */
#define PSAMP_NOALLOC_MAX_N (1 << 26)
psamp_status psamp_per_round_noalloc(void* prio, int64_t n, double alpha, double beta,
                                     const float* u, int64_t k, const float* new_prio,
                                     int32_t* out_idx, float* out_w, double* cdf, double* total,
                                     void* stream);

/* ------------------------------------------------------------------------
 * Measurement aid: the bandwidth ceiling of the CDF scan on this device.
 * out[i] = (double)in[i] for i < n -- the scan's bytes (4 read, 8 written
 * per element) in its access pattern, without its arithmetic or its
 * exchange between workgroups.  rows: 8 (the scan's tile of 8192 elements
 * per workgroup), 4 or 2 (smaller workgroups, more of them per CU); nt: 1
 * for non-temporal stores (as the scan's large tiles use), 0 for plain
 * ones.  n a multiple of 4, 4 <= n <= 2^31 - 1; in and out 16-byte aligned.
 * Errors: E_NULL, E_SIZE, E_PARAM, E_ALIGN, E_LAUNCH.
 * ---------------------------------------------------------------------- */
psamp_status psamp_ceiling_copy(const float* in, double* out, int64_t n, int rows, int nt,
                                 void* stream);

/* ------------------------------------------------------------------------
 * Device-side precondition checks.  The preconditions above that need a
 * sync to check (priorities finite and >= 0 with a positive total,
 * threshold fractions in [0, 1), indices in range, log-weights not NaN or
 * +inf) are checked on the device when checking is on: every entry point
 * then enqueues small check kernels on its stream next to its own, and a
 * violation sets a bit in a per-device word.  The checks change no output
 * and no status code.  Checking starts on when PSAMP_CHECK=1 is in the
 * environment at the library's first use.
 *   psamp_check_enable(1 / 0) turns it on / off and returns the previous
 *   state; psamp_check_enable(-1) only returns the state.
 *   psamp_check_errors copies the word to *bits_host, syncing `stream`
 *   (enqueue it on the stream of the calls it should cover); clear = 1 also
 *   zeroes the word.  Errors: E_NULL, E_LAUNCH.
 * Bits (which entry points check what):
 *   PSAMP_CHECK_PRIORITY   a priority (or new priority) NaN, infinite or < 0
 *                          (float priorities of build_cdf, build_cdf_sample,
 *                          per_round, segtree_build/update, scatter_lww,
 *                          replay insert/update)
 *   PSAMP_CHECK_ZERO_TOTAL the total of the weights is not a positive finite
 *                          number: all weights 0, or a weight or the sum
 *                          past the range of the CDF's type (build_cdf,
 *                          build_cdf_sample, per_round, sample, after
 *                          segtree_build)
 *   PSAMP_CHECK_FRACTION   a float threshold fraction U_i or u_row outside
 *                          [0, 1) (sample, build_cdf_sample, per_round,
 *                          segtree_sample, replay sample, resample_rows,
 *                          pf_step)
 *   PSAMP_CHECK_INDEX      an index outside [0, n) (is_weights)
 *   PSAMP_CHECK_LOGWEIGHT  a log-weight NaN or +inf (resample_rows, pf_step)
 * ---------------------------------------------------------------------- */
#define PSAMP_CHECK_PRIORITY 2u
#define PSAMP_CHECK_ZERO_TOTAL 4u
#define PSAMP_CHECK_FRACTION 8u
#define PSAMP_CHECK_INDEX 16u
#define PSAMP_CHECK_LOGWEIGHT 32u
int psamp_check_enable(int on);
psamp_status psamp_check_errors(uint64_t* bits_host, int clear, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics.  Copies the error bits a workspace of psamp_build_cdf,
 * psamp_build_cdf_sample, psamp_per_round or psamp_is_weights has
 * accumulated (bit 0: a bounded cross-workgroup wait timed out, so some
 * outputs of that call are unspecified; the other bits are always 0) into
 * *bits_host, with a synchronous device-to-host copy on `stream`.  The only
 * call that syncs.  The bits stay set until the caller clears the word.
 * Errors: E_NULL, E_WORKSPACE, E_LAUNCH.
 * ---------------------------------------------------------------------- */
psamp_status psamp_workspace_errors(const void* ws, size_t ws_bytes,
                                    uint64_t* bits_host, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PSAMP_H */
