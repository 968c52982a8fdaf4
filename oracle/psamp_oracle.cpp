// psamp_oracle.cpp -- TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT.
//
// A plain, slow, single-threaded CPU reference for proportional
// (prioritized-replay) sampling.  Only the test suite, the smoke check and
// the CPU-baseline leg of the benchmark may load it.  It shares no source,
// header, table or helper with the GPU library.
//
// Every function below is written from the definition it names, with no
// blocking, fusion or reordering beyond that definition:
//   * floating point is IEEE double (x86-64 SSE, built with
//     -ffp-contract=off -fno-fast-math); the fp32 sum tree works in float
//     because that is the precision its page fixes;
//   * integer work is exact (uint64_t / unsigned __int128).
//
// Sources (page title, then section):
//   [PR615]  "trainer: parallel build_cdf scan + tiled (bitwise-identical)
//            mingru backward", section "1. Parallel build_cdf": the CDF is
//            one serial prefix sum of the B priorities, once per update.
//   [SEGT]   "GPU Segment Tree for PER Sampling": sections "Tree Layout",
//            "Operations" (Update, Sample), "Memory", "Non-Goals".
//   [PF]     POPCORNBENCH particle-filter trace (Kimi-K2.6, l2_p48): the
//            reference model's forward pass -- predict with a linear model
//            plus process noise, a Gaussian observation log-likelihood, the
//            log-weight update -- and its resampling step: weights =
//            exp(log_w - logsumexp), cumsum, u = (arange(P) + rand(B,1)) / P,
//            searchsorted (first index with cumsum >= u), clamp to P-1,
//            gather, log-weights reset to -log(P).
//   [PER]    Prioritized experience replay as named in [SEGT] "Non-Goals"
//            (alpha, beta, IS weights): P(i) = p_i^alpha / sum_j p_j^alpha,
//            IS_i = (N * P(i))^-beta normalised by the largest weight of the
//            batch (Schaul et al., "Prioritized Experience Replay", 2016).
//
// Readings taken where the pages are silent are listed in the design notes
// next to the tests; each is repeated at the function it shapes.
//
// Parity pins: every function here is pinned by a CPU test against closed
// forms, library routines, brute force or invariants; none is "parity
// unpinned".

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <numeric>
#include <vector>

extern "C" {

// ---------------------------------------------------------------------------
// Step 1 -- weights.  [PER]: the sampling weight of item i is p_i^alpha.
// Evaluated with C pow in double (alpha is passed as a double, never as the
// float nearest to it).
// ---------------------------------------------------------------------------
void o_weights_f32(const float* p, int64_t n, double alpha, double* w) {
    for (int64_t i = 0; i < n; ++i) w[i] = std::pow((double)p[i], alpha);
}

// ---------------------------------------------------------------------------
// Step 2 -- inclusive CDF.  [PR615] "1. Parallel build_cdf": one serial
// prefix sum over the B weights; C_i = sum_{j<=i} w_j, T = C_{n-1}.
// Reading: inclusive and unnormalised (the last entry equals the total).
// ---------------------------------------------------------------------------
double o_cdf_f64(const double* w, int64_t n, double* C) {
    double s = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        s += w[i];
        C[i] = s;
    }
    return s;
}

double o_build_cdf_f32(const float* p, int64_t n, double alpha, double* C) {
    std::vector<double> w((size_t)n);
    o_weights_f32(p, n, alpha, w.data());
    return o_cdf_f64(w.data(), n, C);
}

// Integer mode: priorities are exact integers, alpha is not applied (an
// integer to a fractional power is not an integer), and the scan is exact.
uint64_t o_build_cdf_u32(const uint32_t* q, int64_t n, uint64_t* C) {
    uint64_t s = 0;
    for (int64_t i = 0; i < n; ++i) {
        s += (uint64_t)q[i];
        C[i] = s;
    }
    return s;
}

// ---------------------------------------------------------------------------
// Step 3a -- thresholds.
// Stratified: sample i draws its threshold inside stratum i of k equal
// strata of [0, T): t_i = ((i + U_i) / k) * T.  iid: t_i = U_i * T.
// fp: (double)i + (double)U_i is exact, the division by k rounds once (exact
// for power-of-two k), the product with T rounds once.
// ---------------------------------------------------------------------------
void o_thresholds_f64(const float* U, int64_t k, int stratified, double T,
                      double* t) {
    for (int64_t i = 0; i < k; ++i) {
        if (stratified) {
            double a = (double)i + (double)U[i];
            double b = a / (double)k;
            t[i] = b * T;
        } else {
            t[i] = (double)U[i] * T;
        }
    }
}

// Integer mode: U_i = r_i / 2^32 with r_i a uint32.  The threshold is the
// integer ceiling-style map of the same formula onto [1, T]:
//   stratified: t_i = floor(((i * 2^32 + r_i) * T) / (k * 2^32)) + 1
//   iid:        t_i = floor((r_i * T) / 2^32) + 1
// Computed exactly in 128-bit arithmetic.
void o_thresholds_u64(const uint32_t* r, int64_t k, int stratified,
                      uint64_t T, uint64_t* t) {
    typedef unsigned __int128 u128;
    for (int64_t i = 0; i < k; ++i) {
        u128 num;
        u128 den;
        if (stratified) {
            num = (((u128)(uint64_t)i << 32) + (u128)r[i]) * (u128)T;
            den = (u128)(uint64_t)k << 32;
        } else {
            num = (u128)r[i] * (u128)T;
            den = (u128)1 << 32;
        }
        t[i] = (uint64_t)(num / den) + 1;
    }
}

// ---------------------------------------------------------------------------
// Step 3b -- search.  [PF]: searchsorted with right=False returns the first
// index j with C_j >= t (or n if there is none), then the result is clamped
// to n-1.  Done here as a linear merge: thresholds are visited in ascending
// order (a stable argsort), one pointer j only moves forward.
// ---------------------------------------------------------------------------
static std::vector<int64_t> ascending_order_f64(const double* t, int64_t k) {
    std::vector<int64_t> ord((size_t)k);
    std::iota(ord.begin(), ord.end(), (int64_t)0);
    std::stable_sort(ord.begin(), ord.end(),
                     [t](int64_t a, int64_t b) { return t[a] < t[b]; });
    return ord;
}

void o_search_f64(const double* C, int64_t n, const double* t, int64_t k,
                  int32_t* idx) {
    std::vector<int64_t> ord = ascending_order_f64(t, k);
    int64_t j = 0;
    for (int64_t q = 0; q < k; ++q) {
        int64_t i = ord[(size_t)q];
        while (j < n && C[j] < t[i]) ++j;
        idx[i] = (int32_t)(j < n ? j : n - 1);
    }
}

void o_search_u64(const uint64_t* C, int64_t n, const uint64_t* t, int64_t k,
                  int32_t* idx) {
    std::vector<int64_t> ord((size_t)k);
    std::iota(ord.begin(), ord.end(), (int64_t)0);
    std::stable_sort(ord.begin(), ord.end(),
                     [t](int64_t a, int64_t b) { return t[a] < t[b]; });
    int64_t j = 0;
    for (int64_t q = 0; q < k; ++q) {
        int64_t i = ord[(size_t)q];
        while (j < n && C[j] < t[i]) ++j;
        idx[i] = (int32_t)(j < n ? j : n - 1);
    }
}

// Variant searched on an fp32 CDF (the "best possible fp32 CDF" experiment):
// the CDF is the fp64 one rounded to float, thresholds stay fp64.
void o_search_f32cdf(const float* C, int64_t n, const double* t, int64_t k,
                     int32_t* idx) {
    std::vector<int64_t> ord = ascending_order_f64(t, k);
    int64_t j = 0;
    for (int64_t q = 0; q < k; ++q) {
        int64_t i = ord[(size_t)q];
        while (j < n && (double)C[j] < t[i]) ++j;
        idx[i] = (int32_t)(j < n ? j : n - 1);
    }
}

// ---------------------------------------------------------------------------
// Step 4 -- importance-sampling weights.  [PER]: P_i = w_{idx_i} / T,
// v_i = (N * P_i)^-beta, IS_i = v_i / max_j v_j over the k sampled entries.
// Reading: P comes from the priority (w recomputed as p^alpha), not from a
// difference of CDF entries; N is the number of valid items.
// ---------------------------------------------------------------------------
void o_is_weights_f32(const float* p, int64_t N, double alpha, double T,
                      const int32_t* idx, int64_t k, double beta, float* out) {
    std::vector<double> v((size_t)k);
    double vmax = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        double w = std::pow((double)p[idx[i]], alpha);
        double P = w / T;
        v[(size_t)i] = std::pow((double)N * P, -beta);
        if (i == 0 || v[(size_t)i] > vmax) vmax = v[(size_t)i];
    }
    for (int64_t i = 0; i < k; ++i) out[i] = (float)(v[(size_t)i] / vmax);
}

void o_is_weights_u32(const uint32_t* q, int64_t N, uint64_t T,
                      const int32_t* idx, int64_t k, double beta, float* out) {
    std::vector<double> v((size_t)k);
    double vmax = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        double P = (double)q[idx[i]] / (double)T;
        v[(size_t)i] = std::pow((double)N * P, -beta);
        if (i == 0 || v[(size_t)i] > vmax) vmax = v[(size_t)i];
    }
    for (int64_t i = 0; i < k; ++i) out[i] = (float)(v[(size_t)i] / vmax);
}

// ---------------------------------------------------------------------------
// Priority rewrite: p[idx_j] = v_j for j = 0..m-1 in batch order, so the
// last write to a repeated index wins.
// ---------------------------------------------------------------------------
void o_scatter_lww_f32(float* p, int64_t n, const int32_t* idx, const float* v,
                       int64_t m) {
    for (int64_t j = 0; j < m; ++j) {
        int64_t i = idx[j];
        if (i >= 0 && i < n) p[i] = v[j];
    }
}

// ---------------------------------------------------------------------------
// Sum tree.  [SEGT] "Architecture"/"Tree Layout": a binary tree whose leaves
// hold priorities and whose internal nodes hold the sum of their children;
// capacity is rounded up to a power of two.  Here every node is a separate
// object linked by pointers (left, right, parent); the flat heap order of the
// page (root at 1, children of j at 2j and 2j+1, leaf i at cap+i) is only
// produced on export, for comparison.
//
// [SEGT] "Operations -- Update": write the leaf, then recompute every
// ancestor as left + right up to the root (recompute, not add a delta).
// Applied sequentially in batch order, which gives last-write-wins for
// repeated indices.
// [SEGT] "Operations -- Sample": walk root to leaf; go left if the threshold
// is <= the left sum, else subtract the left sum and go right.  Reading: also
// go left when the right sum is 0 (never walk into an empty subtree after
// rounding); the final index is clamped to n_valid - 1.
// ---------------------------------------------------------------------------
}  // extern "C"

namespace {

template <class V>
struct ONode {
    ONode* left = nullptr;
    ONode* right = nullptr;
    ONode* parent = nullptr;
    V sum = V(0);
    int64_t leaf = -1;
};

template <class V>
struct OTree {
    int64_t cap = 0;
    std::vector<ONode<V>> pool;      // owns the nodes; links are pointers
    std::vector<ONode<V>*> leaves;   // leaf i -> its node
    ONode<V>* root = nullptr;
    size_t used = 0;

    ONode<V>* make(int64_t lo, int64_t hi, ONode<V>* parent) {
        ONode<V>* nd = &pool[used++];
        nd->parent = parent;
        if (hi - lo == 1) {
            nd->leaf = lo;
            leaves[(size_t)lo] = nd;
        } else {
            int64_t mid = lo + (hi - lo) / 2;
            nd->left = make(lo, mid, nd);
            nd->right = make(mid, hi, nd);
        }
        return nd;
    }
    explicit OTree(int64_t c) : cap(c), pool((size_t)(2 * c - 1)), leaves((size_t)c) {
        root = make(0, c, nullptr);
    }
    // Recompute all internal sums from the leaves (post-order).
    V rebuild(ONode<V>* nd) {
        if (nd->leaf >= 0) return nd->sum;
        V l = rebuild(nd->left);
        V r = rebuild(nd->right);
        nd->sum = l + r;
        return nd->sum;
    }
    void set_leaf(int64_t i, V val) {
        ONode<V>* nd = leaves[(size_t)i];
        nd->sum = val;
        for (ONode<V>* a = nd->parent; a != nullptr; a = a->parent)
            a->sum = a->left->sum + a->right->sum;
    }
    int64_t descend(V t) const {
        const ONode<V>* nd = root;
        while (nd->leaf < 0) {
            V L = nd->left->sum;
            V R = nd->right->sum;
            if (t <= L || R == V(0)) {
                nd = nd->left;
            } else {
                t = t - L;
                nd = nd->right;
            }
        }
        return nd->leaf;
    }
    // Flat heap order of [SEGT] "Tree Layout": breadth-first numbering.
    void export_flat(V* flat) const {
        flat[0] = V(0);
        std::vector<const ONode<V>*> level{root};
        int64_t pos = 1;
        while (!level.empty()) {
            std::vector<const ONode<V>*> next;
            for (const ONode<V>* nd : level) {
                flat[pos++] = nd->sum;
                if (nd->leaf < 0) {
                    next.push_back(nd->left);
                    next.push_back(nd->right);
                }
            }
            level.swap(next);
        }
    }
};

}  // namespace

extern "C" {

// fp32 leaf value: the float nearest to p^alpha (correctly rounded).  The
// exact power is approximated in 80-bit long double first, whose error
// (about 2^-63 relative) is far below the half-ulp of a float, so rounding
// it to float gives the correctly rounded result except in vanishingly rare
// near-ties.
float o_leaf_f32(float p, double alpha) {
    long double x = powl((long double)p, (long double)alpha);
    return (float)x;
}

void* o_tree_new(int vtype, int64_t cap) {
    if (vtype == 0) return new OTree<float>(cap);
    if (vtype == 1) return new OTree<double>(cap);
    if (vtype == 2) return new OTree<uint64_t>(cap);
    return nullptr;
}

void o_tree_free(int vtype, void* h) {
    if (vtype == 0) delete (OTree<float>*)h;
    if (vtype == 1) delete (OTree<double>*)h;
    if (vtype == 2) delete (OTree<uint64_t>*)h;
}

// Build: leaves 0..n_valid-1 from the priorities, leaves n_valid..cap-1 are 0.
void o_tree_build_f32(void* h, const float* p, int64_t n_valid, double alpha) {
    OTree<float>* t = (OTree<float>*)h;
    for (int64_t i = 0; i < t->cap; ++i)
        t->leaves[(size_t)i]->sum = i < n_valid ? o_leaf_f32(p[i], alpha) : 0.0f;
    t->rebuild(t->root);
}
void o_tree_build_f64(void* h, const float* p, int64_t n_valid, double alpha) {
    OTree<double>* t = (OTree<double>*)h;
    for (int64_t i = 0; i < t->cap; ++i)
        t->leaves[(size_t)i]->sum = i < n_valid ? std::pow((double)p[i], alpha) : 0.0;
    t->rebuild(t->root);
}
void o_tree_build_u64(void* h, const uint32_t* q, int64_t n_valid) {
    OTree<uint64_t>* t = (OTree<uint64_t>*)h;
    for (int64_t i = 0; i < t->cap; ++i)
        t->leaves[(size_t)i]->sum = i < n_valid ? (uint64_t)q[i] : 0;
    t->rebuild(t->root);
}

void o_tree_update_f32(void* h, const int32_t* idx, const float* v, int64_t m,
                       double alpha) {
    OTree<float>* t = (OTree<float>*)h;
    for (int64_t j = 0; j < m; ++j) t->set_leaf(idx[j], o_leaf_f32(v[j], alpha));
}
void o_tree_update_f64(void* h, const int32_t* idx, const float* v, int64_t m,
                       double alpha) {
    OTree<double>* t = (OTree<double>*)h;
    for (int64_t j = 0; j < m; ++j) t->set_leaf(idx[j], std::pow((double)v[j], alpha));
}
void o_tree_update_u64(void* h, const int32_t* idx, const uint32_t* q, int64_t m) {
    OTree<uint64_t>* t = (OTree<uint64_t>*)h;
    for (int64_t j = 0; j < m; ++j) t->set_leaf(idx[j], (uint64_t)q[j]);
}

static int32_t clamp_leaf(int64_t leaf, int64_t n_valid) {
    return (int32_t)(leaf < n_valid ? leaf : n_valid - 1);
}

// fp32 tree thresholds.  iid: t = U * root in float ([SEGT] draws a
// threshold in [0, root) and works in f32).  Stratified: the fp64 stratum
// formula of step 3a, rounded once to float.
void o_tree_sample_f32(void* h, int64_t n_valid, const float* U, int64_t k,
                       int stratified, int32_t* out) {
    OTree<float>* t = (OTree<float>*)h;
    float root = t->root->sum;
    for (int64_t i = 0; i < k; ++i) {
        float th;
        if (stratified) {
            double a = (double)i + (double)U[i];
            double b = a / (double)k;
            th = (float)(b * (double)root);
        } else {
            th = U[i] * root;
        }
        out[i] = clamp_leaf(t->descend(th), n_valid);
    }
}
void o_tree_sample_f64(void* h, int64_t n_valid, const float* U, int64_t k,
                       int stratified, int32_t* out) {
    OTree<double>* t = (OTree<double>*)h;
    std::vector<double> th((size_t)k);
    o_thresholds_f64(U, k, stratified, t->root->sum, th.data());
    for (int64_t i = 0; i < k; ++i) out[i] = clamp_leaf(t->descend(th[(size_t)i]), n_valid);
}
void o_tree_sample_u64(void* h, int64_t n_valid, const uint32_t* r, int64_t k,
                       int stratified, int32_t* out) {
    OTree<uint64_t>* t = (OTree<uint64_t>*)h;
    std::vector<uint64_t> th((size_t)k);
    o_thresholds_u64(r, k, stratified, t->root->sum, th.data());
    for (int64_t i = 0; i < k; ++i) out[i] = clamp_leaf(t->descend(th[(size_t)i]), n_valid);
}

void o_tree_export_f32(void* h, float* flat) { ((OTree<float>*)h)->export_flat(flat); }
void o_tree_export_f64(void* h, double* flat) { ((OTree<double>*)h)->export_flat(flat); }
void o_tree_export_u64(void* h, uint64_t* flat) { ((OTree<uint64_t>*)h)->export_flat(flat); }
float o_tree_root_f32(void* h) { return ((OTree<float>*)h)->root->sum; }
double o_tree_root_f64(void* h) { return ((OTree<double>*)h)->root->sum; }
uint64_t o_tree_root_u64(void* h) { return ((OTree<uint64_t>*)h)->root->sum; }

// ---------------------------------------------------------------------------
// Row-batched systematic resampling.  [PF], the reference model's
// resampling step, per row of P log-weights:
//   new_log_w = log_w - logsumexp(log_w)      (max-shifted, as the fused
//   weights   = exp(new_log_w)                 kernel of the trace does)
//   cumsum    = inclusive prefix sum of the weights
//   u_k       = (k + u_row) / P               (float32, as torch computes
//                                               arange(P) + rand(B,1), / P)
//   anc_k     = first j with cumsum_j >= u_k, clamped to P-1
// Reading: exp, the log-sum and the cumsum are evaluated in double; the
// thresholds keep the pages' float32 arithmetic.  The search is a linear
// merge (the u_k of a row are non-decreasing in k).
// ---------------------------------------------------------------------------
void o_row_cdf(const float* x, int64_t P, double* W, double* C);

void o_resample_rows(const float* lw, int64_t rows, int64_t P, int64_t ld_in,
                     const float* u_row, int32_t* anc, int64_t ld_out) {
    std::vector<double> W((size_t)P), C((size_t)P);
    for (int64_t b = 0; b < rows; ++b) {
        o_row_cdf(lw + b * ld_in, P, W.data(), C.data());
        int64_t j = 0;
        for (int64_t kk = 0; kk < P; ++kk) {
            float uk = ((float)kk + u_row[b]) / (float)P;
            while (j < P && C[(size_t)j] < (double)uk) ++j;
            anc[b * ld_out + kk] = (int32_t)(j < P ? j : P - 1);
        }
    }
}

// ---------------------------------------------------------------------------
// One particle-filter step.  [PF], the reference model's forward pass, per
// row b (one filter of P particles in D dimensions, O observed values):
//   pred_j    = A x_j + sigma_p eps_j          (x @ A^T + sigma_p * noise)
//   y_j       = C pred_j                         (pred @ C^T)
//   ll_j      = -0.5 * sum_o (obs_o - y_jo)^2 / sigma_o^2
//   lw'_j     = lw_j + ll_j
//   anc       = systematic resampling of lw' with u_row[b]  (as above)
//   x_out_k   = pred_{anc_k},   lw_out_k = -log(P)
// Reading: every step up to lw' in float32 as the pages' model computes it,
// each dot product summed in increasing index, the noise term added last,
// ll = (-0.5 * S) / (sigma_o * sigma_o) in that order; the resampling as
// o_resample_rows; -log(P) in double, rounded to float.  The noise eps is
// an input (standard normal draws), like every random number here.
// pred_out and lwn_out (pred and lw', for the pins) may be null.
// ---------------------------------------------------------------------------
void o_pf_step(const float* x, const float* lw, const float* obs, const float* A,
               const float* Cm, const float* eps, float sigma_p, float sigma_o,
               const float* u_row, int64_t rows, int64_t P, int64_t D, int64_t O,
               float* x_out, float* lw_out, int32_t* anc_out, float* pred_out,
               float* lwn_out) {
    std::vector<float> pred((size_t)(P * D)), lwn((size_t)P);
    std::vector<int32_t> anc((size_t)P);
    const float s2 = sigma_o * sigma_o;
    const float neg_log_p = (float)(-std::log((double)P));
    for (int64_t b = 0; b < rows; ++b) {
        const float* xb = x + b * P * D;
        const float* eb = eps + b * P * D;
        const float* ob = obs + b * O;
        for (int64_t j = 0; j < P; ++j) {
            for (int64_t d = 0; d < D; ++d) {
                float acc = 0.0f;
                for (int64_t k = 0; k < D; ++k) acc = acc + A[d * D + k] * xb[j * D + k];
                pred[(size_t)(j * D + d)] = acc + sigma_p * eb[j * D + d];
            }
            float S = 0.0f;
            for (int64_t o = 0; o < O; ++o) {
                float y = 0.0f;
                for (int64_t d = 0; d < D; ++d) y = y + Cm[o * D + d] * pred[(size_t)(j * D + d)];
                const float diff = ob[o] - y;
                S = S + diff * diff;
            }
            const float ll = (-0.5f * S) / s2;
            lwn[(size_t)j] = lw[b * P + j] + ll;
        }
        o_resample_rows(lwn.data(), 1, P, P, u_row + b, anc.data(), P);
        for (int64_t k = 0; k < P; ++k) {
            const int64_t a = anc[(size_t)k];
            for (int64_t d = 0; d < D; ++d) x_out[(b * P + k) * D + d] = pred[(size_t)(a * D + d)];
            lw_out[b * P + k] = neg_log_p;
            if (anc_out) anc_out[b * P + k] = (int32_t)a;
        }
        if (pred_out) std::memcpy(pred_out + b * P * D, pred.data(), sizeof(float) * (size_t)(P * D));
        if (lwn_out) std::memcpy(lwn_out + b * P, lwn.data(), sizeof(float) * (size_t)P);
    }
}

// One row of the resampler: max m, s = sum exp(x - m), lse = m + log s,
// W_j = exp(x_j - lse), C = serial cumsum of W (all double).  Also exposed
// for the pins.
void o_row_cdf(const float* x, int64_t P, double* W, double* C) {
    double m = (double)x[0];
    for (int64_t j = 1; j < P; ++j)
        if ((double)x[j] > m) m = (double)x[j];
    double s = 0.0;
    for (int64_t j = 0; j < P; ++j) s += std::exp((double)x[j] - m);
    double lse = m + std::log(s);
    double c = 0.0;
    for (int64_t j = 0; j < P; ++j) {
        W[j] = std::exp((double)x[j] - lse);
        c += W[j];
        C[j] = c;
    }
}

}  // extern "C"
