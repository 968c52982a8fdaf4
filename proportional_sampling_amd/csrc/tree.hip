// tree.hip -- sum tree ("GPU Segment Tree for PER Sampling").
//
// Layout ([SEGT] "Tree Layout"): flat array of 2*cap nodes, index 0 unused,
// root at 1, children of j at 2j and 2j+1, leaf i at cap+i.  F32 trees hold
// p^alpha rounded to float and float sums (the page's precision); U64 trees
// hold uint32 priorities and exact sums.
//
// Build: passes of up to 11 levels each; a workgroup reduces 2048 nodes of a
// level through LDS and writes every node it forms.
//
// Update ([SEGT] "Operations -- Update": write the leaf, recompute each
// ancestor as left + right).  The page's one-thread-per-update kernel races
// when two updates share an ancestor (a thread can read a stale sibling and
// overwrite a correct parent) and on repeated indices.  Here one 1024-thread
// workgroup handles a batch of up to 1024 updates deterministically:
//   1. sort the (leaf, batch position) keys in LDS (stable radix sort on the
//      leaf);
//   2. keep the last entry of each run of equal leaves (largest batch
//      position: last write wins);
//   3. each winning leaf's thread prefetches the old values of all siblings
//      on its root path at once (one round of loads, no per-level latency);
//   4. level by level, the first winner under each dirty node (its "owner")
//      forms fl(left + right) from its own value, a clean sibling from its
//      registers, or the dirty sibling's value from LDS; each owner also
//      carries the index of the next owner, so it finds that sibling in O(1).
// Every dirty node is written exactly once, after both children are final,
// as fl(left + right): the tree stays bit-equal to a fresh build.
//
// Sample ([SEGT] "Operations -- Sample"): descend from the root, left if
// t <= left sum (or the right sum is 0), else subtract and go right.  The
// top 13 (F32) or 12 (U64) levels are copied into LDS per workgroup; the
// remaining levels load the two children as one vector.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kBuildThreads = 256;
constexpr int kBuildLevels = 11;                 // levels per build pass
constexpr int kUpdThreads = 1024;
constexpr int kUpdWaves = kUpdThreads / kWave;
static_assert(256 * kUpdWaves == 4 * kUpdThreads, "the radix prefix takes 4 counts per thread");

// Inclusive sum over the 64 lanes (uint32; DPP rows, then across rows).
__device__ __forceinline__ uint32_t wave_incl_u32(uint32_t x) {
    x += dpp32<kRowShr1, 0xF, true>(x);
    x += dpp32<kRowShr2, 0xF, true>(x);
    x += dpp32<kRowShr4, 0xF, true>(x);
    x += dpp32<kRowShr8, 0xF, true>(x);
    x += dpp32<kRowBcast15, 0xA, false>(x);
    x += dpp32<kRowBcast31, 0xC, false>(x);
    return x;
}
constexpr int kMaxDepth = 30;                    // cap <= 2^30
constexpr int kSampleTreeThreads = 256;
constexpr int kSampleTreeThreadsBig = 1024;      // large batches: fewer copies of the top levels
constexpr int kSampleTreeDpt = 2;                // draws per thread in large batches

template <class V> struct TreeTop;
template <> struct TreeTop<float> { static constexpr int levels = 13; };
template <> struct TreeTop<uint64_t> { static constexpr int levels = 12; };

__device__ __forceinline__ float leaf_value(float p, double alpha, const MathLds* M) {
    return (float)pow_prio(p, alpha, M);
}
__device__ __forceinline__ uint64_t leaf_value(uint32_t q, double, const MathLds*) {
    return (uint64_t)q;
}

// One build pass.  Input level: `cnt` nodes at tree indices [cnt, 2 cnt)
// (the leaves when FROM_PRIO, whose values are formed from prio).  Each
// workgroup takes 2^s consecutive nodes and writes the s levels above them.
template <class V, class P, bool FROM_PRIO>
__global__ __launch_bounds__(kBuildThreads) void k_tree_build_pass(
    V* __restrict__ tree, int64_t cnt, const P* __restrict__ prio, int64_t n_valid,
    double alpha, int s) {
    __shared__ V buf[2][1 << kBuildLevels];
    __shared__ MathLds M;
    const int tid = threadIdx.x;
    if (FROM_PRIO && sizeof(P) == 4 && sizeof(V) == 4) math_lds_fill(&M, tid, kBuildThreads);
    __syncthreads();
    const int sub = 1 << s;
    const int64_t first = (int64_t)blockIdx.x << s;      // first input node (relative)
    for (int i = tid; i < sub; i += kBuildThreads) {
        const int64_t node = first + i;
        V v;
        if (FROM_PRIO) {
            v = node < n_valid ? leaf_value(prio[node], alpha, &M) : V(0);
            tree[cnt + node] = v;
        } else {
            v = tree[cnt + node];
        }
        buf[0][i] = v;
    }
    __syncthreads();
    int64_t lvl = cnt;                                   // tree index of the level's first node
    for (int d = 1; d <= s; ++d) {
        const int m = sub >> d;
        const V* src = buf[(d - 1) & 1];
        V* dst = buf[d & 1];
        lvl >>= 1;
        for (int q = tid; q < m; q += kBuildThreads) {
            const V x = src[2 * q] + src[2 * q + 1];
            dst[q] = x;
            tree[lvl + (first >> d) + q] = x;
        }
        __syncthreads();
    }
}

template <class V, class P>
__global__ __launch_bounds__(kUpdThreads) void k_tree_update(
    V* __restrict__ tree, int64_t cap, int D, const int32_t* __restrict__ idx,
    const P* __restrict__ prio, int m, double alpha) {
    __shared__ uint64_t keys[kUpdThreads];
    __shared__ uint32_t hist[256 * kUpdWaves];              // (digit, wave) counts, then offsets
    __shared__ uint32_t hsum[kUpdWaves];
    __shared__ uint32_t wcount[kUpdThreads / kWave];
    __shared__ int32_t wl[kUpdThreads];                  // winner leaves, ascending
    __shared__ int32_t wj[kUpdThreads];                  // their batch positions
    __shared__ V vbuf[2][kUpdThreads];
    __shared__ int32_t ebuf[2][kUpdThreads];
    __shared__ uint32_t s_u;
    __shared__ MathLds M;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    if (sizeof(P) == 4 && sizeof(V) == 4) math_lds_fill(&M, tid, kUpdThreads);

    // 1. keys = (leaf << 32) | batch position, sorted.  A stable LSD radix
    // sort on the leaf (8-bit digits; an out-of-range entry takes the key
    // cap, above every leaf, and keeps its all-ones word) leaves equal
    // leaves in batch order, i.e. the array sorted by the whole key: per
    // pass, ballots rank each key among the lanes of its wave with the same
    // digit, and a digit-major prefix over the per-wave counts places it --
    // five barriers a pass and ceil((D + 1) / 8) passes, against the 55
    // compare-exchange steps of a bitonic network.
    uint64_t key = ~0ull;
    if (tid < m) {
        const int32_t l = idx[tid];
        if (l >= 0 && (int64_t)l < cap) key = ((uint64_t)(uint32_t)l << 32) | (uint32_t)tid;
    }
    {
        const uint64_t lane_lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
        const int passes = (D + 1 + 7) / 8;
        for (int ps = 0; ps < passes; ++ps) {
            const uint32_t lp = key == ~0ull ? (uint32_t)cap : (uint32_t)(key >> 32);
            const uint32_t d = (lp >> (8 * ps)) & 255u;
#pragma unroll
            for (int c = 0; c < 4; ++c) hist[4 * tid + c] = 0u;
            __syncthreads();
            uint64_t peers = ~0ull;
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                const uint64_t bal = __ballot((d >> b) & 1u);
                peers &= ((d >> b) & 1u) ? bal : ~bal;
            }
            const uint32_t rank = (uint32_t)__popcll(peers & lane_lt);
            if (rank == 0) hist[d * kUpdWaves + wave] = (uint32_t)__popcll(peers);
            __syncthreads();
            uint32_t h[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) h[c] = hist[4 * tid + c];
            const uint32_t loc = (h[0] + h[1]) + (h[2] + h[3]);
            const uint32_t inc = wave_incl_u32(loc);
            if (lane == kWave - 1) hsum[wave] = inc;
            __syncthreads();
            uint32_t ex = inc - loc;
            for (int w2 = 0; w2 < wave; ++w2) ex += hsum[w2];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                hist[4 * tid + c] = ex;
                ex += h[c];
            }
            __syncthreads();
            keys[hist[d * kUpdWaves + wave] + rank] = key;
            __syncthreads();
            key = keys[tid];
        }
    }

    // 2. winners: the last key of each run of equal leaves.
    const uint64_t my = keys[tid];
    const uint64_t nx = tid + 1 < kUpdThreads ? keys[tid + 1] : ~0ull;
    const bool win = my != ~0ull && (nx >> 32) != (my >> 32);
    const uint64_t bal = __ballot(win);
    if (lane == 0) wcount[wave] = (uint32_t)__popcll(bal);
    __syncthreads();
    uint32_t pos = (uint32_t)__popcll(bal & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
    uint32_t tot = 0;
    for (int w2 = 0; w2 < kUpdThreads / kWave; ++w2) {
        const uint32_t c = wcount[w2];
        if (w2 < wave) pos += c;
        tot += c;
    }
    if (win) {
        wl[pos] = (int32_t)(my >> 32);
        wj[pos] = (int32_t)(uint32_t)my;
    }
    if (tid == 0) s_u = tot;
    __syncthreads();
    const int u = (int)s_u;

    // 3. per-winner state and the prefetch of all path siblings.
    const bool act = tid < u;
    int64_t L = 0, Lp = -1;
    V val = V(0);
    int32_t end = tid + 1;
    V sib[kMaxDepth];
    if (act) {
        L = wl[tid];
        Lp = tid > 0 ? (int64_t)wl[tid - 1] : -1;
        val = leaf_value(prio[wj[tid]], alpha, &M);
#pragma unroll
        for (int d = 0; d < kMaxDepth; ++d)
            if (d < D) sib[d] = tree[((cap + L) >> d) ^ 1];
        tree[cap + L] = val;
        vbuf[0][tid] = val;
        ebuf[0][tid] = end;
    }
    __syncthreads();

    // 4. levels 1..D (unrolled so that sib[] stays in registers).
#pragma unroll
    for (int d = 1; d <= kMaxDepth; ++d) {
        if (d <= D) {
            const int bi = (d - 1) & 1;
            const int bo = d & 1;
            const bool own = act && (tid == 0 || ((cap + Lp) >> d) != ((cap + L) >> d));
            if (own) {
                const int64_t c = (cap + L) >> (d - 1);
                const int64_t N = c >> 1;
                V left, right;
                int32_t ne = end;
                if ((c & 1) == 0) {
                    left = val;
                    const int32_t j = end;
                    if (j < u && ((cap + (int64_t)wl[j]) >> d) == N) {
                        right = vbuf[bi][j];
                        ne = ebuf[bi][j];
                    } else {
                        right = sib[d - 1];
                    }
                } else {
                    left = sib[d - 1];
                    right = val;
                }
                val = left + right;
                end = ne;
                tree[N] = val;
                vbuf[bo][tid] = val;
                ebuf[bo][tid] = end;
            }
            __syncthreads();
        }
    }
}

// The threshold of draw i (see psamp_segtree_sample).
template <class V>
__device__ __forceinline__ V tree_threshold(int64_t i, const void* u, int64_t k, int stratified,
                                            int k_log2, V root) {
    if constexpr (sizeof(V) == 4) {
        const float U = ((const float*)u)[i];
        if (stratified) {
            const double a = (double)i + (double)U;
            const double b = a / (double)k;
            return (float)(b * (double)root);
        }
        return U * root;
    } else {
        return int_threshold((uint64_t)i, ((const uint32_t*)u)[i], (uint64_t)k, root, stratified,
                             k_log2);
    }
}

// DPT draws per thread, descended together level by level (independent
// loads in flight); a workgroup takes NT * DPT consecutive draws.
template <class V, int NT, int DPT>
__global__ __launch_bounds__(NT) void k_tree_sample(
    const V* __restrict__ tree, int64_t cap, int D, int64_t n_valid, const void* __restrict__ u,
    int64_t k, int stratified, int k_log2, int lt, int32_t* __restrict__ out) {
    __shared__ V top[1 << TreeTop<V>::levels];
    const int tid = threadIdx.x;
    const int ntop = 1 << lt;
    for (int i = tid; i < ntop; i += NT) top[i] = i > 0 ? tree[i] : V(0);
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * NT * DPT + tid;
    if (i0 >= k) return;
    const V root = top[1];
    V t[DPT];
    int64_t node[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int64_t i = i0 + (int64_t)j * NT;
        t[j] = tree_threshold<V>(i < k ? i : i0, u, k, stratified, k_log2, root);
        node[j] = 1;
    }
    for (int d = 0; d < D; ++d) {
        V Lv[DPT], Rv[DPT];
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int64_t c = 2 * node[j];
            if (c + 1 < ntop) {
                Lv[j] = top[c];
                Rv[j] = top[c + 1];
            } else if constexpr (sizeof(V) == 4) {
                const float2 pr = *reinterpret_cast<const float2*>(tree + c);
                Lv[j] = pr.x;
                Rv[j] = pr.y;
            } else {
                const ulonglong2 pr = *reinterpret_cast<const ulonglong2*>(tree + c);
                Lv[j] = pr.x;
                Rv[j] = pr.y;
            }
        }
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int64_t c = 2 * node[j];
            if (t[j] <= Lv[j] || Rv[j] == V(0)) {
                node[j] = c;
            } else {
                t[j] = t[j] - Lv[j];
                node[j] = c + 1;
            }
        }
    }
#pragma unroll
    for (int j = 0; j < DPT; ++j) {
        const int64_t i = i0 + (int64_t)j * NT;
        const int64_t leaf = node[j] - cap;
        if (i < k) out[i] = (int32_t)(leaf < n_valid ? leaf : n_valid - 1);
    }
}

template <class V, class P>
static psamp_status launch_build(void* tree, int64_t cap, const void* prio, int64_t n_valid,
                                 double alpha, hipStream_t st) {
    const int D = ilog2_exact(cap);
    int64_t cnt = cap;
    bool from_prio = true;
    if (D == 0) {   // a single leaf is the root
        hipLaunchKernelGGL((k_tree_build_pass<V, P, true>), dim3(1), dim3(kBuildThreads), 0, st,
                           (V*)tree, (int64_t)1, (const P*)prio, n_valid, alpha, 0);
        return launch_status();
    }
    int done = 0;
    while (done < D) {
        const int s = min_(kBuildLevels, D - done);
        const int64_t grid = cnt >> s;
        if (trace_enabled()) trace_launch("k_tree_build_pass", grid, kBuildThreads, cnt);
        if (from_prio)
            hipLaunchKernelGGL((k_tree_build_pass<V, P, true>), dim3((unsigned)grid),
                               dim3(kBuildThreads), 0, st, (V*)tree, cnt, (const P*)prio, n_valid,
                               alpha, s);
        else
            hipLaunchKernelGGL((k_tree_build_pass<V, P, false>), dim3((unsigned)grid),
                               dim3(kBuildThreads), 0, st, (V*)tree, cnt, (const P*)prio, n_valid,
                               alpha, s);
        psamp_status e = launch_status();
        if (e != PSAMP_OK) return e;
        from_prio = false;
        cnt >>= s;
        done += s;
    }
    return PSAMP_OK;
}

}  // namespace psamp

using namespace psamp;

extern "C" int64_t psamp_segtree_cap_pow2(int64_t capacity) {
    if (capacity < 1 || capacity > (int64_t(1) << kMaxDepth)) return 0;
    int64_t c = 1;
    while (c < capacity) c <<= 1;
    return c;
}

static psamp_status tree_types(psamp_dtype tree_t, psamp_dtype prio_t) {
    if (tree_t == PSAMP_F32 && prio_t == PSAMP_F32) return PSAMP_OK;
    if (tree_t == PSAMP_U64 && prio_t == PSAMP_U32) return PSAMP_OK;
    return PSAMP_E_DTYPE;
}

extern "C" psamp_status psamp_segtree_build(void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                            const void* prio, psamp_dtype prio_t, int64_t n_valid,
                                            double alpha, void* stream) {
    if (!tree || !prio) return PSAMP_E_NULL;
    if (!is_pow2(cap_pow2) || cap_pow2 > (int64_t(1) << kMaxDepth) || n_valid < 1 ||
        n_valid > cap_pow2)
        return PSAMP_E_SIZE;
    if (tree_types(tree_t, prio_t) != PSAMP_OK) return PSAMP_E_DTYPE;
    if (tree_t == PSAMP_F32 && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (!aligned(tree, 16) || !aligned(prio, 4)) return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    const bool chk = check_on();
    if (chk && tree_t == PSAMP_F32) check_prio((const float*)prio, n_valid, st);
    const psamp_status e =
        tree_t == PSAMP_F32 ? launch_build<float, float>(tree, cap_pow2, prio, n_valid, alpha, st)
                            : launch_build<uint64_t, uint32_t>(tree, cap_pow2, prio, n_valid, 0.0, st);
    if (chk && e == PSAMP_OK)
        check_total(tree_t == PSAMP_F32 ? (const void*)((const float*)tree + 1)
                                        : (const void*)((const uint64_t*)tree + 1),
                     tree_t, st);
    return e;
}

extern "C" size_t psamp_segtree_update_workspace_size(int64_t cap_pow2, int64_t m) {
    (void)cap_pow2;
    (void)m;
    return 0;
}

extern "C" psamp_status psamp_segtree_update(void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                             const int32_t* idx, const void* prio,
                                             psamp_dtype prio_t, int64_t m, double alpha, void* ws,
                                             size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    if (!is_pow2(cap_pow2) || cap_pow2 > (int64_t(1) << kMaxDepth) || m < 0 || m > kMaxN)
        return PSAMP_E_SIZE;
    if (tree_types(tree_t, prio_t) != PSAMP_OK) return PSAMP_E_DTYPE;
    if (tree_t == PSAMP_F32 && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (m == 0) return PSAMP_OK;
    if (!tree || !idx || !prio) return PSAMP_E_NULL;
    if (!aligned(tree, 16) || !aligned(prio, 4) || !aligned(idx, 4)) return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on() && tree_t == PSAMP_F32) check_prio((const float*)prio, m, st);
    const int D = ilog2_exact(cap_pow2);
    // Batches larger than one workgroup go in order, chunk by chunk: later
    // chunks overwrite earlier ones, which keeps last-write-wins.
    for (int64_t off = 0; off < m; off += kUpdThreads) {
        const int mm = (int)min_<int64_t>(kUpdThreads, m - off);
        if (trace_enabled()) trace_launch("k_tree_update", 1, kUpdThreads, mm);
        if (tree_t == PSAMP_F32)
            hipLaunchKernelGGL((k_tree_update<float, float>), dim3(1), dim3(kUpdThreads), 0, st,
                               (float*)tree, cap_pow2, D, idx + off, (const float*)prio + off, mm,
                               alpha);
        else
            hipLaunchKernelGGL((k_tree_update<uint64_t, uint32_t>), dim3(1), dim3(kUpdThreads), 0,
                               st, (uint64_t*)tree, cap_pow2, D, idx + off,
                               (const uint32_t*)prio + off, mm, 0.0);
        psamp_status e = launch_status();
        if (e != PSAMP_OK) return e;
    }
    return PSAMP_OK;
}

extern "C" psamp_status psamp_segtree_sample(const void* tree, psamp_dtype tree_t,
                                             int64_t cap_pow2, int64_t n_valid, const void* u,
                                             psamp_dtype u_t, int64_t k, int stratified,
                                             int32_t* out_idx, void* stream) {
    if (!is_pow2(cap_pow2) || cap_pow2 > (int64_t(1) << kMaxDepth) || n_valid < 1 ||
        n_valid > cap_pow2 || k < 0 || k > kMaxN)
        return PSAMP_E_SIZE;
    if (stratified != 0 && stratified != 1) return PSAMP_E_PARAM;
    const bool f = tree_t == PSAMP_F32 && u_t == PSAMP_F32;
    const bool in = tree_t == PSAMP_U64 && u_t == PSAMP_U32;
    if (!f && !in) return PSAMP_E_DTYPE;
    if (k == 0) return PSAMP_OK;
    if (!tree || !u || !out_idx) return PSAMP_E_NULL;
    if (!aligned(tree, 16) || !aligned(u, 4) || !aligned(out_idx, 4)) return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on() && f) check_unit((const float*)u, k, st);
    const int D = ilog2_exact(cap_pow2);
    const int k_log2 = is_pow2(k) ? ilog2_exact(k) : -1;
    // Every workgroup copies the top levels (up to 32 KiB) into LDS: large
    // batches use 1024-thread workgroups with 2 draws per thread, so the
    // copies read 8x fewer bytes (2^20 draws over 2^24 leaves: 61 -> 29 us;
    // 4 draws per thread was slower again).
    const bool big = k > 4 * kSampleTreeThreadsBig * kSampleTreeDpt;
    const int nt = big ? kSampleTreeThreadsBig : kSampleTreeThreads;
    const int64_t grid = big ? ceil_div(k, (int64_t)nt * kSampleTreeDpt) : ceil_div(k, nt);
    if (trace_enabled()) trace_launch("k_tree_sample", grid, nt, k);
    if (f) {
        const int lt = min_(TreeTop<float>::levels, D + 1);
        if (big)
            hipLaunchKernelGGL((k_tree_sample<float, kSampleTreeThreadsBig, kSampleTreeDpt>),
                               dim3((unsigned)grid), dim3(nt), 0, st, (const float*)tree,
                               cap_pow2, D, n_valid, u, k, stratified, k_log2, lt, out_idx);
        else
            hipLaunchKernelGGL((k_tree_sample<float, kSampleTreeThreads, 1>),
                               dim3((unsigned)grid), dim3(nt), 0, st, (const float*)tree,
                               cap_pow2, D, n_valid, u, k, stratified, k_log2, lt, out_idx);
    } else {
        const int lt = min_(TreeTop<uint64_t>::levels, D + 1);
        if (big)
            hipLaunchKernelGGL((k_tree_sample<uint64_t, kSampleTreeThreadsBig, kSampleTreeDpt>),
                               dim3((unsigned)grid), dim3(nt), 0, st, (const uint64_t*)tree,
                               cap_pow2, D, n_valid, u, k, stratified, k_log2, lt, out_idx);
        else
            hipLaunchKernelGGL((k_tree_sample<uint64_t, kSampleTreeThreads, 1>),
                               dim3((unsigned)grid), dim3(nt), 0, st, (const uint64_t*)tree,
                               cap_pow2, D, n_valid, u, k, stratified, k_log2, lt, out_idx);
    }
    return launch_status();
}
