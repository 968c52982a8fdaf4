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
// overwrite a correct parent) and on repeated indices.  Here a batch of up
// to 1024 updates is split by subtree: 64 workgroups, one per subtree below
// the top 6 levels, each deterministically
//   1. keeps the entries whose leaf lies in its subtree (about 16 of 1024);
//   2. sorts their (leaf, batch position) keys;
//   3. keeps the last entry of each run of equal leaves (largest batch
//      position: last write wins);
//   4. fetches the old values of the siblings on each winner's path up to
//      the subtree root (all at once, no per-level latency);
//   5. level by level, lets the first winner under each dirty node (its
//      "owner") form fl(left + right) from its own value, a clean sibling,
//      or the dirty sibling's value held by the next owner (found through a
//      carried index, so in O(1)).
// With up to 64 entries (the usual case) one wave does 2-5: a direct ranking
// in registers, the levels with cross-lane reads; above, the whole
// workgroup: a stable radix sort in LDS and the levels through LDS.  Each
// workgroup publishes its subtree's root in the caller's workspace (value
// and presence in one word), and workgroup 0 recomputes the 63 nodes above
// the subtree roots once it has seen all of them.  (A counter that let the
// last workgroup do it needed a release of every workgroup's stores and two
// more round trips.)  Every dirty node is written once per call, after both of
// its children are final, as fl(left + right) (the top levels are formed
// again in full): the tree stays bit-equal to a fresh build.
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
constexpr int kUpdTopLevels = 6;                 // update: 2^6 subtree workgroups
constexpr size_t kUpdWsBytes = 512;              // update: the subtree roots' words (zero between calls)
constexpr int kRootSpin = 1 << 21;               // bounded wait for the roots (about a second)
static_assert((1 << kUpdTopLevels) <= kWave, "the top levels are formed by one wave");
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

// The value of lane + s (lanes past the end get their own).
__device__ __forceinline__ float shfl_down_v(float x, int s) { return __shfl_down(x, (unsigned)s); }
__device__ __forceinline__ uint64_t shfl_down_v(uint64_t x, int s) {
    const uint32_t lo = (uint32_t)__shfl_down((int)(uint32_t)x, (unsigned)s);
    const uint32_t hi = (uint32_t)__shfl_down((int)(uint32_t)(x >> 32), (unsigned)s);
    return ((uint64_t)hi << 32) | lo;
}

// A subtree root as published in the workspace: value and "present" in one
// 64-bit word (0: not yet), so one agent-scope store carries both.  F32:
// the float's bits with bit 32 set; U64: the value plus one (sums of 2^30
// uint32 leaves stay below 2^62).
__device__ __forceinline__ uint64_t root_enc(float v) {
    return (uint64_t(1) << 32) | (uint64_t)__float_as_uint(v);
}
__device__ __forceinline__ uint64_t root_enc(uint64_t v) { return v + 1u; }
__device__ __forceinline__ void root_dec(uint64_t w, float& v) { v = __uint_as_float((uint32_t)w); }
__device__ __forceinline__ void root_dec(uint64_t w, uint64_t& v) { v = w - 1u; }

// A barrier of one wave: its lanes run in lockstep and its LDS accesses
// complete in order; the wavefront-scope fences keep the compiler from
// moving memory accesses across.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Steps 4 and 5 of the update when a subtree has many winners (up to 1024;
// wl, wj: leaves ascending and their batch positions), thread tid < u
// taking winner tid: each prefetches the old values of all siblings on its
// path up to the subtree root; then level by level the first winner under
// each dirty node (its owner) forms fl(left + right) from its own value, a
// clean sibling from its registers, or the dirty sibling's value from LDS
// (the next owner's, found through the carried index).  The subtree's root
// also goes to *s_root, for the workgroup that forms the levels above.
template <class V, class P>
__device__ __forceinline__ void propagate(V* __restrict__ tree, int64_t cap, int Ds, int u,
                                          const int32_t* wl, const int32_t* wj, const P* pbuf,
                                          V (*vbuf)[kUpdThreads], int32_t (*ebuf)[kUpdThreads],
                                          double alpha, const MathLds* M, V* s_root) {
    const int tid = threadIdx.x;
    const bool act = tid < u;
    int64_t L = 0, Lp = -1;
    V val = V(0);
    int32_t end = tid + 1;
    V sib[kMaxDepth];
    if (act) {
        L = wl[tid];
        Lp = tid > 0 ? (int64_t)wl[tid - 1] : -1;
        val = leaf_value(pbuf[wj[tid]], alpha, M);
#pragma unroll
        for (int d = 0; d < kMaxDepth; ++d)
            if (d < Ds) sib[d] = tree[((cap + L) >> d) ^ 1];
        tree[cap + L] = val;
        if (Ds == 0) *s_root = val;
        vbuf[0][tid] = val;
        ebuf[0][tid] = end;
    }
    __syncthreads();
#pragma unroll
    for (int d = 1; d <= kMaxDepth; ++d) {
        if (d <= Ds) {
            const int bi = (d - 1) & 1;
            const int bo = d & 1;
            const bool own = act && (tid == 0 || ((cap + Lp) >> d) != ((cap + L) >> d));
            if (own) {
                const int64_t cn = (cap + L) >> (d - 1);
                const int64_t N = cn >> 1;
                V left, right;
                int32_t ne = end;
                if ((cn & 1) == 0) {
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
                if (d == Ds) *s_root = val;
                vbuf[bo][tid] = val;
                ebuf[bo][tid] = end;
            }
            __syncthreads();
        }
    }
}

// One batch of up to 1024 updates.  Workgroup s of S = 2^T owns the subtree
// below node S + s (the leaves whose top T of D bits are s): it keeps the
// batch entries that fall there, resolves last-write-wins and recomputes
// every dirty node of its subtree up to that node and publishes the
// subtree's root in the workspace; workgroup 0 then waits for all S roots
// and recomputes the T levels above them (and zeroes the words again).  No workgroup
// waits for another, so the grid need not be resident at once.
template <class V, class P>
__global__ __launch_bounds__(kUpdThreads) void k_tree_update(
    V* __restrict__ tree, int64_t cap, int D, int T, const int32_t* __restrict__ idx,
    const P* __restrict__ prio, int m, double alpha, uint64_t* __restrict__ roots) {
    __shared__ uint64_t keys[kUpdThreads];
    __shared__ P pbuf[kUpdThreads];                      // the batch's values, by position
    __shared__ uint32_t hist[256 * kUpdWaves];           // (digit, wave) counts, then offsets
    __shared__ uint32_t hsum[kUpdWaves];
    __shared__ uint32_t wcount[kUpdWaves];
    __shared__ int32_t wl[kUpdThreads];                  // winner leaves, ascending
    __shared__ int32_t wj[kUpdThreads];                  // their batch positions
    __shared__ V vbuf[2][kUpdThreads];
    __shared__ int32_t ebuf[2][kUpdThreads];
    __shared__ uint32_t s_u;
    __shared__ V s_root;                                 // this subtree's root
    __shared__ uint64_t s_sk[kWave];                     // few entries: keys in order,
    __shared__ int32_t s_sp[kWave];                      //   their compact positions,
    __shared__ V s_lv[kWave];                            //   leaf values by position
    __shared__ MathLds M;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const uint64_t lane_lt = lane == 0 ? 0ull : (~0ull >> (64 - lane));
    const int S = 1 << T;
    const int Ds = D - T;                                // levels inside a subtree
    const int sub = (int)blockIdx.x;
    if (sizeof(P) == 4 && sizeof(V) == 4) math_lds_fill(&M, tid, kUpdThreads);
    // the root as it stands (a subtree without entries publishes it as is)
    if (T > 0 && tid == 0) s_root = tree[S + sub];

    // 1. this subtree's entries, keyed (leaf << 32) | batch position (an entry
    // outside [0, cap) belongs to no subtree); the batch's values by position
    uint64_t key = ~0ull;
    P pv = P(0);
    if (tid < m) {
        const int32_t l = idx[tid];
        pv = prio[tid];
        pbuf[tid] = pv;
        if (l >= 0 && (int64_t)l < cap && ((int64_t)l >> Ds) == sub)
            key = ((uint64_t)(uint32_t)l << 32) | (uint32_t)tid;
    }
    const uint64_t sel = __ballot(key != ~0ull);
    if (lane == 0) wcount[wave] = (uint32_t)__popcll(sel);
    __syncthreads();
    uint32_t pos = (uint32_t)__popcll(sel & lane_lt), c = 0;
    for (int w2 = 0; w2 < kUpdWaves; ++w2) {
        const uint32_t cw = wcount[w2];
        if (w2 < wave) pos += cw;
        c += cw;
    }
    if (c == 0) goto done;                               // (uniform: c is the same everywhere)

    if (c <= (uint32_t)kWave) {
        // 2-5, few entries (the usual case, about m / S): one wave does it.
        // Each entry's thread loads its path siblings and forms its leaf
        // value right away (the loads travel while wave 0 ranks the keys)
        // and parks them in LDS by compact position; wave 0 ranks the keys
        // by direct comparison, keeps the last entry of each leaf, and runs
        // the levels in registers, each owner taking the dirty sibling's
        // value from the next owner's lane.
        V* sibl = &vbuf[0][0];                           // [d * kWave + pos]
        V psib[kMaxDepth];
        V lval = V(0);
        if (key != ~0ull) {
            const int64_t L = (int64_t)(key >> 32);
            keys[pos] = key;
#pragma unroll
            for (int d = 0; d < kMaxDepth; ++d)
                if (d < Ds) psib[d] = tree[((cap + L) >> d) ^ 1];
            lval = leaf_value(pv, alpha, &M);
        }
        __syncthreads();
        if (wave == 0) {
            // keys are distinct (batch positions differ): rank = #smaller
            const uint64_t k_i = (uint32_t)lane < c ? keys[lane] : ~0ull;
            uint32_t rank = 0;
            for (int j = 0; j < (int)c; ++j) rank += readlane(k_i, j) < k_i ? 1u : 0u;
            if ((uint32_t)lane < c) {
                s_sk[rank] = k_i;
                s_sp[rank] = lane;
            }
        }
        if (key != ~0ull) {
#pragma unroll
            for (int d = 0; d < kMaxDepth; ++d)
                if (d < Ds) sibl[d * kWave + pos] = psib[d];
            s_lv[pos] = lval;
        }
        __syncthreads();
        if (wave == 0) {
            // winners: the last key of each run of equal leaves, moved to
            // lanes 0..u-1 in leaf order
            const uint64_t sk = (uint32_t)lane < c ? s_sk[lane] : ~0ull;
            const int sp = (uint32_t)lane < c ? s_sp[lane] : 0;
            const uint64_t nk = __shfl_down(sk, 1);
            const bool win = (uint32_t)lane < c &&
                             ((uint32_t)lane + 1 >= c || (nk >> 32) != (sk >> 32));
            const uint64_t wb = __ballot(win);
            const int u = (int)__popcll(wb);
            if (win) {
                const int wr = (int)__popcll(wb & lane_lt);
                wl[wr] = (int32_t)(sk >> 32);
                wj[wr] = sp;
            }
            wave_sync();
            const bool act = lane < u;
            const int p = act ? wj[lane] : 0;
            const int64_t L = act ? (int64_t)wl[lane] : 0;
            V val = act ? s_lv[p] : V(0);
            const V leafv = val;
            // (every lane shuffles: a lane reading from an inactive lane
            // gets 0, so the shuffle must not sit under a branch)
            const int Li = (int)L;                       // leaves < 2^30
            const int Lprev = __shfl(Li, lane > 0 ? lane - 1 : 0);
            const int Lp = lane > 0 ? Lprev : -1;
            int end = lane + 1;
            uint32_t owned = 0;
            // A compact loop (the clean siblings come from LDS, the level
            // values go to LDS, next to them: slot d - 1 of sibl is read
            // before it is written): unrolled over 30 levels the code spread
            // over many more instruction-cache lines, and a global store in
            // the loop would make each level wait for the previous store.
#pragma unroll 1
            for (int d = 1; d <= Ds; ++d) {
                // the next owner's leaf, value and next owner (every lane
                // reads, before any lane updates its own)
                const int j = end < kWave ? end : kWave - 1;
                const int Lj = __shfl(Li, j);
                const V vj = __shfl(val, j);
                const int ej = __shfl(end, j);
                const V sb = sibl[(d - 1) * kWave + p];
                const bool own = act && (lane == 0 || (Lp >> d) != (Li >> d));
                if (own) {
                    V left, right;
                    int ne = end;
                    if (((Li >> (d - 1)) & 1) == 0) {
                        left = val;
                        if (end < u && (Lj >> d) == (Li >> d)) {
                            right = vj;
                            ne = ej;
                        } else {
                            right = sb;
                        }
                    } else {
                        left = sb;
                        right = val;
                    }
                    val = left + right;
                    end = ne;
                    owned |= 1u << d;
                }
                wave_sync();                       // every lane read slot d - 1
                if (act) sibl[(d - 1) * kWave + lane] = val;
            }
            if (act) {
                tree[cap + L] = leafv;
                if (Ds == 0) s_root = leafv;
#pragma unroll 1
                for (int d = 1; d <= Ds; ++d) {
                    if ((owned >> d) & 1u) {
                        const int64_t N = (cap + L) >> d;
                        const V x = sibl[(d - 1) * kWave + lane];
                        tree[N] = x;
                        if (d == Ds) s_root = x;
                    }
                }
            }
        }
        goto done;
    }

    // 2. many entries: sorted by key, so that equal leaves are adjacent in
    // batch order -- a stable LSD radix sort on the leaf over the whole
    // workgroup (8-bit digits; per pass, ballots rank each key among the
    // lanes of its wave with the same digit, and a digit-major prefix over
    // the per-wave counts places it).
    {
        const int passes = (D + 1 + 7) / 8;
        for (int ps = 0; ps < passes; ++ps) {
            const uint32_t lp = key == ~0ull ? (uint32_t)cap : (uint32_t)(key >> 32);
            const uint32_t d = (lp >> (8 * ps)) & 255u;
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) hist[4 * tid + cc] = 0u;
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
            for (int cc = 0; cc < 4; ++cc) h[cc] = hist[4 * tid + cc];
            const uint32_t loc = (h[0] + h[1]) + (h[2] + h[3]);
            const uint32_t inc = wave_incl_u32(loc);
            if (lane == kWave - 1) hsum[wave] = inc;
            __syncthreads();
            uint32_t ex = inc - loc;
            for (int w2 = 0; w2 < wave; ++w2) ex += hsum[w2];
#pragma unroll
            for (int cc = 0; cc < 4; ++cc) {
                hist[4 * tid + cc] = ex;
                ex += h[cc];
            }
            __syncthreads();
            keys[hist[d * kUpdWaves + wave] + rank] = key;
            __syncthreads();
            key = keys[tid];
        }
    }
    {
        // 3. winners: the last key of each run of equal leaves (largest batch
        // position: last write wins)
        const uint64_t my = (uint32_t)tid < c ? keys[tid] : ~0ull;
        const uint64_t nx = (uint32_t)tid + 1 < c ? keys[tid + 1] : ~0ull;
        const bool win = my != ~0ull && (nx >> 32) != (my >> 32);
        const uint64_t bal = __ballot(win);
        if (lane == 0) wcount[wave] = (uint32_t)__popcll(bal);
        __syncthreads();
        uint32_t wp = (uint32_t)__popcll(bal & lane_lt);
        uint32_t tot = 0;
        for (int w2 = 0; w2 < kUpdWaves; ++w2) {
            const uint32_t cw = wcount[w2];
            if (w2 < wave) wp += cw;
            tot += cw;
        }
        if (win) {
            wl[wp] = (int32_t)(my >> 32);
            wj[wp] = (int32_t)(uint32_t)my;
        }
        if (tid == 0) s_u = tot;
        __syncthreads();
    }
    // 4, 5: the whole workgroup (the winners may be up to 1024)
    propagate<V, P>(tree, cap, Ds, (int)s_u, wl, wj, pbuf, vbuf, ebuf, alpha, &M, &s_root);

done:
    if (T == 0) return;
    // 6. publish this subtree's root; workgroup 0 waits for all S of them
    // (value and presence in one word) and recomputes every node of the top
    // T levels from them -- the same fl(left + right) a fresh build forms --
    // then zeroes the words for the next call.  No workgroup waits for
    // another's start: workgroup 0 waits only for roots that the others
    // publish without waiting.
    __syncthreads();
    if (tid == 0) store_agent(roots + sub, root_enc(s_root));
    if (sub != 0 || wave != 0) return;                   // S <= 64: one wave
    // lane i holds node S + i; at stride s, lane i (a multiple of 2s) forms
    // node S / 2s + i / 2s as (its value) + (lane i + s's value): left + right
    V x = V(0);
    {
        const bool need = lane < S;
        uint64_t w = need ? load_agent(roots + lane) : 1u;
        int spins = kRootSpin;
        asm volatile("" : "+s"(spins));                  // (not unrolled)
        while (__any(w == 0)) {
            __builtin_amdgcn_s_sleep(1);
            if (w == 0) w = load_agent(roots + lane);
            if (--spins == 0) break;
        }
        if (need) root_dec(w, x);
    }
    for (int st = 1; st < S; st <<= 1) {
        const V y = shfl_down_v(x, st);                  // (every lane shuffles)
        if ((lane & (2 * st - 1)) == 0 && lane < S) {
            x = x + y;
            tree[S / (2 * st) + lane / (2 * st)] = x;
        }
    }
    if (tid < S) store_agent(roots + tid, 0u);
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

// The update's workspace: one word per subtree root (zero between calls).
extern "C" size_t psamp_segtree_update_workspace_size(int64_t cap_pow2, int64_t m) {
    (void)cap_pow2;
    (void)m;
    return kUpdWsBytes;
}

extern "C" psamp_status psamp_segtree_update(void* tree, psamp_dtype tree_t, int64_t cap_pow2,
                                             const int32_t* idx, const void* prio,
                                             psamp_dtype prio_t, int64_t m, double alpha, void* ws,
                                             size_t ws_bytes, void* stream) {
    if (!is_pow2(cap_pow2) || cap_pow2 > (int64_t(1) << kMaxDepth) || m < 0 || m > kMaxN)
        return PSAMP_E_SIZE;
    if (tree_types(tree_t, prio_t) != PSAMP_OK) return PSAMP_E_DTYPE;
    if (tree_t == PSAMP_F32 && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (m == 0) return PSAMP_OK;
    if (!tree || !idx || !prio) return PSAMP_E_NULL;
    if (!ws || ws_bytes < kUpdWsBytes) return PSAMP_E_WORKSPACE;
    if (!aligned(tree, 16) || !aligned(prio, 4) || !aligned(idx, 4) || !aligned(ws, 8))
        return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on() && tree_t == PSAMP_F32) check_prio((const float*)prio, m, st);
    const int D = ilog2_exact(cap_pow2);
    // S = 2^T subtree workgroups (each subtree keeps at least one level)
    const int T = D - 1 < kUpdTopLevels ? (D > 1 ? D - 1 : 0) : kUpdTopLevels;
    // Batches larger than one workgroup go in order, chunk by chunk: later
    // chunks overwrite earlier ones, which keeps last-write-wins.
    for (int64_t off = 0; off < m; off += kUpdThreads) {
        const int mm = (int)min_<int64_t>(kUpdThreads, m - off);
        if (trace_enabled()) trace_launch("k_tree_update", int64_t(1) << T, kUpdThreads, mm);
        if (tree_t == PSAMP_F32)
            hipLaunchKernelGGL((k_tree_update<float, float>), dim3(1u << T), dim3(kUpdThreads), 0,
                               st, (float*)tree, cap_pow2, D, T, idx + off,
                               (const float*)prio + off, mm, alpha, (uint64_t*)ws);
        else
            hipLaunchKernelGGL((k_tree_update<uint64_t, uint32_t>), dim3(1u << T),
                               dim3(kUpdThreads), 0, st, (uint64_t*)tree, cap_pow2, D, T,
                               idx + off, (const uint32_t*)prio + off, mm, 0.0, (uint64_t*)ws);
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
