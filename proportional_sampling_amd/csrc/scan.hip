// scan.hip -- p^alpha fused into a single-pass inclusive CDF scan.
//
// What it computes: [PR615] "1. Parallel build_cdf" -- the prefix sum of the
// B priorities that a sampler searches, once per update; [PER] weights
// w_i = p_i^alpha.  fp mode: float priorities, weights and sums in double,
// CDF stored as double (or float).  Integer mode: uint32 priorities, exact
// uint64 sums.
//
// How (MI355X design, not the page's two-level block scan):
//  * one pass over HBM: each element is read once (4 B) and its CDF entry
//    written once (8 B); no block-sums buffer and no second kernel, so there
//    is no size limit beyond int32 indexing;
//  * a tile of 256 threads x IPT elements is read with 16-byte loads (thread
//    t holds 4 consecutive elements of each 1024-element row of the tile);
//  * tile-local scan: serial over each thread's 4 elements, wave64 DPP scan,
//    LDS across the 4 waves;
//  * one workgroup per tile, tiles in blockIdx order (workgroups are
//    dispatched in increasing order on each XCD, so a tile only waits on
//    tiles dispatched before it; no per-tile atomic on a shared counter,
//    which would serialise the grid); tiles exchange sums through 64-bit
//    status words (value and ready flag in one word: relaxed agent-scope
//    atomics suffice across XCDs); every wait is bounded;
//  * fixed-association lookback: tile j in group g (64 tiles per group)
//    adds the published sums of the earlier tiles of its group and the
//    published totals of the earlier groups, each with a fixed DPP tree.
//    No sum depends on timing, so the fp64 CDF is the same bits on every
//    run, and each tile looks back in one round trip;
//  * the status words alternate between two parities from call to call;
//    each call zeroes the other parity, so the workspace needs no reset.
#include "psamp_host.h"
#include "scan_tile.h"

namespace psamp {

// The first b in [lo, n] with C[b] >= t (n if none) of a non-decreasing
// array in LDS, every b < lo being known to lie below t.  A thread's later
// draws land at or after its earlier ones, so it starts at its previous
// result: one read when the draw lands on the same element again (an
// element that takes many draws), a binary search over the rest otherwise.
template <class Acc>
__device__ __forceinline__ int lds_lower_bound_from(const Acc* C, int lo, int n, Acc t) {
    if (lo < n && !(C[lo] < t)) return lo;
    int b = lo + 1, len = n - lo - 1;
    while (len > 1) {
        const int half = len >> 1;
        b = (C[b + half - 1] < t) ? b + half : b;
        len -= half;
    }
    if (len == 1) b += (C[b] < t) ? 1 : 0;
    return b > n ? n : b;
}


constexpr int kScanPark = 4;     // rows of an 8-row tile parked in LDS during the lookback

template <class Out, class Acc>
__device__ __forceinline__ Out to_out(Acc v) { return (Out)v; }

// Four CDF values with 16-byte stores.  NT: streamed out (non-temporal), for
// the large tiles: below 2^20 elements the CDF fits in L2, where a search
// that follows finds it (streaming it out made the PER-mid update as four
// calls 5% slower); above, streaming takes the scan of 2^22 elements from
// 21.6 to 20.0 us and leaves larger scans unchanged.
template <bool NT>
__device__ __forceinline__ void store4(double* p, const double (&o)[4]) {
    if constexpr (NT) {
        store_nt(p, o[0], o[1]);
        store_nt(p + 2, o[2], o[3]);
    } else {
        reinterpret_cast<double2*>(p)[0] = make_double2(o[0], o[1]);
        reinterpret_cast<double2*>(p)[1] = make_double2(o[2], o[3]);
    }
}
template <bool NT>
__device__ __forceinline__ void store4(uint64_t* p, const uint64_t (&o)[4]) {
    if constexpr (NT) {
        store_nt(p, o[0], o[1]);
        store_nt(p + 2, o[2], o[3]);
    } else {
        reinterpret_cast<ulonglong2*>(p)[0] = make_ulonglong2(o[0], o[1]);
        reinterpret_cast<ulonglong2*>(p)[1] = make_ulonglong2(o[2], o[3]);
    }
}
template <bool NT>
__device__ __forceinline__ void store4(float* p, const float (&o)[4]) {
    if constexpr (NT) store_nt(p, o[0], o[1], o[2], o[3]);
    else *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

// The draws of the fused scan + stratified sample (unused otherwise).
struct SampleArgs {
    const void* u;        // float U_i (fp mode) or uint32 r_i (integer mode)
    int64_t k;
    int k_log2;           // log2 k if k is a power of two, else -1 (integer mode)
    int32_t* out;
    // PER (the fused update, fp mode): the priorities (read, then rewritten),
    // the new priorities (may be null), the weights (the drawn priorities'
    // bits are parked there for k_isw_from_slots)
    float* prio = nullptr;
    const float* newp = nullptr;
    float* out_w = nullptr;
};

// One workgroup per tile, tiles in blockIdx order.  VEC: see load_tile.
// SAMPLE: every tile sum and group total and T are already published (by
// k_tile_sums, which also advanced the call counter), so the lookback's
// words are fetched up front and never waited for; the tile then draws its own
// stratified samples -- the thresholds in (excl_j, excl_{j+1}] -- from an
// LDS copy of its CDF values.
// FAST (fp mode, 8-row tiles, alpha <= kFastPowMaxAlpha): p^alpha from
// per-workgroup tables (pow_prio_fast), built while the tile's loads travel.
// PER (with SAMPLE, fp mode): the rest of a PER update for this tile's draws
// -- park each drawn priority's bits in out_w, fold the smallest into this
// call's draw-minimum slots, then rewrite the last draw of each index.
// Plain scans of 8-row tiles with 16-byte loads run three workgroups per CU
// (at most 168 registers; see kScanPark): a workgroup waiting for its
// predecessors' sums no longer leaves its CU's share of HBM idle as often.
// 2^24 elements: 57.2 -> 53.6 us (fp), 56.8 -> 51.8 us (integer).  (The
// element-wise loads of unaligned input need a few more registers.)
template <int R, bool VEC, bool SAMPLE>
constexpr int scan_waves_per_simd() { return (R > 1 && VEC && !SAMPLE) ? 3 : 2; }

template <int IPT, bool VEC, class In, class Out, bool SAMPLE = false, bool FAST = false,
          bool PER = false, bool KEEP = false>
__global__ __launch_bounds__(kScanThreads, (scan_waves_per_simd<IPT / 4, VEC, SAMPLE>())) void k_build_cdf(
    const In* __restrict__ in, int64_t n, double alpha, Out* __restrict__ cdf,
    Out* __restrict__ total, uint64_t* __restrict__ ws, int n_tiles,
    uint64_t max_slots, int vec_ok, SampleArgs sa) {
    using Acc = typename ScanAcc<In>::type;
    constexpr bool kFp = std::is_same<In, float>::value;
    constexpr int R = IPT / 4;                    // rows per tile
    constexpr int ROW = kScanThreads * 4;         // elements per row
    constexpr int TILE = ROW * R;

    static_assert(!FAST || std::is_same<In, float>::value, "FAST is for fp mode");
    __shared__ MathLds M;
    __shared__ PowLds PL;
    __shared__ Acc s_wtot[4][R];
    __shared__ double s_wmax[4][R];
    __shared__ Acc s_excl[2];
    __shared__ Acc s_C[SAMPLE ? TILE : 1];
    __shared__ Acc s_T;
    __shared__ int64_t s_range[2];
    __shared__ uint32_t s_mn[4];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int tile = (int)blockIdx.x;
    const int64_t base = (int64_t)tile * TILE;
    const int tlen = (int)min_<int64_t>(TILE, n - base);   // valid elements, >= 1

    // ws[kHdrCalls] counts calls; its parity selects this call's status
    // words.  The workgroup that owns the last tile advances it once its
    // lookback has seen every other tile's sum -- by then every workgroup
    // has read it.  All first loads (counter, high-water mark, pow tables,
    // priorities) are issued together, so their latencies overlap.
    // (The priorities go first: the counter words are made uniform, which
    // makes the compiler wait for them where they are loaded.  FAST: the
    // small pow tables go first instead, so the per-workgroup tables can be
    // built while the priorities are on their way.)
    In v[R][4];
    MathRegs mr;
    if constexpr (FAST) {
        mr = math_load(tid);
        asm volatile("" ::: "memory");
    }
    load_tile<R, VEC, In>(in + base, tlen, v);
    asm volatile("" ::: "memory");
    if (kFp && !FAST) mr = math_load(tid);
    const uint64_t calls_w = load_agent(&ws[kHdrCalls]);
    const uint64_t hw_w = load_agent(&ws[kHdrHw]);
    // SAMPLE: T is already published (parity of this call); its word goes
    // with the first loads
    const uint64_t t0_w = SAMPLE ? load_agent(&ws[kHdrT + 0]) : 0;
    const uint64_t t1_w = SAMPLE ? load_agent(&ws[kHdrT + 1]) : 0;
    if (kFp) math_store(&M, tid, mr);
    __syncthreads();
    PowCoef pc;
    if constexpr (FAST) {
        pow_tables_build(&PL, &M, alpha, tid, kScanThreads);
        pc = pow_coef(alpha);
        __syncthreads();
    }
    // SAMPLE: k_tile_sums has already advanced the call counter, so this
    // call's parity is that of calls - 1; every sum is published, so wave 0
    // fetches its lookback words now, behind the tile's own loads
    const uint32_t calls = SAMPLE ? (uint32_t)calls_w - 1u : (uint32_t)calls_w;
    const int par = (int)(calls & 1u);
    uint64_t pre[kLbGtWords + 2];
    if constexpr (SAMPLE) {
        if (wave == 0) lb_preload(tile, par, ws, pre);
    }

    // ---- weights and the thread-local prefix of each row
    // (Each row's values are pinned where they are formed: left to itself
    // the compiler sinks every pow's tail to the tile scan and keeps all 32
    // half-done pows live at once.)
    Acc q[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            Acc w;
            if constexpr (FAST) w = pow_prio_fast(v[r][c], &PL, pc);
            else w = to_weight(v[r][c], alpha, &M);
            q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
        }
        if constexpr (kFp) {
#pragma unroll
            for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(q[r][c]));
        }
    }

    // ---- tile-local scan: DPP across the wave, LDS across the 4 waves
    Acc X[R];
    Acc A;
    tile_scan_256<R, Acc>(q, X, A, s_wtot);

    // ---- publish the tile sum; the local values (running max in fp mode)
    // while it travels; then look back (wave 0) while the other waves clear
    // the other parity
    if (tid == 0) store_agent(&ws[a_off((uint32_t)tile, par)], status_enc(A));
    tile_local_values<R, Acc>(q, X, s_wmax);
    // The first kScanPark rows' values wait in LDS during the lookback (plain
    // scans of 8-row tiles), which keeps the kernel within 168 registers.
    constexpr int PK = (R > 1 && !SAMPLE) ? kScanPark : 0;
    __shared__ Acc s_park[PK ? PK * 4 : 1][PK ? kScanThreads : 1];
#pragma unroll
    for (int r = 0; r < PK; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) s_park[r * 4 + c][tid] = q[r][c];
    if (wave == 0)
        lookback<Acc, SAMPLE>(tile, n_tiles, par, A, ws, calls, s_excl, pre);
    else
        clear_other_parity(ws, par, n_tiles, max_slots, hw_w, tid - kWave, kScanThreads - kWave);
    __syncthreads();

    // ---- outputs (monotone and tile-consistent in fp mode); tile-local
    // 32-bit offsets
    const Acc excl = s_excl[0], next = s_excl[1];
    const bool full = vec_ok && tlen == TILE;
    // (t4 is formed again here, so that the 8 row offsets derived from it for
    // the loads are not kept live through the tile; lastk: element (r, k)
    // is the tile's last iff r*ROW + k == lastk)
    Out* __restrict__ tout = cdf + base;
    int t4 = 4 * tid;
    asm volatile("" : "+v"(t4));
    const int lastk = tlen - 1 - t4;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e0 = r * ROW + t4;
        Out o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const Acc x = r < PK ? s_park[r * 4 + k][t4 >> 2] : q[r][k];
            const Acc c = tile_value<Acc>(x, excl, next, r * ROW + k == lastk);
            o[k] = to_out<Out>(c);
            if constexpr (SAMPLE) s_C[e0 + k] = c;
        }
        if (full) {
            store4<(R > 1 && !KEEP)>(tout + e0, o);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (r * ROW + k <= lastk) tout[e0 + k] = o[k];
        }
        // T = C_{n-1}, written by the thread that owns element n-1.
        if (tile == n_tiles - 1) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (r * ROW + k == lastk) total[0] = o[k];
        }
    }

    if constexpr (SAMPLE) {
        // this tile's draws: [first t_i > excl_j, first t_i > excl_{j+1})
        const KDiv kd(sa.k);
        if (wave == 0) {
            uint64_t tw = readlane(par ? t1_w : t0_w, 0);   // normally already present
            const uint32_t off[1] = {(uint32_t)(kHdrT + par)};
            const bool need[1] = {lane == 0 && tw == 0};
            uint64_t w[1];
            wait_words<1>(ws, off, need, w);
            if (tw == 0) tw = readlane(w[0], 0);
            Acc T;
            status_dec(tw, T);
            int64_t rr;
            if constexpr (kFp)
                rr = first_above2(excl, next, T, StratFp{(const float*)sa.u, kd, T}, sa.k);
            else
                rr = first_above2(excl, next, T,
                                  StratInt{(const uint32_t*)sa.u, sa.k, T, sa.k_log2}, sa.k);
            if (lane == 0) {
                s_range[0] = tile == 0 ? 0 : rr;
                s_T = T;
            }
            if (lane == 32) s_range[1] = tile == n_tiles - 1 ? sa.k : rr;
        }
        __syncthreads();
        const int64_t i_lo = s_range[0], i_hi = s_range[1];
        const Acc T = s_T;
        uint32_t mn = 0xFFFFFFFFu;
        // Four draws a round, their fractions (and then their drawn
        // priorities) loaded together; each search starts at the thread's
        // previous element, since its draws land in increasing order (one
        // LDS read per draw when an element takes many).
        int bp = 0;
        for (int64_t i0 = i_lo + tid; i0 < i_hi; i0 += 4 * kScanThreads) {
            uint32_t uq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + q * kScanThreads;
                uq[q] = ((const uint32_t*)sa.u)[i < i_hi ? i : i0];
            }
            int bq[4] = {0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t i = i0 + q * kScanThreads;
                if (i < i_hi) {
                    Acc t;
                    if constexpr (kFp)
                        t = strat_threshold(i, __uint_as_float(uq[q]), kd, T);
                    else
                        t = int_threshold((uint64_t)i, uq[q], (uint64_t)sa.k, T, 1, sa.k_log2);
                    int b = lds_lower_bound_from(s_C, bp, tlen, t);
                    if (b >= tlen) b = tlen - 1;
                    bp = b;
                    bq[q] = b;
                    sa.out[i] = (int32_t)(base + b);
                }
            }
            if constexpr (PER) {
                // the drawn priorities, as read before any rewrite of this tile
                uint32_t kq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) kq[q] = __float_as_uint(sa.prio[base + bq[q]]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t i = i0 + q * kScanThreads;
                    if (i < i_hi) {
                        reinterpret_cast<uint32_t*>(sa.out_w)[i] = kq[q];
                        mn = kq[q] < mn ? kq[q] : mn;
                    }
                }
            }
        }
        if constexpr (PER) {
            mn = wave_min_u32(mn);
            if (lane == 0) s_mn[wave] = mn;
            __syncthreads();          // every drawn priority has been read
            if (tid == 0) {
                const uint32_t m = min_(min_(s_mn[0], s_mn[1]), min_(s_mn[2], s_mn[3]));
                if (m != 0xFFFFFFFFu)
                    fetch_max_agent(&ws[kHdrDrawMin + kDrawMinSlots * par + (tile & 3)],
                                    (uint64_t)(~m));
            }
            // rewrite: draw i is the last of its index unless draw i + 1 (in
            // this tile) lands on the same element -- the search's own test
            if (sa.newp != nullptr) {
                for (int64_t i0 = i_lo + tid; i0 < i_hi; i0 += 4 * kScanThreads) {
                    int32_t bq[4];
                    float un[4], nq[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {      // loads first, in range
                        const int64_t i = i0 + q * kScanThreads;
                        const int64_t ic = i < i_hi ? i : i0;
                        bq[q] = sa.out[ic] - (int32_t)base;
                        un[q] = ((const float*)sa.u)[ic + 1 < i_hi ? ic + 1 : ic];
                        nq[q] = sa.newp[ic];
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t i = i0 + q * kScanThreads;
                        if (i < i_hi) {
                            const int b = bq[q];
                            // (draw i + 1 lands on b or later; on the tile's
                            // last element it can only land on b)
                            bool last = i + 1 >= i_hi;
                            if (!last && b < tlen - 1) {
                                const Acc tn = strat_threshold(i + 1, un[q], kd, T);
                                last = s_C[b] < tn;
                            }
                            if (last) sa.prio[base + b] = nq[q];
                        }
                    }
                }
            }
        }
    }
}

// The first pass of a reduce-then-scan: the tile sums A_j (the same
// arithmetic as the scan's), published in the scan's status words.  Tiles
// count per group of 64 (the group's MIN words of this parity serve as the
// counters; the next call zeroes them): the tile that completes a group
// publishes its total GT_g, and the group that completes last forms T with
// the scan's association, publishes it and advances the call counter (every
// tile has read it by then: each counted itself in after reading it).  One counter per group keeps the
// atomics on 64-tile-wide addresses apart instead of serialising all tiles
// on one word.
template <int IPT, bool VEC, class In, bool FAST = false>
__global__ __launch_bounds__(kScanThreads) void k_tile_sums(const In* __restrict__ in, int64_t n,
                                                            double alpha,
                                                            uint64_t* __restrict__ ws,
                                                            int n_tiles) {
    using Acc = typename ScanAcc<In>::type;
    constexpr bool kFp = std::is_same<In, float>::value;
    constexpr int R = IPT / 4;
    constexpr int TILE = kScanThreads * 4 * R;

    __shared__ MathLds M;
    __shared__ PowLds PL;
    __shared__ Acc s_wtot[4][R];
    __shared__ int s_role;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int tile = (int)blockIdx.x;
    const int g = tile / kScanGroup;
    const int G = (n_tiles + kScanGroup - 1) / kScanGroup;
    const int64_t base = (int64_t)tile * TILE;
    const int tlen = (int)min_<int64_t>(TILE, n - base);

    In v[R][4];
    MathRegs mr;
    if constexpr (FAST) {
        mr = math_load(tid);
        asm volatile("" ::: "memory");
    }
    load_tile<R, VEC, In>(in + base, tlen, v);
    asm volatile("" ::: "memory");
    if (kFp && !FAST) mr = math_load(tid);
    const uint64_t calls_w = load_agent(&ws[kHdrCalls]);
    if (kFp) math_store(&M, tid, mr);
    __syncthreads();
    PowCoef pc;
    if constexpr (FAST) {
        pow_tables_build(&PL, &M, alpha, tid, kScanThreads);
        pc = pow_coef(alpha);
        __syncthreads();
    }
    const int par = (int)(calls_w & 1u);

    Acc q[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            Acc w;
            if constexpr (FAST) w = pow_prio_fast(v[r][c], &PL, pc);
            else w = to_weight(v[r][c], alpha, &M);
            q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
        }
        if constexpr (kFp) {
#pragma unroll
            for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(q[r][c]));
        }
    }
    Acc X[R];
    Acc A;
    tile_scan_256<R, Acc>(q, X, A, s_wtot);
    if (tid == 0) {
        store_agent(&ws[a_off((uint32_t)tile, par)], status_enc(A));
        const uint64_t in_group = (uint64_t)min_(kScanGroup, n_tiles - g * kScanGroup);
        s_role = fetch_add_agent(&ws[min_off((uint32_t)(g * kScanGroup), par)], 1) ==
                 in_group - 1;
    }
    __syncthreads();
    if (!s_role || wave != 0) return;

    // the tile that completes group g: GT_g = the DPP tree over its sums
    {
        const int t = g * kScanGroup + lane;
        const uint32_t off[1] = {a_off((uint32_t)(t < n_tiles ? t : 0), par)};
        const bool need[1] = {t < n_tiles};
        uint64_t w[1];
        wait_words<1>(ws, off, need, w);
        const Acc gt = wave_sum(need[0] ? status_value<Acc>(w[0]) : Acc(0));
        int last = 0;
        if (lane == 0) {
            store_agent(&ws[gt_off((uint32_t)g, par)], status_enc(gt));
            last = fetch_add_agent(&ws[kHdrExit], 1) == (uint64_t)G - 1;
        }
        if (!__builtin_amdgcn_readfirstlane(last)) return;
    }
    // the group that completes last: T = Outer(GT_0, ..., GT_{G-1}) (lane h
    // mod 64 adds its leaves in increasing h, then the tree) -- the value the
    // scan's last tile forms as C_{n-1}
    Acc acc = Acc(0);
    for (int s0 = 0; s0 * kWave < G; ++s0) {
        const int h = s0 * kWave + lane;
        const uint32_t off[1] = {gt_off((uint32_t)(h < G ? h : 0), par)};
        const bool need[1] = {h < G};
        uint64_t w[1];
        wait_words<1>(ws, off, need, w);
        if (need[0]) acc = acc + status_value<Acc>(w[0]);
    }
    const Acc T = wave_sum(acc);
    if (lane == 0) {
        store_agent(&ws[kHdrT + par], status_enc(T));
        store_agent(&ws[kHdrExit], 0);
        store_agent(&ws[kHdrCalls], (uint64_t)((uint32_t)calls_w + 1u));
    }
}

// The table-driven pow for fp mode on 8-row tiles when alpha allows it.
template <int IPT, class In>
static bool use_fast_pow(double alpha) {
    return IPT == 32 && std::is_same<In, float>::value && alpha <= kFastPowMaxAlpha;
}

template <int IPT, class In, class Out, bool FAST, bool KEEP>
static psamp_status launch_scan_t(const void* prio, int64_t n, double alpha, void* cdf,
                                  void* total, void* ws, uint64_t max_slots, int vec_ok,
                                  hipStream_t st) {
    const int tiles = (int)ceil_div(n, kScanThreads * IPT);
    if (trace_enabled()) trace_launch("k_build_cdf", tiles, kScanThreads, n);
    const bool vec_in = aligned(prio, 16) && n % 4 == 0;
    if (vec_in)
        hipLaunchKernelGGL((k_build_cdf<IPT, true, In, Out, false, FAST, false, KEEP>), dim3(tiles),
                           dim3(kScanThreads), 0, st, (const In*)prio, n, alpha, (Out*)cdf,
                           (Out*)total, (uint64_t*)ws, tiles, max_slots, vec_ok, SampleArgs{});
    else
        hipLaunchKernelGGL((k_build_cdf<IPT, false, In, Out, false, FAST, false, KEEP>), dim3(tiles),
                           dim3(kScanThreads), 0, st, (const In*)prio, n, alpha, (Out*)cdf,
                           (Out*)total, (uint64_t*)ws, tiles, max_slots, vec_ok, SampleArgs{});
    return launch_status();
}

template <int IPT, class In, class Out, bool KEEP>
static psamp_status launch_scan(const void* prio, int64_t n, double alpha, void* cdf, void* total,
                                void* ws, uint64_t max_slots, int vec_ok, hipStream_t st) {
    if constexpr (IPT == 32 && std::is_same<In, float>::value) {
        if (use_fast_pow<IPT, In>(alpha))
            return launch_scan_t<IPT, In, Out, true, KEEP>(prio, n, alpha, cdf, total, ws,
                                                           max_slots, vec_ok, st);
    }
    return launch_scan_t<IPT, In, Out, false, KEEP>(prio, n, alpha, cdf, total, ws, max_slots,
                                                    vec_ok, st);
}

// KEEP: large tiles store the CDF like small ones (not streamed out), so that
// a search right after it finds it in the Infinity Cache.
template <class In, class Out, bool KEEP = false>
static psamp_status launch_build_cdf(const void* prio, int64_t n, double alpha, void* cdf,
                                     void* total, void* ws, size_t ws_bytes, hipStream_t st) {
    const uint64_t max_slots = ws_tile_capacity(ws_bytes);
    const int vec_ok = aligned(cdf, 16);   // 16-byte stores of whole tiles
    if (scan_rows_for(n) == 1)
        return launch_scan<4, In, Out, KEEP>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok,
                                             st);
    return launch_scan<32, In, Out, KEEP>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok, st);
}

// The fused scan + stratified sample: k_tile_sums, then the scan with
// SAMPLE.  CDF, T and indices are the bits of psamp_build_cdf + psamp_sample.
template <int IPT, class In, bool FAST>
static psamp_status launch_scan_sample_t(const void* prio, int64_t n, double alpha, void* cdf,
                                         void* total, void* ws, uint64_t max_slots, int vec_ok,
                                         SampleArgs sa, hipStream_t st) {
    using Acc = typename ScanAcc<In>::type;
    const int tiles = (int)ceil_div(n, kScanThreads * IPT);
    if (trace_enabled()) trace_launch("k_tile_sums+k_build_cdf<sample>", tiles, kScanThreads, n);
    const bool vec_in = aligned(prio, 16) && n % 4 == 0;
    if (vec_in) {
        hipLaunchKernelGGL((k_tile_sums<IPT, true, In, FAST>), dim3(tiles), dim3(kScanThreads), 0,
                           st, (const In*)prio, n, alpha, (uint64_t*)ws, tiles);
        hipLaunchKernelGGL((k_build_cdf<IPT, true, In, Acc, true, FAST>), dim3(tiles),
                           dim3(kScanThreads), 0, st, (const In*)prio, n, alpha, (Acc*)cdf,
                           (Acc*)total, (uint64_t*)ws, tiles, max_slots, vec_ok, sa);
    } else {
        hipLaunchKernelGGL((k_tile_sums<IPT, false, In, FAST>), dim3(tiles), dim3(kScanThreads), 0,
                           st, (const In*)prio, n, alpha, (uint64_t*)ws, tiles);
        hipLaunchKernelGGL((k_build_cdf<IPT, false, In, Acc, true, FAST>), dim3(tiles),
                           dim3(kScanThreads), 0, st, (const In*)prio, n, alpha, (Acc*)cdf,
                           (Acc*)total, (uint64_t*)ws, tiles, max_slots, vec_ok, sa);
    }
    return launch_status();
}

template <int IPT, class In>
static psamp_status launch_scan_sample(const void* prio, int64_t n, double alpha, void* cdf,
                                       void* total, void* ws, uint64_t max_slots, int vec_ok,
                                       SampleArgs sa, hipStream_t st) {
    if constexpr (IPT == 32 && std::is_same<In, float>::value) {
        if (use_fast_pow<IPT, In>(alpha))
            return launch_scan_sample_t<IPT, In, true>(prio, n, alpha, cdf, total, ws, max_slots,
                                                       vec_ok, sa, st);
    }
    return launch_scan_sample_t<IPT, In, false>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok,
                                                sa, st);
}

// The IS weights of a fused update whose draws parked their priorities in
// out_w (k_build_cdf with PER): the smallest drawn priority is read from
// this call's draw-minimum slots, then IS_i = (p_min / p_i)^(alpha beta) with
// the arithmetic of psamp_is_weights.
constexpr int kIswSlotThreads = 1024;
constexpr int kIswSlotPer = 4;
__global__ __launch_bounds__(kIswSlotThreads) void k_isw_from_slots(int64_t k, double e,
                                                                   const uint64_t* __restrict__ ws,
                                                                   float* __restrict__ out) {
    __shared__ MathLds M;
    const int tid = threadIdx.x;
    math_lds_fill(&M, tid, kIswSlotThreads);
    __syncthreads();
    // k_tile_sums of this call has advanced the counter
    const int par = (int)((load_agent(&ws[kHdrCalls]) - 1u) & 1u);
    uint64_t mx = 0;
#pragma unroll
    for (int q = 0; q < kDrawMinSlots; ++q)
        mx = max_(mx, load_agent(&ws[kHdrDrawMin + kDrawMinSlots * par + q]));
    const double pmin = (double)__uint_as_float(~(uint32_t)mx);
    const double lpmin = pmin > 0.0 ? log2_sig32(pmin, &M) : 0.0;
    const int64_t b0 = (int64_t)blockIdx.x * kIswSlotThreads * kIswSlotPer;
#pragma unroll
    for (int j = 0; j < kIswSlotPer; ++j) {
        const int64_t i = b0 + j * kIswSlotThreads + tid;
        if (i < k) {
            const double p = (double)__uint_as_float(reinterpret_cast<const uint32_t*>(out)[i]);
            out[i] = is_weight(pmin, lpmin, p, e, &M);
        }
    }
}

template <int IPT, bool FAST>
static psamp_status launch_per_update_t(float* prio, int64_t n, double alpha, double ab,
                                        const float* u, int64_t k, const float* newp,
                                        int32_t* out_idx, float* out_w, double* cdf,
                                        double* total, uint64_t* ws, uint64_t max_slots,
                                        int vec_ok, hipStream_t st) {
    const int tiles = (int)ceil_div(n, kScanThreads * IPT);
    if (trace_enabled()) trace_launch("k_tile_sums+k_build_cdf<per>+k_isw", tiles, kScanThreads, n);
    SampleArgs sa{u, k, -1, out_idx};
    sa.prio = prio;
    sa.newp = newp;
    sa.out_w = out_w;
    if (aligned(prio, 16) && n % 4 == 0) {
        hipLaunchKernelGGL((k_tile_sums<IPT, true, float, FAST>), dim3(tiles), dim3(kScanThreads),
                           0, st, prio, n, alpha, ws, tiles);
        hipLaunchKernelGGL((k_build_cdf<IPT, true, float, double, true, FAST, true>), dim3(tiles),
                           dim3(kScanThreads), 0, st, prio, n, alpha, cdf, total, ws, tiles,
                           max_slots, vec_ok, sa);
    } else {
        hipLaunchKernelGGL((k_tile_sums<IPT, false, float, FAST>), dim3(tiles), dim3(kScanThreads),
                           0, st, prio, n, alpha, ws, tiles);
        hipLaunchKernelGGL((k_build_cdf<IPT, false, float, double, true, FAST, true>), dim3(tiles),
                           dim3(kScanThreads), 0, st, prio, n, alpha, cdf, total, ws, tiles,
                           max_slots, vec_ok, sa);
    }
    psamp_status s = launch_status();
    if (s != PSAMP_OK) return s;
    const int64_t g = ceil_div(k, (int64_t)kIswSlotThreads * kIswSlotPer);
    hipLaunchKernelGGL(k_isw_from_slots, dim3((unsigned)g), dim3(kIswSlotThreads), 0, st, k, ab,
                       ws, out_w);
    return launch_status();
}

psamp_status launch_per_update(float* prio, int64_t n, double alpha, double beta, const float* u,
                               int64_t k, const float* newp, int32_t* out_idx, float* out_w,
                               double* cdf, double* total, void* ws, size_t ws_bytes,
                               hipStream_t st) {
    const uint64_t max_slots = ws_tile_capacity(ws_bytes);
    const int vec_ok = aligned(cdf, 16);
    uint64_t* w = (uint64_t*)ws;
    const double ab = alpha * beta;
    if (scan_rows_for(n) == 1)
        return launch_per_update_t<4, false>(prio, n, alpha, ab, u, k, newp, out_idx, out_w, cdf,
                                             total, w, max_slots, vec_ok, st);
    if (use_fast_pow<32, float>(alpha))
        return launch_per_update_t<32, true>(prio, n, alpha, ab, u, k, newp, out_idx, out_w, cdf,
                                             total, w, max_slots, vec_ok, st);
    return launch_per_update_t<32, false>(prio, n, alpha, ab, u, k, newp, out_idx, out_w, cdf,
                                          total, w, max_slots, vec_ok, st);
}

}  // namespace psamp

using namespace psamp;

// psamp_build_cdf after its argument checks (KEEP: see launch_build_cdf).
template <bool KEEP>
static psamp_status build_cdf_checked(const void* prio, psamp_dtype prio_t, int64_t n,
                                      double alpha, void* cdf, psamp_dtype cdf_t, void* total,
                                      void* ws, size_t ws_bytes, void* stream) {
    const bool in = prio_t == PSAMP_U32;
    hipStream_t st = as_stream(stream);
    const bool chk = check_on();
    if (chk && !in) check_prio((const float*)prio, n, st);
    psamp_status e;
    if (in)
        e = launch_build_cdf<uint32_t, uint64_t, KEEP>(prio, n, 0.0, cdf, total, ws, ws_bytes, st);
    else if (cdf_t == PSAMP_F64)
        e = launch_build_cdf<float, double, KEEP>(prio, n, alpha, cdf, total, ws, ws_bytes, st);
    else e = launch_build_cdf<float, float, KEEP>(prio, n, alpha, cdf, total, ws, ws_bytes, st);
    if (chk && e == PSAMP_OK) check_total(total, cdf_t, st);
    return e;
}

extern "C" size_t psamp_build_cdf_workspace_size(int64_t n) {
    if (n < 1 || n > kMaxN) return 0;
    return ws_bytes_for_tiles(ceil_div(n, kMinTile));
}

extern "C" psamp_status psamp_build_cdf(const void* prio, psamp_dtype prio_t, int64_t n,
                                        double alpha, void* cdf, psamp_dtype cdf_t, void* total,
                                        void* ws, size_t ws_bytes, void* stream) {
    if (!prio || !cdf || !total) return PSAMP_E_NULL;
    if (n < 1 || n > kMaxN) return PSAMP_E_SIZE;
    const bool fp = prio_t == PSAMP_F32 && (cdf_t == PSAMP_F64 || cdf_t == PSAMP_F32);
    const bool in = prio_t == PSAMP_U32 && cdf_t == PSAMP_U64;
    if (!fp && !in) return PSAMP_E_DTYPE;
    if (fp && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (!ws) return PSAMP_E_WORKSPACE;
    if (ws_bytes < psamp_build_cdf_workspace_size(n)) return PSAMP_E_WORKSPACE;
    const size_t osz = cdf_t == PSAMP_F32 ? 4 : 8;
    if (!aligned(prio, 4) || !aligned(cdf, osz) || !aligned(total, osz) || !aligned(ws, 8))
        return PSAMP_E_ALIGN;
    return build_cdf_checked<false>(prio, prio_t, n, alpha, cdf, cdf_t, total, ws, ws_bytes,
                                    stream);
}

extern "C" psamp_status psamp_build_cdf_sample(const void* prio, psamp_dtype prio_t, int64_t n,
                                               double alpha, const void* u, psamp_dtype u_t,
                                               int64_t k, void* cdf, psamp_dtype cdf_t,
                                               void* total, int32_t* out_idx, void* ws,
                                               size_t ws_bytes, void* stream) {
    if (!prio || !cdf || !total) return PSAMP_E_NULL;
    if (n < 1 || n > kMaxN || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    const bool fp = prio_t == PSAMP_F32 && u_t == PSAMP_F32 &&
                    (cdf_t == PSAMP_F64 || cdf_t == PSAMP_F32);
    const bool in = prio_t == PSAMP_U32 && u_t == PSAMP_U32 && cdf_t == PSAMP_U64;
    if (!fp && !in) return PSAMP_E_DTYPE;
    if (fp && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (k > 0 && (!u || !out_idx)) return PSAMP_E_NULL;
    if (!ws) return PSAMP_E_WORKSPACE;
    if (ws_bytes < psamp_build_cdf_workspace_size(n)) return PSAMP_E_WORKSPACE;
    const size_t osz = cdf_t == PSAMP_F32 ? 4 : 8;
    if (!aligned(prio, 4) || !aligned(cdf, osz) || !aligned(total, osz) || !aligned(ws, 8) ||
        (k > 0 && (!aligned(u, 4) || !aligned(out_idx, 4))))
        return PSAMP_E_ALIGN;
    // The two calls (same results) when there is nothing to draw, for a
    // float CDF (whose rounding breaks the tiles' ownership of the
    // thresholds), and for large tiles with dense draws: there the one
    // kernel's draw phase (a search per draw in the tile's LDS copy, behind
    // a search for the tile's first draw) lengthens every tile's life at two
    // workgroups per CU by more than the CDF-side sampler takes to re-read
    // the CDF -- measured 100.1 us against 82.9 us for 2^20 draws over 2^24
    // LogNormal priorities, while up to 2^20 priorities the one kernel is
    // 1-3 us faster.
    if (k == 0 || cdf_t == PSAMP_F32 || (scan_rows_for(n) != 1 && 64 * k >= n)) {
        // (the CDF kept in the Infinity Cache for the sample that reads it)
        psamp_status s = k == 0 ? build_cdf_checked<false>(prio, prio_t, n, alpha, cdf, cdf_t,
                                                           total, ws, ws_bytes, stream)
                                : build_cdf_checked<true>(prio, prio_t, n, alpha, cdf, cdf_t,
                                                          total, ws, ws_bytes, stream);
        if (s != PSAMP_OK || k == 0) return s;
        return psamp_sample(cdf, cdf_t, n, total, u, u_t, k, 1, out_idx, stream);
    }
    hipStream_t st = as_stream(stream);
    const uint64_t max_slots = ws_tile_capacity(ws_bytes);
    const int vec_ok = aligned(cdf, 16);
    const SampleArgs sa{u, k, is_pow2(k) ? ilog2_exact(k) : -1, out_idx};
    const bool chk = check_on();
    if (chk && fp) {
        check_prio((const float*)prio, n, st);
        check_unit((const float*)u, k, st);
    }
    psamp_status e;
    if (in) {
        if (scan_rows_for(n) == 1)
            e = launch_scan_sample<4, uint32_t>(prio, n, 0.0, cdf, total, ws, max_slots, vec_ok,
                                                sa, st);
        else
            e = launch_scan_sample<32, uint32_t>(prio, n, 0.0, cdf, total, ws, max_slots, vec_ok,
                                                 sa, st);
    } else if (scan_rows_for(n) == 1) {
        e = launch_scan_sample<4, float>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok, sa,
                                         st);
    } else {
        e = launch_scan_sample<32, float>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok, sa,
                                          st);
    }
    if (chk && e == PSAMP_OK) check_total(total, cdf_t, st);
    return e;
}
