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
//  * tiles follow blockIdx (workgroups are dispatched in increasing order on
//    each XCD, so a tile only waits on tiles dispatched before it; no
//    per-tile atomic on a shared counter, which serialises the grid); a
//    workgroup that owns several tiles loads the next one before it scans,
//    looks back and stores the current one; tiles exchange sums through
//    64-bit status words (value and ready flag in one word: relaxed
//    agent-scope atomics suffice across XCDs); every wait is bounded;
//  * fixed-association lookback: tile j in group g (64 tiles per group)
//    adds the published sums of the earlier tiles of its group and the
//    published totals of the earlier groups, each with a fixed DPP tree.
//    No sum depends on timing, so the fp64 CDF is the same bits on every
//    run, and no wait chain is longer than two hops;
//  * the status words alternate between two parities from call to call;
//    each call zeroes the other parity, so the workspace needs no reset.
#include <type_traits>

#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kScanThreads = 256;
constexpr int kScanGroup = 64;           // tiles per lookback group
constexpr int kWsHeaderWords = 32;       // 256-byte header
constexpr int kSlotWords = 4;            // {A par0, A par1, GT par0, GT par1}
constexpr int kMinTile = kScanThreads * 4;
constexpr int kSpinLimit = 1 << 21;      // bounded waits (about a second)

template <class In> struct ScanAcc;
template <> struct ScanAcc<float> { using type = double; };
template <> struct ScanAcc<uint32_t> { using type = uint64_t; };

__device__ __forceinline__ double to_weight(float p, double alpha, const MathLds* M) {
    return pow_prio(p, alpha, M);
}
__device__ __forceinline__ uint64_t to_weight(uint32_t q, double, const MathLds*) {
    return (uint64_t)q;
}

template <class Out, class Acc>
__device__ __forceinline__ Out to_out(Acc v) { return (Out)v; }

template <class Out>
__device__ __forceinline__ void store4(Out* p, const Out (&o)[4]);
template <>
__device__ __forceinline__ void store4<double>(double* p, const double (&o)[4]) {
    reinterpret_cast<double2*>(p)[0] = make_double2(o[0], o[1]);
    reinterpret_cast<double2*>(p)[1] = make_double2(o[2], o[3]);
}
template <>
__device__ __forceinline__ void store4<uint64_t>(uint64_t* p, const uint64_t (&o)[4]) {
    reinterpret_cast<ulonglong2*>(p)[0] = make_ulonglong2(o[0], o[1]);
    reinterpret_cast<ulonglong2*>(p)[1] = make_ulonglong2(o[2], o[3]);
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float (&o)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
}

template <int R, class In>
__device__ __forceinline__ void load_tile(const In* __restrict__ in, int64_t n, int64_t base,
                                          bool vec_ok, In (&v)[R][4]) {
    constexpr int ROW = kScanThreads * 4;
    const int tid = threadIdx.x;
    if (vec_ok && base + (int64_t)R * ROW <= n) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const uint4 x = *reinterpret_cast<const uint4*>(in + base + r * ROW + 4 * tid);
            v[r][0] = __builtin_bit_cast(In, x.x);
            v[r][1] = __builtin_bit_cast(In, x.y);
            v[r][2] = __builtin_bit_cast(In, x.z);
            v[r][3] = __builtin_bit_cast(In, x.w);
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t i = base + r * ROW + 4 * tid + c;
                v[r][c] = i < n ? in[i] : In(0);
            }
    }
}

// Lookback of one tile (called by wave 0).  Tile j of group g needs the
// sums A of tiles g*64 .. j-1 and the group totals GT of groups 0 .. g-1.
// Every status word it needs is requested in the same round trip (one word
// of A and up to kGtWords words of GT per lane), then the wave waits until
// all have arrived.  The sums are then folded in a fixed order -- A by one
// DPP tree over the lanes, GT by one DPP tree per word, words in order -- so
// the result does not depend on timing.  The tile that ends a group
// publishes that group's total; the last tile advances the call counter.
constexpr int kGtWords = 4;          // group totals per lane per round

template <class Acc>
__device__ __forceinline__ void lookback(int tile, int n_tiles, int par, Acc A, uint64_t* slots,
                                         uint64_t* hdr, uint32_t calls, Acc* s_excl) {
    const int lane = threadIdx.x & 63;
    const int g = tile / kScanGroup;
    const int first = g * kScanGroup;
    const int cnt = tile - first;
    const bool need_a = lane < cnt;
    const uint64_t* pa = &slots[kSlotWords * (uint64_t)(first + lane) + par];
    Acc F = Acc(0);
    Acc P = Acc(0);
    bool have_p = false;
    for (int h0 = 0; h0 < g || !have_p; h0 += kGtWords * kWave) {
        bool need_g[kGtWords];
        const uint64_t* pg[kGtWords];
        uint64_t wg[kGtWords];
        uint64_t wa = 0;
        if (!have_p && need_a) wa = load_agent(pa);
#pragma unroll
        for (int w = 0; w < kGtWords; ++w) {
            const int h = h0 + w * kWave + lane;
            need_g[w] = h < g;
            pg[w] = &slots[kSlotWords * (uint64_t)h * kScanGroup + 2 + par];
            wg[w] = need_g[w] ? load_agent(pg[w]) : 0;
        }
        int polls = 0;
        for (;;) {
            bool missing = !have_p && need_a && wa == 0;
#pragma unroll
            for (int w = 0; w < kGtWords; ++w) missing = missing || (need_g[w] && wg[w] == 0);
            if (!__any(missing)) break;
            if (++polls > kSpinLimit) {
                if (lane == 0)
                    __hip_atomic_fetch_or(&hdr[2], (uint64_t)1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
            if (!have_p && need_a && wa == 0) wa = load_agent(pa);
#pragma unroll
            for (int w = 0; w < kGtWords; ++w)
                if (need_g[w] && wg[w] == 0) wg[w] = load_agent(pg[w]);
        }
        if (!have_p) {
            Acc a = Acc(0);
            if (need_a) status_dec(wa, a);
            P = wave_sum(a);
            have_p = true;
            if (cnt == kScanGroup - 1 && lane == 0)
                store_agent(&slots[kSlotWords * (uint64_t)first + 2 + par], status_enc(P + A));
        }
#pragma unroll
        for (int w = 0; w < kGtWords; ++w) {
            Acc x = Acc(0);
            if (need_g[w]) status_dec(wg[w], x);
            if (h0 + w * kWave < g) F = F + wave_sum(x);
        }
    }
    if (lane == 0) {
        *s_excl = F + P;
        if (tile == n_tiles - 1) store_agent(&hdr[0], (uint64_t)(calls + 1u));
    }
}

// Workgroup b handles tiles b, b + G, b + 2G, ... (G = grid size; with
// G = number of tiles each workgroup owns one tile).  The input of the next
// tile is loaded before the current tile's scan, lookback and stores, so HBM
// reads stay in flight while a tile waits on its predecessors.
template <int IPT, class In, class Out>
__global__ __launch_bounds__(kScanThreads) void k_build_cdf(
    const In* __restrict__ in, int64_t n, double alpha, Out* __restrict__ cdf,
    Out* __restrict__ total, uint64_t* __restrict__ ws, int n_tiles,
    uint64_t max_slots, int vec_ok) {
    using Acc = typename ScanAcc<In>::type;
    constexpr bool kFp = std::is_same<In, float>::value;
    constexpr int R = IPT / 4;                    // rows per tile
    constexpr int ROW = kScanThreads * 4;         // elements per row
    constexpr int TILE = ROW * R;

    __shared__ MathLds M;
    __shared__ Acc s_wtot[4][R];
    __shared__ Acc s_excl;
    __shared__ uint32_t s_calls;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int G = (int)gridDim.x;
    uint64_t* hdr = ws;
    uint64_t* slots = ws + kWsHeaderWords;

    // hdr[0] counts calls; its parity selects this call's status words.  The
    // workgroup that owns the last tile advances it once its lookback has
    // seen every other tile's sum -- by then every workgroup has read it.
    if (tid == 0) s_calls = (uint32_t)load_agent(&hdr[0]);
    if (kFp) math_lds_fill(&M, tid, kScanThreads);

    int tile = (int)blockIdx.x;
    In v[R][4];
    load_tile<R, In>(in, n, (int64_t)tile * TILE, vec_ok, v);
    __syncthreads();
    const uint32_t calls = s_calls;
    const int par = (int)(calls & 1u);

    // Zero the other parity for the next call, up to the high-water mark of
    // slots any call has used (never beyond the workspace).
    {
        uint64_t hw = load_agent(&hdr[1]);
        if (hw < (uint64_t)n_tiles) hw = (uint64_t)n_tiles;
        if (hw > max_slots) hw = max_slots;
        if (blockIdx.x == 0 && tid == 0) fetch_max_agent(&hdr[1], (uint64_t)n_tiles);
        const int op = par ^ 1;
        for (uint64_t s = (uint64_t)blockIdx.x * kScanThreads + tid; s < hw;
             s += (uint64_t)G * kScanThreads) {
            slots[kSlotWords * s + op] = 0;
            slots[kSlotWords * s + 2 + op] = 0;
        }
    }

    for (; tile < n_tiles; tile += G) {
        const int64_t base = (int64_t)tile * TILE;

        // ---- weights and the thread-local prefix of each row
        Acc q[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const Acc w = to_weight(v[r][c], alpha, &M);
                q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
            }
        // ---- prefetch the next tile of this workgroup
        if (tile + G < n_tiles) load_tile<R, In>(in, n, (int64_t)(tile + G) * TILE, vec_ok, v);

        // ---- tile-local scan: DPP across the wave, LDS across the 4 waves
        Acc X[R];
        Acc A;
        tile_scan_256<R, Acc>(q, X, A, s_wtot);

        // ---- publish the tile sum, then look back (wave 0)
        if (tid == 0) store_agent(&slots[kSlotWords * (uint64_t)tile + par], status_enc(A));
        if (wave == 0) lookback<Acc>(tile, n_tiles, par, A, slots, hdr, calls, &s_excl);
        __syncthreads();
        const Acc excl = s_excl;

        // ---- outputs
        Out o[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) o[r][c] = to_out<Out>(excl + (X[r] + q[r][c]));

        if (vec_ok && base + TILE <= n) {
#pragma unroll
            for (int r = 0; r < R; ++r) store4<Out>(cdf + base + r * ROW + 4 * tid, o[r]);
        } else {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int64_t i = base + r * ROW + 4 * tid + c;
                    if (i < n) cdf[i] = o[r][c];
                }
        }
        // T = C_{n-1}, written by the thread that owns element n-1.
        const int64_t last = n - 1;
        if (last >= base && last < base + TILE) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (base + r * ROW + 4 * tid + c == last) total[0] = o[r][c];
        }
    }
}

static size_t ws_bytes_for_tiles(int64_t tiles) {
    return (size_t)kWsHeaderWords * 8 + (size_t)tiles * kSlotWords * 8;
}

// Grid: one workgroup per tile (dispatch order alone guarantees progress),
// or, when kScanPersistent, at most one resident wave of workgroups that
// loop over tiles with the next tile prefetched.
constexpr bool kScanPersistent = false;
constexpr int kScanBigIpt = 32;

template <int IPT, class In, class Out>
static psamp_status launch_scan(const void* prio, int64_t n, double alpha, void* cdf, void* total,
                                void* ws, uint64_t max_slots, int vec_ok, hipStream_t st) {
    const int tiles = (int)ceil_div(n, kScanThreads * IPT);
    int grid = tiles;
    if (kScanPersistent) {
        const int cap = resident_grid(reinterpret_cast<const void*>(&k_build_cdf<IPT, In, Out>),
                                      kScanThreads);
        if (cap > 0 && cap < tiles) grid = cap;
    }
    if (trace_enabled()) trace_launch("k_build_cdf", grid, kScanThreads, n);
    hipLaunchKernelGGL((k_build_cdf<IPT, In, Out>), dim3(grid), dim3(kScanThreads), 0, st,
                       (const In*)prio, n, alpha, (Out*)cdf, (Out*)total, (uint64_t*)ws, tiles,
                       max_slots, vec_ok);
    return launch_status();
}

template <class In, class Out>
static psamp_status launch_build_cdf(const void* prio, int64_t n, double alpha, void* cdf,
                                     void* total, void* ws, size_t ws_bytes, hipStream_t st) {
    const uint64_t max_slots = (ws_bytes - (size_t)kWsHeaderWords * 8) / (kSlotWords * 8);
    const int vec_ok = aligned(prio, 16) && aligned(cdf, 16);
    if (n <= (int64_t(1) << 20))
        return launch_scan<4, In, Out>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok, st);
    return launch_scan<kScanBigIpt, In, Out>(prio, n, alpha, cdf, total, ws, max_slots, vec_ok,
                                             st);
}

}  // namespace psamp

using namespace psamp;

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
    hipStream_t st = as_stream(stream);
    if (in) return launch_build_cdf<uint32_t, uint64_t>(prio, n, 0.0, cdf, total, ws, ws_bytes, st);
    if (cdf_t == PSAMP_F64)
        return launch_build_cdf<float, double>(prio, n, alpha, cdf, total, ws, ws_bytes, st);
    return launch_build_cdf<float, float>(prio, n, alpha, cdf, total, ws, ws_bytes, st);
}
