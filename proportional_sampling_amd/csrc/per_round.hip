// per_round.hip -- one prioritized-replay minibatch update in one kernel.
//
// What it computes is exactly the composition of the separate calls:
//   psamp_build_cdf (p^alpha, inclusive CDF, T)      [PR615] "1. Parallel
//   psamp_sample    (k stratified draws)               build_cdf"; [PF]
//   psamp_is_weights(IS = (p_min / p_i)^(alpha beta))  searchsorted; [PER]
//   psamp_scatter_lww(prio[idx_i] = new_i, grouped)    [SEGT] "Integration"
// -- the PER update the PufferLib page runs once per minibatch (32 to 128
// times per train call), the hot loop of the trainer.
//
// Why one kernel: once T is known, everything a stratified draw needs lies
// in one tile.  The CDF of scan_tile.h is exactly monotone and every tile j
// owns the thresholds in (excl_j, excl_{j+1}], so after the scan each tile
// (one workgroup) keeps its CDF values and priorities in LDS and
//   1. waits for T (published by the last tile after its lookback);
//   2. finds its samples: the stratified thresholds are non-decreasing in i,
//      so they form one index range, located from the stratum estimate
//      i ~ B k / T and checked exactly on a 32-wide window;
//   3. searches each sample's threshold in LDS and writes the index;
//   4. publishes the smallest priority it drew and waits for every tile's;
//   5. writes the IS weights and, for the last draw of each index (draws of
//      one index are adjacent and all in this tile), the new priority --
//      only this tile ever reads that part of the priority array, so no
//      other synchronisation is needed.
// The grid is one workgroup per tile and must be resident at once (two
// grid-wide waits); the host checks the occupancy and otherwise runs the
// separate kernels, which give the same bits.
#include <mutex>

#include "psamp_host.h"
#include "scan_tile.h"

namespace psamp {

constexpr int kULds = 8192;   // k up to this: the thresholds' fractions are staged in LDS

// UL: U (k <= kULds values) is copied to LDS at the start, so locating and
// searching the draws touches no global memory.  VEC: see load_tile.  FAST:
// p^alpha from per-workgroup tables, as the scan does on the same tiles.
template <int R, bool UL, bool VEC, bool FAST = false>
__global__ __launch_bounds__(kScanThreads) void k_per_round(
    float* __restrict__ prio, int64_t n, double alpha, double ab, const float* __restrict__ U,
    int64_t k, const float* __restrict__ newp, int32_t* __restrict__ out_idx,
    float* __restrict__ out_w, double* __restrict__ cdf, double* __restrict__ total,
    uint64_t* __restrict__ ws, int n_tiles, uint64_t max_slots, int vec_ok) {
    constexpr int ROW = kScanThreads * 4;
    constexpr int TILE = ROW * R;

    __shared__ MathLds M;
    __shared__ PowLds PL;
    __shared__ double s_wtot[4][R];
    __shared__ double s_wmax[4][R];
    __shared__ double s_lb[3];
    __shared__ double s_C[TILE];
    __shared__ float s_p[TILE];
    __shared__ float s_U[UL ? kULds : 1];
    __shared__ int64_t s_range[2];
    __shared__ uint32_t s_min, s_gmin;
    __shared__ int s_b[kScanThreads + 1];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int tile = (int)blockIdx.x;
    const bool last_tile = tile == n_tiles - 1;
    const int64_t base = (int64_t)tile * TILE;
    const int tlen = (int)min_<int64_t>(TILE, n - base);

    // All first loads (counter, high-water mark, pow tables, priorities) are
    // issued together, so their latencies overlap.
    // (The priorities go first: the counter words are made uniform, which
    // makes the compiler wait for them where they are loaded.)
    float v[R][4];
    MathRegs mr;
    if constexpr (FAST) {
        mr = math_load(tid);
        asm volatile("" ::: "memory");
    }
    load_tile<R, VEC, float>(prio + base, tlen, v);
    asm volatile("" ::: "memory");
    if constexpr (!FAST) mr = math_load(tid);
    const uint64_t calls_w = load_agent(&ws[kHdrCalls]);
    const uint64_t hw_w = load_agent(&ws[kHdrHw]);
    math_store(&M, tid, mr);
    if (tid == 0) s_min = 0xFFFFFFFFu;
    const float* Us = UL ? s_U : U;
    __syncthreads();
    PowCoef pc;
    if constexpr (FAST) {
        pow_tables_build(&PL, &M, alpha, tid, kScanThreads);
        pc = pow_coef(alpha);
        __syncthreads();
    }
    const uint32_t calls = (uint32_t)calls_w;
    const int par = (int)(calls & 1u);
    const KDiv kd(k);

    // ---- 1. scan (as psamp_build_cdf); every tile learns T in its lookback
    double q[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            double w;
            if constexpr (FAST) w = pow_prio_fast(v[r][c], &PL, pc);
            else w = pow_prio(v[r][c], alpha, &M);
            q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
            s_p[r * ROW + 4 * tid + c] = v[r][c];
        }
        // (pinned where formed: see the scan)
#pragma unroll
        for (int c = 0; c < 4; ++c) asm volatile("" : "+v"(q[r][c]));
    }
    // U is loaded now, behind the priorities, and written to LDS during the
    // lookback: its latency hides under the scan.  (The empty asm keeps the
    // compiler from hoisting these loads above the pow.)
    constexpr int kUR = UL ? kULds / kScanThreads : 1;
    float ureg[kUR];
    if constexpr (UL) {
        asm volatile("" ::: "memory");
#pragma unroll
        for (int m = 0; m < kUR; ++m) {
            const int i = m * kScanThreads + tid;
            const bool ok = i < (int)k;
            const float x = U[ok ? i : 0];      // issued unconditionally (k >= 1)
            ureg[m] = ok ? x : 0.0f;
        }
    }
    double X[R];
    double A;
    tile_scan_256<R, double>(q, X, A, s_wtot);
    if (tid == 0) store_agent(&ws[a_off((uint32_t)tile, par)], status_enc(A));
    tile_local_values<R, double>(q, X, s_wmax);
    if (wave != 0) {
        if constexpr (UL) {
#pragma unroll
            for (int m = 0; m < kUR; ++m) s_U[m * kScanThreads + tid] = ureg[m];
        }
        clear_other_parity(ws, par, n_tiles, max_slots, hw_w, tid - kWave, kScanThreads - kWave);
    }
    if (wave == 0) {
        lookback_all<double>(tile, n_tiles, par, A, ws, calls, s_lb);
        if constexpr (UL) {
#pragma unroll
            for (int m = 0; m < kUR; ++m) s_U[m * kScanThreads + tid] = ureg[m];
        }
    }
    __syncthreads();
    const double excl = s_lb[0];
    const double excl_next = s_lb[1];
    const double T = s_lb[2];

    // ---- 2. this tile's samples: the thresholds in (excl, excl_next]
    if (wave == 0) {
        const int64_t r = first_above2(excl, excl_next, T, StratFp{Us, kd, T}, k);
        if (lane == 0) s_range[0] = (tile == 0) ? 0 : r;
        if (lane == 32) s_range[1] = last_tile ? k : r;
    }
    // the tile's CDF values, kept in q; the LDS copy serves the search, the
    // global stores wait until the local minimum is on its way
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int cc = 0; cc < 4; ++cc) {
            const int e = r * ROW + 4 * tid + cc;
            q[r][cc] = tile_value<double>(q[r][cc], excl, excl_next, e == tlen - 1);
            s_C[e] = q[r][cc];
        }
    __syncthreads();
    const int64_t i_lo = s_range[0];
    const int64_t i_hi = s_range[1];

    // ---- 3. search in LDS, write the indices, local minimum of p.  With at
    // most one draw per thread (the usual case) each thread keeps its draw's
    // index, the log2 of its priority and its new priority (fetched while it
    // searches) in registers, and publishes the index in LDS for its
    // neighbour.
    const bool one_pass = i_hi - i_lo <= kScanThreads;
    const int64_t i1 = i_lo + tid;
    float my_new = 0.0f;
    if (one_pass && newp != nullptr && i1 < i_hi) my_new = newp[i1];
    int my_b = -1;
    double my_lp = 0.0;
    uint32_t mn = 0xFFFFFFFFu;
    for (int64_t i = i1; i < i_hi; i += kScanThreads) {
        const double t = strat_threshold(i, Us[i], kd, T);
        int b = 0, len = tlen;
        while (len > 1) {
            const int half = len >> 1;
            b = (s_C[b + half - 1] < t) ? b + half : b;
            len -= half;
        }
        b += (s_C[b] < t) ? 1 : 0;
        if (b >= tlen) b = tlen - 1;
        out_idx[i] = (int32_t)(base + b);
        my_b = b;
        const float pb = s_p[b];
        const uint32_t key = __float_as_uint(pb);
        mn = key < mn ? key : mn;
    }
    if (one_pass) s_b[tid] = my_b;
    mn = wave_min_u32(mn);
    if (lane == 0) atomicMin(&s_min, mn);
    __syncthreads();

    // ---- 4. publish the local minimum; while the others arrive, store the
    // CDF and rewrite the last draw of each index (draws of one index are
    // adjacent and all in this tile, and only this tile reads that part of
    // the priority array)
    if (tid == 0) store_agent(&ws[min_off((uint32_t)tile, par)], (uint64_t)s_min + 1);
    // (the drawn priority's log2, for its IS weight, only now: off the path
    // to the published minimum)
    if (one_pass && my_b >= 0) {
        const float pb = s_p[my_b];
        if (pb > 0.0f) my_lp = log2_sig32((double)pb, &M);
    }
    const bool vec_out = vec_ok && tlen == TILE;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e0 = r * ROW + 4 * tid;
        if (vec_out) {
            double2* o = reinterpret_cast<double2*>(cdf + base + e0);
            o[0] = make_double2(q[r][0], q[r][1]);
            o[1] = make_double2(q[r][2], q[r][3]);
        } else {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                if (e0 + cc < tlen) cdf[base + e0 + cc] = q[r][cc];
        }
        if (last_tile) {
#pragma unroll
            for (int cc = 0; cc < 4; ++cc)
                if (e0 + cc == tlen - 1) total[0] = q[r][cc];
        }
    }
    if (newp != nullptr) {
        if (one_pass) {
            if (i1 < i_hi) {
                const bool winner = i1 + 1 >= i_hi || s_b[tid + 1] != my_b;
                if (winner) prio[base + my_b] = my_new;
            }
        } else {
            for (int64_t i = i1; i < i_hi; i += kScanThreads) {
                const int32_t b = out_idx[i];
                const bool winner = i + 1 >= i_hi || out_idx[i + 1] != b;
                if (winner) prio[b] = newp[i];
            }
        }
    }
    if (wave == 0) {
        uint32_t g = 0xFFFFFFFFu;
#pragma nounroll
        for (int t0 = 0; t0 < n_tiles; t0 += kAllWords * kWave) {
            uint32_t off[kAllWords];
            bool need[kAllWords];
            uint64_t w[kAllWords];
#pragma unroll
            for (int j = 0; j < kAllWords; ++j) {
                const int tt = t0 + j * kWave + lane;
                need[j] = tt < n_tiles;
                off[j] = min_off((uint32_t)(need[j] ? tt : 0), par);
            }
            wait_words<kAllWords>(ws, off, need, w);
#pragma unroll
            for (int j = 0; j < kAllWords; ++j)
                if (need[j]) {
                    const uint32_t key = (uint32_t)(w[j] - 1);
                    g = key < g ? key : g;
                }
        }
        g = wave_min_u32(g);
        if (lane == 0) s_gmin = g;
    }
    __syncthreads();

    // ---- 5. IS weights
    const double pmin = (double)__uint_as_float(s_gmin);
    const double lpmin = pmin > 0.0 ? log2_sig32(pmin, &M) : 0.0;
    if (one_pass) {
        if (i1 < i_hi) out_w[i1] = is_weight_lp(pmin, lpmin, (double)s_p[my_b], my_lp, ab, &M);
    } else {
        for (int64_t i = i1; i < i_hi; i += kScanThreads) {
            const int b = (int)(out_idx[i] - base);
            out_w[i] = is_weight(pmin, lpmin, (double)s_p[b], ab, &M);
        }
    }
}

template <int R, bool UL, bool FAST>
static int per_round_capacity() {
    // VEC does not change the resources.
    return resident_grid(reinterpret_cast<const void*>(&k_per_round<R, UL, true, FAST>),
                         kScanThreads);
}

template <int R, bool UL, bool FAST>
static psamp_status launch_per_round(void* prio, int64_t n, double alpha, double ab,
                                     const float* u, int64_t k, const float* newp,
                                     int32_t* out_idx, float* out_w, double* cdf, double* total,
                                     void* ws, uint64_t max_slots, int vec_ok, hipStream_t st) {
    const int tiles = (int)ceil_div(n, kScanThreads * 4 * R);
    if (trace_enabled()) trace_launch("k_per_round", tiles, kScanThreads, n);
    if (aligned(prio, 16) && n % 4 == 0)
        hipLaunchKernelGGL((k_per_round<R, UL, true, FAST>), dim3(tiles), dim3(kScanThreads), 0, st,
                           (float*)prio, n, alpha, ab, u, k, newp, out_idx, out_w, cdf, total,
                           (uint64_t*)ws, tiles, max_slots, vec_ok);
    else
        hipLaunchKernelGGL((k_per_round<R, UL, false, FAST>), dim3(tiles), dim3(kScanThreads), 0, st,
                           (float*)prio, n, alpha, ab, u, k, newp, out_idx, out_w, cdf, total,
                           (uint64_t*)ws, tiles, max_slots, vec_ok);
    return launch_status();
}

}  // namespace psamp

using namespace psamp;

// The scan's workspace: the fused kernel keeps its draw minima in the
// header, and the three-kernel path forms the weights from the scan's slots.
extern "C" size_t psamp_per_round_workspace_size(int64_t n, int64_t k) {
    if (k < 0 || k > kMaxN) return 0;
    return psamp_build_cdf_workspace_size(n);
}

static psamp_status per_round_impl(void* prio, int64_t n, double alpha, double beta,
                                   const float* u, int64_t k, const float* new_prio,
                                   int32_t* out_idx, float* out_w, double* cdf, double* total,
                                   void* ws, size_t ws_bytes, void* stream);

extern "C" psamp_status psamp_per_round(void* prio, int64_t n, double alpha, double beta,
                                        const float* u, int64_t k, const float* new_prio,
                                        int32_t* out_idx, float* out_w, double* cdf,
                                        double* total, void* ws, size_t ws_bytes, void* stream) {
    const bool chk = check_on();
    const psamp_status e = per_round_impl(prio, n, alpha, beta, u, k, new_prio, out_idx, out_w,
                                          cdf, total, ws, ws_bytes, stream);
    if (chk && e == PSAMP_OK) check_total(total, PSAMP_F64, as_stream(stream));
    return e;
}

static psamp_status per_round_impl(void* prio, int64_t n, double alpha, double beta,
                                   const float* u, int64_t k, const float* new_prio,
                                   int32_t* out_idx, float* out_w, double* cdf, double* total,
                                   void* ws, size_t ws_bytes, void* stream) {
    if (!prio || !cdf || !total) return PSAMP_E_NULL;
    if (n < 1 || n > kMaxN || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    if (!(finite_d(alpha) && alpha > 0.0) || !(finite_d(beta) && beta >= 0.0)) return PSAMP_E_PARAM;
    if (!ws || ws_bytes < psamp_per_round_workspace_size(n, k)) return PSAMP_E_WORKSPACE;
    if (!aligned(prio, 4) || !aligned(cdf, 8) || !aligned(total, 8) || !aligned(ws, 256))
        return PSAMP_E_ALIGN;
    if (k > 0 && (!u || !out_idx || !out_w)) return PSAMP_E_NULL;
    if (k > 0 && (!aligned(u, 4) || !aligned(out_idx, 4) || !aligned(out_w, 4) ||
                  (new_prio && !aligned(new_prio, 4))))
        return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on()) {
        // (checked before the update rewrites the drawn priorities)
        check_prio((const float*)prio, n, st);
        if (k > 0) check_unit(u, k, st);
        if (k > 0 && new_prio) check_prio(new_prio, k, st);
    }
    // The clearing of the other parity runs up to the largest tile count any
    // call on this workspace has used, which can exceed this call's: the
    // bound is the workspace's own capacity, not the one this n needs.
    const uint64_t max_slots = ws_tile_capacity(ws_bytes);
    const int vec_ok = aligned(cdf, 16);   // 16-byte stores of whole tiles
    if (k > 0) {
        // The scan's own tiling (so the CDF is the same bits as psamp_build_cdf's);
        // U in LDS when it fits and the grid still is resident.
#define PSAMP_PER_ROUND_TRY(RR, UU, FF)                                                     \
    if (ceil_div(n, kScanThreads * 4 * RR) <= per_round_capacity<RR, UU, FF>())            \
        return launch_per_round<RR, UU, FF>(prio, n, alpha, alpha * beta, u, k, new_prio,  \
                                            out_idx, out_w, cdf, total, ws, max_slots,     \
                                            vec_ok, st);
        if (scan_rows_for(n) == 1) {
            if (k <= kULds) PSAMP_PER_ROUND_TRY(1, true, false)
            PSAMP_PER_ROUND_TRY(1, false, false)
        } else {
            // the scan's pow on these tiles (same bits as psamp_build_cdf)
            if (alpha <= kFastPowMaxAlpha) {
                PSAMP_PER_ROUND_TRY(8, false, true)
            } else {
                PSAMP_PER_ROUND_TRY(8, false, false)
            }
        }
#undef PSAMP_PER_ROUND_TRY
    }
    // Too large to be resident at once: three kernels (the tile sums; the
    // scan with the draws, the drawn priorities and the rewrite; the IS
    // weights), the same results as the four separate calls.
    if (k > 0)
        return launch_per_update((float*)prio, n, alpha, beta, u, k, new_prio, out_idx, out_w,
                                 cdf, total, ws, ws_bytes, st);
    return psamp_build_cdf(prio, PSAMP_F32, n, alpha, cdf, PSAMP_F64, total, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// psamp_per_round_noalloc: psamp_per_round for callers that cannot allocate
// device memory.  Its workspace is `scratch`, a file-scope device array, one
// copy on every GPU the library runs on, held until the process ends.  Host
// code never passes the array's name to a kernel or a copy (on the host it
// is only a stand-in for the symbol): it takes the array's device address on
// each device from hipGetSymbolAddress, once, and uses that.
// ---------------------------------------------------------------------------
namespace psamp {

constexpr int64_t kNoAllocMaxN = PSAMP_NOALLOC_MAX_N;
constexpr size_t kNoAllocBytes = ws_bytes_for_tiles((kNoAllocMaxN + kMinTile - 1) / kMinTile);
static_assert(kNoAllocBytes % 8 == 0, "scratch is an array of 64-bit words");

static __device__ __align__(256) uint64_t scratch[kNoAllocBytes / 8];

__global__ void k_zero_words(uint64_t* __restrict__ p, int64_t words) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

constexpr int kNoAllocMaxDevices = 64;

// The device address of this device's scratch, found once per device.  On
// that first call the array is also cleared by a kernel on the caller's
// stream (it starts zeroed as a zero-initialised static; the kernel only
// makes that explicit) -- unless the stream is being captured, where the
// static zero state is the one the first call finds.
static psamp_status noalloc_scratch(hipStream_t st, uint64_t** out) {
    static std::mutex mu;
    static uint64_t* ptr[kNoAllocMaxDevices] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocMaxDevices) {
        (void)hipGetLastError();
        return PSAMP_E_LAUNCH;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PSAMP_E_LAUNCH;
        }
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing(st, &cap) != hipSuccess) {
            (void)hipGetLastError();
            return PSAMP_E_LAUNCH;
        }
        if (cap == hipStreamCaptureStatusNone) {
            hipLaunchKernelGGL(k_zero_words, dim3(256), dim3(256), 0, st, (uint64_t*)p,
                               (int64_t)(kNoAllocBytes / 8));
            if (launch_status() != PSAMP_OK) return PSAMP_E_LAUNCH;
        }
        ptr[dev] = (uint64_t*)p;
    }
    *out = ptr[dev];
    return PSAMP_OK;
}

}  // namespace psamp

extern "C" psamp_status psamp_per_round_noalloc(void* prio, int64_t n, double alpha, double beta,
                                                const float* u, int64_t k,
                                                const float* new_prio, int32_t* out_idx,
                                                float* out_w, double* cdf, double* total,
                                                void* stream) {
    if (n > kNoAllocMaxN) return PSAMP_E_SIZE;
    // the checks of psamp_per_round that need no workspace, before set-up
    if (!prio || !cdf || !total) return PSAMP_E_NULL;
    if (n < 1 || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    if (!(finite_d(alpha) && alpha > 0.0) || !(finite_d(beta) && beta >= 0.0)) return PSAMP_E_PARAM;
    uint64_t* ws = nullptr;
    const psamp_status e = noalloc_scratch(as_stream(stream), &ws);
    if (e != PSAMP_OK) return e;
    return psamp_per_round(prio, n, alpha, beta, u, k, new_prio, out_idx, out_w, cdf, total, ws,
                           kNoAllocBytes, stream);
}
