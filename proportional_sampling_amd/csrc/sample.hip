// sample.hip -- thresholds and searchsorted onto the CDF.
//
// [PF]: searchsorted(cumsum, u) with right=False gives the first index whose
// cumsum is >= u (n if none), clamped to n-1.  Thresholds: stratified
// t_i = ((i + U_i) / k) * T or iid t_i = U_i * T, in double (one rounding per
// operation, the same operations as the serial definition); integer mode
// uses the exact integer map onto [1, T].
//
// Kernel: one thread per sample, a branch-free lower_bound whose trip count
// depends only on n (no divergence).  Consecutive stratified samples search
// neighbouring regions, so the upper levels of the search hit L2 for the
// whole wave and the lower levels touch about one line per sample.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kSampleThreads = 256;

// First position p in [0, n] with C[p] >= t (n if none).  The loop runs
// ceil(log2 n) times for every lane.
template <class CdfT, class ThrT>
__device__ __forceinline__ int64_t lower_bound_dev(const CdfT* __restrict__ C, int64_t n, ThrT t) {
    int64_t b = 0;
    int64_t len = n;
    while (len > 1) {
        const int64_t half = len >> 1;
        b = ((ThrT)C[b + half - 1] < t) ? b + half : b;
        len -= half;
    }
    return b + (((ThrT)C[b] < t) ? 1 : 0);
}

template <class CdfT>
__global__ __launch_bounds__(kSampleThreads) void k_sample_fp(
    const CdfT* __restrict__ cdf, int64_t n, const CdfT* __restrict__ total,
    const float* __restrict__ U, int64_t k, int stratified, int32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kSampleThreads + threadIdx.x;
    if (i >= k) return;
    const double T = (double)total[0];
    const double u = (double)U[i];
    double t;
    if (stratified) {
        const double a = (double)i + u;
        const double b = a / (double)k;
        t = b * T;
    } else {
        t = u * T;
    }
    const int64_t p = lower_bound_dev<CdfT, double>(cdf, n, t);
    out[i] = (int32_t)(p < n ? p : n - 1);
}

__global__ __launch_bounds__(kSampleThreads) void k_sample_int(
    const uint64_t* __restrict__ cdf, int64_t n, const uint64_t* __restrict__ total,
    const uint32_t* __restrict__ r, int64_t k, int stratified, int k_log2,
    int32_t* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * kSampleThreads + threadIdx.x;
    if (i >= k) return;
    const uint64_t T = total[0];
    const uint64_t t = int_threshold((uint64_t)i, r[i], (uint64_t)k, T, stratified, k_log2);
    const int64_t p = lower_bound_dev<uint64_t, uint64_t>(cdf, n, t);
    out[i] = (int32_t)(p < n ? p : n - 1);
}

// ---------------------------------------------------- stratified draws
// Stratified thresholds are non-decreasing in i, so the search can run from
// the CDF's side: element e (a non-decreasing CDF, as psamp_build_cdf
// produces) is the index of exactly the draws i with C_{e-1} < t_i <= C_e,
// i.e. i in [F(C_{e-1}), F(C_e)) with F(x) = #{i : t_i <= x}; element 0
// also takes every t_i <= C_0 and element n-1 every t_i above C_{n-1} (the
// clamp).  Each thread reads 4 consecutive CDF values once (coalesced) and
// counts the thresholds at or below them from the stratum estimate x k / T,
// checked on the thresholds themselves -- every CDF line is read once
// instead of once per search level, and the thresholds' fractions come from
// L1/L2 (neighbouring threads need neighbouring ones).  The result is the
// binary search's, bit for bit.  (For a CDF that is not non-decreasing the
// ranges are kept non-empty-or-empty by a running max, so every index is
// still written with some value in [0, n).)
constexpr int kStratThreads = 256;
constexpr int kStratWin = 8;       // thresholds a thread tests directly
constexpr int kStratHeavy = 32;    // a window this wide is placed by the whole wave

// F(x) for fp thresholds t_i = ((i + U_i) / k) * T (double; for a
// power-of-two k the division is a multiplication by 1/k, the same bits).
struct StratCountFp {
    const float* __restrict__ U;
    int64_t k;
    double T, kT, inv_k;
    bool pow2;
    using Raw = float;
    __device__ __forceinline__ float raw(int64_t i) const { return U[i]; }
    __device__ __forceinline__ double thr_raw(int64_t i, float u) const {
        const double a = (double)(int32_t)i + (double)u;        // i < k <= 2^31 - 1
        const double b = pow2 ? a * inv_k : a / (double)k;
        return b * T;
    }
    __device__ __forceinline__ double thr(int64_t i) const { return thr_raw(i, U[i]); }
    __device__ __forceinline__ int64_t estimate(double x) const {
        const double e = floor(x * kT);
        return !(e > 0.0) ? 0 : (e >= (double)k ? k : (int64_t)e);
    }
    __device__ __forceinline__ uint32_t estimate32(double x) const {   // the same, k < 2^31
        const double e = floor(x * kT);
        return !(e > 0.0) ? 0u : (e >= (double)k ? (uint32_t)k : (uint32_t)(int32_t)e);
    }
};

// F(x) for integer thresholds (the exact map onto [1, T]).
struct StratCountInt {
    const uint32_t* __restrict__ r;
    int64_t k;
    uint64_t T;
    double kT;
    int k_log2;
    using Raw = uint32_t;
    __device__ __forceinline__ uint32_t raw(int64_t i) const { return r[i]; }
    __device__ __forceinline__ uint64_t thr_raw(int64_t i, uint32_t u) const {
        return int_threshold((uint64_t)i, u, (uint64_t)k, T, 1, k_log2);
    }
    __device__ __forceinline__ uint64_t thr(int64_t i) const { return thr_raw(i, r[i]); }
    __device__ __forceinline__ int64_t estimate(uint64_t x) const {
        const double e = floor((double)x * kT);
        return !(e > 0.0) ? 0 : (e >= (double)k ? k : (int64_t)e);
    }
    __device__ __forceinline__ uint32_t estimate32(uint64_t x) const {
        const double e = floor((double)x * kT);
        return !(e > 0.0) ? 0u : (e >= (double)k ? (uint32_t)k : (uint32_t)(int32_t)e);
    }
};

// #{i : t_i <= x}: the count c with t_{c-1} <= x < t_c, from the estimate
// (off by at most one) or, if that misses, a binary search.
template <class Cnt, class V>
__device__ __forceinline__ int64_t strat_count(const Cnt& F, V x) {
    const int64_t k = F.k;
    const int64_t c = F.estimate(x);
    const bool below = c == 0 || F.thr(c - 1) <= x;
    const bool above = c == k || F.thr(c) > x;
    if (below && above) return c;
    if (below && (c + 1 == k || F.thr(c + 1) > x)) return c + 1;
    if (!below && (c == 1 || F.thr(c - 2) <= x)) return c - 1;
    int64_t lo = 0, hi = k;
    while (lo < hi) {
        const int64_t mid = lo + ((hi - lo) >> 1);
        if (F.thr(mid) > x) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

// PER consecutive CDF values of a thread, as 16-byte vectors (VEC) or one
// by one (clamped to the array).
template <int PER, bool VEC, class CdfT, class V>
__device__ __forceinline__ void load_elems(const CdfT* __restrict__ cdf, int64_t e0, int64_t n,
                                           V (&x)[PER]) {
    if constexpr (VEC) {
        if constexpr (sizeof(CdfT) == 8) {
#pragma unroll
            for (int h = 0; h < PER / 2; ++h) {
                const ulonglong2 a = reinterpret_cast<const ulonglong2*>(cdf + e0)[h];
                x[2 * h] = (V)__builtin_bit_cast(CdfT, a.x);
                x[2 * h + 1] = (V)__builtin_bit_cast(CdfT, a.y);
            }
        } else {
#pragma unroll
            for (int h = 0; h < PER / 4; ++h) {
                const float4 a = reinterpret_cast<const float4*>(cdf + e0)[h];
                x[4 * h] = (V)a.x; x[4 * h + 1] = (V)a.y; x[4 * h + 2] = (V)a.z; x[4 * h + 3] = (V)a.w;
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < PER; ++j) x[j] = (V)cdf[e0 + j < n ? e0 + j : n - 1];
    }
}

// VEC: the CDF is 16-byte aligned and n % PER == 0.  Each thread takes PER
// consecutive elements (4 up to 2^20 elements, where more threads hide
// more latency; 8 above, where fewer thresholds per element pay).  The
// draws it owns are those with x_before < t_i <= x_last (element 0 also
// owns every t_i <= C_0, element n-1 every t_i above C_{n-1}), and they lie
// in a short window [estimate(x_before) - 1, estimate(x_last) + 1]: the
// thread forms the window's thresholds once (checking that the one below
// the window is at or below x_before and the one above it beyond x_last).
// Each owned draw's index is then the thread's first element plus the
// number of its values below the threshold -- the first element at or
// above it, as the search would find -- with no per-element loop: the
// wave's widest window bounds the loop over the window's draws (mostly 2
// or 3 slots), kStratWin thresholds at a time.  A window of kStratHeavy
// draws or more (heavy elements), a failed check or a last thread whose
// draws reach past the window is handed to the whole wave: it counts the
// thresholds at the thread's boundaries (strat_count, on up to PER + 1
// lanes at once) and 64 lanes write each element's range together -- one
// element holding half the mass of 2^24 priorities took 92 ms for 2^20
// draws on its one lane, and the old per-element loops were as serial.
template <int PER, bool VEC, class CdfT, class V, class Cnt>
__device__ __forceinline__ void strat_place(const CdfT* __restrict__ cdf, int64_t n, const Cnt& F,
                                            int32_t* __restrict__ out) {
    const int lane = (int)(threadIdx.x & (kWave - 1));
    const int64_t e0 = ((int64_t)blockIdx.x * kStratThreads + threadIdx.x) * PER;
    // (a thread past the end stays in the wave, idle: the wave fills
    // heavy ranges together below)
    const bool valid = e0 < n;
    V x[PER];
    load_elems<PER, VEC, CdfT, V>(cdf, valid ? e0 : 0, n, x);   // past the end: C_{n-1}
    // valid elements of this thread (VEC: n % PER == 0, so all of them)
    const int nv = !valid ? 0 : (VEC ? PER : (int)min_<int64_t>(PER, n - e0));
    const bool first = e0 == 0;
    const bool last = valid && e0 + nv == n;
    const V xp = (first || !valid) ? V(0) : (V)cdf[e0 - 1];
    V xl = x[PER - 1];
    if constexpr (!VEC) {
        xl = x[0];
#pragma unroll
        for (int j = 1; j < PER; ++j) xl = j < nv ? x[j] : xl;
    }
    // window arithmetic in 32 bits (k <= 2^31 - 1, so every index below
    // k + kStratWin + 1 fits an unsigned 32-bit word)
    const uint32_t kk = (uint32_t)F.k;
    const uint32_t ca = first ? 0u : F.estimate32(xp);
    const uint32_t cb = F.estimate32(xl);
    const uint32_t wlo = ca > 0 ? ca - 1 : 0u;
    const uint32_t whi = cb + 1 < kk ? cb + 1 : kk - 1;
    const int span = (int)(whi - wlo);              // < 0 only where the CDF decreases
    // the first kStratWin thresholds of the window and the two checks: every
    // fraction load unconditional (index clamped below k), so that all are
    // in flight at once (a load under a branch is waited for inside it); a
    // threshold past the window is formed but never used
    using Raw = typename Cnt::Raw;
    auto at = [&](uint32_t i) { return (int64_t)(i < kk ? i : kk - 1); };
    Raw u[kStratWin];
#pragma unroll
    for (int w = 0; w < kStratWin; ++w) u[w] = F.raw(at(wlo + w));
    const Raw ulo = F.raw(at(wlo - 1));                 // (wlo = 0: unused)
    const Raw uhi = F.raw(at(whi + 1));
    V t[kStratWin];
#pragma unroll
    for (int w = 0; w < kStratWin; ++w) t[w] = F.thr_raw(wlo + w, u[w]);
    bool win = valid && !(last && whi + 1 < kk);
    if (!first && wlo > 0 && !(F.thr_raw(wlo - 1, ulo) <= xp)) win = false;
    if (whi + 1 < kk && !(F.thr_raw(whi + 1, uhi) > xl)) win = false;
    // a wide window (heavy elements) or a failed check: the wave places this
    // thread's draws together, below
    const bool coop = valid && (!win || span >= kStratHeavy);
    const bool own_win = win && !coop;
    // the widest window of the wave bounds the loop for every lane
    int smax = own_win ? span : -1;
    smax = wave_max_i32(smax);
    const int32_t eb = (int32_t)e0;
    for (int b = 0; b <= smax; b += kStratWin) {          // (uniform in the wave)
        if (b > 0) {
#pragma unroll
            for (int w = 0; w < kStratWin; ++w) u[w] = F.raw(at(wlo + b + w));
#pragma unroll
            for (int w = 0; w < kStratWin; ++w) t[w] = F.thr_raw(wlo + b + w, u[w]);
        }
#pragma unroll
        for (int w = 0; w < kStratWin; ++w) {
            if (b + w > smax) break;
            const V tw = t[w];
            const bool own = own_win && b + w <= span && (first || tw > xp) && (last || tw <= xl);
            int p = 0;
#pragma unroll
            for (int j = 0; j < PER; ++j) p += x[j] < tw ? 1 : 0;
            p = p < nv ? p : nv - 1;                          // past C_{n-1}: the clamp
            if (own) out[wlo + (uint32_t)(b + w)] = eb + p;
        }
    }
    // The other threads, one at a time: lanes 0..nv of the wave count the
    // thresholds at or below its boundaries (x_before, then each value;
    // the last element of the array takes every draw), and the whole wave
    // writes each element's range of draws.  (A value outside [x_before,
    // x_last] -- only in a CDF that decreases somewhere -- is counted as the
    // nearest end, so that neighbouring threads agree on the count at their
    // shared boundary and every draw is written once more than zero times.)
    uint64_t cm = __ballot(coop);
    while (cm != 0) {                                     // (uniform in the wave)
        const int h = __builtin_ctzll(cm);
        cm &= cm - 1;
        const int64_t he0 = (int64_t)__builtin_amdgcn_readlane((int)e0, h);
        const int hnv = __builtin_amdgcn_readlane(nv, h);
        const bool hfirst = he0 == 0;
        const V hxp = readlane(xp, h);
        const V hxl = readlane(xl, h);
        V v = hxp;
#pragma unroll
        for (int j = 1; j <= PER; ++j) {
            const V xj = readlane(x[j - 1], h);
            v = lane == j ? xj : v;
        }
        int64_t c = 0;
        if (lane <= hnv) {
            if (lane > 0 && he0 + lane - 1 == n - 1) {
                c = F.k;
            } else if (!(lane == 0 && hfirst)) {
                v = v > hxl ? hxl : v;
                if (!hfirst) v = v < hxp ? hxp : v;
                c = strat_count(F, v);
            }
        }
        int64_t lo = (int64_t)readlane((uint64_t)c, 0);
        for (int j = 0; j < hnv; ++j) {
            int64_t hi = (int64_t)readlane((uint64_t)c, j + 1);
            hi = hi > lo ? hi : lo;
            for (int64_t i = lo + lane; i < hi; i += kWave) out[i] = (int32_t)(he0 + j);
            lo = hi;
        }
    }
}

template <int PER, bool VEC, class CdfT>
__global__ __launch_bounds__(kStratThreads) void k_sample_strat_fp(
    const CdfT* __restrict__ cdf, int64_t n, const CdfT* __restrict__ total,
    const float* __restrict__ U, int64_t k, int32_t* __restrict__ out) {
    const double T = (double)total[0];
    const StratCountFp F{U, k, T, (double)k / T, 1.0 / (double)k, (k & (k - 1)) == 0};
    strat_place<PER, VEC, CdfT, double>(cdf, n, F, out);
}

template <int PER, bool VEC>
__global__ __launch_bounds__(kStratThreads) void k_sample_strat_int(
    const uint64_t* __restrict__ cdf, int64_t n, const uint64_t* __restrict__ total,
    const uint32_t* __restrict__ r, int64_t k, int k_log2, int32_t* __restrict__ out) {
    const uint64_t T = total[0];
    const StratCountInt F{r, k, T, (double)k / (double)T, k_log2};
    strat_place<PER, VEC, uint64_t, uint64_t>(cdf, n, F, out);
}

template <int PER>
static psamp_status launch_strat(const void* cdf, psamp_dtype cdf_t, int64_t n, const void* total,
                                 const void* u, int64_t k, int32_t* out_idx, hipStream_t st) {
    const int64_t g = ceil_div(n, (int64_t)kStratThreads * PER);
    const bool vec = n % PER == 0 && aligned(cdf, 16);
    if (trace_enabled()) trace_launch("k_sample_strat", g, kStratThreads, n);
#define PSAMP_STRAT_LAUNCH(V)                                                                     \
    if (cdf_t == PSAMP_U64)                                                                      \
        hipLaunchKernelGGL((k_sample_strat_int<PER, V>), dim3((unsigned)g), dim3(kStratThreads), 0, \
                           st, (const uint64_t*)cdf, n, (const uint64_t*)total, (const uint32_t*)u,  \
                           k, is_pow2(k) ? ilog2_exact(k) : -1, out_idx);                         \
    else if (cdf_t == PSAMP_F64)                                                                 \
        hipLaunchKernelGGL((k_sample_strat_fp<PER, V, double>), dim3((unsigned)g),                \
                           dim3(kStratThreads), 0, st, (const double*)cdf, n,                     \
                           (const double*)total, (const float*)u, k, out_idx);                    \
    else                                                                                         \
        hipLaunchKernelGGL((k_sample_strat_fp<PER, V, float>), dim3((unsigned)g),                 \
                           dim3(kStratThreads), 0, st, (const float*)cdf, n, (const float*)total, \
                           (const float*)u, k, out_idx);
    if (vec) {
        PSAMP_STRAT_LAUNCH(true)
    } else {
        PSAMP_STRAT_LAUNCH(false)
    }
#undef PSAMP_STRAT_LAUNCH
    return launch_status();
}

// Stratified draws from the CDF's side when they are not too sparse in it
// (each CDF line read once, against k searches of log2 n dependent loads,
// the lower levels of which touch about three lines per draw).  Measured
// against the searches: B = 262144 with 8192 draws 7.1 -> 4.9 us; 2^24
// with 2^20 draws 55 -> 50 us and 314 -> 145 MB of HBM traffic; placing
// the window's draws directly (no per-element count loop) and issuing its
// fraction loads together then took 2^24 / 2^20 LogNormal priorities from
// 48.7 to 28.3 us back to back (604 -> 269 VALU instructions per wave).
// For sparse draws the searches read less.
inline bool strat_from_cdf(int64_t n, int64_t k) {
    return 64 * k >= n;
}

}  // namespace psamp

using namespace psamp;

extern "C" psamp_status psamp_sample(const void* cdf, psamp_dtype cdf_t, int64_t n,
                                     const void* total, const void* u, psamp_dtype u_t, int64_t k,
                                     int stratified, int32_t* out_idx, void* stream) {
    if (n < 1 || n > kMaxN || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    if (stratified != 0 && stratified != 1) return PSAMP_E_PARAM;
    const bool fp = (cdf_t == PSAMP_F64 || cdf_t == PSAMP_F32) && u_t == PSAMP_F32;
    const bool in = cdf_t == PSAMP_U64 && u_t == PSAMP_U32;
    if (!fp && !in) return PSAMP_E_DTYPE;
    if (k == 0) return PSAMP_OK;
    if (!cdf || !total || !u || !out_idx) return PSAMP_E_NULL;
    const size_t csz = cdf_t == PSAMP_F32 ? 4 : 8;
    if (!aligned(cdf, csz) || !aligned(total, csz) || !aligned(u, 4) || !aligned(out_idx, 4))
        return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on()) {
        if (fp) check_unit((const float*)u, k, st);
        check_total(total, cdf_t, st);
    }
    if (stratified && strat_from_cdf(n, k)) {
        if (n <= ((int64_t)1 << 20)) return launch_strat<4>(cdf, cdf_t, n, total, u, k, out_idx, st);
        return launch_strat<8>(cdf, cdf_t, n, total, u, k, out_idx, st);
    }
    const int64_t grid = ceil_div(k, kSampleThreads);
    if (trace_enabled()) trace_launch("k_sample", grid, kSampleThreads, k);
    if (in) {
        const int k_log2 = is_pow2(k) ? ilog2_exact(k) : -1;
        hipLaunchKernelGGL(k_sample_int, dim3((unsigned)grid), dim3(kSampleThreads), 0, st,
                           (const uint64_t*)cdf, n, (const uint64_t*)total, (const uint32_t*)u, k,
                           stratified, k_log2, out_idx);
    } else if (cdf_t == PSAMP_F64) {
        hipLaunchKernelGGL(k_sample_fp<double>, dim3((unsigned)grid), dim3(kSampleThreads), 0, st,
                           (const double*)cdf, n, (const double*)total, (const float*)u, k,
                           stratified, out_idx);
    } else {
        hipLaunchKernelGGL(k_sample_fp<float>, dim3((unsigned)grid), dim3(kSampleThreads), 0, st,
                           (const float*)cdf, n, (const float*)total, (const float*)u, k,
                           stratified, out_idx);
    }
    return launch_status();
}
