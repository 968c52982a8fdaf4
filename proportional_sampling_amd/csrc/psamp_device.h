// psamp_device.h -- device building blocks shared by the libpsamp kernels
// (gfx950 / CDNA4, wave64).
//
//  * wave64 inclusive scans built from DPP row shifts and row broadcasts;
//  * 64-bit status words for the single-pass scan (value and "ready" flag in
//    one word, so relaxed agent-scope atomics are enough to pass them
//    between workgroups on different XCDs);
//  * a table-driven fp64 log2 / exp2 (range reduction after Tang's method,
//    Taylor kernels on the reduced argument) used for p^alpha, exp and the
//    importance-sampling weights.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pow_tables.h"

namespace psamp {

constexpr int kWave = 64;

// ------------------------------------------------------------------ DPP
// DPP control words (GFX9 encoding).
enum : int {
    kRowShr1 = 0x111,
    kRowShr2 = 0x112,
    kRowShr4 = 0x114,
    kRowShr8 = 0x118,
    kWaveShr1 = 0x138,
    kRowBcast15 = 0x142,
    kRowBcast31 = 0x143,
};

// Lanes that have no source (or whose row is masked off) receive 0.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint32_t dpp32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, BOUND_ZERO);
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ double dpp(double x) {
    uint32_t lo = dpp32<CTRL, ROW_MASK, BOUND_ZERO>((uint32_t)__double2loint(x));
    uint32_t hi = dpp32<CTRL, ROW_MASK, BOUND_ZERO>((uint32_t)__double2hiint(x));
    return __hiloint2double((int)hi, (int)lo);
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ uint64_t dpp(uint64_t x) {
    uint32_t lo = dpp32<CTRL, ROW_MASK, BOUND_ZERO>((uint32_t)x);
    uint32_t hi = dpp32<CTRL, ROW_MASK, BOUND_ZERO>((uint32_t)(x >> 32));
    return ((uint64_t)hi << 32) | lo;
}

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp(float x) {
    return __uint_as_float(dpp32<CTRL, ROW_MASK, BOUND_ZERO>(__float_as_uint(x)));
}

// Inclusive sum over the 64 lanes: Kogge-Stone inside each 16-lane row,
// then row 0 -> row 1, row 2 -> row 3 (bcast15) and rows 0..1 -> rows 2..3
// (bcast31).  The association is fixed, so the result is deterministic.
template <class T>
__device__ __forceinline__ T wave_incl_scan(T x) {
    x = x + dpp<kRowShr1, 0xF, true>(x);
    x = x + dpp<kRowShr2, 0xF, true>(x);
    x = x + dpp<kRowShr4, 0xF, true>(x);
    x = x + dpp<kRowShr8, 0xF, true>(x);
    x = x + dpp<kRowBcast15, 0xA, false>(x);
    x = x + dpp<kRowBcast31, 0xC, false>(x);
    return x;
}

// Value of lane-1 (lane 0 gets 0): turns an inclusive scan into an exclusive one.
template <class T>
__device__ __forceinline__ T wave_shr1(T x) {
    return dpp<kWaveShr1, 0xF, true>(x);
}

__device__ __forceinline__ double readlane(double x, int lane) {
    int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
    int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
    return __hiloint2double(hi, lo);
}
__device__ __forceinline__ uint64_t readlane(uint64_t x, int lane) {
    uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, lane);
    uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ float readlane(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Sum of all 64 lanes, same association as wave_incl_scan (lane 63's value).
template <class T>
__device__ __forceinline__ T wave_sum(T x) {
    return readlane(wave_incl_scan(x), kWave - 1);
}

// N independent wave_sums, step by step together: the same bits as N calls,
// in the time of about one (each step of one sum waits for the last).
template <class T, int N>
__device__ __forceinline__ void wave_sums(T (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowShr1, 0xF, true>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowShr2, 0xF, true>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowShr4, 0xF, true>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowShr8, 0xF, true>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowBcast15, 0xA, false>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = x[i] + dpp<kRowBcast31, 0xC, false>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = readlane(x[i], kWave - 1);
}

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// ------------------------------------------------------- atomics / status
__device__ __forceinline__ uint64_t load_agent(const uint64_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_agent(uint64_t* p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch_add_agent(uint64_t* p, uint64_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t fetch_max_agent(uint64_t* p, uint64_t v) {
    return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A status word is 0 while not ready; a published value v is stored as
// enc(v) != 0.  Doubles: bit pattern + 1 (NaN first made canonical, so the
// all-ones pattern never appears).  uint64: v + 1 (sums stay below 2^63).
__device__ __forceinline__ uint64_t status_enc(double v) {
    uint64_t b = (uint64_t)__double_as_longlong(v);
    if (v != v) b = 0x7FF8000000000000ull;
    return b + 1;
}
__device__ __forceinline__ uint64_t status_enc(uint64_t v) { return v + 1; }
__device__ __forceinline__ void status_dec(uint64_t w, double& v) {
    v = __longlong_as_double((long long)(w - 1));
}
__device__ __forceinline__ void status_dec(uint64_t w, uint64_t& v) { v = w - 1; }

// ------------------------------------------------------------ fp64 math
// log2 and exp2 in double: exp2 within 2.3e-16 relative (normal results),
// log2 within 2.6e-16 of max(1, |log2 x|) (both measured on the host
// against long double over every float exponent) -- far below what the
// sampling contract needs (about 1e-9 on the weights).  Tables live in LDS
// (one copy per workgroup): entry k of the log table holds {c_k, -log2(c_k)}.
// Bit views, usable on the host too (the math below is also compiled for the
// host, where its error bounds are tested against long double).
__host__ __device__ __forceinline__ uint64_t bits_of(double x) {
    return __builtin_bit_cast(uint64_t, x);
}
__host__ __device__ __forceinline__ double double_of(uint64_t b) {
    return __builtin_bit_cast(double, b);
}
__host__ __device__ __forceinline__ double double_of_hi(uint32_t hi, uint32_t lo) {
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__host__ __device__ __forceinline__ float float_of(uint32_t b) {
    return __builtin_bit_cast(float, b);
}
__host__ __device__ __forceinline__ double2 dpair(double x, double y) {
    double2 r;
    r.x = x;
    r.y = y;
    return r;
}

struct MathLds {
    double2 log_tab[128];
    double exp_tab[64];
};

__host__ __device__ __forceinline__ void math_lds_fill(MathLds* m, int tid, int nthreads) {
    for (int i = tid; i < 128; i += nthreads)
        m->log_tab[i] = dpair(double_of(kLog2Tab[i][0]), double_of(kLog2Tab[i][1]));
    for (int i = tid; i < 64; i += nthreads)
        m->exp_tab[i] = double_of(kExp2Tab[i][0]);
}

// The same in two steps for blocks of at least 128 threads: math_load()
// issues the table loads (to be issued together with the kernel's other
// first loads, so their latencies overlap), math_store() writes LDS.
struct MathRegs {
    double2 lg;
    double ex;
};
__device__ __forceinline__ MathRegs math_load(int tid) {
    // Unconditional loads (indices wrapped): a guarded load would be merged
    // with its guarded LDS store and waited for on the spot.
    MathRegs r;
    r.lg = dpair(double_of(kLog2Tab[tid & 127][0]), double_of(kLog2Tab[tid & 127][1]));
    r.ex = double_of(kExp2Tab[tid & 63][0]);
    return r;
}
__device__ __forceinline__ void math_store(MathLds* m, int tid, const MathRegs& r) {
    if (tid < 128) m->log_tab[tid] = r.lg;
    if (tid < 64) m->exp_tab[tid] = r.ex;
}

constexpr double kLog2e = 1.4426950408889634074;   // 1/ln 2
constexpr double kLn2 = 0.69314718055994530942;

// log2(x) for a positive, finite, normal double whose significand has at
// most 32 significant bits (every float and every uint32 converts to one).
// x = 2^e * m, m in [1,2); k = top 7 fraction bits of m; c_k ~ 1/m (21
// bits) so r = m*c_k - 1 is exact and |r| < 2^-8; ln(1+r) by Taylor to r^6
// (truncation < 3e-18).
__host__ __device__ __forceinline__ double log2_sig32(double x, const MathLds* M) {
    uint64_t b = bits_of(x);
    int e = (int)(b >> 52) - 1023;
    int k = (int)(b >> 45) & 127;
    double m = double_of((b & 0x000FFFFFFFFFFFFFull) | 0x3FF0000000000000ull);
    double2 ct = M->log_tab[k];
    double r = fma(m, ct.x, -1.0);
    double q = fma(r, -1.0 / 6.0, 0.2);
    q = fma(r, q, -0.25);
    q = fma(r, q, 1.0 / 3.0);
    q = fma(r, q, -0.5);
    double ln1p = fma(r * r, q, r);
    return ((double)e + ct.y) + ln1p * kLog2e;
}

// 2^y.  y = N/64 + f with N = rint(64 y), |f| <= 1/128 (f exact);
// 2^f = e^g, g = f ln2, |g| < 0.0055, Taylor to g^5 (truncation < 4e-17);
// 2^(j/64) from the table; the power of two by ldexp.  Branch-free: y is
// clamped to [-1100, 1100] first, where ldexp already saturates to +inf
// (y >= 1024) or to 0 (y < -1075); a NaN y is passed through.
__host__ __device__ __forceinline__ double exp2_tab(double y, const MathLds* M) {
    const double yc = fmin(fmax(y, -1100.0), 1100.0);
    double N = rint(yc * 64.0);
    double f = fma(N, -1.0 / 64.0, yc);
    int Ni = (int)N;
    int j = Ni & 63;
    int n = Ni >> 6;
    double g = f * kLn2;
    double q = fma(g, 1.0 / 120.0, 1.0 / 24.0);
    q = fma(g, q, 1.0 / 6.0);
    q = fma(g, q, 0.5);
    q = fma(g, q, 1.0);
    double em1 = g * q;                  // e^g - 1
    double s = M->exp_tab[j];
    const double r = ldexp(fma(s, em1, s), n);
    return (y != y) ? y : r;
}

// p^alpha for a float priority p >= 0 and alpha > 0 (double), as
// 2^(alpha log2 p).  The error of y = alpha log2 p (log2's and the
// product's roundings, about 3.7e-16 |y|) becomes a relative error of
// about 2.6e-16 (|y| + 1) in the power: below 3e-13 for every normal
// result (|y| < 1075).  Branch-free: the power is formed for every lane
// (from 1 where p is not positive and finite) and the special cases are
// selected: 0 -> 0, +inf -> +inf, negative or NaN -> NaN.
__host__ __device__ __forceinline__ double pow_prio(float p, double alpha, const MathLds* M) {
    const float inf = float_of(0x7F800000u);
    const bool fin = p > 0.0f && p < inf;
    const double r = exp2_tab(alpha * log2_sig32((double)(fin ? p : 1.0f), M), M);
    const uint32_t sp_hi = (p == 0.0f) ? 0u : (p == inf) ? 0x7FF00000u : 0x7FF80000u;
    const double sp = double_of_hi(sp_hi, 0u);
    return fin ? r : sp;
}

// p^alpha with per-workgroup tables for one alpha (large tiles).  A float
// p > 0 is 2^e m with m in [1, 2) and e in [-149, 127] (subnormals
// normalised by the conversion to double); k = the top 7 fraction bits of m
// and c_k the table's 21-bit reciprocal, so r = m c_k - 1 is exact and
// |r| < 2^-8 + 2^-21.  Then p^alpha = 2^(alpha e) * c_k^(-alpha) * (1 + r)^alpha
// with the first two factors from the tables and (1 + r)^alpha from the
// binomial series to r^7 (truncation below 7e-16 relative for alpha <= 16).
// Tables, formed once per workgroup with pow_prio's own log2 / exp2:
// gk[k] = (c_k, c_k^(-alpha)), ex[e + 149] = (2^(alpha e - S_e), S_e) with
// S_e the multiple of 64 below alpha e (alpha e split exactly into a rounded
// part and its remainder), so that the table entry lies in [1, 2^64) and the
// product never overflows or loses bits below DBL_MIN before the final
// ldexp by 2^S_e, which rounds once where the result is subnormal and gives
// +inf where it overflows.  Wherever the result is a normal double the
// scaling is exact.  About 11 fp64 operations per element instead of ~27,
// and no rounding of alpha log2(p) (the main error of pow_prio): within
// 3e-15 relative for normal results, the rounding of alpha (-log2 c_k) in
// the table (|alpha log2 c_k| <= 16) being the largest part.
constexpr double kFastPowMaxAlpha = 16.0;
constexpr int kPowExpMin = -149;
constexpr int kPowExpCount = 277;                 // e in [-149, 127]

struct PowLds {
    double2 gk[128];
    double2 ex[kPowExpCount];                     // (2^(alpha e - S_e), S_e as int bits)
};

struct PowCoef {
    double b[8];                                  // b[i] = binomial(alpha, i), i = 1..7
};

__host__ __device__ __forceinline__ PowCoef pow_coef(double alpha) {
    PowCoef c;
    c.b[0] = 1.0;
    c.b[1] = alpha;
    const double inv[8] = {0.0, 1.0, 0.5, 1.0 / 3.0, 0.25, 0.2, 1.0 / 6.0, 1.0 / 7.0};
#pragma unroll
    for (int i = 2; i < 8; ++i) c.b[i] = c.b[i - 1] * (alpha - (double)(i - 1)) * inv[i];
    return c;
}

// Every thread of the workgroup takes part; M must be filled and visible.
// A barrier must follow before the tables are read.
__host__ __device__ __forceinline__ void pow_tables_build(PowLds* P, const MathLds* M, double alpha,
                                                 int tid, int nthreads) {
    for (int i = tid; i < 128 + kPowExpCount; i += nthreads) {
        if (i < 128) {
            const double2 ct = M->log_tab[i];           // (c_k, -log2 c_k)
            P->gk[i] = dpair(ct.x, exp2_tab(alpha * ct.y, M));
        } else {
            const double e = (double)(i - 128 + kPowExpMin);
            const double hi = alpha * e;
            const double lo = fma(alpha, e, -hi);         // alpha e = hi + lo exactly
            const double S = 64.0 * floor(hi * (1.0 / 64.0));
            const double E = exp2_tab(hi - S, M);         // hi - S in [0, 64), exact
            P->ex[i - 128] = dpair(fma(E, lo * kLn2, E),  // 2^lo = 1 + lo ln2 (|lo| <= 2^-41)
                                   double_of((uint64_t)(uint32_t)(int)S));
        }
    }
}

__host__ __device__ __forceinline__ double pow_prio_fast(float p, const PowLds* P,
                                                        const PowCoef& c) {
    const float inf = float_of(0x7F800000u);
    const bool fin = p > 0.0f && p < inf;
    const double d = (double)(fin ? p : 1.0f);
    const uint64_t db = bits_of(d);
    const uint32_t hi = (uint32_t)(db >> 32);
    const int e = (int)(hi >> 20) - 1023;
    const int k = (int)(hi >> 13) & 127;
    const double m = double_of_hi((hi & 0x000FFFFFu) | 0x3FF00000u, (uint32_t)db);
    const double2 g = P->gk[k];
    const double2 Es = P->ex[e - kPowExpMin];
    const double r = fma(m, g.x, -1.0);
    double s = fma(c.b[7], r, c.b[6]);
    s = fma(s, r, c.b[5]);
    s = fma(s, r, c.b[4]);
    s = fma(s, r, c.b[3]);
    s = fma(s, r, c.b[2]);
    s = fma(s, r, c.b[1]);
    const double t = r * s;                              // (1 + r)^alpha - 1
    const double ge = g.y * Es.x;                        // in [1, 2^80)
    const double w = ldexp(fma(ge, t, ge), (int)(uint32_t)bits_of(Es.y));
    const uint32_t sp_hi = (p == 0.0f) ? 0u : (p == inf) ? 0x7FF00000u : 0x7FF80000u;
    const double sp = double_of_hi(sp_hi, 0u);
    return fin ? w : sp;
}

// e^x for a finite double x (the particle weights).
__host__ __device__ __forceinline__ double exp_d(double x, const MathLds* M) {
    return exp2_tab(x * kLog2e, M);
}

// ------------------------------------------------ integer thresholds
// floor(((i 2^32 + r) T) / (k 2^32)) + 1  (stratified) or
// floor((r T) / 2^32) + 1 (iid), exactly, with T < 2^63 and k < 2^31.
__device__ __forceinline__ uint64_t int_threshold(uint64_t i, uint32_t r, uint64_t k, uint64_t T,
                                                  int stratified, int k_log2) {
    if (!stratified) {
        const uint64_t lo = (uint64_t)r * T;
        const uint64_t hi = __umul64hi((uint64_t)r, T);
        return ((hi << 32) | (lo >> 32)) + 1;
    }
    const uint64_t a = (i << 32) | (uint64_t)r;      // < 2^63
    const uint64_t lo = a * T;
    const uint64_t hi = __umul64hi(a, T);            // product < 2^126
    const uint64_t h2 = hi >> 32;                    // x = floor(prod / 2^32) = h2:l2
    const uint64_t l2 = (hi << 32) | (lo >> 32);
    uint64_t q;
    if (k_log2 >= 0) {
        q = (k_log2 == 0) ? l2 : ((l2 >> k_log2) | (h2 << (64 - k_log2)));
    } else {
        // floor(x / k) < 2^63 implies h2 < k: long division in 32-bit digits.
        uint64_t cur = (h2 << 32) | (l2 >> 32);
        const uint64_t q1 = cur / k;
        const uint64_t rem = cur - q1 * k;
        cur = (rem << 32) | (l2 & 0xFFFFFFFFull);
        const uint64_t q0 = cur / k;
        q = (q1 << 32) | q0;
    }
    return q + 1;
}

// ------------------------------------------------- 256-thread tile scan
// A tile of 256 threads x R rows x 4 elements: thread t holds elements
// r*1024 + 4t + c (c = 0..3) of row r.  On entry q[r][c] is the thread-local
// inclusive prefix of its 4 elements.  On exit X[r] is the sum of everything
// before the thread's 4 elements of row r (so element (r, c) has inclusive
// prefix X[r] + q[r][c]) and A is the tile total.  Association is fixed:
// DPP inside each wave, then the 4 wave totals in order, rows in order.
// s_wtot: LDS scratch of 4 x R values; the call contains one barrier.
template <int R, class Acc>
__device__ __forceinline__ void tile_scan_256(const Acc (&q)[R][4], Acc (&X)[R], Acc& A,
                                              Acc (*s_wtot)[R]) {
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    Acc iex[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const Acc I = wave_incl_scan(q[r][3]);
        iex[r] = wave_shr1(I);
        const Acc wt = readlane(I, kWave - 1);
        if (lane == 0) s_wtot[wave][r] = wt;
    }
    __syncthreads();
    A = Acc(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        Acc pw = Acc(0), rt = Acc(0);
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const Acc t = s_wtot[w2][r];
            if (w2 < wave) pw = pw + t;
            rt = rt + t;
        }
        X[r] = A + (pw + iex[r]);
        A = A + rt;
    }
}

// ------------------------------------------------- IS weights
// IS = (pmin / p)^e.  p == 0 forces pmin == 0: 0/0 -> NaN; pmin == 0 < p -> 0.
__device__ __forceinline__ float is_weight(double pmin, double lpmin, double p, double e,
                                           const MathLds* M) {
    if (!(p > 0.0)) return __int_as_float(0x7FC00000);
    if (!(pmin > 0.0)) return 0.0f;
    return (float)exp2_tab(e * (lpmin - log2_sig32(p, M)), M);
}
// The same with lp = log2(p) already known.
__device__ __forceinline__ float is_weight_lp(double pmin, double lpmin, double p, double lp,
                                              double e, const MathLds* M) {
    if (!(p > 0.0)) return __int_as_float(0x7FC00000);
    if (!(pmin > 0.0)) return 0.0f;
    return (float)exp2_tab(e * (lpmin - lp), M);
}

// Minimum over the 64 lanes (every lane active), in every lane: the DPP
// steps of wave_incl_scan with min (lanes without a source take the
// identity), then lane 63's value -- register-to-register moves instead of
// six round trips through the LDS crossbar.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp32_or(uint32_t old, uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)x, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
    constexpr uint32_t I = 0xFFFFFFFFu;
    auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
    x = mn(x, dpp32_or<kRowShr1, 0xF>(I, x));
    x = mn(x, dpp32_or<kRowShr2, 0xF>(I, x));
    x = mn(x, dpp32_or<kRowShr4, 0xF>(I, x));
    x = mn(x, dpp32_or<kRowShr8, 0xF>(I, x));
    x = mn(x, dpp32_or<kRowBcast15, 0xA>(I, x));
    x = mn(x, dpp32_or<kRowBcast31, 0xC>(I, x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, kWave - 1);
}
// Maximum over the 64 lanes (every lane active), in every lane, the same way.
__device__ __forceinline__ int wave_max_i32(int x) {
    constexpr uint32_t I = 0x80000000u;                  // INT_MIN
    auto mx = [](int a, int b) { return a > b ? a : b; };
    x = mx(x, (int)dpp32_or<kRowShr1, 0xF>(I, (uint32_t)x));
    x = mx(x, (int)dpp32_or<kRowShr2, 0xF>(I, (uint32_t)x));
    x = mx(x, (int)dpp32_or<kRowShr4, 0xF>(I, (uint32_t)x));
    x = mx(x, (int)dpp32_or<kRowShr8, 0xF>(I, (uint32_t)x));
    x = mx(x, (int)dpp32_or<kRowBcast15, 0xA>(I, (uint32_t)x));
    x = mx(x, (int)dpp32_or<kRowBcast31, 0xC>(I, (uint32_t)x));
    return __builtin_amdgcn_readlane(x, kWave - 1);
}
__device__ __forceinline__ float wave_max_f32(float x) {
    constexpr uint32_t I = 0xFF800000u;                  // -inf
    auto f = [](float v) { return __float_as_uint(v); };
    auto g = [](uint32_t v) { return __uint_as_float(v); };
    x = fmaxf(x, g(dpp32_or<kRowShr1, 0xF>(I, f(x))));
    x = fmaxf(x, g(dpp32_or<kRowShr2, 0xF>(I, f(x))));
    x = fmaxf(x, g(dpp32_or<kRowShr4, 0xF>(I, f(x))));
    x = fmaxf(x, g(dpp32_or<kRowShr8, 0xF>(I, f(x))));
    x = fmaxf(x, g(dpp32_or<kRowBcast15, 0xA>(I, f(x))));
    x = fmaxf(x, g(dpp32_or<kRowBcast31, 0xC>(I, f(x))));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kWave - 1));
}

// ------------------------------------------------------ streaming stores
// Non-temporal 16-byte stores for large output streams that no later step
// of the same kernel reads: they stream through L2 instead of settling in
// it, so less dirty data is left for the write-back at the kernel's end
// (measured: scan of 2^22 elements 21.6 -> 20.0 us, row resampling of
// 1024 x 4096 19.4 -> 17.6 us).
typedef double nt_f64x2 __attribute__((ext_vector_type(2)));
typedef unsigned long long nt_u64x2 __attribute__((ext_vector_type(2)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef int nt_i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store_nt(double* p, double a, double b) {
    const nt_f64x2 v = {a, b};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_f64x2*>(p));
}
__device__ __forceinline__ void store_nt(uint64_t* p, uint64_t a, uint64_t b) {
    const nt_u64x2 v = {(unsigned long long)a, (unsigned long long)b};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_u64x2*>(p));
}
__device__ __forceinline__ void store_nt(float* p, float a, float b, float c, float d) {
    const nt_f32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_f32x4*>(p));
}
__device__ __forceinline__ void store_nt(int32_t* p, int a, int b, int c, int d) {
    const nt_i32x4 v = {a, b, c, d};
    __builtin_nontemporal_store(v, reinterpret_cast<nt_i32x4*>(p));
}

// ------------------------------------------------------------- helpers
template <class T>
__host__ __device__ __forceinline__ T min_(T a, T b) { return a < b ? a : b; }
template <class T>
__host__ __device__ __forceinline__ T max_(T a, T b) { return a > b ? a : b; }

}  // namespace psamp
