// resample_row.h -- the ancestors of one row of systematic resampling,
// shared by the row resampler and the particle-filter step.
//
// POPCORNBENCH particle-filter trace (Kimi-K2.6, l2_p48), the reference
// model's resampling step, per row of P log-weights:
//   new_log_w = log_w - logsumexp(log_w);  weights = exp(new_log_w);
//   cumsum;  u_k = (k + u_row) / P  (float);  anc_k = searchsorted(cumsum,
//   u_k) (first index with cumsum >= u_k), clamped to P-1.
// Here: the max in float (exact), exp and the sums in double (the weights
// must be good to ~1e-9 for the ancestors to agree with an exact-arithmetic
// reading), W_j = exp(lw_j - m) / s with s = sum_j exp(lw_j - m) (equal to
// exp(lw_j - lse) with lse = m + log s, one exp per particle instead of
// two), thresholds in float exactly as the page computes them.
//
// One 256-thread workgroup per row; reads and writes are 16-byte vectors.
// No search: the thresholds are non-decreasing in k, so particle j is the
// ancestor of exactly the k with M_{j-1} < t_k <= M_j, where M is the
// running max of the row CDF ("first j with C_j >= t" is "first j with
// M_j >= t"), and the last particle also of every k with t_k > M_{P-1}.
// The number of thresholds <= x comes from its estimate x P - u, checked on
// the exact float thresholds.  Each particle with a non-empty range marks
// its first k (the first k's of non-empty ranges are distinct) and a
// block-wide max-scan over k fills every k with its particle: one heavy
// particle (hundreds of offspring are common here) costs no serial loop.
#pragma once
#include "psamp_device.h"
#include "scan_tile.h"

namespace psamp {

constexpr int kResThreads = 256;

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

// Threshold k of a row, in float exactly as the page forms it: fl(fl(k + u)
// / P).  For P a power of two, fl(a * (1/P)) is the same float (1/P is exact
// and both round the same exact quotient), without the division sequence.
template <bool POW2>
__device__ __forceinline__ double res_threshold(int k, float ub, float Pf, float invP) {
    const float a = __fadd_rn((float)k, ub);
    return (double)(POW2 ? __fmul_rn(a, invP) : __fdiv_rn(a, Pf));
}

// #{k in [0, P) : t_k <= x}.  fl(k + u) is within 2^-12 of k + u (k < 2^13)
// and t_k P equals it for a power-of-two P (else the division adds at most
// 2^-11 more), so t_k P lies within d = 2^-12 (2^-10) of k + u, and y =
// x P - u in double within 2^-39 of its exact value.  When y is at least
// eps = 2^-11 (2^-9) away from every integer, the count is floor(y) + 1
// clamped to [0, P] with no threshold formed; otherwise at most one k can be
// counted differently by that estimate, and one check on each side fixes
// it.  (A wave takes the checks for some lane on a few per cent of the
// counts.)
template <bool POW2>
__device__ __forceinline__ int res_count_le(double x, float ub, float Pf, float invP, int P) {
    constexpr double kEps = POW2 ? 0x1p-11 : 0x1p-9;
    const double y = x * (double)P - (double)ub;
    const double e = floor(y);
    const double fr = y - e;                          // exact (Sterbenz)
    const int k = !(e >= 0.0) ? 0 : (e >= (double)P ? P : (int)e + 1);
    const bool sure = (fr >= kEps && fr <= 1.0 - kEps) || e >= (double)P || e <= -2.0;
    if (__builtin_expect(sure, 1)) return k;
    const bool over = k > 0 && res_threshold<POW2>(k - 1, ub, Pf, invP) > x;
    const bool under = k < P && res_threshold<POW2>(k, ub, Pf, invP) <= x;
    return k - (over ? 1 : 0) + (under ? 1 : 0);
}

// exp(x) for x <= 0 (finite; a NaN passes through): exp2_tab without its
// clamp and NaN select, the same bits -- for x below the range that the
// clamp guards the integer conversion saturates and ldexp still gives 0.
__device__ __forceinline__ double exp_nonpos(double x, const MathLds* M) {
    const double y = x * kLog2e;
    const double N = rint(y * 64.0);
    const double f = fma(N, -1.0 / 64.0, y);
    const int Ni = (int)N;
    const double g = f * kLn2;
    double q = fma(g, 1.0 / 120.0, 1.0 / 24.0);
    q = fma(g, q, 1.0 / 6.0);
    q = fma(g, q, 0.5);
    q = fma(g, q, 1.0);
    const double s = M->exp_tab[Ni & 63];
    return ldexp(fma(s, g * q, s), Ni >> 6);
}

template <int R>
struct ResLds {
    // first-offspring marks: O[k] = j + 1 if particle j's offspring start at k
    __attribute__((aligned(16))) uint16_t O[R * kResThreads * 4];
    uint32_t s_wm[4][R];
    uint32_t s_lastk[4][R];
    double s_wtot[4][R];
    double s_wmax[4][R];
    float s_max[4];
    double s_sum[4];
};

// The ancestors of one row.  v: this thread's log-weights r*1024 + 4t + c
// (-inf past the end of the row).  On return anc[r][c] is the ancestor of
// offspring k = r*1024 + 4t + c (k < P).  M must be written and visible
// after the first barrier (the caller stores it before calling).
// POW2: P is a power of two (see res_threshold).
template <int R, bool POW2>
__device__ __forceinline__ void res_ancestors(const float (&v)[R][4], int Pi, float ub,
                                              const MathLds* M, ResLds<R>& L,
                                              uint32_t (&anc)[R][4]) {
    constexpr int ROW = kResThreads * 4;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const float ninf = __int_as_float(0xFF800000);

    // max (float, exact)
    float mx = ninf;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) mx = fmaxf(mx, v[r][c]);
    mx = wave_max_f32(mx);
    if (lane == 0) L.s_max[wave] = mx;
    __syncthreads();
    const double m =
        (double)fmaxf(fmaxf(L.s_max[0], L.s_max[1]), fmaxf(L.s_max[2], L.s_max[3]));

    // e_j = exp(lw_j - m) in double, thread-local prefixes, row sum s
    double q[R][4];
    double ssum = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const double e = (v[r][c] == ninf) ? 0.0 : exp_nonpos((double)v[r][c] - m, M);
            q[r][c] = e;
            ssum = ssum + e;
        }
    ssum = wave_sum(ssum);
    if (lane == 0) L.s_sum[wave] = ssum;
    __syncthreads();
    const double s = ((L.s_sum[0] + L.s_sum[1]) + L.s_sum[2]) + L.s_sum[3];
    const double inv_s = 1.0 / s;

    // W_j = e_j / s; inclusive scan of W (double); M = its running max
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const double w = q[r][c] * inv_s;
            q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
        }
    double X[R];
    double A;
    tile_scan_256<R, double>(q, X, A, L.s_wtot);
    tile_local_values<R, double>(q, X, L.s_wmax);

    // ancestors: particle j takes k in [#{t <= M_{j-1}}, #{t <= M_j}); the
    // last particle also every k above.  O[k] = j + 1 at the first k of each
    // non-empty range, 0 elsewhere.  kc: the counts at this thread's values;
    // kp[r]: the count at the element before its first element of row r
    // (the neighbour's last count, through DPP and, across waves and rows,
    // LDS).
    const float Pf = (float)Pi;
    const float invP = 1.0f / Pf;              // exact when POW2
    uint32_t kc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = r * ROW + 4 * tid + c;
            kc[r][c] = (uint32_t)((j >= Pi - 1) ? Pi : res_count_le<POW2>(q[r][c], ub, Pf, invP, Pi));
        }
    uint32_t kp[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        kp[r] = dpp32<kWaveShr1, 0xF, true>(kc[r][3]);
        if (lane == kWave - 1) L.s_lastk[wave][r] = kc[r][3];
        *reinterpret_cast<uint2*>(&L.O[r * ROW + 4 * tid]) = make_uint2(0u, 0u);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (lane == 0)
            kp[r] = wave > 0 ? L.s_lastk[wave - 1][r] : (r > 0 ? L.s_lastk[3][r - 1] : 0u);
        const int j0 = r * ROW + 4 * tid;
        uint32_t k0 = j0 == 0 ? 0u : kp[r];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = j0 + c;
            const uint32_t k1 = kc[r][c];
            if (j < Pi && k1 > k0) L.O[k0] = (uint16_t)(j + 1);
            k0 = k1 > k0 ? k1 : k0;
        }
    }
    __syncthreads();

    // inclusive max-scan over k (rows, then threads, then columns): the
    // particle of every k
    uint32_t a[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint2 t2 = *reinterpret_cast<const uint2*>(&L.O[r * ROW + 4 * tid]);
        a[r][0] = t2.x & 0xFFFFu;
        a[r][1] = max_(a[r][0], t2.x >> 16);
        a[r][2] = max_(a[r][1], t2.y & 0xFFFFu);
        a[r][3] = max_(a[r][2], t2.y >> 16);
    }
    uint32_t ex[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t y = a[r][3];
        y = max_(y, dpp32<kRowShr1, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr2, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr4, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr8, 0xF, true>(y));
        y = max_(y, dpp32<kRowBcast15, 0xA, false>(y));
        y = max_(y, dpp32<kRowBcast31, 0xC, false>(y));
        ex[r] = dpp32<kWaveShr1, 0xF, true>(y);
        const uint32_t wm = (uint32_t)__builtin_amdgcn_readlane((int)y, kWave - 1);
        if (lane == 0) L.s_wm[wave][r] = wm;
    }
    __syncthreads();
    uint32_t carry = 0u;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        uint32_t pm = carry, rm = carry;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
            const uint32_t t = L.s_wm[w2][r];
            if (w2 < wave) pm = max_(pm, t);
            rm = max_(rm, t);
        }
        pm = max_(pm, ex[r]);
        carry = rm;
#pragma unroll
        for (int c = 0; c < 4; ++c) anc[r][c] = max_(a[r][c], pm) - 1u;
    }
}

}  // namespace psamp
