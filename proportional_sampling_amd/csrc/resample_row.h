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
// two), thresholds in float exactly as the page computes them.  The scan
// runs over the unnormalised e_j = exp(lw_j - m), its total is s, and the
// division by s goes into the threshold counts (C_j = E_j / s).
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

// Threshold k of a row, in float exactly as the page forms it: fl(fl(k + u)
// / P).  For P a power of two, fl(a * (1/P)) is the same float (1/P is exact
// and both round the same exact quotient), without the division sequence.
template <bool POW2>
__device__ __forceinline__ double res_threshold(int k, float ub, float Pf, float invP) {
    const float a = __fadd_rn((float)k, ub);
    return (double)(POW2 ? __fmul_rn(a, invP) : __fdiv_rn(a, Pf));
}

// #{k in [0, P) : t_k <= x} for x = E inv_s, E an unnormalised CDF value,
// sP = P inv_s and omu = 1 - u (exact).  fl(k + u) is within 2^-12 of k + u
// (k < 2^13) and t_k P equals it for a power-of-two P (else the division adds
// at most 2^-11 more), so t_k P lies within d = 2^-12 (2^-10) of k + u.
// z = E sP + (1 - u) in double (one rounding) is x P - u + 1 to within 2^-38,
// and positive (E >= 0, u < 1): its truncation is floor(x P - u) + 1 and its
// fraction that of x P - u.  When that fraction is at least eps = 2^-11
// (2^-9) away from 0 and 1, the count is the truncation clamped to P, with
// no threshold formed; otherwise at most one k can be counted differently by
// that estimate, and one check on each side (against x itself) fixes it.
// (A wave takes the checks for some lane on a few per cent of the counts.)
template <bool POW2>
__device__ __forceinline__ int res_count_le(double E, double inv_s, double sP, double omu,
                                            float ub, float Pf, float invP, int P) {
    constexpr double kEps = POW2 ? 0x1p-11 : 0x1p-9;
    const double z = fma(E, sP, omu);                  // one rounding
    const int k = min_((int)z, P);                    // (the conversion gives 0 for NaN)
    const double fr = __builtin_amdgcn_fract(z);      // z - floor(z), exact
    // fr in [eps, 1 - eps] (fr - 0.5 is exact: fr is a multiple of 2^-40)
    if (__builtin_expect(fabs(fr - 0.5) <= 0.5 - kEps, 1)) return k;
    const double x = E * inv_s;
    const bool over = k > 0 && res_threshold<POW2>(k - 1, ub, Pf, invP) > x;
    const bool under = k < P && res_threshold<POW2>(k, ub, Pf, invP) <= x;
    return k - (over ? 1 : 0) + (under ? 1 : 0);
}

// exp(x) for x in [-2^20, 0] in double, within 2e-13 relative where the
// result is a normal double (the weights need about 1e-9 for the ancestors
// to follow an exact-arithmetic reading):
// x = N ln2/256 + g with |g| <= ln2/512 (to within a rounding), exp(x) =
// 2^(N/256) e^g, 2^(j/256) from a 256-entry table (correctly rounded), e^g
// from its cubic Taylor polynomial (truncation below 1.4e-13 relative);
// ln2/256 rounded to double adds at most |N| 2^-61 to g.  N is rounded to
// an integer by adding 1.5 2^52 (the sum's unit is 1), which also leaves N in
// the sum's low word.  Below the double range the result is 0 (ldexp
// underflows); a NaN passes through.  The caller keeps x at or above -2^20.
__host__ __device__ __forceinline__ double exp_row(double x, const double* __restrict__ tab) {
    constexpr double kShift = 0x1.8p52;
    const double t = fma(x, 0x1.71547652b82fep+8, kShift);   // 256 / ln 2
    const double N = t - kShift;                              // exact
    const int Ni = (int)(uint32_t)bits_of(t);                 // N, two's complement
    const double g = fma(N, -0x1.62e42fefa39efp-9, x);        // ln 2 / 256
    const double b = fma(g, fma(g, 1.0 / 6.0, 0.5), 1.0);
    const double s = tab[Ni & 255];
    return ldexp(fma(s, g * b, s), Ni >> 8);
}

// The table of exp_row, one entry per thread of a 256-thread block: each
// thread loads its entry with its first loads and stores it to LDS later.
__host__ __device__ __forceinline__ double exp_row_tab_load(int tid) {
    return double_of(kExp2Tab256[tid & 255]);
}

template <int R>
struct ResLds {
    // first-offspring marks: O[k] = j + 1 if particle j's offspring start at k
    __attribute__((aligned(16))) uint16_t O[R * kResThreads * 4];
    uint32_t s_wm[4][R];
    uint32_t s_lastk[4][R];
    double s_wtot[4][R];
    float s_max[4];
    double etab[256];          // the table of exp_row (the caller stores it)
};

// The ancestors of one row.  v: this thread's log-weights r*1024 + 4t + c
// (-inf past the end of the row).  On return anc[r][c] is the ancestor of
// offspring k = r*1024 + 4t + c (k < P).  L.etab must be written (thread t
// entry t, exp_row_tab_load) and is read after the first barrier.
// POW2: P is a power of two (see res_threshold).
template <int R, bool POW2>
__device__ __forceinline__ void res_ancestors(const float (&v)[R][4], int Pi, float ub,
                                              ResLds<R>& L, uint32_t (&anc)[R][4]) {
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

    // e_j = exp(lw_j - m) in double and their thread-local prefixes; the
    // unnormalised CDF E (double) and its total s
    double q[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            // (-inf, and a NaN, weigh 0: exp(-1000) is 0 in double)
            const double e = exp_row(fmax((double)v[r][c] - m, -1000.0), L.etab);
            q[r][c] = (c == 0) ? e : q[r][c - 1] + e;
        }
    double X[R];
    double s;
    tile_scan_256<R, double>(q, X, s, L.s_wtot);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) q[r][c] = X[r] + q[r][c];
    const double inv_s = 1.0 / s;
    const double sP = (double)Pi / s;

    // ancestors: with M_j = max_{i <= j} C_i, particle j takes the k in
    // [#{t <= M_{j-1}}, #{t <= M_j}), the last particle also every k above
    // ("first j with C_j >= t" is "first j with M_j >= t").  The count is
    // non-decreasing in its argument, so #{t <= M_j} = max_{i <= j} #{t <=
    // C_i}: a running max of integers over the counts at the C values, which
    // need not be monotone themselves.  O[k] = j + 1 at the first k of each
    // non-empty range, 0 elsewhere.
    const float Pf = (float)Pi;
    const float invP = 1.0f / Pf;              // exact when POW2
    const double omu = 1.0 - (double)ub;
    uint32_t kc[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = r * ROW + 4 * tid + c;
            kc[r][c] = (uint32_t)((j >= Pi - 1) ? Pi
                                                : res_count_le<POW2>(q[r][c], inv_s, sP, omu, ub, Pf, invP, Pi));
        }
    // running max in element order: within the thread's 4, across the
    // wave's lanes (DPP), then across waves and rows (LDS)
    uint32_t kx[R];                            // max over the elements before the thread's first in row r, within its wave
#pragma unroll
    for (int r = 0; r < R; ++r) {
        kc[r][1] = max_(kc[r][0], kc[r][1]);
        kc[r][2] = max_(kc[r][1], kc[r][2]);
        kc[r][3] = max_(kc[r][2], kc[r][3]);
        uint32_t y = kc[r][3];
        y = max_(y, dpp32<kRowShr1, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr2, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr4, 0xF, true>(y));
        y = max_(y, dpp32<kRowShr8, 0xF, true>(y));
        y = max_(y, dpp32<kRowBcast15, 0xA, false>(y));
        y = max_(y, dpp32<kRowBcast31, 0xC, false>(y));
        kx[r] = dpp32<kWaveShr1, 0xF, true>(y);
        const uint32_t wm = (uint32_t)__builtin_amdgcn_readlane((int)y, kWave - 1);
        if (lane == 0) L.s_lastk[wave][r] = wm;
        *reinterpret_cast<uint2*>(&L.O[r * ROW + 4 * tid]) = make_uint2(0u, 0u);
    }
    __syncthreads();
    {
        uint32_t carry = 0u;                   // max over the earlier rows
#pragma unroll
        for (int r = 0; r < R; ++r) {
            uint32_t pm = carry, rm = carry;
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
                const uint32_t t = L.s_lastk[w2][r];
                if (w2 < wave) pm = max_(pm, t);
                rm = max_(rm, t);
            }
            carry = rm;
            uint32_t k0 = max_(pm, kx[r]);
            const int j0 = r * ROW + 4 * tid;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = j0 + c;
                const uint32_t k1 = max_(kc[r][c], k0);
                if (j < Pi && k1 > k0) L.O[k0] = (uint16_t)(j + 1);
                k0 = k1;
            }
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
