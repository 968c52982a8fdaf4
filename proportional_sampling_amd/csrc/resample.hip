// resample.hip -- row-batched systematic resampling.
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
// One 256-thread workgroup per row; the row's CDF stays in LDS (8 B per
// particle) for the searches; reads and writes are 16-byte vectors.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kResThreads = 256;

__device__ __forceinline__ float wave_max_f32(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
    return x;
}

template <int R>
__global__ __launch_bounds__(kResThreads) void k_resample_rows(
    const float* __restrict__ lw, int64_t P, int64_t ld_in, const float* __restrict__ u_row,
    int32_t* __restrict__ anc, int64_t ld_out, int vec_ok) {
    constexpr int ROW = kResThreads * 4;
    __shared__ double C[R * ROW];
    __shared__ double s_wtot[4][R];
    __shared__ float s_max[4];
    __shared__ double s_sum[4];
    __shared__ MathLds M;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int64_t b = blockIdx.x;
    const float* x = lw + b * ld_in;
    math_lds_fill(&M, tid, kResThreads);

    const float ninf = __int_as_float(0xFF800000);
    const bool full = P == (int64_t)R * ROW;
    float v[R][4];
    if (full && vec_ok) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float4 t = *reinterpret_cast<const float4*>(x + r * ROW + 4 * tid);
            v[r][0] = t.x; v[r][1] = t.y; v[r][2] = t.z; v[r][3] = t.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t j = (int64_t)r * ROW + 4 * tid + c;
                v[r][c] = j < P ? x[j] : ninf;
            }
    }

    // max (float, exact)
    float mx = ninf;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) mx = fmaxf(mx, v[r][c]);
    mx = wave_max_f32(mx);
    if (lane == 0) s_max[wave] = mx;
    __syncthreads();
    const double m = (double)fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));

    // e_j = exp(lw_j - m) in double, thread-local prefixes, row sum s
    double q[R][4];
    double ssum = 0.0;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const double e = (v[r][c] == ninf) ? 0.0 : exp_d((double)v[r][c] - m, &M);
            q[r][c] = e;
            ssum = ssum + e;
        }
    ssum = wave_sum(ssum);
    if (lane == 0) s_sum[wave] = ssum;
    __syncthreads();
    const double s = ((s_sum[0] + s_sum[1]) + s_sum[2]) + s_sum[3];
    const double inv_s = 1.0 / s;

    // W_j = e_j / s; inclusive scan of W (double) into LDS
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const double w = q[r][c] * inv_s;
            q[r][c] = (c == 0) ? w : q[r][c - 1] + w;
        }
    double X[R];
    double A;
    tile_scan_256<R, double>(q, X, A, s_wtot);
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) C[r * ROW + 4 * tid + c] = X[r] + q[r][c];
    __syncthreads();

    // thresholds u_k = (k + u_row) / P in float; lower_bound in the LDS CDF
    const float ub = u_row[b];
    const float Pf = (float)P;
    int32_t o[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int kk = r * ROW + 4 * tid + c;
            const float uk = __fdiv_rn(__fadd_rn((float)kk, ub), Pf);
            const double t = (double)uk;
            int lo = 0;
            int len = (int)P;
            while (len > 1) {
                const int half = len >> 1;
                lo = (C[lo + half - 1] < t) ? lo + half : lo;
                len -= half;
            }
            lo += (C[lo] < t) ? 1 : 0;
            o[r][c] = lo < P ? lo : (int32_t)(P - 1);
        }
    int32_t* out = anc + b * ld_out;
    if (full && vec_ok) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            *reinterpret_cast<int4*>(out + r * ROW + 4 * tid) =
                make_int4(o[r][0], o[r][1], o[r][2], o[r][3]);
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int64_t j = (int64_t)r * ROW + 4 * tid + c;
                if (j < P) out[j] = o[r][c];
            }
    }
}

template <int R>
static void launch_rows(const float* logw, int64_t rows, int64_t P, int64_t ld_in,
                        const float* u_row, int32_t* out, int64_t ld_out, int vec_ok,
                        hipStream_t st) {
    if (trace_enabled()) trace_launch("k_resample_rows", rows, kResThreads, P);
    hipLaunchKernelGGL(k_resample_rows<R>, dim3((unsigned)rows), dim3(kResThreads), 0, st, logw, P,
                       ld_in, u_row, out, ld_out, vec_ok);
}

}  // namespace psamp

using namespace psamp;

extern "C" psamp_status psamp_resample_rows(const float* logw, int64_t rows, int64_t P,
                                            int64_t ld_in, const float* u_row, int32_t* out_anc,
                                            int64_t ld_out, void* stream) {
    if (!logw || !u_row || !out_anc) return PSAMP_E_NULL;
    if (rows < 1 || rows > kMaxN || P < 1 || P > 8192 || ld_in < P || ld_out < P)
        return PSAMP_E_SIZE;
    if (!aligned(logw, 4) || !aligned(u_row, 4) || !aligned(out_anc, 4)) return PSAMP_E_ALIGN;
    const int vec_ok = aligned(logw, 16) && aligned(out_anc, 16) && ld_in % 4 == 0 &&
                       ld_out % 4 == 0;
    hipStream_t st = as_stream(stream);
    const int64_t R = ceil_div(P, kResThreads * 4);
    if (R <= 1) launch_rows<1>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else if (R <= 2) launch_rows<2>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else if (R <= 4) launch_rows<4>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else launch_rows<8>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    return launch_status();
}
