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
