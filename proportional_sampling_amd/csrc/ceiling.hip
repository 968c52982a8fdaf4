// ceiling.hip -- a measurement aid: the bandwidth ceiling of the CDF scan.
//
// The scan reads 4 bytes and writes 8 bytes per element.  This kernel moves
// exactly those bytes (f32 in, the same value as f64 out) with no arithmetic
// and no exchange between workgroups, in the scan's own access pattern
// (256 threads, rows of 1024 elements, each thread 4 consecutive elements of
// a row as one 16-byte load and two 16-byte non-temporal stores), so the time
// it takes on a box is the best the scan's bytes can do there.  Two
// geometries: the scan's tile (8 rows, 8192 elements per workgroup) and a
// smaller one (4 rows), which lets more workgroups share a CU.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

template <int R, bool NT>
__global__ __launch_bounds__(256) void k_ceiling_copy(const float* __restrict__ in,
                                                      double* __restrict__ out, int64_t n) {
    constexpr int ROW = 256 * 4;
    const int64_t base = (int64_t)blockIdx.x * ROW * R + 4 * (int64_t)threadIdx.x;
    float4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t e = base + (int64_t)r * ROW;
        v[r] = e < n ? *reinterpret_cast<const float4*>(in + e) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t e = base + (int64_t)r * ROW;
        if (e < n) {
            if constexpr (NT) {
                store_nt(out + e, (double)v[r].x, (double)v[r].y);
                store_nt(out + e + 2, (double)v[r].z, (double)v[r].w);
            } else {
                reinterpret_cast<double2*>(out + e)[0] = make_double2(v[r].x, v[r].y);
                reinterpret_cast<double2*>(out + e)[1] = make_double2(v[r].z, v[r].w);
            }
        }
    }
}

template <int R, bool NT>
static void launch_copy(const float* in, double* out, int64_t n, hipStream_t st) {
    const int64_t grid = ceil_div(n, (int64_t)1024 * R);
    hipLaunchKernelGGL((k_ceiling_copy<R, NT>), dim3((unsigned)grid), dim3(256), 0, st, in, out,
                       n);
}

}  // namespace psamp

using namespace psamp;

extern "C" psamp_status psamp_ceiling_copy(const float* in, double* out, int64_t n, int rows,
                                           int nt, void* stream) {
    if (!in || !out) return PSAMP_E_NULL;
    if (n < 4 || n > kMaxN || n % 4 != 0) return PSAMP_E_SIZE;
    if ((rows != 2 && rows != 4 && rows != 8) || (nt != 0 && nt != 1)) return PSAMP_E_PARAM;
    if (!aligned(in, 16) || !aligned(out, 16)) return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (nt) {
        if (rows == 8) launch_copy<8, true>(in, out, n, st);
        else if (rows == 4) launch_copy<4, true>(in, out, n, st);
        else launch_copy<2, true>(in, out, n, st);
    } else {
        if (rows == 8) launch_copy<8, false>(in, out, n, st);
        else if (rows == 4) launch_copy<4, false>(in, out, n, st);
        else launch_copy<2, false>(in, out, n, st);
    }
    return launch_status();
}
