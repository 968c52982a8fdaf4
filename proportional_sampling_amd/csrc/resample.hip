// resample.hip -- row-batched systematic resampling (the per-row ancestor
// computation is in resample_row.h).
#include "psamp_device.h"
#include "psamp_host.h"
#include "resample_row.h"

namespace psamp {

template <int R, bool POW2>
__global__ __launch_bounds__(kResThreads) void k_resample_rows(
    const float* __restrict__ lw, int64_t P, int64_t ld_in, const float* __restrict__ u_row,
    int32_t* __restrict__ anc, int64_t ld_out, int vec_ok) {
    constexpr int ROW = kResThreads * 4;
    __shared__ ResLds<R> L;

    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const float* x = lw + b * ld_in;
    const double et = exp_row_tab_load(tid);     // (the exp table, with the first loads)
    const float ub = u_row[b];

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
                const float t = x[j < P ? j : 0];
                v[r][c] = j < P ? t : ninf;
            }
    }
    L.etab[tid] = et;

    const int Pi = (int)P;
    uint32_t a[R][4];
    res_ancestors<R, POW2>(v, Pi, ub, L, a);

    int32_t* out = anc + b * ld_out;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int e0 = r * ROW + 4 * tid;
        if (full && vec_ok) {
            store_nt(out + e0, (int)a[r][0], (int)a[r][1], (int)a[r][2], (int)a[r][3]);
        } else {
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (e0 + c < Pi) out[e0 + c] = (int32_t)a[r][c];
        }
    }
}

template <int R>
static void launch_rows(const float* logw, int64_t rows, int64_t P, int64_t ld_in,
                        const float* u_row, int32_t* out, int64_t ld_out, int vec_ok,
                        hipStream_t st) {
    if (trace_enabled()) trace_launch("k_resample_rows", rows, kResThreads, P);
    if ((P & (P - 1)) == 0)
        hipLaunchKernelGGL((k_resample_rows<R, true>), dim3((unsigned)rows), dim3(kResThreads), 0,
                           st, logw, P, ld_in, u_row, out, ld_out, vec_ok);
    else
        hipLaunchKernelGGL((k_resample_rows<R, false>), dim3((unsigned)rows), dim3(kResThreads),
                           0, st, logw, P, ld_in, u_row, out, ld_out, vec_ok);
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
    if (check_on()) {
        check_f32(logw, rows, P, ld_in, kChkLogw, PSAMP_CHECK_LOGWEIGHT, st);
        check_unit(u_row, rows, st);
    }
    const int64_t R = ceil_div(P, kResThreads * 4);
    if (R <= 1) launch_rows<1>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else if (R <= 2) launch_rows<2>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else if (R <= 4) launch_rows<4>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    else launch_rows<8>(logw, rows, P, ld_in, u_row, out_anc, ld_out, vec_ok, st);
    return launch_status();
}
