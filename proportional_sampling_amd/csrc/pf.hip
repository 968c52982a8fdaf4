// pf.hip -- one particle-filter step, fused: predict, Gaussian observation
// log-likelihood, log-weight update, systematic resampling, gather.
//
// POPCORNBENCH particle-filter trace (Kimi-K2.6, l2_p48), the reference
// model's forward pass, per filter b of P particles in D dimensions with O
// observed values:
//   pred_j = A x_j + sigma_p eps_j;  y_j = C pred_j;
//   ll_j = -0.5 sum_o (obs_o - y_jo)^2 / sigma_o^2;  lw'_j = lw_j + ll_j;
//   anc = systematic resampling of lw' (resample_row.h);
//   x_out_k = pred_{anc_k};  lw_out_k = -log P.
// Everything up to lw' in float32 in a fixed order (each dot product summed
// in increasing index starting from +0, the noise term added last,
// ll = (-0.5 S) / sigma_o^2 with a correctly rounded division); the
// resampling as psamp_resample_rows.
//
// One 256-thread workgroup per filter.  Particles are read and written one
// per lane (consecutive lanes, consecutive particles: 16-byte vectors when
// D = 4), pred is kept in LDS component by component (pred_S[d][j]), the
// weights in the resampler's layout (4 consecutive particles per thread) are
// formed from LDS, and the gather reads the ancestor's pred from LDS.  HBM:
// x, eps and lw in, x_out and lw_out (and the ancestors) out, once each.
#include "psamp_device.h"
#include "psamp_host.h"
#include "resample_row.h"

namespace psamp {

constexpr int kPfMaxO = 8;
constexpr int kPfMaxLds = 16384;    // floats of pred per workgroup (P * D)

template <int D>
struct PVec {
    float v[D];
};

// One particle's D floats at p (16-byte aligned when D >= 4, 8-byte when
// D = 2).
template <int D>
__device__ __forceinline__ PVec<D> load_particle(const float* p) {
    PVec<D> r;
    if constexpr (D == 1) {
        r.v[0] = p[0];
    } else if constexpr (D == 2) {
        const float2 t = *reinterpret_cast<const float2*>(p);
        r.v[0] = t.x; r.v[1] = t.y;
    } else {
#pragma unroll
        for (int h = 0; h < D / 4; ++h) {
            const float4 t = *reinterpret_cast<const float4*>(p + 4 * h);
            r.v[4 * h] = t.x; r.v[4 * h + 1] = t.y; r.v[4 * h + 2] = t.z; r.v[4 * h + 3] = t.w;
        }
    }
    return r;
}

template <int D>
__device__ __forceinline__ void store_particle(float* p, const PVec<D>& r) {
    if constexpr (D == 1) {
        p[0] = r.v[0];
    } else if constexpr (D == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(r.v[0], r.v[1]);
    } else {
#pragma unroll
        for (int h = 0; h < D / 4; ++h)
            *reinterpret_cast<float4*>(p + 4 * h) =
                make_float4(r.v[4 * h], r.v[4 * h + 1], r.v[4 * h + 2], r.v[4 * h + 3]);
    }
}

// x, lw and their outputs may be the same arrays (every read of a filter
// precedes a barrier that precedes its writes), so they are not restrict.
template <int R, bool POW2, int D>
__global__ __launch_bounds__(kResThreads) void k_pf_step(
    const float* x, const float* lw, const float* __restrict__ obs,
    const float* __restrict__ A, const float* __restrict__ Cm, const float* __restrict__ eps,
    float sigma_p, float s2, float neg_log_p, const float* __restrict__ u_row, int64_t P, int O,
    float* x_out, float* lw_out, int32_t* __restrict__ anc_out, int lw_vec) {
    constexpr int ROW = kResThreads * 4;
    constexpr int RW = R * ROW;               // particles a workgroup can hold
    static_assert(RW * D <= kPfMaxLds, "pred does not fit the LDS budget");
    __shared__ __attribute__((aligned(16))) float predS[D * RW];
    __shared__ ResLds<R> L;

    const int tid = threadIdx.x;
    const int64_t b = blockIdx.x;
    const int Pi = (int)P;
    const float* xb = x + b * P * D;
    const float* eb = eps + b * P * D;
    const float* lb = lw + b * P;
    const float* ob = obs + (int64_t)b * O;
    const double et = exp_row_tab_load(tid);     // (the exp table, with the first loads)
    const float ub = u_row[b];
    const float ninf = __int_as_float(0xFF800000);

    // this thread's log-weights, resampler layout (r*1024 + 4t + c)
    float lwv[R][4];
    if (lw_vec && Pi == RW) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float4 t = *reinterpret_cast<const float4*>(lb + r * ROW + 4 * tid);
            lwv[r][0] = t.x; lwv[r][1] = t.y; lwv[r][2] = t.z; lwv[r][3] = t.w;
        }
    } else {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = r * ROW + 4 * tid + c;
                lwv[r][c] = lb[j < Pi ? j : 0];
            }
    }

    // predict, one particle per lane: j = r*1024 + 256c + t (loads clamped
    // to the row and issued together; the stores are guarded)
    PVec<D> xs[R][4], es[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = r * ROW + c * kResThreads + tid;
            const int jc = j < Pi ? j : Pi - 1;
            xs[r][c] = load_particle<D>(xb + (int64_t)jc * D);
            es[r][c] = load_particle<D>(eb + (int64_t)jc * D);
        }
    float Am[D][D];
#pragma unroll
    for (int d = 0; d < D; ++d)
#pragma unroll
        for (int k = 0; k < D; ++k) Am[d][k] = A[d * D + k];
    L.etab[tid] = et;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = r * ROW + c * kResThreads + tid;
#pragma unroll
            for (int d = 0; d < D; ++d) {
                float acc = 0.0f;
#pragma unroll
                for (int k = 0; k < D; ++k) acc = acc + Am[d][k] * xs[r][c].v[k];
                const float pd = acc + sigma_p * es[r][c].v[d];
                if (j < Pi) predS[d * RW + j] = pd;
            }
        }
    __syncthreads();

    // likelihood and updated log-weights, resampler layout
    float v[R][4];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float pr[D][4];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const float4 t = *reinterpret_cast<const float4*>(&predS[d * RW + r * ROW + 4 * tid]);
            pr[d][0] = t.x; pr[d][1] = t.y; pr[d][2] = t.z; pr[d][3] = t.w;
        }
        float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int o = 0; o < O; ++o) {
            const float obv = ob[o];
            float Cr[D];
#pragma unroll
            for (int d = 0; d < D; ++d) Cr[d] = Cm[o * D + d];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float y = 0.0f;
#pragma unroll
                for (int d = 0; d < D; ++d) y = y + Cr[d] * pr[d][c];
                const float diff = obv - y;
                S[c] = S[c] + diff * diff;
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = r * ROW + 4 * tid + c;
            const float ll = __fdiv_rn(-0.5f * S[c], s2);
            v[r][c] = j < Pi ? lwv[r][c] + ll : ninf;
        }
    }

    uint32_t a[R][4];
    res_ancestors<R, POW2>(v, Pi, ub, L, a);

    // every read of L.O happened before the last barrier of res_ancestors:
    // reuse it to hand the ancestors to the gather layout
#pragma unroll
    for (int r = 0; r < R; ++r)
        *reinterpret_cast<uint2*>(&L.O[r * ROW + 4 * tid]) =
            make_uint2(a[r][0] | (a[r][1] << 16), a[r][2] | (a[r][3] << 16));
    __syncthreads();

    float* xo = x_out + b * P * D;
    float* lo = lw_out + b * P;
    int32_t* ao = anc_out ? anc_out + b * P : nullptr;
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int k = r * ROW + c * kResThreads + tid;
            if (k < Pi) {
                const int an = (int)L.O[k];
                PVec<D> pv;
#pragma unroll
                for (int d = 0; d < D; ++d) pv.v[d] = predS[d * RW + an];
                store_particle<D>(xo + (int64_t)k * D, pv);
                lo[k] = neg_log_p;
                if (ao) ao[k] = an;
            }
        }
}

template <int R, bool POW2, int D>
static void launch_pf(const float* x, const float* lw, const float* obs, const float* A,
                      const float* Cm, const float* eps, float sigma_p, float s2, float nlp,
                      const float* u_row, int64_t rows, int64_t P, int O, float* x_out,
                      float* lw_out, int32_t* anc, int lw_vec, hipStream_t st) {
    hipLaunchKernelGGL((k_pf_step<R, POW2, D>), dim3((unsigned)rows), dim3(kResThreads), 0, st,
                       x, lw, obs, A, Cm, eps, sigma_p, s2, nlp, u_row, P, O, x_out, lw_out, anc,
                       lw_vec);
}

template <int R, int D>
static void launch_pf_p2(bool pow2, const float* x, const float* lw, const float* obs,
                         const float* A, const float* Cm, const float* eps, float sigma_p,
                         float s2, float nlp, const float* u_row, int64_t rows, int64_t P, int O,
                         float* x_out, float* lw_out, int32_t* anc, int lw_vec, hipStream_t st) {
    if (pow2)
        launch_pf<R, true, D>(x, lw, obs, A, Cm, eps, sigma_p, s2, nlp, u_row, rows, P, O, x_out,
                              lw_out, anc, lw_vec, st);
    else
        launch_pf<R, false, D>(x, lw, obs, A, Cm, eps, sigma_p, s2, nlp, u_row, rows, P, O,
                               x_out, lw_out, anc, lw_vec, st);
}

// false when (R, D) has no instantiation (P * D over the LDS budget)
template <int R>
static bool launch_pf_d(int64_t D, bool pow2, const float* x, const float* lw, const float* obs,
                        const float* A, const float* Cm, const float* eps, float sigma_p,
                        float s2, float nlp, const float* u_row, int64_t rows, int64_t P, int O,
                        float* x_out, float* lw_out, int32_t* anc, int lw_vec, hipStream_t st) {
#define PF_D(DD)                                                                              \
    launch_pf_p2<R, DD>(pow2, x, lw, obs, A, Cm, eps, sigma_p, s2, nlp, u_row, rows, P, O, x_out, \
                        lw_out, anc, lw_vec, st)
    if (D == 1) {
        PF_D(1);
        return true;
    }
    if (D == 2) {
        PF_D(2);
        return true;
    }
    if constexpr (R * kResThreads * 4 * 4 <= kPfMaxLds) {
        if (D == 4) {
            PF_D(4);
            return true;
        }
    }
    if constexpr (R * kResThreads * 4 * 8 <= kPfMaxLds) {
        if (D == 8) {
            PF_D(8);
            return true;
        }
    }
#undef PF_D
    return false;
}

}  // namespace psamp

using namespace psamp;

extern "C" psamp_status psamp_pf_step(const float* x, const float* logw, const float* obs,
                                      const float* A, const float* C, const float* eps,
                                      float sigma_p, float sigma_o, const float* u_row,
                                      int64_t rows, int64_t P, int64_t D, int64_t O, float* x_out,
                                      float* logw_out, int32_t* anc_out, void* stream) {
    if (!x || !logw || !obs || !A || !C || !eps || !u_row || !x_out || !logw_out)
        return PSAMP_E_NULL;
    if (rows < 1 || rows > kMaxN || P < 1 || P > 8192 || O < 1 || O > kPfMaxO ||
        !(D == 1 || D == 2 || D == 4 || D == 8) || P * D > kPfMaxLds)
        return PSAMP_E_SIZE;
    if (!(sigma_o > 0.0f) || !(sigma_o - sigma_o == 0.0f) || !(sigma_p - sigma_p == 0.0f))
        return PSAMP_E_PARAM;
    if (!aligned(x, 16) || !aligned(eps, 16) || !aligned(x_out, 16) || !aligned(logw, 4) ||
        !aligned(logw_out, 4) || !aligned(obs, 4) || !aligned(A, 4) || !aligned(C, 4) ||
        !aligned(u_row, 4) || (anc_out && !aligned(anc_out, 4)))
        return PSAMP_E_ALIGN;
    const float s2 = sigma_o * sigma_o;
    const float nlp = (float)(-std::log((double)P));
    const int lw_vec = aligned(logw, 16) && P % 4 == 0;
    const bool pow2 = (P & (P - 1)) == 0;
    hipStream_t st = as_stream(stream);
    if (check_on()) {
        check_f32(logw, rows, P, P, kChkLogw, PSAMP_CHECK_LOGWEIGHT, st);
        check_unit(u_row, rows, st);
    }
    const int64_t R = ceil_div(P, kResThreads * 4);
    if (trace_enabled()) trace_launch("k_pf_step", rows, kResThreads, P);
    bool ok;
    if (R <= 1)
        ok = launch_pf_d<1>(D, pow2, x, logw, obs, A, C, eps, sigma_p, s2, nlp, u_row, rows, P,
                       (int)O, x_out, logw_out, anc_out, lw_vec, st);
    else if (R <= 2)
        ok = launch_pf_d<2>(D, pow2, x, logw, obs, A, C, eps, sigma_p, s2, nlp, u_row, rows, P,
                       (int)O, x_out, logw_out, anc_out, lw_vec, st);
    else if (R <= 4)
        ok = launch_pf_d<4>(D, pow2, x, logw, obs, A, C, eps, sigma_p, s2, nlp, u_row, rows, P,
                       (int)O, x_out, logw_out, anc_out, lw_vec, st);
    else
        ok = launch_pf_d<8>(D, pow2, x, logw, obs, A, C, eps, sigma_p, s2, nlp, u_row, rows, P,
                       (int)O, x_out, logw_out, anc_out, lw_vec, st);
    if (!ok) return PSAMP_E_SIZE;
    return launch_status();
}
