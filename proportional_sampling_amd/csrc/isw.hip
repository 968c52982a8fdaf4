// isw.hip -- importance-sampling weights of a sampled batch.
//
// [PER] (named in "GPU Segment Tree for PER Sampling", "Non-Goals"):
// P_i = w_{idx_i} / T, v_i = (N P_i)^-beta, IS_i = v_i / max_j v_j.
// Since N and T cancel, IS_i = (w_min / w_i)^beta with w_min the smallest
// sampled weight; with w = p^alpha that is (p_min / p_i)^(alpha beta) (fp
// mode) and (q_min / q_i)^beta in integer mode (alpha not applied).  The
// minimum is taken exactly on the raw priorities (uint32 order of the
// non-negative float bits), the power in double via log2 / exp2, and the
// largest weight comes out as exactly 1.
//
// One kernel while its blocks can all be resident at once: blocks of 1024
// (k <= 8192) or 4096 samples gather their priorities on different CUs at
// once and exchange their minima.  Larger batches use two kernels:
// per-block minima with a last-block reduction (the gathered priorities are
// parked in the output array), then the weights from the parked values --
// the priority array is gathered once either way.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kIswThreads = 1024;
constexpr int kIswPerThread = 4;
constexpr int kIswBlock = kIswThreads * kIswPerThread;   // samples per block
constexpr int64_t kIswSingleMax = 8192;            // blocks of 1024 samples up to this many
constexpr int kIswHdrWords = 64;                        // 256-byte header (uint32)
constexpr int kIswSpinLimit = 1 << 21;                  // bounded waits (about a second)

template <class P>
__device__ __forceinline__ uint32_t prio_key(P x);
template <>
__device__ __forceinline__ uint32_t prio_key<float>(float x) { return __float_as_uint(x); }
template <>
__device__ __forceinline__ uint32_t prio_key<uint32_t>(uint32_t x) { return x; }

template <class P>
__device__ __forceinline__ double prio_val(uint32_t key);
template <>
__device__ __forceinline__ double prio_val<float>(uint32_t key) { return (double)__uint_as_float(key); }
template <>
__device__ __forceinline__ double prio_val<uint32_t>(uint32_t key) { return (double)key; }

__device__ __forceinline__ int64_t clamp_idx(int32_t i, int64_t n) {
    return i < 0 ? 0 : (i >= n ? n - 1 : (int64_t)i);
}

// The one-kernel path: PT samples per thread in blocks of 1024 threads,
// nblocks <= 64 * PW blocks, all resident at once (the host checks).  Each
// block gathers its priorities (one round trip for the indices, one for the
// priorities), publishes its minimum in its slot, tagged with this call's
// number, and polls the other blocks' slots until every one carries the
// tag; then each block writes its own weights from the keys it holds in
// registers.  Block 0 advances the call number once it has seen every slot
// -- by then every block has read it.  No data but the minima crosses
// between blocks, so no fences.  Waits are bounded (bit 0 of the
// workspace's error word instead of a hang).
// (k <= 8192: one workgroup gathering all 8192 took 12 us -- a single CU's
// request rate bounds 8192 scattered loads; a last-block variant that
// formed every weight in one workgroup, 10 us.  2^20 samples: the two
// kernels took 26 us.)
// Workspace, as 64-bit words: [2] error bits (where psamp_workspace_errors
// reads them), [4] the call number, [8, 16) the slots of blocks of 1024
// samples, [32, 32 + kIswExMax) those of blocks of 4096; the two-kernel path
// uses the first two 32-bit words and the 32-bit words from kIswPartWord on.
constexpr int kIswErrWord = 2;
constexpr int kIswCallWord = 4;
constexpr int kIswSlotSmall = 8;
constexpr int kIswSlotBig = 32;
constexpr int kIswExMax = 1024;                              // blocks of the one-kernel path
constexpr int kIswPartWord = kIswHdrWords + 2 * kIswExMax;   // 32-bit index

template <class P, int PT, int PW>
__global__ __launch_bounds__(kIswThreads) void k_isw_exch(const P* __restrict__ prio, int64_t n,
                                                          const int32_t* __restrict__ idx,
                                                          int64_t k, double e,
                                                          uint64_t* __restrict__ ws, int slot0,
                                                          int nblocks, float* __restrict__ out) {
    __shared__ MathLds M;
    __shared__ uint32_t s_min;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const MathRegs mr = math_load(tid);
    if (tid == 0) s_min = 0xFFFFFFFFu;
    const int64_t b0 = (int64_t)blockIdx.x * kIswThreads * PT;
    const uint32_t call = (uint32_t)load_agent(&ws[kIswCallWord]);
    uint32_t key[PT];
    uint32_t mk = 0xFFFFFFFFu;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int64_t i = b0 + j * kIswThreads + tid;
        key[j] = i < k ? prio_key<P>(prio[clamp_idx(idx[i], n)]) : 0xFFFFFFFFu;
        mk = min_(mk, key[j]);
    }
    math_store(&M, tid, mr);
    const uint32_t mn = wave_min_u32(mk);
    __syncthreads();
    if (lane == 0) atomicMin(&s_min, mn);
    __syncthreads();
    if (nblocks > 1 && tid < kWave) {
        const uint32_t tag = call + 1u;
        if (tid == 0) store_agent(&ws[slot0 + blockIdx.x], ((uint64_t)tag << 32) | s_min);
        // every slot of this call (lane l polls slots l, l + 64, ...)
        bool need[PW];
        uint64_t w[PW];
#pragma unroll
        for (int m = 0; m < PW; ++m) {
            const int b = m * kWave + lane;
            need[m] = b < nblocks;
            w[m] = load_agent(&ws[slot0 + (need[m] ? b : 0)]);
        }
        int limit = kIswSpinLimit;
        asm volatile("" : "+s"(limit));
        for (int polls = 0;; ++polls) {
            bool pend = false;
#pragma unroll
            for (int m = 0; m < PW; ++m) pend |= need[m] && (uint32_t)(w[m] >> 32) != tag;
            if (!__any(pend)) break;
            if (polls > limit) {
                if (lane == 0)
                    __hip_atomic_fetch_or(&ws[kIswErrWord], (uint64_t)1, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            __builtin_amdgcn_s_sleep(1);
#pragma unroll
            for (int m = 0; m < PW; ++m)
                if (need[m] && (uint32_t)(w[m] >> 32) != tag)
                    w[m] = load_agent(&ws[slot0 + m * kWave + lane]);
        }
        uint32_t g = 0xFFFFFFFFu;
#pragma unroll
        for (int m = 0; m < PW; ++m) g = min_(g, need[m] ? (uint32_t)w[m] : 0xFFFFFFFFu);
        g = wave_min_u32(g);
        if (lane == 0) {
            s_min = min_(s_min, g);
            if (blockIdx.x == 0) store_agent(&ws[kIswCallWord], (uint64_t)tag);
        }
    }
    __syncthreads();
    const double pmin = prio_val<P>(s_min);
    const double lpmin = pmin > 0.0 ? log2_sig32(pmin, &M) : 0.0;
#pragma unroll
    for (int j = 0; j < PT; ++j) {
        const int64_t i = b0 + j * kIswThreads + tid;
        if (i < k) out[i] = is_weight(pmin, lpmin, prio_val<P>(key[j]), e, &M);
    }
}

// Pass 1: per-block minimum; the last block to finish reduces them into
// hdr[1] (the block counter hdr[0] wraps back to 0 on the last block).  Each
// gathered priority's bits are parked in out[i] for pass 2.
template <class P>
__global__ __launch_bounds__(kIswThreads) void k_isw_min(const P* __restrict__ prio, int64_t n,
                                                         const int32_t* __restrict__ idx, int64_t k,
                                                         uint32_t* __restrict__ ws, int nblocks,
                                                         uint32_t* __restrict__ park) {
    __shared__ uint32_t s_min;
    __shared__ int s_last;
    const int tid = threadIdx.x;
    if (tid == 0) s_min = 0xFFFFFFFFu;
    __syncthreads();
    uint32_t mn = 0xFFFFFFFFu;
    const int64_t b0 = (int64_t)blockIdx.x * kIswBlock;
#pragma unroll
    for (int j = 0; j < kIswPerThread; ++j) {
        const int64_t i = b0 + j * kIswThreads + tid;
        if (i < k) {
            const uint32_t key = prio_key<P>(prio[clamp_idx(idx[i], n)]);
            park[i] = key;
            mn = min_(mn, key);
        }
    }
    atomicMin(&s_min, mn);
    __syncthreads();
    uint32_t* hdr = ws;
    uint32_t* part = ws + kIswPartWord;
    if (tid == 0) {
        part[blockIdx.x] = s_min;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const uint32_t t = __builtin_amdgcn_atomic_inc32(&hdr[0], (uint32_t)(nblocks - 1),
                                                         __ATOMIC_RELAXED, "agent");
        s_last = (t == (uint32_t)(nblocks - 1));
        if (s_last) s_min = 0xFFFFFFFFu;
    }
    __syncthreads();
    if (!s_last) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    uint32_t m2 = 0xFFFFFFFFu;
    for (int b = tid; b < nblocks; b += kIswThreads)
        m2 = min_(m2, __hip_atomic_load(&part[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    atomicMin(&s_min, m2);
    __syncthreads();
    if (tid == 0) hdr[1] = s_min;
}

// Pass 2: the weights from the parked priorities (read and overwritten in
// place, each by its own thread).
template <class P>
__global__ __launch_bounds__(kIswThreads) void k_isw_apply(int64_t k, double e,
                                                           const uint32_t* __restrict__ ws,
                                                           float* __restrict__ out) {
    __shared__ MathLds M;
    const int tid = threadIdx.x;
    math_lds_fill(&M, tid, kIswThreads);
    __syncthreads();
    const double pmin = prio_val<P>(ws[1]);
    const double lpmin = pmin > 0.0 ? log2_sig32(pmin, &M) : 0.0;
    const int64_t b0 = (int64_t)blockIdx.x * kIswBlock;
#pragma unroll
    for (int j = 0; j < kIswPerThread; ++j) {
        const int64_t i = b0 + j * kIswThreads + tid;
        if (i < k) {
            const double p = prio_val<P>(__float_as_uint(out[i]));
            out[i] = is_weight(pmin, lpmin, p, e, &M);
        }
    }
}

template <class P>
static psamp_status launch_isw(const void* prio, int64_t n, const int32_t* idx, int64_t k,
                               double e, float* out, void* ws, hipStream_t st) {
    if (k <= kIswSingleMax) {
        const int nb = (int)ceil_div(k, kIswThreads);
        if (trace_enabled()) trace_launch("k_isw_exch<1>", nb, kIswThreads, k);
        hipLaunchKernelGGL((k_isw_exch<P, 1, 1>), dim3(nb), dim3(kIswThreads), 0, st,
                           (const P*)prio, n, idx, k, e, (uint64_t*)ws, kIswSlotSmall, nb, out);
        return launch_status();
    }
    const int64_t nb = ceil_div(k, kIswBlock);
    constexpr int kPW = kIswExMax / kWave;
    if (nb <= kIswExMax &&
        nb <= resident_grid(reinterpret_cast<const void*>(&k_isw_exch<P, kIswPerThread, kPW>),
                            kIswThreads)) {
        if (trace_enabled()) trace_launch("k_isw_exch<4>", nb, kIswThreads, k);
        hipLaunchKernelGGL((k_isw_exch<P, kIswPerThread, kPW>), dim3((unsigned)nb),
                           dim3(kIswThreads), 0, st, (const P*)prio, n, idx, k, e, (uint64_t*)ws,
                           kIswSlotBig, (int)nb, out);
        return launch_status();
    }
    if (trace_enabled()) trace_launch("k_isw_min+apply", nb, kIswThreads, k);
    hipLaunchKernelGGL(k_isw_min<P>, dim3((unsigned)nb), dim3(kIswThreads), 0, st, (const P*)prio,
                       n, idx, k, (uint32_t*)ws, (int)nb, reinterpret_cast<uint32_t*>(out));
    psamp_status s = launch_status();
    if (s != PSAMP_OK) return s;
    hipLaunchKernelGGL(k_isw_apply<P>, dim3((unsigned)nb), dim3(kIswThreads), 0, st, k, e,
                       (const uint32_t*)ws, out);
    return launch_status();
}

}  // namespace psamp

using namespace psamp;

extern "C" size_t psamp_is_weights_workspace_size(int64_t k) {
    if (k < 0 || k > kMaxN) return 0;
    if (k == 0) return 0;
    if (k <= kIswSingleMax) return (size_t)kIswHdrWords * 4;   // call number, error bits, 8 slots
    return (size_t)kIswPartWord * 4 + (size_t)ceil_div(k, kIswBlock) * 4;
}

extern "C" psamp_status psamp_is_weights(const void* prio, psamp_dtype prio_t, int64_t n,
                                         double alpha, const int32_t* idx, int64_t k, double beta,
                                         float* out_w, void* ws, size_t ws_bytes, void* stream) {
    if (n < 1 || n > kMaxN || k < 0 || k > kMaxN) return PSAMP_E_SIZE;
    if (prio_t != PSAMP_F32 && prio_t != PSAMP_U32) return PSAMP_E_DTYPE;
    if (!(finite_d(beta) && beta >= 0.0)) return PSAMP_E_PARAM;
    if (prio_t == PSAMP_F32 && !(finite_d(alpha) && alpha > 0.0)) return PSAMP_E_PARAM;
    if (k == 0) return PSAMP_OK;
    if (!prio || !idx || !out_w) return PSAMP_E_NULL;
    const size_t need = psamp_is_weights_workspace_size(k);
    if (need > 0 && (!ws || ws_bytes < need)) return PSAMP_E_WORKSPACE;
    if (!aligned(prio, 4) || !aligned(idx, 4) || !aligned(out_w, 4) || (need && !aligned(ws, 8)))
        return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on()) check_i32(idx, k, n, st);
    if (prio_t == PSAMP_F32) return launch_isw<float>(prio, n, idx, k, alpha * beta, out_w, ws, st);
    return launch_isw<uint32_t>(prio, n, idx, k, beta, out_w, ws, st);
}
