// scatter.hip -- last-write-wins priority rewrite.
//
// After sampling, the trainer rewrites the sampled items' priorities (the
// scatter of "GPU Segment Tree for PER Sampling", "Integration with
// GpuReplayBuffer" -- update_priorities_gpu).  Sequential semantics:
// prio[idx_j] = vals_j for j = 0..m-1, so on a repeated index the largest j
// wins.  When the caller promises grouped indices (equal ones adjacent) the
// last entry of each run wins, decided from its neighbour alone.  Otherwise
// two kernels make the order explicit:
//   claim: owner[idx_j] = max(owner[idx_j], j + 1)   (atomic max)
//   apply: the entry whose j + 1 is the owner writes its value and zeroes
//          the owner word again (it is the only writer of that word).
// The owner array (one uint32 per item) is therefore all-zero between
// calls: it must be zeroed once after allocation and never again.
#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

constexpr int kScatThreads = 256;

__global__ __launch_bounds__(kScatThreads) void k_scatter_claim(
    const int32_t* __restrict__ idx, int64_t m, int64_t n, uint32_t* __restrict__ owner) {
    const int64_t j = (int64_t)blockIdx.x * kScatThreads + threadIdx.x;
    if (j >= m) return;
    const int32_t i = idx[j];
    if (i < 0 || (int64_t)i >= n) return;
    atomicMax(&owner[i], (uint32_t)(j + 1));
}

template <class T>
__global__ __launch_bounds__(kScatThreads) void k_scatter_apply(
    T* __restrict__ prio, const int32_t* __restrict__ idx, const T* __restrict__ vals, int64_t m,
    int64_t n, uint32_t* __restrict__ owner) {
    const int64_t j = (int64_t)blockIdx.x * kScatThreads + threadIdx.x;
    if (j >= m) return;
    const int32_t i = idx[j];
    if (i < 0 || (int64_t)i >= n) return;
    if (owner[i] == (uint32_t)(j + 1)) {
        prio[i] = vals[j];
        owner[i] = 0u;
    }
}

// Grouped indices (equal indices adjacent, e.g. the non-decreasing output
// of stratified sampling): the winner of a run is its last entry, known from
// the next index alone -- one kernel, no atomics, no workspace.
__global__ __launch_bounds__(kScatThreads) void k_scatter_grouped(
    uint32_t* __restrict__ prio, const int32_t* __restrict__ idx,
    const uint32_t* __restrict__ vals, int64_t m, int64_t n) {
    const int64_t j = (int64_t)blockIdx.x * kScatThreads + threadIdx.x;
    if (j >= m) return;
    const int32_t i = idx[j];
    if (i < 0 || (int64_t)i >= n) return;
    if (j + 1 < m && idx[j + 1] == i) return;
    prio[i] = vals[j];
}

}  // namespace psamp

using namespace psamp;

extern "C" size_t psamp_scatter_workspace_size(int64_t n, int64_t m) {
    (void)m;
    if (n < 1 || n > kMaxN) return 0;
    return (size_t)n * 4;
}

extern "C" psamp_status psamp_scatter_lww(void* prio, psamp_dtype prio_t, int64_t n,
                                          const int32_t* idx, const void* vals, int64_t m,
                                          int flags, void* ws, size_t ws_bytes, void* stream) {
    if (n < 1 || n > kMaxN || m < 0 || m > kMaxN - 1) return PSAMP_E_SIZE;
    if (prio_t != PSAMP_F32 && prio_t != PSAMP_U32) return PSAMP_E_DTYPE;
    if (flags & ~PSAMP_SCATTER_GROUPED) return PSAMP_E_PARAM;
    if (m == 0) return PSAMP_OK;
    if (!prio || !idx || !vals) return PSAMP_E_NULL;
    const bool grouped = (flags & PSAMP_SCATTER_GROUPED) != 0;
    if (!grouped && (!ws || ws_bytes < psamp_scatter_workspace_size(n, m)))
        return PSAMP_E_WORKSPACE;
    if (!aligned(prio, 4) || !aligned(idx, 4) || !aligned(vals, 4) || (!grouped && !aligned(ws, 4)))
        return PSAMP_E_ALIGN;
    hipStream_t st = as_stream(stream);
    if (check_on() && prio_t == PSAMP_F32) check_prio((const float*)vals, m, st);
    const int64_t grid = ceil_div(m, kScatThreads);
    if (grouped) {
        if (trace_enabled()) trace_launch("k_scatter_grouped", grid, kScatThreads, m);
        hipLaunchKernelGGL(k_scatter_grouped, dim3((unsigned)grid), dim3(kScatThreads), 0, st,
                           (uint32_t*)prio, idx, (const uint32_t*)vals, m, n);
        return launch_status();
    }
    if (trace_enabled()) trace_launch("k_scatter_claim+apply", grid, kScatThreads, m);
    hipLaunchKernelGGL(k_scatter_claim, dim3((unsigned)grid), dim3(kScatThreads), 0, st, idx, m, n,
                       (uint32_t*)ws);
    psamp_status s = launch_status();
    if (s != PSAMP_OK) return s;
    // The value is moved as raw 32-bit words: float and uint32 alike.
    hipLaunchKernelGGL(k_scatter_apply<uint32_t>, dim3((unsigned)grid), dim3(kScatThreads), 0, st,
                       (uint32_t*)prio, idx, (const uint32_t*)vals, m, n, (uint32_t*)ws);
    return launch_status();
}
