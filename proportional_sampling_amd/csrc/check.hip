// check.hip -- optional device-side checks of the preconditions the library
// cannot check on the host without a sync: priorities finite and >= 0 with
// a positive, finite total, threshold fractions in [0, 1), indices in range,
// log-weights that are not NaN or +inf.  [SEGT] "Operations -- Update" has
// every update thread work on its own index, independently of the others,
// and [PR615] "1. Parallel build_cdf" keeps the CDF rebuild free of
// allocations and host syncs -- so a bad input cannot be refused when the
// call is made; it can only be recorded on the device.
//
// When checking is on (PSAMP_CHECK=1 in the environment when the library is
// first used, or psamp_check_enable(1)), each entry point enqueues small
// check kernels on its stream next to its own kernels.  A violation sets a
// bit in a per-device word (`check_bits`, a file-scope device variable);
// psamp_check_errors copies it to the host (syncing the stream) and can
// clear it.  The checks never change an output.
#include <float.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>

#include "psamp_device.h"
#include "psamp_host.h"

namespace psamp {

static __device__ __align__(8) uint64_t check_bits;

constexpr int kCheckThreads = 256;
constexpr int kCheckMaxGrid = 1024;

__device__ __forceinline__ void check_flag(bool bad, uint64_t bit) {
    if (__any(bad) && lane_id() == 0)
        __hip_atomic_fetch_or(&check_bits, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// rows x P floats with row stride ld; mode: kChkPrio, kChkUnit or kChkLogw.
__global__ __launch_bounds__(kCheckThreads) void k_check_f32(const float* __restrict__ a,
                                                             int64_t rows, int64_t P, int64_t ld,
                                                             int mode, uint64_t bit) {
    bool bad = false;
    const int64_t total = rows * P;
    for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * kCheckThreads) {
        const int64_t r = i / P;
        const float x = a[r * ld + (i - r * P)];
        if (mode == kChkPrio) bad = bad || !(x >= 0.0f && x <= 3.402823466e38f);
        else if (mode == kChkUnit) bad = bad || !(x >= 0.0f && x < 1.0f);
        else bad = bad || x != x || x > 3.402823466e38f;
    }
    check_flag(bad, bit);
}

__global__ __launch_bounds__(kCheckThreads) void k_check_i32(const int32_t* __restrict__ idx,
                                                             int64_t m, int64_t hi, uint64_t bit) {
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * kCheckThreads + threadIdx.x; i < m;
         i += (int64_t)gridDim.x * kCheckThreads) {
        const int64_t v = idx[i];
        bad = bad || v < 0 || v >= hi;
    }
    check_flag(bad, bit);
}

// The total of a CDF or the root of a sum tree: > 0 (and not NaN).
__global__ void k_check_total(const void* __restrict__ t, int kind, uint64_t bit) {
    bool bad;
    if (kind == PSAMP_F64) {
        const double x = *(const double*)t;
        bad = !(x > 0.0 && x <= DBL_MAX);                 // zero, NaN or overflowed
    } else if (kind == PSAMP_F32) {
        const float x = *(const float*)t;
        bad = !(x > 0.0f && x <= FLT_MAX);
    } else {
        bad = *(const uint64_t*)t == 0;
    }
    check_flag(bad && threadIdx.x == 0, bit);
}

__global__ void k_check_clear() { check_bits = 0; }

static std::atomic<int>& check_state() {
    static std::atomic<int> on([] {
        const char* e = getenv("PSAMP_CHECK");
        return (e && e[0] == '1') ? 1 : 0;
    }());
    return on;
}

bool check_on() { return check_state().load(std::memory_order_relaxed) != 0; }

static unsigned check_grid(int64_t n) {
    const int64_t g = ceil_div(n, (int64_t)kCheckThreads * 8);
    return (unsigned)(g < 1 ? 1 : (g > kCheckMaxGrid ? kCheckMaxGrid : g));
}

void check_f32(const float* a, int64_t rows, int64_t P, int64_t ld, int mode, uint64_t bit,
               hipStream_t st) {
    if (!a || rows < 1 || P < 1) return;
    hipLaunchKernelGGL(k_check_f32, dim3(check_grid(rows * P)), dim3(kCheckThreads), 0, st, a,
                       rows, P, ld, mode, bit);
}

void check_i32(const int32_t* idx, int64_t m, int64_t hi, hipStream_t st) {
    if (!idx || m < 1) return;
    hipLaunchKernelGGL(k_check_i32, dim3(check_grid(m)), dim3(kCheckThreads), 0, st, idx, m, hi,
                       (uint64_t)PSAMP_CHECK_INDEX);
}

void check_total(const void* t, int kind, hipStream_t st) {
    if (!t) return;
    hipLaunchKernelGGL(k_check_total, dim3(1), dim3(64), 0, st, t, kind,
                       (uint64_t)PSAMP_CHECK_ZERO_TOTAL);
}

// The address of this device's check word, found once per device.
static uint64_t* check_word() {
    static std::mutex mu;
    static uint64_t* ptr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_bits)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        ptr[dev] = (uint64_t*)p;
    }
    return ptr[dev];
}

}  // namespace psamp

using namespace psamp;

extern "C" int psamp_check_enable(int on) {
    if (on < 0) return check_state().load();
    return check_state().exchange(on ? 1 : 0);
}

extern "C" psamp_status psamp_check_errors(uint64_t* bits_host, int clear, void* stream) {
    if (!bits_host) return PSAMP_E_NULL;
    uint64_t* w = check_word();
    if (!w) return PSAMP_E_LAUNCH;
    hipStream_t st = as_stream(stream);
    uint64_t v = 0;
    if (hipMemcpyAsync(&v, w, sizeof(v), hipMemcpyDeviceToHost, st) != hipSuccess) {
        (void)hipGetLastError();
        return PSAMP_E_LAUNCH;
    }
    if (clear) {
        hipLaunchKernelGGL(k_check_clear, dim3(1), dim3(1), 0, st);
        if (launch_status() != PSAMP_OK) return PSAMP_E_LAUNCH;
    }
    if (hipStreamSynchronize(st) != hipSuccess) return PSAMP_E_LAUNCH;
    *bits_host = v;
    return PSAMP_OK;
}
