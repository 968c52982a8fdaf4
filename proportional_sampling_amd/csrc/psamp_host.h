// psamp_host.h -- host-side helpers shared by the libpsamp entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/psamp.h"

namespace psamp {

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void* p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline bool finite_d(double x) { return x == x && x - x == 0.0; }

// Report a launch failure (never aborts).
inline psamp_status launch_status() {
    hipError_t e = hipGetLastError();
    return e == hipSuccess ? PSAMP_OK : PSAMP_E_LAUNCH;
}

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int ilog2_exact(int64_t x) {   // x must be a power of two
    int r = 0;
    while ((int64_t(1) << r) < x) ++r;
    return r;
}

inline bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

constexpr int64_t kMaxN = 0x7FFFFFFFll;   // int32 indices

// Workgroups of `block` threads of kernel `fn` that fit on the current
// device at once (CUs x resident per CU).  Cached per (kernel, device).
int resident_grid(const void* fn, int block);

// One PER update (CDF, stratified draws, IS weights, rewrite of the drawn
// priorities) whose grid need not be resident: the tile sums, the scan with
// the draws, the drawn priorities and the rewrite, then the IS weights --
// three kernels, the bits of the separate calls (scan.hip).  ws: the scan's
// workspace.
psamp_status launch_per_update(float* prio, int64_t n, double alpha, double beta, const float* u,
                               int64_t k, const float* newp, int32_t* out_idx, float* out_w,
                               double* cdf, double* total, void* ws, size_t ws_bytes,
                               hipStream_t st);

// Optional device-side precondition checks (check.hip).  check_on() is
// cheap; the check_* launchers enqueue a check kernel on `st`.
enum : int { kChkPrio = 0, kChkUnit = 1, kChkLogw = 2 };
bool check_on();
void check_f32(const float* a, int64_t rows, int64_t P, int64_t ld, int mode, uint64_t bit,
               hipStream_t st);
inline void check_prio(const float* p, int64_t n, hipStream_t st) {
    check_f32(p, 1, n, n, kChkPrio, PSAMP_CHECK_PRIORITY, st);
}
inline void check_unit(const float* u, int64_t n, hipStream_t st) {
    check_f32(u, 1, n, n, kChkUnit, PSAMP_CHECK_FRACTION, st);
}
void check_i32(const int32_t* idx, int64_t m, int64_t hi, hipStream_t st);
void check_total(const void* t, int kind, hipStream_t st);

// Optional launch trace: PSAMP_TRACE=1 prints one line per launch.
bool trace_enabled();
void trace_launch(const char* kernel, int64_t grid, int block, int64_t n);

}  // namespace psamp
