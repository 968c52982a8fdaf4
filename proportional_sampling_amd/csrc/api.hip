// api.hip -- library-wide entry points: status strings, ABI version,
// launch tracing (PSAMP_TRACE=1) and the workspace error query.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "psamp_host.h"

namespace psamp {

bool trace_enabled() {
    static const int on = [] {
        const char* e = getenv("PSAMP_TRACE");
        return (e && e[0] == '1') ? 1 : 0;
    }();
    return on != 0;
}

// A small lock-protected cache: occupancy depends only on the kernel and the
// device, so it is computed once per pair.
int resident_grid(const void* fn, int block) {
    struct Entry {
        const void* fn;
        int dev;
        int block;
        int value;
    };
    static std::mutex mu;
    static Entry cache[64];
    static int used = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    {
        std::lock_guard<std::mutex> lock(mu);
        for (int i = 0; i < used; ++i)
            if (cache[i].fn == fn && cache[i].dev == dev && cache[i].block == block)
                return cache[i].value;
    }
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, block, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    const int value = per_cu * cus;
    std::lock_guard<std::mutex> lock(mu);
    if (used < 64) cache[used++] = Entry{fn, dev, block, value};
    return value;
}

void trace_launch(const char* kernel, int64_t grid, int block, int64_t n) {
    fprintf(stderr, "[psamp] %s grid=%lld block=%d n=%lld\n", kernel, (long long)grid, block,
            (long long)n);
}

}  // namespace psamp

using namespace psamp;

extern "C" const char* psamp_status_string(psamp_status s) {
    // A C caller may pass any int: its bits are read as an int, since loading
    // a value outside the enumerators' range as the enum type is undefined
    // in C++.
    int v = 0;
    memcpy(&v, &s, sizeof(v) < sizeof(s) ? sizeof(v) : sizeof(s));
    switch (v) {
        case PSAMP_OK: return "ok";
        case PSAMP_E_NULL: return "null pointer";
        case PSAMP_E_SIZE: return "size out of range";
        case PSAMP_E_DTYPE: return "unsupported dtype";
        case PSAMP_E_PARAM: return "parameter out of range";
        case PSAMP_E_WORKSPACE: return "workspace missing or too small";
        case PSAMP_E_ALIGN: return "misaligned pointer";
        case PSAMP_E_LAUNCH: return "kernel launch failed";
        case PSAMP_E_UNSUPPORTED: return "unsupported";
        default: break;
    }
    return "unknown status";
}

extern "C" int psamp_abi_version(void) { return 1; }

extern "C" psamp_status psamp_workspace_errors(const void* ws, size_t ws_bytes, uint64_t* bits_host,
                                               void* stream) {
    if (!ws || !bits_host) return PSAMP_E_NULL;
    if (ws_bytes < 256) return PSAMP_E_WORKSPACE;
    hipStream_t st = as_stream(stream);
    uint64_t v = 0;
    if (hipMemcpyAsync(&v, (const uint64_t*)ws + 2, sizeof(v), hipMemcpyDeviceToHost, st) !=
        hipSuccess)
        return PSAMP_E_LAUNCH;
    if (hipStreamSynchronize(st) != hipSuccess) return PSAMP_E_LAUNCH;
    *bits_host = v;
    return PSAMP_OK;
}
