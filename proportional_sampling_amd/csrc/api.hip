// api.hip -- library-wide entry points: status strings, ABI version,
// launch tracing (PSAMP_TRACE=1) and the workspace error query.
#include <stdio.h>
#include <stdlib.h>

#include "psamp_host.h"

namespace psamp {

bool trace_enabled() {
    static const int on = [] {
        const char* e = getenv("PSAMP_TRACE");
        return (e && e[0] == '1') ? 1 : 0;
    }();
    return on != 0;
}

void trace_launch(const char* kernel, int64_t grid, int block, int64_t n) {
    fprintf(stderr, "[psamp] %s grid=%lld block=%d n=%lld\n", kernel, (long long)grid, block,
            (long long)n);
}

}  // namespace psamp

using namespace psamp;

extern "C" const char* psamp_status_string(psamp_status s) {
    switch (s) {
        case PSAMP_OK: return "ok";
        case PSAMP_E_NULL: return "null pointer";
        case PSAMP_E_SIZE: return "size out of range";
        case PSAMP_E_DTYPE: return "unsupported dtype";
        case PSAMP_E_PARAM: return "parameter out of range";
        case PSAMP_E_WORKSPACE: return "workspace missing or too small";
        case PSAMP_E_ALIGN: return "misaligned pointer";
        case PSAMP_E_LAUNCH: return "kernel launch failed";
        case PSAMP_E_UNSUPPORTED: return "unsupported";
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
