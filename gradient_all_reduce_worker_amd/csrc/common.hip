// common.hip -- host-side error reporting shared by every entry point.
#include "common.hpp"

namespace ga {

static thread_local char g_err[512] = "";

ga_status fail(ga_status code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

ga_status check_launch(const char* what) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(GA_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
    return GA_OK;
}

ga_status check_workers(const void* const* bufs, int32_t P, size_t align, const char* what) {
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (!bufs) return fail(GA_EINVAL, "%s: null pointer array", what);
    for (int i = 0; i < P; i++) {
        if (!bufs[i]) return fail(GA_EINVAL, "%s: worker %d pointer is null", what, i);
        if (!aligned(bufs[i], align))
            return fail(GA_EINVAL, "%s: worker %d pointer not aligned to %zu bytes", what, i, align);
    }
    return GA_OK;
}

}  // namespace ga

extern "C" const char* ga_last_error(void) { return ga::g_err; }
