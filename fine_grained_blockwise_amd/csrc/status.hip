// status.hip -- thread-local error text and version of libfgb.
#include <stdarg.h>
#include <stdio.h>

#include "fgb_internal.h"

namespace fgb {

static thread_local char g_err[512] = "";

int set_error(int code, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_err[0] = '\0'; }

} // namespace fgb

extern "C" const char *fgb_last_error(void) { return fgb::g_err; }

extern "C" const char *fgb_version(void) { return "fgb 0.1 gfx950"; }
