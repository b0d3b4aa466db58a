// Per-thread error text behind gdn_last_error().
#include <cstdio>

#include "gdn_internal.h"

namespace gdn {

static thread_local char g_error[512] = "";

void clear_error() { g_error[0] = '\0'; }

gdn_status fail(gdn_status code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return code;
}

}  // namespace gdn

extern "C" const char *gdn_last_error(void) { return gdn::g_error; }
