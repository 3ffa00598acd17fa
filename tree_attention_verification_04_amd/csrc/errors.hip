// Thread-local error text behind tree_last_error().
#include <stdarg.h>
#include <stdio.h>

#include "tv_common.h"

namespace tv {

static thread_local char g_last_error[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace tv

extern "C" const char* tree_last_error(void) { return tv::g_last_error; }
