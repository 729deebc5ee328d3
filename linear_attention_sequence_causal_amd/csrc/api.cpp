// api.cpp -- error reporting and device queries of libgdn.
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "gdn_internal.h"

namespace gdn {

static thread_local char g_last_error[512] = "";
static thread_local int g_seg_chunks = 0;

int segment_chunks_override() { return g_seg_chunks; }

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_last_error[0] = '\0'; }

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace gdn

extern "C" const char* gdn_last_error(void) { return gdn::g_last_error; }

// Test hook, deliberately absent from gdn.h: forces the segment length of the
// chunk plans made on the calling thread (workspace queries included) to
// `chunks` 64-token chunks; 0 restores the default plan.  Returns the
// previous value.
extern "C" int gdn_testing_set_segment_chunks(int chunks) {
  const int prev = gdn::g_seg_chunks;
  gdn::g_seg_chunks = chunks > 0 ? chunks : 0;
  return prev;
}
