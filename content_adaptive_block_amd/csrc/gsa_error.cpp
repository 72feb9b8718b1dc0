// Status strings, the thread-local detail of the last failure, and the zlib version.
// No HIP calls: the host gzip stage links against this file alone in its CPU-only
// sanitizer builds.
#include <cstdarg>
#include <cstdio>
#include <string>

#include <zlib.h>

#include "gsa_internal.hpp"

namespace gsa {

static thread_local std::string g_last_error;

gsa_status fail(gsa_status st, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

void clear_error() { g_last_error.clear(); }

}  // namespace gsa

extern "C" {

const char *gsa_status_str(int32_t s) {
  switch (s) {
    case GSA_OK: return "GSA_OK";
    case GSA_ERR_ARG: return "GSA_ERR_ARG";
    case GSA_ERR_SHAPE: return "GSA_ERR_SHAPE";
    case GSA_ERR_ZLIB: return "GSA_ERR_ZLIB";
    case GSA_ERR_HIP: return "GSA_ERR_HIP";
    case GSA_ERR_UNSUPPORTED: return "GSA_ERR_UNSUPPORTED";
    default: return "GSA_ERR_UNKNOWN";
  }
}

const char *gsa_last_error(void) { return gsa::g_last_error.c_str(); }

const char *gsa_zlib_version(void) { return zlibVersion(); }

}  // extern "C"
