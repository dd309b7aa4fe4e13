// Library-wide C entry points: ABI version, status names, last-error detail.
#include <cstdarg>
#include <cstdio>
#include <string>

#include "status.h"

namespace ringattn {

static thread_local std::string g_last_error;

int32_t fail(int32_t code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int32_t ok() {
  g_last_error.clear();
  return CP_OK;
}

}  // namespace ringattn

extern "C" int32_t cp_abi_version(void) { return RINGATTN_ABI_VERSION; }

extern "C" const char* cp_status_string(int32_t status) {
  switch (status) {
    case CP_OK: return "CP_OK";
    case CP_EINVAL: return "CP_EINVAL: invalid argument";
    case CP_EDTYPE: return "CP_EDTYPE: unknown dtype";
    case CP_EUNSUPPORTED: return "CP_EUNSUPPORTED: no kernel for this shape";
    case CP_EHIP: return "CP_EHIP: HIP runtime error";
    default: return "unknown status";
  }
}

extern "C" const char* cp_last_error(void) { return ringattn::g_last_error.c_str(); }
