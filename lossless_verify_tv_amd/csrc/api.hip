// Library-level entry points of the C ABI (version, error strings).
#include "../../include/lvtv.h"

extern "C" int lvtv_version(void) { return 1; }

extern "C" const char* lvtv_strerror(int code) {
  switch (code) {
    case LVTV_OK: return "ok";
    case LVTV_ERR_NULL: return "a required pointer is NULL";
    case LVTV_ERR_SHAPE: return "a size is outside the supported range";
    case LVTV_ERR_DTYPE: return "unknown dtype";
    case LVTV_ERR_WORKSPACE: return "workspace is NULL, misaligned or smaller than required";
    case LVTV_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    default: return "unknown error code";
  }
}
