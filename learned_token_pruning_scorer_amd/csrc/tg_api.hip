// Library-level entry points of the C ABI: version and status text.
#include "tg_common.h"

extern "C" int32_t tg_abi_version(void) { return TG_ABI_VERSION; }

extern "C" const char* tg_status_string(tg_status status) {
  switch (status) {
    case TG_OK: return "TG_OK";
    case TG_ERR_INVALID_ARG: return "TG_ERR_INVALID_ARG: invalid argument";
    case TG_ERR_UNSUPPORTED: return "TG_ERR_UNSUPPORTED: shape or alignment not supported by this library";
    case TG_ERR_WORKSPACE: return "TG_ERR_WORKSPACE: workspace too small";
    case TG_ERR_HIP: return "TG_ERR_HIP: HIP runtime error at launch";
    case TG_ERR_INCOMPLETE:
      return "TG_ERR_INCOMPLETE: a selection on this workspace gave up waiting for its workgroups (or found the "
             "workspace not zero-filled); its outputs are invalid and the workspace must be zero-filled again";
    default: return "unknown tg_status";
  }
}
