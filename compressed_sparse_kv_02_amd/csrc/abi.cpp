// Version and status text of the C ABI declared in include/cskv.h.
#include "abi_common.h"

extern "C" int cskv_version(void) { return 10000 * 0 + 100 * 2 + 0; }

extern "C" const char* cskv_status_string(int status) {
  switch (status) {
    case CSKV_OK: return "ok";
    case CSKV_ERR_INVALID_ARG: return "invalid argument (null pointer or bad enum/value)";
    case CSKV_ERR_BAD_SHAPE: return "bad shape (sizes inconsistent or out of range)";
    case CSKV_ERR_BAD_DTYPE: return "bad dtype (expected CSKV_BF16 or CSKV_F32)";
    case CSKV_ERR_MISALIGNED: return "misaligned pointer (16-byte alignment required)";
    case CSKV_ERR_WORKSPACE: return "workspace missing or too small";
    case CSKV_ERR_UNSUPPORTED: return "unsupported request for this build";
    case CSKV_ERR_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}
