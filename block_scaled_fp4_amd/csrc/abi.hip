// Status strings and version of the C ABI.
#include "fp4mi.h"

extern "C" const char* fp4_status_string(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_EINVAL: return "invalid argument (null pointer, enum or group size)";
    case FP4_ESHAPE: return "invalid shape (negative size or block/group rule broken)";
    case FP4_EALIGN: return "misaligned pointer";
    case FP4_EDTYPE: return "unknown dtype";
    case FP4_EHIP: return "HIP launch failure";
    case FP4_EOVERLAP: return "output overlaps an input";
    default: return "unknown status";
  }
}

extern "C" int fp4_abi_version(void) { return FP4MI_ABI_VERSION; }
