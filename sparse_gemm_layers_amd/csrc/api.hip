// Status strings and ABI version of the C interface.
#include "common.h"

extern "C" const char* sg_status_str(sg_status s) {
  switch (s) {
    case SG_OK: return "SG_OK";
    case SG_ERR_NULL: return "SG_ERR_NULL: a required pointer is NULL";
    case SG_ERR_SHAPE: return "SG_ERR_SHAPE: a size or leading dimension is out of range";
    case SG_ERR_UNSUPPORTED: return "SG_ERR_UNSUPPORTED: granularity, dtype or output form not supported";
    case SG_ERR_ALIGN: return "SG_ERR_ALIGN: a pointer or leading dimension is misaligned";
    case SG_ERR_HIP: return "SG_ERR_HIP: the HIP runtime reported an error at launch";
  }
  return "unknown sg_status";
}

extern "C" int sg_abi_version(void) { return 3; }
