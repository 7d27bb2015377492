// Return-code text for the C ABI (host only).
#include "bqmm.h"

extern "C" const char *bqm_strerror(int rc) {
    if (rc == BQM_OK) return "ok";
    if (rc == BQM_EINVAL) return "invalid argument (null pointer or size out of range)";
    if (rc == BQM_EUNSUPPORTED) return "unsupported shape or alignment";
    if (rc >= BQM_EHIP_BASE) return "HIP launch error (rc - 10000 is the hipError_t)";
    return "unknown error";
}
