// Version and status strings of the libmxq C ABI.
#include "mxq.h"

extern "C" const char *mxq_status_string(mxq_status s)
{
    switch (s) {
    case MXQ_OK: return "ok";
    case MXQ_ERR_NULL: return "a required pointer is NULL";
    case MXQ_ERR_SHAPE: return "invalid size (negative, or not a multiple of 32 along the block axis)";
    case MXQ_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case MXQ_ERR_UNSUPPORTED: return "unsupported option or combination";
    case MXQ_ERR_DEVICE: return "HIP launch failed";
    case MXQ_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
    }
}

extern "C" int32_t mxq_abi_version(void) { return MXQ_ABI_VERSION; }
