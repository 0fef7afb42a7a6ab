// xv_api.hip -- library-wide C entry points of libxv (version and status text).
#include "xv_common.h"

extern "C" int xv_abi_version(void) { return XV_ABI_VERSION; }

extern "C" const char* xv_status_string(int status) {
    switch (status) {
        case XV_OK: return "ok";
        case XV_ERR_NULL: return "a required pointer is NULL";
        case XV_ERR_SHAPE: return "a size is outside the supported set";
        case XV_ERR_ALIGN: return "a pointer breaks its alignment rule";
        case XV_ERR_WORKSPACE: return "workspace too small";
        case XV_ERR_LAUNCH: return "kernel launch failed";
        case XV_ERR_ALIAS: return "an output aliases an input it must not overwrite";
        default: return "unknown status";
    }
}
