// Status strings and small host-side helpers of libqgemv.
#include "common.h"
#include "gemv_device.h"

extern "C" const char *qg_status_string(int status) {
    switch (status) {
        case QG_OK: return "ok";
        case QG_ERR_NULL: return "a required pointer is NULL";
        case QG_ERR_SHAPE: return "a size is out of the supported range";
        case QG_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case QG_ERR_FORMAT: return "unknown weight format";
        case QG_ERR_WORKSPACE: return "workspace too small";
        case QG_ERR_LAUNCH: return "kernel launch failed";
        default: break;
    }
    return "unknown status";
}

namespace qg {

// Compute units of the current device, queried once per device.
int device_cu_count() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

}  // namespace qg
