// Status strings and small host-side helpers of libqgemv.
#include "common.h"

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
