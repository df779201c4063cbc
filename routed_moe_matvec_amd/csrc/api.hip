// Status strings and the small host-side state of libqgemv: per-device
// facts and one-time kernel attributes, kept behind one lock.
#include <mutex>

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

namespace {

// (key, device) pairs whose one-time set-up has succeeded: an open-addressed
// table of fixed size (no allocation), guarded by one mutex.  A full table
// only means the set-up is repeated (every set-up here is idempotent).
constexpr int kOnceSlots = 1024;
struct OnceSlot {
    const void *key;
    int dev;
};
std::mutex g_once_mu;
OnceSlot g_once[kOnceSlots];

constexpr int kMaxDevices = 64;
int g_cus[kMaxDevices];  // compute units per device, 0 = not yet queried (under g_once_mu)

unsigned slot_hash(const void *key, int dev) {
    uint64_t h = (uint64_t)(uintptr_t)key * 0x9E3779B97F4A7C15ull ^ (uint64_t)(unsigned)dev * 0xC2B2AE3D27D4EB4Full;
    return (unsigned)(h >> 40) % kOnceSlots;
}

}  // namespace

int current_device(int *dev) {
    return hipGetDevice(dev) == hipSuccess && *dev >= 0 ? QG_OK : QG_ERR_LAUNCH;
}

int once_per_device(const void *key, int (*init)(const void *key, int arg), int arg) {
    int dev = 0;
    if (current_device(&dev) != QG_OK) return QG_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_once_mu);
    const unsigned h0 = slot_hash(key, dev);
    int free_slot = -1;
    for (int i = 0; i < kOnceSlots; ++i) {
        const unsigned s = (h0 + (unsigned)i) % kOnceSlots;
        if (g_once[s].key == key && g_once[s].dev == dev) return QG_OK;
        if (g_once[s].key == nullptr) {
            free_slot = (int)s;
            break;
        }
    }
    const int rc = init(key, arg);
    if (rc != QG_OK) return rc;
    if (free_slot >= 0) g_once[free_slot] = OnceSlot{key, dev};
    return QG_OK;
}

static int raise_lds(const void *kern, int bytes) {
    return hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes) == hipSuccess
               ? QG_OK
               : QG_ERR_LAUNCH;
}

int ensure_lds_limit(const void *kern, int bytes) { return once_per_device(kern, raise_lds, bytes); }

// Compute units of the current device, queried once per device.
int device_cu_count() {
    int dev = 0;
    if (current_device(&dev) != QG_OK || dev >= kMaxDevices) return 256;
    std::lock_guard<std::mutex> lock(g_once_mu);
    if (g_cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        g_cus[dev] = n;
    }
    return g_cus[dev];
}

}  // namespace qg
