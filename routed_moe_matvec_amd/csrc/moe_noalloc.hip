// The routed MoE for callers that cannot allocate device memory: the same
// call as moe_routed_qgemv_fmt, with its workspace taken from a fixed array
// in device memory that the library holds on every device it runs on until
// the process ends.
#include "common.h"

namespace qg {

// The workspace of moe_routed_qgemv_noalloc; each device holds its own copy.
static __device__ __align__(256) uint8_t scratch[QG_MOE_SCRATCH_BYTES];

constexpr int kScratchDevices = 64;
// Device address of `scratch` per device, set once per device (under the
// library lock, by once_per_device) before its first use.
static void *g_scratch_ptr[kScratchDevices];

static int scratch_init(const void *, int dev) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QG_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
    return QG_OK;
}

static const char g_scratch_key = 0;  // its address keys the set-up

}  // namespace qg

extern "C" int moe_routed_qgemv_noalloc(int fmt, const int8_t *qx, const float *dx, const int32_t *sx, int T, int D,
                                        int F, int E, int topk, const int32_t *ids, const float *rw,
                                        const void *const *gate, const void *const *up, const void *const *down,
                                        float *y, int32_t *d_status, void *stream) {
    if (fmt != QG_FMT_Q4K && fmt != QG_FMT_FP8_E4M3_B128 && fmt != QG_FMT_FP4_E2M1_MX) return QG_ERR_FORMAT;
    const size_t need = moe_routed_workspace_bytes(T, topk, E, D, F);
    if (need == 0) return QG_ERR_SHAPE;
    if (need > (size_t)QG_MOE_SCRATCH_BYTES) return QG_ERR_WORKSPACE;
    int dev = 0;
    if (qg::current_device(&dev) != QG_OK || dev >= qg::kScratchDevices) return QG_ERR_LAUNCH;
    if (qg::once_per_device(&qg::g_scratch_key, qg::scratch_init, dev) != QG_OK) return QG_ERR_LAUNCH;
    return moe_routed_qgemv_fmt(fmt, qx, dx, sx, T, D, F, E, topk, ids, rw, gate, up, down, y,
                                qg::g_scratch_ptr[dev], (size_t)QG_MOE_SCRATCH_BYTES, d_status, stream);
}
