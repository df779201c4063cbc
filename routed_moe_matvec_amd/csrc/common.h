// Device helpers shared by the libqgemv kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

constexpr int kWave = 64;

// Weights per "group": the unit one lane decodes at a time.  For Q8_0 that
// is 8 blocks (8 x 34 = 272 bytes, a multiple of 16), for Q4_K one superblock
// (144 bytes).  Both cover 256 consecutive weights of a row, so rows with
// K % 256 == 0 are whole numbers of groups and stay 16-byte aligned.
constexpr int kGroupWeights = 256;


template <int FMT>
struct GroupBytes;
template <>
struct GroupBytes<QG_FMT_Q8_0> {
    static constexpr int value = 272;
};
template <>
struct GroupBytes<QG_FMT_Q4K> {
    static constexpr int value = 144;
};

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

// low 32 bits of ({hi, lo} >> 8 * shift), shift in 0..3
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t shift) {
    return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}

__device__ __forceinline__ float fmaf_exact(float a, float b, float c) { return __builtin_fmaf(a, b, c); }

// 16-byte global -> LDS copy of one chunk per lane, written to
// lds_base + 16 * lane (lds_base must be wave-uniform).
__device__ __forceinline__ void global_to_lds16(const void *gsrc, void *lds_base) {
    __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Wait until every outstanding vector-memory operation of this wave (including
// global->LDS copies) has completed.  gfx9 s_waitcnt encoding: vmcnt = 0,
// expcnt = 7 (no wait), lgkmcnt = 15 (no wait).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// A wave-uniform read of memory that no thread of the kernel writes (tables
// built by an earlier launch): through the constant address space it becomes
// a scalar load, which waits on its own counter instead of queueing behind
// the vector loads in flight.
template <class T>
__device__ __forceinline__ T load_uniform(const T *p) {
    return *(const __attribute__((address_space(4))) T *)p;
}

// A pointer into device (global) memory.  Loads through a pointer that was
// itself read from memory (the routed experts' matrices) are otherwise
// generic "flat" loads, which also count against the LDS wait counter: every
// LDS wait would then wait for the weights in flight as well.
template <class T>
__device__ __forceinline__ const __attribute__((address_space(1))) T *as_global(const void *p) {
    return (const __attribute__((address_space(1))) T *)p;
}

// Workgroup barrier that orders LDS accesses only.  __syncthreads() also
// waits for every global load and store of the wave to complete; here the
// caller's global loads (weights in flight) and stores stay outstanding.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Host-side state (api.hip), all of it per device and behind one lock:
//  - once_per_device runs init(key, arg) once per (key, current device) and
//    remembers its success (a failure is retried on the next call);
//  - ensure_lds_limit raises a kernel's dynamic-LDS limit that way;
//  - device_cu_count gives the current device's compute units.
// Each returns QG_OK or QG_ERR_LAUNCH.
int current_device(int *dev);
// Clears an error that an earlier, unrelated HIP call left for this thread, so
// that the check after a launch (hipGetLastError) reports that launch only.
inline void clear_stale_error() { (void)hipGetLastError(); }
int once_per_device(const void *key, int (*init)(const void *key, int arg), int arg);
int ensure_lds_limit(const void *kern, int bytes);
int device_cu_count();

template <class T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, kWave);
}

}  // namespace qg
