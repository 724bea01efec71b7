// common.h -- internal helpers shared by the HIP sources of libbps.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "bps.h"

namespace bps {

// ---- error reporting (host) -------------------------------------------------

void set_error(const char *fmt, ...);
void clear_error();

#define BPS_FAIL(code, ...)              \
    do {                                 \
        ::bps::set_error(__VA_ARGS__);   \
        return (code);                   \
    } while (0)

#define BPS_HIP(call)                                                              \
    do {                                                                           \
        hipError_t e_ = (call);                                                    \
        if (e_ != hipSuccess)                                                      \
            BPS_FAIL(BPS_EHIP, "%s failed: %s", #call, hipGetErrorString(e_));     \
    } while (0)

// After a kernel launch: report a launch failure (does not synchronise).
#define BPS_LAUNCHED(name)                                                         \
    do {                                                                           \
        hipError_t e_ = hipGetLastError();                                         \
        if (e_ != hipSuccess)                                                      \
            BPS_FAIL(BPS_EHIP, "launch of %s failed: %s", name, hipGetErrorString(e_)); \
    } while (0)

// Kernel attributes of the current device, set once per device by the first
// call that needs them: every kernel whose launches may use more than the
// default 64 KiB of dynamic LDS is allowed its largest launch.  Host-side
// only (no stream work, no allocation), so it may run inside a graph capture.
// Also gives the device address of the current device's scratch array (the
// work memory of the allocation-free entry point) when scratch_dev is set.
bps_status prepare_device(void **scratch_dev = nullptr);
hipError_t spike_prepare_device();     // penta_spike.hip
hipError_t hines_prepare_device();     // hines.hip

inline hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

inline bool aligned(const void *p, size_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

inline size_t dtype_size(int dtype) {
    return dtype == BPS_F64 ? 8 : dtype == BPS_F32 ? 4 : 0;
}

// One wavefront of gfx950.
constexpr int kWave = 64;

// ---- device helpers ------------------------------------------------------------

template <typename T>
__device__ __forceinline__ bool bad_pivot(T v) {
    return v == T(0) || !isfinite(v);
}

// Grid-stride-free 1-D index of this lane.
__device__ __forceinline__ int64_t lane_id() {
    return int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
}

}  // namespace bps
