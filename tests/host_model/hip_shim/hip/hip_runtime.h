// Host stand-in for <hip/hip_runtime.h>, used only by the CPU build of the
// library's host layer (tests/host_model).  It declares the few HIP types
// and calls the host layer uses, and emulates the wave-wide intrinsics of the
// plan builder on 64 host threads running in lockstep (lanes.cpp), so that
// the device's own plan code can run on the CPU under the sanitizers.
#pragma once

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#define __device__
#define __host__
#define __global__
#define __forceinline__ inline
#define __launch_bounds__(...)

typedef enum hipError_t {
    hipSuccess = 0,
    hipErrorInvalidValue = 1,
    hipErrorLaunchFailure = 719,
} hipError_t;

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;

hipError_t hipEventRecord(hipEvent_t event, hipStream_t stream);
hipError_t hipGetLastError(void);

struct HostThreadIdx {
    unsigned x, y, z;
};
extern thread_local HostThreadIdx threadIdx;

// Wave-wide operations: every one of the 64 emulated lanes must make the same
// sequence of these calls (the plan builder's loops around them are uniform).
int __shfl_up(int v, unsigned delta, int width);
int __shfl(int v, int src_lane, int width);
unsigned long long __ballot(int pred);
