// mla_decode_noalloc: mla_decode with the split plan and the partial results
// kept in a fixed device array of this library instead of a caller-provided
// workspace, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code its name is only a host-side stand-in, so the device address is looked
// up once per device (hipGetSymbolAddress, with that device current) on the
// entry point's first call there, and that address is what the kernels get.
// Every call on one GPU shares that GPU's array: calls that overlap in time on
// one GPU (two streams, two threads) race on it.  Nothing in it needs to start
// at zero: the kernels write the plan and every partial before reading them.
#include "../../include/mla355.h"
#include "mla355_internal.h"

#include <mutex>

namespace mla355 {
namespace {

constexpr size_t kScratchBytes = (size_t)MLA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];  // device address of `scratch` per device (nullptr: not yet looked up)

// The calling thread's current device's copy of `scratch`, or nullptr.
void* device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lk(scratch_mu);
    if (scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        scratch_ptr[dev] = p;
    }
    return scratch_ptr[dev];
}

}  // namespace
}  // namespace mla355

#pragma GCC visibility push(default)
extern "C" {

mla_status_t mla_decode_noalloc(mla_dtype_t dtype, int b, int h, int t_max, const void* q_prime,
                                const void* cache, const int32_t* seqlens, float softmax_scale, void* out,
                                float* lse, void* stream)
{
    const size_t need = mla_decode_workspace_bytes(dtype, b, h, t_max);
    if (need == 0) return MLA_ERR_INVALID_ARGUMENT;
    if (need > mla355::kScratchBytes) return MLA_ERR_WORKSPACE_TOO_SMALL;
    void* ws = mla355::device_scratch();
    if (ws == nullptr) return MLA_ERR_HIP;
    return mla_decode(dtype, b, h, t_max, q_prime, cache, seqlens, softmax_scale, out, lse, ws,
                      mla355::kScratchBytes, stream);
}

}  // extern "C"
#pragma GCC visibility pop
