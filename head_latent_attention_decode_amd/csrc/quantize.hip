// Per-token fp8 (OCP e4m3) form of latent cache rows, for the fp8 decode path.
//
// The pages do not define a quantised cache; this is the plainest form that
// keeps every scale out of the inner products: one fp32 scale per cached
// token (per 576-wide row), scale = max_i |x_i| / 448 (448 is the largest
// finite e4m3 magnitude), code_i = e4m3(x_i / scale) rounded to nearest even,
// with the quotient clamped to [-448, 448] (0 codes when the row is all zero).
// The decode kernel multiplies each token's score and probability by its
// scale, so the codes enter the MFMAs as exact bf16 values.
#include "mla355_internal.h"

namespace mla355 {
namespace {

constexpr int kRowsPerBlock = 4;        // one wave per row
constexpr long long kMaxBlocks = 1 << 20;  // larger inputs loop (grid stride)

__global__ __launch_bounds__(64 * kRowsPerBlock) void quantize_fp8_kernel(long long n_rows,
                                                                          const __bf16* __restrict__ x,
                                                                          unsigned char* __restrict__ codes,
                                                                          float* __restrict__ scale)
{
    const int lane = threadIdx.x & 63;
    const long long stride = (long long)gridDim.x * kRowsPerBlock;
    for (long long row = (long long)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); row < n_rows; row += stride) {
        const __bf16* xr = x + row * kDqk;
        constexpr int PER = kDqk / 64;  // 9 values per lane: columns lane + 64 j
        float v[PER];
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            v[j] = (float)xr[lane + 64 * j];
            a = fmaxf(a, fabsf(v[j]));
        }
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off, 64));
        const float s = a / 448.0f;
        unsigned char* cr = codes + row * kDqk;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            float q = s > 0.f ? v[j] / s : 0.f;
            q = fminf(fmaxf(q, -448.0f), 448.0f);
            cr[lane + 64 * j] = (unsigned char)(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFF);
        }
        if (lane == 0) scale[row] = s;
    }
}

}  // namespace

hipError_t launch_quantize_fp8(long long n_rows, const void* x, void* codes, float* scale,
                               hipStream_t stream)
{
    long long grid = (n_rows + kRowsPerBlock - 1) / kRowsPerBlock;
    if (grid > kMaxBlocks) grid = kMaxBlocks;
    quantize_fp8_kernel<<<(unsigned)grid, 64 * kRowsPerBlock, 0, stream>>>(
        n_rows, (const __bf16*)x, (unsigned char*)codes, scale);
    return hipGetLastError();
}

}  // namespace mla355
