// Query and output absorption (per-head batched matrix products).
//
// Glossary "Multi-head Latent Attention", section on why decode absorbs:
//   q absorb: qbar_h = q^C_h (W^UK_h)^T, a 512-wide latent-space query, which
//             the FlashMLA issue-16 answer concatenates with the 64-wide rope
//             query into the 576-wide attention input;
//   o absorb: (sum_t p_t c_t) W^UV_h, the value up-projection applied once to
//             the 512-wide attention output.
// Both are weight-read bound at decode batch sizes (each head's 128 x 512
// weight block is used by only b query rows), so they run on the vector ALU
// with fp32 accumulation: one workgroup per (head, block of 16 batch rows)
// streams that head's weights once with coalesced vector loads and keeps the
// 16 rows' inputs in LDS.
#include "mla355_internal.h"

namespace mla355 {
namespace {

constexpr int kRows = 16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
    typedef float type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec4<__bf16> {
    typedef __bf16 type __attribute__((ext_vector_type(4)));
};

// q'[r,h,0:512] = q_nope[r,h,:] . W_UK[h] ;  q'[r,h,512:576] = q_rope[r,h,:]
// 128 threads; thread t owns latent columns 4t .. 4t+3 for the 16 rows.
template <typename T>
__global__ __launch_bounds__(128) void absorb_q_kernel(int b, int h, const T* __restrict__ q_nope,
                                                       const T* __restrict__ w_uk,
                                                       const T* __restrict__ q_rope,
                                                       T* __restrict__ q_prime)
{
    typedef typename Vec4<T>::type v4;
    __shared__ float qs[kRows][kDk];
    const int head = blockIdx.x % h;
    const int r0 = (blockIdx.x / h) * kRows;
    const int nrows = min(kRows, b - r0);
    const int t = threadIdx.x;
    for (int i = t; i < kRows * kDk; i += 128) {
        const int rr = i / kDk, j = i % kDk;
        qs[rr][j] = rr < nrows ? to_f32(q_nope[((size_t)(r0 + rr) * h + head) * kDk + j]) : 0.f;
    }
    __syncthreads();
    float acc[kRows][4];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rr][e] = 0.f;
    const T* w = w_uk + (size_t)head * kDk * kDc + 4 * t;
    for (int j = 0; j < kDk; ++j) {
        const v4 wv = *(const v4*)(w + (size_t)j * kDc);
        const float w0 = to_f32(wv[0]), w1 = to_f32(wv[1]), w2 = to_f32(wv[2]), w3 = to_f32(wv[3]);
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
            const float q = qs[rr][j];
            acc[rr][0] = fmaf(q, w0, acc[rr][0]);
            acc[rr][1] = fmaf(q, w1, acc[rr][1]);
            acc[rr][2] = fmaf(q, w2, acc[rr][2]);
            acc[rr][3] = fmaf(q, w3, acc[rr][3]);
        }
    }
    for (int rr = 0; rr < nrows; ++rr) {
        v4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(acc[rr][e]);
        *(v4*)(q_prime + ((size_t)(r0 + rr) * h + head) * kDqk + 4 * t) = o;
    }
    for (int i = t; i < nrows * kDr; i += 128) {
        const int rr = i / kDr, j = i % kDr;
        q_prime[((size_t)(r0 + rr) * h + head) * kDqk + kDc + j] =
            q_rope[((size_t)(r0 + rr) * h + head) * kDr + j];
    }
}

// y[r,h,:] = o[r,h,:] . W_UV[h]
// 128 threads; thread t owns output column t for the 16 rows.
template <typename T>
__global__ __launch_bounds__(128) void absorb_o_kernel(int b, int h, const T* __restrict__ o,
                                                       const T* __restrict__ w_uv,
                                                       T* __restrict__ y)
{
    __shared__ float os[kRows][kDc];
    const int head = blockIdx.x % h;
    const int r0 = (blockIdx.x / h) * kRows;
    const int nrows = min(kRows, b - r0);
    const int t = threadIdx.x;
    for (int i = t; i < kRows * kDc; i += 128) {
        const int rr = i / kDc, c = i % kDc;
        os[rr][c] = rr < nrows ? to_f32(o[((size_t)(r0 + rr) * h + head) * kDc + c]) : 0.f;
    }
    __syncthreads();
    float acc[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) acc[rr] = 0.f;
    const T* w = w_uv + (size_t)head * kDc * kDv + t;
    for (int c = 0; c < kDc; ++c) {
        const float wv = to_f32(w[(size_t)c * kDv]);
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) acc[rr] = fmaf(os[rr][c], wv, acc[rr]);
    }
    for (int rr = 0; rr < nrows; ++rr) y[((size_t)(r0 + rr) * h + head) * kDv + t] = from_f32<T>(acc[rr]);
}

}  // namespace

hipError_t launch_absorb_q(bool bf16, int b, int h, const void* q_nope, const void* w_uk,
                           const void* q_rope, void* q_prime, hipStream_t stream)
{
    const unsigned grid = (unsigned)h * (unsigned)((b + kRows - 1) / kRows);
    if (bf16)
        absorb_q_kernel<__bf16><<<grid, 128, 0, stream>>>(b, h, (const __bf16*)q_nope,
                                                          (const __bf16*)w_uk, (const __bf16*)q_rope,
                                                          (__bf16*)q_prime);
    else
        absorb_q_kernel<float><<<grid, 128, 0, stream>>>(b, h, (const float*)q_nope,
                                                         (const float*)w_uk, (const float*)q_rope,
                                                         (float*)q_prime);
    return hipGetLastError();
}

hipError_t launch_absorb_o(bool bf16, int b, int h, const void* o, const void* w_uv, void* y,
                           hipStream_t stream)
{
    const unsigned grid = (unsigned)h * (unsigned)((b + kRows - 1) / kRows);
    if (bf16)
        absorb_o_kernel<__bf16><<<grid, 128, 0, stream>>>(b, h, (const __bf16*)o,
                                                          (const __bf16*)w_uv, (__bf16*)y);
    else
        absorb_o_kernel<float><<<grid, 128, 0, stream>>>(b, h, (const float*)o,
                                                         (const float*)w_uv, (float*)y);
    return hipGetLastError();
}

}  // namespace mla355
