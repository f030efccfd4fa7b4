// Split-KV planning and log-sum-exp combine for libmla355.
//
// Split-KV ("flash-decoding") is an exact regrouping of the softmax-weighted
// sum: attention over a token set A u B equals the e^{lse}-weighted mix of the
// two halves' normalised outputs, with lse = logaddexp(lse_A, lse_B).  The
// glossary page ("Multi-head Latent Attention", capacity and cost section)
// notes that online softmax still applies to MLA once the content and RoPE
// score parts are summed; the Polish glossary notes attention parallelises over
// tokens.  The split itself is this library's scheduling choice.
#include "mla355_internal.h"

#include <math.h>

namespace mla355 {
namespace {

constexpr int kPlanThreads = 1024;

// Inclusive block scan of one int per thread (Hillis-Steele in LDS).
__device__ int block_inclusive_scan(int x, int* buf)
{
    const int tid = threadIdx.x;
    buf[tid] = x;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
        const int y = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += y;
        __syncthreads();
    }
    const int r = buf[tid];
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens,
                                                            int b, int t_max, int n_chunks,
                                                            int min_chunk, int32_t* plan)
{
    __shared__ int buf[kPlanThreads];
    __shared__ int carry_s;
    PlanView v{plan, b};
    const int tid = threadIdx.x;

    // Pass 1: cu[] = prefix sums of the clamped lengths.
    int carry = 0;
    if (tid == 0) v.cu()[0] = 0;
    for (int base = 0; base < b; base += kPlanThreads) {
        const int i = base + tid;
        int L = 0;
        if (i < b) {
            L = seqlens[i];
            L = L < 0 ? 0 : (L > t_max ? t_max : L);
        }
        const int inc = block_inclusive_scan(L, buf);
        if (i < b) v.cu()[i + 1] = carry + inc;
        if (tid == kPlanThreads - 1) carry_s = inc;
        __syncthreads();
        carry += carry_s;
        __syncthreads();
    }
    const int total = carry;
    int chunk = (int)(((long long)total + n_chunks - 1) / n_chunks);
    if (chunk < min_chunk) chunk = min_chunk;
    if (tid == 0) {
        plan[0] = total;
        plan[1] = chunk;
        plan[2] = n_chunks;
        plan[3] = 0;
    }
    for (int k = tid; k < n_chunks; k += kPlanThreads) v.chunk_row()[k] = -1;
    __syncthreads();

    // Pass 2: segments per row, first partial slot per row, and for every
    // chunk the row holding its first token.
    carry = 0;
    for (int base = 0; base < b; base += kPlanThreads) {
        const int i = base + tid;
        int ns = 0;
        if (i < b) {
            const int lo = v.cu()[i], hi = v.cu()[i + 1];
            if (hi > lo) {
                ns = (hi - 1) / chunk - lo / chunk + 1;
                for (int k = (lo + chunk - 1) / chunk; k * chunk < hi; ++k) v.chunk_row()[k] = i;
            }
            v.nsplit()[i] = ns;
        }
        const int inc = block_inclusive_scan(ns, buf);
        if (i < b) v.base()[i] = carry + inc - ns;
        if (tid == kPlanThreads - 1) carry_s = inc;
        __syncthreads();
        carry += carry_s;
        __syncthreads();
    }
}

__device__ inline void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }

__device__ inline float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }

__device__ inline float4 load4(const __bf16* p)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
}

__device__ inline void store4(__bf16* p, float4 v)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 o;
    o[0] = (__bf16)v.x;
    o[1] = (__bf16)v.y;
    o[2] = (__bf16)v.z;
    o[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4*>(p) = o;
}

// One workgroup: two heads of one batch row; 128 threads per head, 4 latent
// columns per thread.  Rows with one segment were finished by the decode
// kernel; rows with none get out = 0, lse = -inf.
template <typename OutT>
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ plan, int b,
                                                      int h, const float* __restrict__ plse,
                                                      const OutT* __restrict__ po,
                                                      OutT* __restrict__ out,
                                                      float* __restrict__ lse)
{
    PlanView v{const_cast<int32_t*>(plan), b};
    const int hpairs = (h + 1) / 2;
    const int r = blockIdx.x / hpairs;
    const int head = (blockIdx.x % hpairs) * 2 + (threadIdx.x >> 7);
    if (r >= b || head >= h) return;
    const int c = (threadIdx.x & 127) * 4;
    const int ns = v.nsplit()[r];
    if (ns == 1) return;
    OutT* o = out + ((size_t)r * h + head) * kDc + c;
    if (ns == 0) {
        store4(o, make_float4(0.f, 0.f, 0.f, 0.f));
        if (c == 0) lse[(size_t)r * h + head] = -INFINITY;
        return;
    }
    const int s0 = v.base()[r];
    float mx = -INFINITY;
    for (int s = 0; s < ns; ++s) mx = fmaxf(mx, plse[(size_t)(s0 + s) * h + head]);
    float sum = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
        const float w = expf(plse[(size_t)(s0 + s) * h + head] - mx);
        const float4 x = load4(po + ((size_t)(s0 + s) * h + head) * kDc + c);
        sum += w;
        acc.x += w * x.x;
        acc.y += w * x.y;
        acc.z += w * x.z;
        acc.w += w * x.w;
    }
    const float inv = 1.0f / sum;
    store4(o, make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv));
    if (c == 0) lse[(size_t)r * h + head] = mx + logf(sum);
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, int b, int t_max, int n_chunks, int min_chunk,
                       int32_t* plan, hipStream_t stream)
{
    plan_kernel<<<1, kPlanThreads, 0, stream>>>(seqlens, b, t_max, n_chunks, min_chunk, plan);
    return hipGetLastError();
}

hipError_t launch_combine(bool bf16, const int32_t* plan, int b, int h, const float* plse,
                          const void* po, void* out, float* lse, hipStream_t stream)
{
    const unsigned grid = (unsigned)b * (unsigned)((h + 1) / 2);
    if (bf16)
        combine_kernel<__bf16><<<grid, 256, 0, stream>>>(plan, b, h, plse, (const __bf16*)po,
                                                         (__bf16*)out, lse);
    else
        combine_kernel<float><<<grid, 256, 0, stream>>>(plan, b, h, plse, (const float*)po,
                                                        (float*)out, lse);
    return hipGetLastError();
}

}  // namespace mla355
