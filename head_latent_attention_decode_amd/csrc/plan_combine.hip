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
#include "plan_build.h"

#include <math.h>

namespace mla355 {
namespace {

constexpr int kPlanThreads = 256;
constexpr int kPlanMaxRowBlocks = 2048;

// Workgroup 0, wave 0 builds the plan; workgroups 1.. give every row with no
// tokens out = 0 and lse = -inf.
template <typename OutT>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens,
                                                            int b, int h, int t_max, int n_chunks,
                                                            int min_chunk, int align, int32_t* plan,
                                                            OutT* out, float* lse)
{
    if (blockIdx.x > 0) {
        zero_empty_rows([&](int r) { return clamped_len(seqlens, r, t_max); }, b, h, out, lse, blockIdx.x - 1,
                        gridDim.x - 1, threadIdx.x, kPlanThreads);
        return;
    }
    if (threadIdx.x >= 64) return;
    build_plan(seqlens, b, t_max, n_chunks, min_chunk, align, plan);
}

typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

typedef float f32x8_v __attribute__((ext_vector_type(8)));

// Eight consecutive elements of a partial row as loaded (one 16- or 32-byte
// load); they are converted to fp32 only where they are used, which keeps
// the bf16 rows in flight at four registers each.
template <typename T>
struct Vec8;
template <>
struct Vec8<__bf16> {
    typedef bf16x8_v type;
};
template <>
struct Vec8<float> {
    typedef f32x8_v type;
};

__device__ inline void store8(float* p, const float (&x)[8])
{
    reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

__device__ inline void store8(__bf16* p, const float (&x)[8])
{
    bf16x8_v v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = (__bf16)x[e];
    *reinterpret_cast<bf16x8_v*>(p) = v;
}

constexpr int kCombineThreads = 256;  // 4 waves = 4 heads of one batch row
constexpr int kCombineUnroll = 8;     // partial rows in flight per wave

// One wave per (batch row, head) of a row cut into several segments; no LDS
// and no barrier.  Every partial row (512 columns) is one coalesced load,
// lane l taking columns 8l .. 8l+7.  The slots are taken kCombineUnroll at a
// time with a running max m, running sum l and unnormalised sum acc (the
// usual online log-sum-exp): each round requests its slots' lse values
// together with their partial rows, so a row with up to kCombineUnroll
// segments waits on memory once after reading the plan.  Rows with one
// segment were finished by the attention kernel, rows with none by whichever
// kernel built the plan (plan_kernel, or the wide attention kernel itself).
template <typename OutT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(const int32_t* __restrict__ plan,
                                                                  int b, int h,
                                                                  const float* __restrict__ plse,
                                                                  const OutT* __restrict__ po,
                                                                  OutT* __restrict__ out,
                                                                  float* __restrict__ lse)
{
    PlanView v{const_cast<int32_t*>(plan), b};
    const int groups = (h + 3) / 4;
    // Workgroups go to the 8 XCDs round-robin by id, and the attention kernel
    // handles the chunks of the batch's eighth x on XCD x: the workgroups of
    // row r take ids on that XCD, whose L2 may still hold the row's partials.
    const int b8 = b / 8;
    int rg = blockIdx.x;
    if ((int)blockIdx.x < 8 * b8 * groups) {
        const int x = blockIdx.x % 8, j = blockIdx.x / 8;
        rg = (x * b8 + j / groups) * groups + j % groups;
    }
    const int r = rg / groups;
    // the head is the same for the whole wave: keep it, and every address
    // built on it but the lane's 16 bytes, in scalar registers
    const int head = __builtin_amdgcn_readfirstlane((rg % groups) * 4 + (threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    if (head >= h) return;
    const int ns = v.nsplit()[r];
    if (ns <= 1) return;
    const int s0 = v.base()[r];
    const float* pl = plse + (size_t)s0 * h + head;
    const OutT* prow = po + ((size_t)s0 * h + head) * kDc;

    float m = -INFINITY, l = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s = 0; s < ns; s += kCombineUnroll) {
        // slots past the end re-read the last one and take no part below
        float ls[kCombineUnroll];
        typename Vec8<OutT>::type x[kCombineUnroll];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int sl = min(s + u, ns - 1);
            ls[u] = pl[(size_t)sl * h];
            x[u] = reinterpret_cast<const typename Vec8<OutT>::type*>(prow + (size_t)sl * h * kDc)[lane];
        }
        float mb = m;
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u)
            if (s + u < ns) mb = fmaxf(mb, ls[u]);
        if (mb == -INFINITY) continue;  // no segment so far saw a token
        const float scale = expf(m - mb);  // 0 while m is still -inf
        l *= scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= scale;
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const float w = s + u < ns ? expf(ls[u] - mb) : 0.f;
            l += w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[u][e];
        }
        m = mb;
    }
    OutT* o = out + ((size_t)r * h + head) * kDc + 8 * lane;
    if (m == -INFINITY) {
        // no segment saw a token (a causal query row with an empty prefix)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        store8(o, acc);
        if (lane == 0) lse[(size_t)r * h + head] = -INFINITY;
        return;
    }
    const float inv = 1.0f / l;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8(o, acc);
    if (lane == 0) lse[(size_t)r * h + head] = m + logf(l);
}

// Rows cut into many segments: one workgroup per (row, head).  Wave w takes
// slots w, w + 4, w + 8, ... with the online log-sum-exp above
// (kCombineUnroll of its slots per round), and the four (m, l, acc) are
// merged through LDS by wave 0.
template <typename OutT>
__global__ __launch_bounds__(kCombineThreads) void combine_split_kernel(const int32_t* __restrict__ plan,
                                                                        int b, int h,
                                                                        const float* __restrict__ plse,
                                                                        const OutT* __restrict__ po,
                                                                        OutT* __restrict__ out,
                                                                        float* __restrict__ lse)
{
    constexpr int NW = kCombineThreads / 64;
    __shared__ float wm[NW], wl[NW];
    __shared__ float wacc[NW][8 * 64];  // [wave][element * 64 + lane]
    PlanView v{const_cast<int32_t*>(plan), b};
    const int r = blockIdx.x / h;
    const int head = blockIdx.x % h;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int ns = v.nsplit()[r];
    if (ns <= 1) return;  // the same for the whole workgroup
    const int s0 = v.base()[r];
    const float* pl = plse + (size_t)s0 * h + head;
    const OutT* prow = po + ((size_t)s0 * h + head) * kDc;

    float m = -INFINITY, l = 0.f;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    for (int s = wave; s < ns; s += NW * kCombineUnroll) {
        // this wave's slots s, s + NW, ...; past the end it re-reads slot s
        // (weight 0 below)
        float ls[kCombineUnroll];
        typename Vec8<OutT>::type x[kCombineUnroll];
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const int sl = s + NW * u < ns ? s + NW * u : s;
            ls[u] = pl[(size_t)sl * h];
            x[u] = reinterpret_cast<const typename Vec8<OutT>::type*>(prow + (size_t)sl * h * kDc)[lane];
        }
        float mb = m;
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u)
            if (s + NW * u < ns) mb = fmaxf(mb, ls[u]);
        if (mb == -INFINITY) continue;
        const float scale = expf(m - mb);
        l *= scale;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] *= scale;
#pragma unroll
        for (int u = 0; u < kCombineUnroll; ++u) {
            const float w = s + NW * u < ns ? expf(ls[u] - mb) : 0.f;
            l += w;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += w * (float)x[u][e];
        }
        m = mb;
    }
    if (lane == 0) {
        wm[wave] = m;
        wl[wave] = l;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) wacc[wave][e * 64 + lane] = acc[e];
    __syncthreads();
    if (wave != 0) return;

    float mx = wm[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, wm[w]);
    OutT* o = out + ((size_t)r * h + head) * kDc + 8 * lane;
    if (mx == -INFINITY) {
        // no segment saw a token (a causal query row with an empty prefix)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = 0.f;
        store8(o, acc);
        if (lane == 0) lse[(size_t)r * h + head] = -INFINITY;
        return;
    }
    float lt = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const float f = wm[w] == -INFINITY ? 0.f : expf(wm[w] - mx);
        lt += wl[w] * f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += f * wacc[w][e * 64 + lane];
    }
    const float inv = 1.0f / lt;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= inv;
    store8(o, acc);
    if (lane == 0) lse[(size_t)r * h + head] = mx + logf(lt);
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, int b, int h, int t_max, int n_chunks, int min_chunk,
                       int align, int32_t* plan, bool bf16, void* out, float* lse, hipStream_t stream)
{
    const unsigned grid = 1u + (unsigned)(b < kPlanMaxRowBlocks ? b : kPlanMaxRowBlocks);
    if (bf16)
        plan_kernel<__bf16><<<grid, kPlanThreads, 0, stream>>>(seqlens, b, h, t_max, n_chunks, min_chunk,
                                                               align, plan, (__bf16*)out, lse);
    else
        plan_kernel<float><<<grid, kPlanThreads, 0, stream>>>(seqlens, b, h, t_max, n_chunks, min_chunk,
                                                              align, plan, (float*)out, lse);
    return hipGetLastError();
}

hipError_t launch_combine(bool bf16, const int32_t* plan, int b, int h, int n_chunks, const float* plse,
                          const void* po, void* out, float* lse, hipStream_t stream)
{
    // Sixteen or more segments per row on average: a workgroup per (row, head)
    // so that the slots are read four waves at a time.
    if ((long long)n_chunks >= 16LL * b) {
        const unsigned grid = (unsigned)b * (unsigned)h;
        if (bf16)
            combine_split_kernel<__bf16><<<grid, kCombineThreads, 0, stream>>>(plan, b, h, plse, (const __bf16*)po,
                                                                               (__bf16*)out, lse);
        else
            combine_split_kernel<float><<<grid, kCombineThreads, 0, stream>>>(plan, b, h, plse, (const float*)po,
                                                                              (float*)out, lse);
        return hipGetLastError();
    }
    const unsigned grid = (unsigned)b * (unsigned)((h + 3) / 4);
    if (bf16)
        combine_kernel<__bf16><<<grid, kCombineThreads, 0, stream>>>(plan, b, h, plse, (const __bf16*)po,
                                                                     (__bf16*)out, lse);
    else
        combine_kernel<float><<<grid, kCombineThreads, 0, stream>>>(plan, b, h, plse, (const float*)po,
                                                                    (float*)out, lse);
    return hipGetLastError();
}

}  // namespace mla355
