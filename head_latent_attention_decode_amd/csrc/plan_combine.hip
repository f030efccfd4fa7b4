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

constexpr int kPlanThreads = 256;
constexpr int kPlanMaxRowBlocks = 2048;

// Inclusive scan across the 64 lanes of a wave.
__device__ int wave_inclusive_scan(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

__device__ int clamped_len(const int32_t* seqlens, int i, int t_max)
{
    const int L = seqlens[i];
    return L < 0 ? 0 : (L > t_max ? t_max : L);
}

// Workgroup 0, wave 0 builds the plan (two scans over the clamped lengths, 64
// rows per step).  Workgroups 1.. give every row with no tokens out = 0 and
// lse = -inf.  With align > 1 the plan is laid over the lengths rounded up to
// a multiple of align, and the chunk too, so that every segment starts at a
// multiple of align inside its row (the paged cache needs whole tiles inside
// one block); the kernel masks the padding with the true lengths.
template <typename OutT>
__global__ __launch_bounds__(kPlanThreads) void plan_kernel(const int32_t* __restrict__ seqlens,
                                                            int b, int h, int t_max, int n_chunks,
                                                            int min_chunk, int align, int32_t* plan,
                                                            OutT* out, float* lse)
{
    auto planned_len = [&](int i) { return (clamped_len(seqlens, i, t_max) + align - 1) / align * align; };
    const int tid = threadIdx.x;
    if (blockIdx.x > 0) {
        for (int r = blockIdx.x - 1; r < b; r += gridDim.x - 1) {
            if (clamped_len(seqlens, r, t_max) != 0) continue;
            OutT* o = out + (size_t)r * h * kDc;
            for (int i = tid; i < h * kDc; i += kPlanThreads) o[i] = (OutT)0.f;
            for (int i = tid; i < h; i += kPlanThreads) lse[(size_t)r * h + i] = -INFINITY;
        }
        return;
    }
    if (tid >= 64) return;
    PlanView v{plan, b};
    const int lane = tid;

    // Pass 1: cu[] = prefix sums of the clamped lengths.
    int carry = 0;
    if (lane == 0) v.cu()[0] = 0;
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        const int L = i < b ? planned_len(i) : 0;
        const int inc = wave_inclusive_scan(L);
        if (i < b) v.cu()[i + 1] = carry + inc;
        carry += __shfl(inc, 63, 64);
    }
    const int total = carry;
    int chunk = (int)(((long long)total + n_chunks - 1) / n_chunks);
    if (chunk < min_chunk) chunk = min_chunk;
    chunk = (chunk + align - 1) / align * align;
    if (lane == 0) {
        plan[0] = total;
        plan[1] = chunk;
        plan[2] = n_chunks;
        plan[3] = 0;
    }
    // Chunks starting at or past the last token are idle.  Every other chunk
    // k starts inside exactly one non-empty row (the one holding token
    // k * chunk), written in pass 2; the two sets are disjoint.
    const int first_idle = (total + chunk - 1) / chunk;
    for (int k = first_idle + lane; k < n_chunks; k += 64) v.chunk_row()[k] = -1;

    // Pass 2 (the lengths are scanned again rather than read back): segments
    // per row, first partial slot per row, and the starting row of every chunk.
    carry = 0;
    int slots = 0;
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        const int L = i < b ? planned_len(i) : 0;
        const int inc = wave_inclusive_scan(L);
        const int hi = carry + inc, lo = hi - L;
        int ns = 0, k_lo = 0, k_hi = 0;  // chunks k_lo .. k_hi-1 start inside row i
        if (i < b && L > 0) {
            ns = (hi - 1) / chunk - lo / chunk + 1;
            k_lo = (int)(((long long)lo + chunk - 1) / chunk);
            k_hi = (int)(((long long)hi + chunk - 1) / chunk);
        }
        // a lane writes its own row's few chunk starts; rows holding many are
        // written by the whole wave, one row at a time
        constexpr int kLaneChunks = 4;
        if (k_hi - k_lo <= kLaneChunks)
            for (int k = k_lo; k < k_hi; ++k) v.chunk_row()[k] = i;
        unsigned long long many = __ballot(k_hi - k_lo > kLaneChunks);
        while (many) {
            const int j = __builtin_ctzll(many);
            many &= many - 1;
            const int a = __shfl(k_lo, j, 64), z = __shfl(k_hi, j, 64);
            for (int k = a + lane; k < z; k += 64) v.chunk_row()[k] = base + j;
        }
        const int ns_inc = wave_inclusive_scan(ns);
        if (i < b) {
            v.nsplit()[i] = ns;
            v.base()[i] = slots + ns_inc - ns;
        }
        carry += __shfl(inc, 63, 64);
        slots += __shfl(ns_inc, 63, 64);
    }
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
// segment were finished by the decode kernel, rows with none by plan_kernel.
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
    const int r = blockIdx.x / groups;
    // the head is the same for the whole wave: keep it, and every address
    // built on it but the lane's 16 bytes, in scalar registers
    const int head = __builtin_amdgcn_readfirstlane((blockIdx.x % groups) * 4 + (threadIdx.x >> 6));
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

hipError_t launch_combine(bool bf16, const int32_t* plan, int b, int h, const float* plse,
                          const void* po, void* out, float* lse, hipStream_t stream)
{
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
