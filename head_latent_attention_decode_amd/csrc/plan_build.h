// The split plan, built by one wave: shared by plan_kernel (which writes it to
// the workspace) and by the attention kernels that build their own copy in
// LDS.  Layout (int32): [total, chunk, n_chunks, 0], cu[b + 1] (prefix sums of
// the planned lengths), base[b] (first partial slot of each row), nsplit[b]
// (segments per row), chunk_row[n_chunks] (row in which chunk k starts, -1 for
// idle chunks); see PlanView.
#pragma once

#include "mla355_internal.h"

namespace mla355 {

__device__ __forceinline__ int clamped_len(const int32_t* seqlens, int i, int t_max)
{
    const int L = seqlens[i];
    return L < 0 ? 0 : (L > t_max ? t_max : L);
}

// Inclusive scan across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int x)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    return x;
}

// Called by all 64 lanes of one wave.  P: int32_t* (global) or an LDS pointer.
// Two scans over the clamped lengths, 64 rows per step.  With align > 1 the
// plan is laid over the lengths rounded up to a multiple of align, and the
// chunk too, so that every segment starts at a multiple of align inside its
// row (the paged cache needs whole tiles inside one block); the attention
// kernel masks the padding with the true lengths.
template <typename P>
__device__ void build_plan(const int32_t* __restrict__ seqlens, int b, int t_max, int n_chunks,
                           int min_chunk, int align, P plan)
{
    auto planned_len = [&](int i) { return (clamped_len(seqlens, i, t_max) + align - 1) / align * align; };
    const int lane = threadIdx.x & 63;
    P cu = plan + 4;
    P base_of = plan + 4 + (b + 1);
    P nsplit = plan + 4 + (b + 1) + b;
    P chunk_row = plan + 4 + (b + 1) + 2 * b;

    // Pass 1: cu[] = prefix sums of the planned lengths.  The first 64 rows'
    // lengths stay in a register for pass 2.
    const int len0 = lane < b ? planned_len(lane) : 0;
    int carry = 0;
    if (lane == 0) cu[0] = 0;
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        const int L = base == 0 ? len0 : (i < b ? planned_len(i) : 0);
        const int inc = wave_inclusive_scan(L);
        if (i < b) cu[i + 1] = carry + inc;
        carry += __shfl(inc, 63, 64);
    }
    // Totals stay below 2^31 (the host bounds b * t_max), so every rounded-up
    // quotient below is exact in unsigned 32-bit arithmetic.
    const int total = carry;
    int chunk = (int)(((unsigned)total + (unsigned)n_chunks - 1u) / (unsigned)n_chunks);
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
    const int first_idle = (int)(((unsigned)total + (unsigned)chunk - 1u) / (unsigned)chunk);
    for (int k = first_idle + lane; k < n_chunks; k += 64) chunk_row[k] = -1;

    // Pass 2: segments per row, first partial slot per row, and the starting
    // row of every chunk.
    carry = 0;
    int slots = 0;
    for (int base = 0; base < b; base += 64) {
        const int i = base + lane;
        const int L = base == 0 ? len0 : (i < b ? planned_len(i) : 0);
        const int inc = wave_inclusive_scan(L);
        const int hi = carry + inc, lo = hi - L;
        int ns = 0, k_lo = 0, k_hi = 0;  // chunks k_lo .. k_hi-1 start inside row i
        if (i < b && L > 0) {
            ns = (hi - 1) / chunk - lo / chunk + 1;
            k_lo = (int)(((unsigned)lo + (unsigned)chunk - 1u) / (unsigned)chunk);
            k_hi = (int)(((unsigned)hi + (unsigned)chunk - 1u) / (unsigned)chunk);
        }
        // a lane writes its own row's few chunk starts; rows holding many are
        // written by the whole wave, one row at a time
        constexpr int kLaneChunks = 4;
        if (k_hi - k_lo <= kLaneChunks)
            for (int k = k_lo; k < k_hi; ++k) chunk_row[k] = i;
        unsigned long long many = __ballot(k_hi - k_lo > kLaneChunks);
        while (many) {
            const int j = __builtin_ctzll(many);
            many &= many - 1;
            const int a = __shfl(k_lo, j, 64), z = __shfl(k_hi, j, 64);
            for (int k = a + lane; k < z; k += 64) chunk_row[k] = base + j;
        }
        const int ns_inc = wave_inclusive_scan(ns);
        if (i < b) {
            nsplit[i] = ns;
            base_of[i] = slots + ns_inc - ns;
        }
        carry += __shfl(inc, 63, 64);
        slots += __shfl(ns_inc, 63, 64);
    }
}

// out = 0, lse = -inf for every row r = first, first + stride, ... with no
// tokens (no attention workgroup touches such a row), h rows of 512 outputs
// each; `tid` of `nthreads` threads.  len(r): the row's (clamped) length.
template <typename OutT, typename LenFn>
__device__ void zero_empty_rows(LenFn len, int b, int h, OutT* out, float* lse, int first, int stride,
                                int tid, int nthreads)
{
    for (int r = first; r < b; r += stride) {
        if (len(r) != 0) continue;
        OutT* o = out + (size_t)r * h * kDc;
        for (int i = tid; i < h * kDc; i += nthreads) o[i] = (OutT)0.f;
        for (int i = tid; i < h; i += nthreads) lse[(size_t)r * h + i] = -INFINITY;
    }
}

}  // namespace mla355
