// Split-KV absorbed-MLA decode, fp32 throughout (IEEE fp32 FMAs on the vector
// ALU; no reduced-precision matrix mode anywhere).  Same operation, plan and
// partial format as the bf16 kernel; this instance serves fp32 callers, where
// accuracy rather than speed is the point.
//
// One workgroup (256 threads) = one token chunk x 16 heads.  Per 16-token
// tile: thread (head = t/16, token = t%16) forms one 576-wide score; the
// 16 lanes of a head reduce max and sum with cross-lane steps; then thread
// (head = t/16) accumulates 32 latent columns (t%16 + 16 j) of the weighted
// sum.
#include "mla355_internal.h"

#include <math.h>

namespace mla355 {
namespace {

constexpr int kHeads = 16;
constexpr int kTok = 16;
constexpr int kPitch = kDqk + 1;  // padded LDS row (floats) against bank conflicts
constexpr float kNegBig = -1.0e30f;

__global__ __launch_bounds__(256) void decode_f32_kernel(DecodeParams p)
{
    __shared__ float q_s[kHeads * kPitch];
    __shared__ float k_s[kTok * kPitch];
    __shared__ float p_s[kHeads * kTok];

    const int t = threadIdx.x;
    const int hh = t / kTok;  // head inside the group
    const int tt = t % kTok;  // token inside the tile (scores) / column phase (output)
    const int k = blockIdx.x / p.n_hg;
    const int hg = blockIdx.x % p.n_hg;
    const PlanView pv{const_cast<int32_t*>(p.plan), p.b};
    const int total = p.plan[0];
    const int chunk = p.plan[1];
    int r = pv.chunk_row()[k];
    if (r < 0) return;
    int pos = k * chunk;
    const int end = pos + min(chunk, total - pos);  // no int overflow near 2^31 tokens
    const float* qg = (const float*)p.q;
    const float* cg = (const float*)p.cache;
    const int head = hg * kHeads + hh;
    const bool head_ok = head < p.h;

    while (true) {
        const int row_lo = pv.cu()[r];
        const int row_hi = pv.cu()[r + 1];
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        const int seg_len = seg_end - pos;
        const int split_j = k - row_lo / chunk;
        const bool final_out = pv.nsplit()[r] == 1;
        const int slot = pv.base()[r] + split_j;

        __syncthreads();
        for (int i = t; i < kHeads * kDqk; i += 256) {
            const int h2 = i / kDqk, c = i % kDqk;
            const int hd = hg * kHeads + h2;
            q_s[h2 * kPitch + c] = hd < p.h ? qg[((size_t)r * p.h + hd) * kDqk + c] : 0.f;
        }
        float m_run = kNegBig, l_run = 0.f;
        float acc[kDc / kTok];
#pragma unroll
        for (int j = 0; j < kDc / kTok; ++j) acc[j] = 0.f;

        for (int t0 = 0; t0 < seg_len; t0 += kTok) {
            const int nvalid = min(kTok, seg_len - t0);
            __syncthreads();
            for (int i = t; i < kTok * kDqk; i += 256) {
                const int rr = i / kDqk, c = i % kDqk;
                const int tok = seg_a + t0 + min(rr, nvalid - 1);
                k_s[rr * kPitch + c] = cg[((size_t)r * p.t_max + tok) * kDqk + c];
            }
            __syncthreads();
            float s = 0.f;
            for (int c = 0; c < kDqk; ++c) s = fmaf(q_s[hh * kPitch + c], k_s[tt * kPitch + c], s);
            s = (tt < nvalid) ? s * p.scale_log2 : -INFINITY;
            float mx = s;
#pragma unroll
            for (int off = 1; off < kTok; off <<= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            const float m_new = fmaxf(m_run, mx);
            const float alpha = exp2f(m_run - m_new);
            const float e = exp2f(s - m_new);
            float se = e;
#pragma unroll
            for (int off = 1; off < kTok; off <<= 1) se += __shfl_xor(se, off, 64);
            l_run = l_run * alpha + se;
            m_run = m_new;
            p_s[hh * kTok + tt] = e;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < kDc / kTok; ++j) acc[j] *= alpha;
            for (int u = 0; u < nvalid; ++u) {
                const float pu = p_s[hh * kTok + u];
#pragma unroll
                for (int j = 0; j < kDc / kTok; ++j) acc[j] = fmaf(pu, k_s[u * kPitch + tt + kTok * j], acc[j]);
            }
        }

        if (head_ok) {
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + log2f(l_run)) * 0.69314718055994531f : -INFINITY;
            float* dst = final_out ? (float*)p.out + ((size_t)r * p.h + head) * kDc
                                   : (float*)p.po + ((size_t)slot * p.h + head) * kDc;
#pragma unroll
            for (int j = 0; j < kDc / kTok; ++j) dst[tt + kTok * j] = acc[j] * inv;
            if (tt == 0) {
                if (final_out)
                    p.lse[(size_t)r * p.h + head] = lse_v;
                else
                    p.plse[(size_t)slot * p.h + head] = lse_v;
            }
        }

        pos = seg_end;
        if (pos >= end) break;
        ++r;
        while (pv.cu()[r + 1] <= pos) ++r;
    }
}

}  // namespace

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream)
{
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    decode_f32_kernel<<<grid, 256, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace mla355
