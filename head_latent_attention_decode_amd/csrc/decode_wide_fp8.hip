// Split-KV absorbed-MLA decode over an fp8 (OCP e4m3) latent cache for groups
// of 128 heads: scores on the gfx950 FP8 matrix cores, the weighted sum on the
// bf16 ones.
//
// Same operation, plan and partial format as the bf16 kernels (the glossary
// page "Multi-head Latent Attention", section on why decode absorbs the
// matrices: absorbed query heads score directly against the shared latent
// rows, and the softmax-weighted sum of the c_KV parts is the output).  The
// cache holds one e4m3 code per element and one fp32 scale s_t per token (the
// library's per-token quantiser, quantize.hip).
//
//  * Scores use v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales.  That
//    instruction takes both operands in e4m3, so each workgroup quantises its
//    row's queries on entry, per (batch row, head) over all 576 channels:
//      sigma = max|q'| / 448,  code = e4m3(clamp(q' * (448 / max|q'|), +-448))
//    (fp32 quotient and product, rounded to the nearest code, ties to even;
//    an all-zero query gets sigma = 0 and zero codes).  A score is then
//    sigma * s_t * (code_q . code_t).
//  * The weighted sum runs on bf16 MFMAs: every e4m3 code is exactly a bf16
//    value (converted in registers after a transposed 8-bit LDS read), and
//    the token scale folds into the probability (P^T entry bf16(p * s_t)).
//  * Layout of the work as in the bf16 wide kernel: one workgroup = one token
//    chunk x 128 heads, 32 heads per wave, queries in VGPRs (72 of them as
//    codes), each wave's 512 x 32 fp32 outputs in AGPRs.  32-token tiles of
//    18.3 KB stream into a four-deep LDS ring by direct-to-LDS DMA; the
//    queries are fetched first, so their quantisation overlaps the first
//    tiles' DMA.
#include "bf16_common.h"
#include "plan_build.h"

#include <math.h>

namespace mla355 {
namespace {

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2f = 0.69314718055994531f;
constexpr float kE4m3Max = 448.0f;

// Region A of a tile (channels 0..511, 512-byte rows): 16-byte chunk c of row
// r sits at chunk position c ^ sw8(r).  sw8 permutes the low four bits of r:
// 16 consecutive rows read at one chunk land in 16 distinct 16-byte bank
// groups, and each half-wave of the transposed reads (8 rows whose bit 2
// agrees, two adjacent chunks) covers all 64 banks once, since those 8 rows
// get 8 distinct values of one parity.
__device__ __forceinline__ int sw8(int r) { return ((r >> 2) & 1) | ((r & 1) << 1) | (((r >> 1) & 1) << 2) | (r & 8); }

template <int STAGES>
struct WideF8Tiling {
    static constexpr int NW = 4;
    static constexpr int THREADS = NW * 64;
    static constexpr int HG = 32 * NW;               // heads per workgroup
    static constexpr int N = 32;                     // tokens per tile
    static constexpr int ROW8 = kDqk;                // bytes of an e4m3 row in HBM
    static constexpr int A_BYTES = N * 512;          // region A: channels 0..511
    static constexpr int B_OFF = A_BYTES;            // region B: channels 512..575, 64-byte rows
    static constexpr int SCL_OFF = B_OFF + N * 64;   // the tile's 32 token scales (64 slots)
    static constexpr int TILE_BYTES = SCL_OFF + 64 * 4;
    static constexpr int LOADS_A = 16 / NW;          // two rows per DMA instruction
    // plus two instructions per wave: a region-B block of 16 rows (waves w
    // and w + 2 the same rows) and the 32 scales (every wave the same bytes)
    static constexpr int LOADS = LOADS_A + 2;
    static constexpr int KS = kDqk / 64;             // 9 score steps of 64 channels
    static constexpr int MBLK = kDc / 32;            // 16 output blocks of 32 columns
    static constexpr int STG_ROW = 512 + 16;         // epilogue staging row (bf16 half rows)
    static_assert(32 * STG_ROW <= TILE_BYTES, "a wave's epilogue staging fits one stage");
    static_assert(STAGES >= NW && STAGES <= 6, "one stage per wave for the epilogue; LDS budget");
    static_assert((STAGES - 2) * LOADS <= 63, "vmcnt range");
    static_assert(LOADS <= KS, "refill spread over the score steps");
};

// Score MFMAs (S^T += K . Q'^T, 32 tokens x 64 channels x 32 heads, both
// operands e4m3, unit block scales: `one` holds the E8M0 code 127) with the
// accumulator in VGPRs.  The 256 AGPRs hold the output accumulators and the
// compiler picks one register form for every MFMA of a kernel, so these are
// written as inline asm; the hazard recognizer does not look inside asm, so
// score8_wait() supplies the wait states between the last score MFMA (16
// passes) and the first vector-ALU access to its result.
__device__ __forceinline__ f32x16_t score8_first(i32x8_t a, i32x8_t b, int one)
{
    f32x16_t d;
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, 0, %3, %3 op_sel_hi:[0,0,0]"
                 : "=&v"(d)
                 : "v"(a), "v"(b), "v"(one));
    return d;
}
__device__ __forceinline__ void score8_acc(f32x16_t& acc, i32x8_t a, i32x8_t b, int one)
{
    asm volatile("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3 op_sel_hi:[0,0,0]"
                 : "+v"(acc)
                 : "v"(a), "v"(b), "v"(one));
}
__device__ __forceinline__ void score8_wait(f32x16_t& acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Four fp32 values -> four e4m3 codes (one dword, first value in the low byte).
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d)
{
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

template <int STAGES>
__device__ __forceinline__ void decode_wide_fp8_body(const DecodeParams& p)
{
    using T = WideF8Tiling<STAGES>;
    using M = Mfma<32>;
    typedef f32x16_t acc_t;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31;    // head inside the wave's 32
    const int grp = lane >> 5;   // k-slot group of the MFMA operand layouts

    int k, hg;
    block_work(p.n_chunks, p.n_hg, k, hg);
    // The split plan: plan_kernel's copy in the workspace or, with
    // plan_in_kernel, this workgroup's own copy in LDS built by wave 0
    // (workgroup 0 also leaves it in the workspace for the combine).
    __shared__ int32_t lplan[kPlanLdsInts];
    const bool lds_plan = p.plan_in_kernel != 0;
    if (lds_plan) {
        if (wave == 0)
            build_plan(p.seqlens, p.b, p.t_max, p.n_chunks, p.plan_min_chunk, p.plan_align,
                       (LDS_AS int32_t*)lplan);
        __syncthreads();
        if (blockIdx.x == 0) {
            const int n = 4 + (p.b + 1) + 2 * p.b + p.n_chunks;
            for (int i = threadIdx.x; i < n; i += T::THREADS)
                const_cast<int32_t*>(p.plan)[i] = ((const LDS_AS int32_t*)lplan)[i];
        }
    }
    auto pl = [&](int idx) {
        return __builtin_amdgcn_readfirstlane(lds_plan ? ((const LDS_AS int32_t*)lplan)[idx] : p.plan[idx]);
    };
    auto pl_cu = [&](int row) { return pl(4 + row); };
    auto pl_base = [&](int row) { return pl(4 + (p.b + 1) + row); };
    auto pl_nsplit = [&](int row) { return pl(4 + (p.b + 1) + p.b + row); };
    auto plan_duties = [&]() {
        if (!lds_plan) return;
        zero_empty_rows([&](int row) { return pl_cu(row + 1) - pl_cu(row); }, p.b, p.h, (__bf16*)p.out, p.lse,
                        blockIdx.x, gridDim.x, threadIdx.x, T::THREADS);
    };
    const int total = pl(0);
    const int chunk = pl(1);
    int r = pl(4 + (p.b + 1) + 2 * p.b + k);
    if (r < 0) {
        plan_duties();
        return;
    }
    int pos = k * chunk;
    const int end = pos + min(chunk, total - pos);

    const __bf16* __restrict__ qg = (const __bf16*)p.q;
    const unsigned char* __restrict__ cg = (const unsigned char*)p.cache;
    const int head = hg * T::HG + wave * 32 + hl;
    const bool head_ok = head < p.h;
    const float c2 = p.scale_log2;

    // ---- per-lane LDS offsets --------------------------------------------
    // Scores, step j < 8: row rr = lane & 31, chunks 4j + 2grp and 4j + 2grp + 1
    // (channels 64j + 32grp .. +31, the A operand's 32 bytes).  With
    // u = 2grp ^ sw8(rr) the first sits at chunk position 4j ^ u, i.e. for
    // j = 4a + b at rr*512 + 16(u & 3) + 64(b ^ (u >> 2)) + 256a, and the
    // second at that position ^ 1.
    // The offsets are recomputed where they are used, from a thread index
    // the compiler cannot see through, so that none of them stays live across
    // the tile loop (every register is taken there).
    auto opaque_lane = [&]() {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        return t & 63;
    };
    struct KOffsets {
        int koff[4], kflip, kb0, kb1, soff;
    };
    auto k_offsets = [&]() {
        KOffsets o;
        const int l = opaque_lane();
        const int rr = l & 31, g = l >> 5;
        const int ku = (2 * g) ^ sw8(rr);
#pragma unroll
        for (int b = 0; b < 4; ++b) o.koff[b] = rr * 512 + 16 * (ku & 3) + 64 * (b ^ (ku >> 2));
        o.kflip = (ku & 1) ? -16 : 16;
        // Step 8 (channels 512..575): region B, chunk c of row r at c ^ ((r >> 2) & 3).
        o.kb0 = T::B_OFF + rr * 64 + 16 * ((2 * g) ^ ((rr >> 2) & 3));
        o.kb1 = T::B_OFF + rr * 64 + 16 * ((2 * g + 1) ^ ((rr >> 2) & 3));
        // Token scales of the lane's accumulator entries (tokens 8q + 4g .. +3).
        o.soff = T::SCL_OFF + 16 * g;
        return o;
    };
    // Weighted sum: ds_read_b64_tr_b8 hands output lane i of a 16-lane group
    // byte i % 8 of source lanes 2e + i / 8 (e = 0..7), so source lane pair e
    // supplies the 16 bytes of k slot e.  Group G = lane >> 4 builds the A
    // operand of columns 32mb + 16(G & 1) .. +15 and k slots 8(G >> 1) .. +7,
    // whose tokens follow the P^T layout (k slot e of group half g: token
    // 8(e >> 2) + 4g + (e & 3), +16 for the tile's second half): source lane s
    // reads token t0 = 8(e >> 2) + 4(G >> 1) + (e & 3), e = s >> 1, channels
    // 32mb + 16(G & 1) + 8(s & 1) .. +7, i.e. chunk 2mb + (G & 1) at position
    // 2mb ^ w, w = (G & 1) ^ sw8(t0): for mb = 8a + b at
    // t0*512 + 16(w & 1) + 8(s & 1) + 32(b ^ (w >> 1)) + 256a (+8192 for the
    // second half).
    struct VOffsets {
        int voff[8];
    };
    auto v_offsets = [&]() {
        VOffsets o;
        const int l = opaque_lane();
        const int G = l >> 4, sl = l & 15, e = sl >> 1;
        const int t0 = 8 * (e >> 2) + 4 * (G >> 1) + (e & 3);
        const int w = (G & 1) ^ sw8(t0);
#pragma unroll
        for (int b = 0; b < 8; ++b) o.voff[b] = t0 * 512 + 16 * (w & 1) + 8 * (sl & 1) + 32 * (b ^ (w >> 1));
        return o;
    };

    while (true) {
        const int row_lo = pl_cu(r);
        const int row_hi = pl_cu(r + 1);
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        const int seg_len = seg_end - pos;
        const int split_j = k - row_lo / chunk;
        const bool final_out = pl_nsplit(r) == 1;
        const int slot = pl_base(r) + split_j;
        const unsigned char* seg_base = cg + ((size_t)r * p.t_max + seg_a) * T::ROW8;
        const float* seg_scale = p.cache_scale + (size_t)r * p.t_max + seg_a;
        const int n_tiles = (seg_len + T::N - 1) / T::N;

        // DMA instruction `li` (0 .. LOADS-1) of this wave's share of `tile`
        // into stage SC.  Rows past the segment end re-read its last row
        // (their scores are masked), so every code access stays inside the
        // segment; scales past the end read as 0 (outside the resource).  A
        // tile past the last one gets an empty resource: the instructions
        // are still issued (zeros land in a free stage, no memory is read),
        // so every step issues the same DMA count and the compiler's own
        // waits need not assume a shorter queue.
        auto issue_load = [&](auto SC, int tile, int li) {
            const int t0 = tile * T::N;
            // uniform (a scalar value: a resource built from a vector register
            // would need a loop over lanes)
            const int last = __builtin_amdgcn_readfirstlane((tile < n_tiles ? min(T::N, seg_len - t0) : 0) - 1);
            lds_byte* st = stage_lds<T::TILE_BYTES, decltype(SC)::value>();
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(seg_base + (size_t)t0 * T::ROW8), (short)0, (last + 1) * T::ROW8, kBufferFlags);
            const int ln = opaque_lane();
            if (li < T::LOADS_A) {
                // rows 2q, 2q + 1 (lanes 0..31, 32..63); lane position l & 31
                // holds logical chunk (l & 31) ^ sw8(row)
                const int q = wave + li * T::NW;
                const int row = 2 * q + (ln >> 5);
                const int srow = min(row, last);
                const int c = (ln & 31) ^ sw8(row);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(st + q * 1024), 16,
                                                         (unsigned)(srow * T::ROW8 + c * 16), 0, 0, 0);
            } else if (li == T::LOADS_A) {
                // region B rows 16 bw .. +15, bw = wave & 1: lane -> row
                // 16 bw + l / 4, position l % 4 (waves 2 and 3 write the same
                // bytes as waves 0 and 1)
                const int bw = wave & 1;
                const int row = 16 * bw + (ln >> 2);
                const int srow = min(row, last);
                const int c = (ln & 3) ^ ((row >> 2) & 3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(st + T::B_OFF + bw * 1024), 16,
                                                         (unsigned)(srow * T::ROW8 + 512 + c * 16), 0, 0, 0);
            } else {
                // the tile's scales, 4 bytes per lane (dword bounds checks:
                // tokens past the segment end read 0; lanes 32..63 fill the
                // unused rest of the scale area); every wave writes the same
                // bytes.  Every wave thus issues the same instruction kinds
                // in the same order: with a wave-dependent choice between the
                // region-B and the scale DMA here, the compiler drained the
                // whole ring before the first stage's scale reads.
                const __amdgpu_buffer_rsrc_t rsc = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(seg_scale + t0), (short)0, (last + 1) * 4, kBufferFlags);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rsc, (LDS_AS void*)(st + T::SCL_OFF), 4,
                                                         (unsigned)(ln * 4), 0, 0, 0);
            }
        };
        auto issue_tile = [&](auto SC, int tile) {
#pragma unroll
            for (int li = 0; li < T::LOADS; ++li) issue_load(SC, tile, li);
        };
        // Wait until this wave's share of tile t has landed: tiles t+1 ..
        // t+STAGES-2 (real or empty) were issued after it.
        auto wait_tile = [&]() { wait_vmcnt<(STAGES - 2) * T::LOADS>(); };

        // Queries first (bf16, lane -> head hl, channels 64j + 32grp .. +31 of
        // step j), then the first STAGES-1 tiles, which land while the
        // queries are quantised.  A lane past the last head reads head 0.
        bf16x8_t qb[4 * T::KS];
        {
            const bf16x8_t* qrow = (const bf16x8_t*)(qg + ((size_t)r * p.h + (head_ok ? head : 0)) * kDqk);
#pragma unroll
            for (int j = 0; j < T::KS; ++j)
#pragma unroll
                for (int v = 0; v < 4; ++v) qb[4 * j + v] = qrow[8 * j + 4 * grp + v];
        }
        issue_tile(IC<0>{}, 0);
        issue_tile(IC<1>{}, 1);
        if (STAGES > 3) issue_tile(IC<(STAGES > 3 ? 2 : 0)>{}, 2);
        if (STAGES > 4) issue_tile(IC<(STAGES > 4 ? 3 : 0)>{}, 3);
        if (STAGES > 5) issue_tile(IC<(STAGES > 5 ? 4 : 0)>{}, 4);

        // Quantise: the head's max |q'| over its 576 channels (this lane holds
        // half of them, the lane 32 away the other half).
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 4 * T::KS; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qb[i][e]));
        amax = max_xor32(amax);
        const float inv = amax > 0.f ? kE4m3Max / amax : 0.f;
        const float sigma = amax / kE4m3Max;
        i32x8_t q8[T::KS];
#pragma unroll
        for (int j = 0; j < T::KS; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int h2 = 0; h2 < 2; ++h2) {
                    float x[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        x[e] = fminf(fmaxf((float)qb[4 * j + v][4 * h2 + e] * inv, -kE4m3Max), kE4m3Max);
                    q8[j][2 * v + h2] = pack4_e4m3(x[0], x[1], x[2], x[3]);
                }
        const float c2s = c2 * sigma;  // log2-domain factor of a code product, before the token scale

        // outputs: zero blocks pinned one by one in AGPRs (left alone the
        // compiler feeds one shared zero block to every first MFMA)
        acc_t o[T::MBLK];
#pragma unroll
        for (int mb = 0; mb < T::MBLK; ++mb) {
            o[mb] = (acc_t){};
            asm volatile("" : "+a"(o[mb]));
        }
        int one = 127;  // E8M0 unit scale of the score MFMAs, in a VGPR
        asm volatile("" : "+v"(one));
        float m_run = kNegBig;
        float l_run = 0.f;

        // One tile: tile index i in stage SC.
        auto step = [&](auto SC, int i) {
            constexpr int S = decltype(SC)::value;
            constexpr int SR = (S + STAGES - 1) % STAGES;  // stage of tile i-1 = refill target
            lds_byte* tb = stage_lds<T::TILE_BYTES, S>();
            wait_tile();
            lds_exchange_barrier();  // tile i visible to all; everyone is done with tile i-1

            const KOffsets ko = k_offsets();
            f32x4_t sc[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) sc[q] = *(const LDS_AS f32x4_t*)(tb + ko.soff + 32 * q);

            // ---- scores: S^T = K . Q'^T on the FP8 cores, the refill DMA of
            // tile i+STAGES-1 spread over the first steps
            acc_t sacc;
            auto k_frag = [&](int j) -> i32x8_t {
                i32x4_t lo, hi;
                if (j < 8) {
                    const int o0 = ko.koff[j & 3] + 256 * (j >> 2);
                    lo = *(const LDS_AS i32x4_t*)(tb + o0);
                    hi = *(const LDS_AS i32x4_t*)(tb + o0 + ko.kflip);
                } else {
                    lo = *(const LDS_AS i32x4_t*)(tb + ko.kb0);
                    hi = *(const LDS_AS i32x4_t*)(tb + ko.kb1);
                }
                return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            };
            {
                constexpr int PF = 2;
                i32x8_t kring[PF];
#pragma unroll
                for (int j = 0; j < PF; ++j) kring[j] = k_frag(j);
#pragma unroll
                for (int j = 0; j < T::KS; ++j) {
                    const i32x8_t kf = kring[j % PF];
                    if (j + PF < T::KS) kring[j % PF] = k_frag(j + PF);
                    if (j == 0)
                        sacc = score8_first(kf, q8[0], one);
                    else
                        score8_acc(sacc, kf, q8[j], one);
                    if (j < T::LOADS) issue_load(IC<SR>{}, i + STAGES - 1, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
                score8_wait(sacc);
            }

            // ---- online softmax; sacc[e]: token (e/4)*8 + 4grp + e%4, head hl
            float x[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) x[e] = sacc[e] * (c2s * sc[e >> 2][e & 3]);
            const int tvalid = __builtin_amdgcn_readfirstlane(seg_len - i * T::N);
            if (tvalid < T::N) {
                const int lim = tvalid - 4 * grp;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if ((e >> 2) * 8 + (e & 3) >= lim) x[e] = -INFINITY;
            }
            float tm = fmaxf(fmaxf(x[0], x[1]), x[2]);
#pragma unroll
            for (int e = 3; e < 16; ++e) tm = fmaxf(tm, x[e]);
            const float tmax = max_xor32(tm);
            const float m_new = fmaxf(m_run, tmax);
            if (i == 0) {
                m_run = m_new;  // first tile: nothing accumulated yet
            } else if (__any(m_new > m_run + kRescaleThreshold)) {
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
                // one accumulator block at a time through VGPRs (the empty asm
                // statements keep the compiler from moving all of them at once)
#pragma unroll
                for (int mb = 0; mb < T::MBLK; ++mb) {
                    acc_t t = o[mb];
                    asm volatile("" : "+v"(t));
                    t *= alpha;
                    asm volatile("" : "+a"(t));
                    o[mb] = t;
                }
                m_run = m_new;
            }
            // P^T entries bf16(p * s_t): the first 16 tokens now, the second
            // 16 between the first weighted-sum MFMAs
            bf16x8_t pb[2];
            auto prob = [&](int e) {
                const float pe = exp2_fast(x[e] - m_run);
                l_run += pe;
                pb[e >> 3][e & 7] = (__bf16)(pe * sc[e >> 2][e & 3]);
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) prob(e);

            // ---- weighted sum: O^T += V^T . P^T (codes converted to bf16)
            constexpr int NPV = 2 * T::MBLK;
            constexpr int PFV = 4;
            const VOffsets vo = v_offsets();
            auto v_frag = [&](int idx) -> i32x2_t {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (LDS_AS i32x2_t*)(tb + vo.voff[mb & 7] + 8192 * u + 256 * (mb >> 3)));
            };
            i32x2_t vring[PFV];
#pragma unroll
            for (int j = 0; j < PFV; ++j) vring[j] = v_frag(j);
#pragma unroll
            for (int idx = 0; idx < NPV; ++idx) {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                const bf16x8_t a = cvt8_e4m3(__builtin_bit_cast(unsigned long long, vring[idx % PFV]));
                if (idx + PFV < NPV) vring[idx % PFV] = v_frag(idx + PFV);
                o[mb] = M::mma(a, pb[u], o[mb]);
                if (idx < 8) prob(8 + idx);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // The steps form one chain (each reachable only from the one before),
        // so the compiler's own DMA bookkeeping sees the same queue on every
        // path into a step and adds no wait of its own.  n_tiles >= 1.
        for (int i0 = 0;; i0 += STAGES) {
            step(IC<0>{}, i0);
            if (i0 + 1 >= n_tiles) break;
            step(IC<1>{}, i0 + 1);
            if (i0 + 2 >= n_tiles) break;
            if constexpr (STAGES > 2) {
                step(IC<(STAGES > 2 ? 2 : 0)>{}, i0 + 2);
                if (i0 + 3 >= n_tiles) break;
            }
            if constexpr (STAGES > 3) {
                step(IC<(STAGES > 3 ? 3 : 0)>{}, i0 + 3);
                if (i0 + 4 >= n_tiles) break;
            }
            if constexpr (STAGES > 4) {
                step(IC<(STAGES > 4 ? 4 : 0)>{}, i0 + 4);
                if (i0 + 5 >= n_tiles) break;
            }
            if constexpr (STAGES > 5) {
                step(IC<(STAGES > 5 ? 5 : 0)>{}, i0 + 5);
                if (i0 + 6 >= n_tiles) break;
            }
        }

        // ---- segment epilogue ----------------------------------------------
        // A row finished here writes out/lse; otherwise its slot's partial
        // (normalised, bf16) and partial lse.  Each wave stages half of its
        // 32 x 512 outputs at a time in its own ring stage (free once every
        // wave is past the last tile) and stores whole 512-byte half rows.
        l_run += __shfl_xor(l_run, 32, 64);
        wait_vmcnt<0>();         // the empty refills past the last tile have landed
        lds_exchange_barrier();
        {
            // head and column group from the (opaque) thread index again, not
            // kept live across the tile loop
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int e_lane = tid & 63;
            const int e_grp = (tid >> 5) & 1;
            const int e_hl = tid & 31;
            const int head0 = hg * T::HG + wave * 32;
            const float inv_l = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2f : -INFINITY;
            __bf16* obase = (final_out ? (__bf16*)p.out + (size_t)r * p.h * kDc
                                       : (__bf16*)p.po + (size_t)slot * p.h * kDc) + (size_t)head0 * kDc;
            lds_byte* stg = wave == 0   ? stage_lds<T::TILE_BYTES, 0>()
                            : wave == 1 ? stage_lds<T::TILE_BYTES, 1>()
                            : wave == 2 ? stage_lds<T::TILE_BYTES, 2>()
                                        : stage_lds<T::TILE_BYTES, 3>();
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // accumulator entry e of block mb: column 32mb + (e/4)*8 + 4grp + e%4
#pragma unroll
                for (int mb = half * T::MBLK / 2; mb < (half + 1) * T::MBLK / 2; ++mb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        bf16x4_t v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[mb][q4 * 4 + e] * inv_l);
                        const int col = (mb - half * T::MBLK / 2) * 32 + q4 * 8 + e_grp * 4;
                        *(LDS_AS bf16x4_t*)(stg + e_hl * T::STG_ROW + 2 * col) = v;
                    }
                // a wave's LDS accesses complete in order: the reads below see
                // the writes above, and the next half's writes follow these reads
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 2 * i + (e_lane >> 5);
                    const bf16x8_t v = *(const LDS_AS bf16x8_t*)(stg + row * T::STG_ROW + 16 * e_hl);
                    if (head0 + row < p.h)
                        *(bf16x8_t*)(obase + (size_t)row * kDc + half * (kDc / 2) + 8 * e_hl) = v;
                }
            }
            if (e_grp == 0 && head0 + e_hl < p.h)
                (final_out ? p.lse + (size_t)r * p.h : p.plse + (size_t)slot * p.h)[head0 + e_hl] = lse_v;
        }

        pos = seg_end;
        if (pos >= end) break;
        wg_barrier();  // every wave is done with the stages before they are refilled
        ++r;
        while (pl_cu(r + 1) <= pos) ++r;
    }
    plan_duties();
}

constexpr int kF8Stages = 4;

__global__ __launch_bounds__(256) void decode_wide_fp8_kernel(DecodeParams p)
{
    clock_stamp(p.clock_stamps, 0);
    decode_wide_fp8_body<kF8Stages>(p);
    clock_stamp(p.clock_stamps, 1);
}

}  // namespace

hipError_t launch_decode_wide_fp8(const DecodeParams& p, hipStream_t stream)
{
    using T = WideF8Tiling<kF8Stages>;
    if (p.plan_in_kernel && (p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks))
        return hipErrorInvalidValue;  // no room for the plan in this kernel's LDS
    if (p.cache_scale == nullptr || p.block_table != nullptr || p.q_len != 1) return hipErrorInvalidValue;
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    decode_wide_fp8_kernel<<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace mla355
