// Split-KV absorbed-MLA decode, bf16 in / fp32 accumulate, for groups of 128
// heads: the column-split, software-pipelined kernel.
//
// Same operation, plan and partial format as the other bf16 kernels (the
// glossary page "Multi-head Latent Attention", section on why decode absorbs
// the matrices: absorbed query heads score directly against the shared latent
// rows, and the softmax-weighted sum of the c_KV parts is the output; its
// capacity-and-cost section: online softmax applies once the score parts are
// summed).
//
// One workgroup = 4 waves = one token chunk x 128 heads.  The work of a tile
// of 32 latent rows is split two ways:
//  * scores: wave w owns heads 32w .. 32w+31.  Their 576-wide queries stay in
//    VGPRs (the B operand of v_mfma_f32_32x32x16_bf16), the tile rows are the
//    A operand (ds_read_b128), and the online softmax of those heads is
//    lane-local (one head per lane, one cross-lane step for the tile max);
//  * weighted sum: wave w owns output columns 128w .. 128w+127 of all 128
//    heads (16 accumulator blocks of 32 columns x 32 heads, 256 AGPRs).  Its
//    A operand is a 32-column strip of the tile read transposed
//    (ds_read_b64_tr_b16), used for four MFMAs (four head groups): each latent
//    value is read from LDS once per workgroup for the weighted sum instead of
//    once per wave.  Its B operand, the probabilities of all 128 heads, comes
//    from LDS, where each wave leaves its own heads' probabilities in the
//    exact register layout of that operand (conflict-free 16-byte reads).
//
// Pipelining.  Iteration i consumes tile i's weighted sum and tile i+1's
// scores: the 36 score MFMAs of tile i+1 are interleaved with the first 16
// weighted-sum MFMAs of tile i (two independent accumulator chains, so the
// score chain never waits on its own result), and the softmax of tile i+1
// runs on the vector ALU between the last 16 weighted-sum MFMAs of tile i.
// The probabilities of tile i+1 (and, when a head's running max grew past
// the lazy-rescale threshold, its rescale factor) go to LDS; one barrier per
// tile then publishes them, the landed tile i+2, and the release of tile i's
// stage.  Tiles stream HBM -> LDS by direct-to-LDS DMA in a 3-stage ring
// (tile i+2 in flight while tiles i and i+1 are read), with the LDS layout of
// the wide-wave kernel (region A rows rotated inside 128 bytes of padding,
// region B swizzled).
//
// Rescaling.  The running max of a head lives with its score wave; when it
// grows by more than 2^8 the wave writes the factor exp2(m_old - m_new) for
// that head, and every wave multiplies its 4 column blocks of that head's
// group by it before adding the next tile.  The final normalisation divides
// by the running sum of the same maxima, so the result is exact.
#include "bf16_common.h"
#include "plan_build.h"

#include <math.h>

namespace mla355 {
namespace {

constexpr float kLn2c = 0.69314718055994531f;

// Chunk rotation of region-A row r (as in the wide-wave kernel).
__device__ __forceinline__ int rot16c(int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); }

struct ColTiling {
    static constexpr int NW = 4;
    static constexpr int THREADS = NW * 64;
    static constexpr int HG = 128;                     // heads per workgroup
    static constexpr int STAGES = 3;
    static constexpr int N = 32;                       // tokens per tile
    static constexpr int ROW_A = 1024 + 128;           // LDS stride of a region-A row (rotated)
    static constexpr int A_BYTES = N * ROW_A;
    static constexpr int TILE_BYTES = A_BYTES + N * 128;
    static constexpr int LOADS_A = N / NW;             // region-A DMA instructions per wave
    static constexpr int LOADS_B = (N / 8) / NW;       // region-B DMA instructions per wave
    static constexpr int LOADS = LOADS_A + LOADS_B;
    static constexpr int KS = kDqk / 16;               // 36 score k-steps
    static constexpr int KSA = kDc / 16;               // 32 of them in region A
    static constexpr int CB = 4;                       // 32-column blocks per wave (128 columns)
    static constexpr int G = 4;                        // head groups of 32
    // probabilities: [buffer 2][writer wave 4][token half 2][lane 64] x 16 B
    static constexpr int P_BYTES = 2 * NW * 2 * 64 * 16;
    // rescale factors [buffer 2][group 4][32] fp32, then flags [buffer 2][group 4] int
    static constexpr int A_OFF_FLAGS = 2 * G * 32 * 4;
    static constexpr int AUX_BYTES = A_OFF_FLAGS + 2 * G * 4;
    // epilogue: 1/l and lse of the 128 heads
    static constexpr int EPI_BYTES = 2 * HG * 4;
    // epilogue staging: 64 rows (heads) of 128 outputs (bf16) per wave, rows
    // padded by 16 B
    static constexpr int STG_ROW = 256 + 16;
    static_assert(2 * 64 * STG_ROW <= TILE_BYTES, "epilogue staging: two waves per ring stage");
    static_assert((N / 8) % NW == 0, "region-B groups split evenly over waves");
    static_assert(LOADS <= KS, "refill spread over the score steps");
    static_assert(STAGES * TILE_BYTES + P_BYTES + AUX_BYTES + EPI_BYTES + kPlanLdsInts * 4 <= 160 * 1024,
                  "LDS budget");
};

typedef const __attribute__((address_space(4))) int32_t cint32c_t;

template <bool PAGED>
__device__ __forceinline__ void colsplit_body(const DecodeParams& p)
{
    using T = ColTiling;
    using M = Mfma<32>;
    typedef f32x16_t acc_t;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31;    // head inside a group of 32
    const int grp = lane >> 5;   // k-slot group (0/1) of the MFMA operand layouts

    int k, hg;
    block_work(p.n_chunks, p.n_hg, k, hg);
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
    auto seqlen_of = [&](int row) { return __builtin_amdgcn_readfirstlane(p.seqlens[row]); };
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
    const int head = hg * T::HG + wave * 32 + hl;   // this lane's score head
    const bool head_ok = head < p.h;
    const float c2 = p.scale_log2;

    lds_byte* const pbuf = stage_lds<T::P_BYTES, 8>();
    lds_byte* const aux = stage_lds<T::AUX_BYTES, 9>();
    lds_byte* const epi = stage_lds<T::EPI_BYTES, 10>();

    // Per-lane LDS offsets (layout as in the wide-wave kernel).  They are
    // derived where they are used from an opaque copy of the thread index, so
    // the compiler recomputes them (a few integer ops) instead of keeping them
    // live across the tile loop, where every register is taken.
    // The transposed-read offset is the exception: computed once, because a
    // transposed read whose address derives from the opaque value loses track
    // of which LDS array it reads, and the compiler then waits for every tile
    // DMA in flight before it.
    int vA;
    {
        const int row0 = grp * 4 + ((lane & 15) >> 2);
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        vA = row0 * T::ROW_A + 16 * (cc + rot16c(row0)) + ((lane & 1) << 3) + 256 * wave;
    }
    struct LaneOffs {
        int lane, kA, kB;
    };
    auto lane_offs = [&]() {
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        LaneOffs lo;
        lo.lane = tid & 63;
        const int g2 = lo.lane >> 5;
        const int rr = lo.lane & 31;
        lo.kA = rr * T::ROW_A + 16 * (g2 + rot16c(rr));
        const int xbv = xb(rr & 15);
        lo.kB = T::A_BYTES + rr * 128 + 32 * (xbv >> 1) + 16 * (g2 ^ (xbv & 1));
        return lo;
    };

    while (true) {
        const int row_lo = pl_cu(r);
        const int row_hi = pl_cu(r + 1);
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        int seg_len = seg_end - pos;
        if (PAGED) {
            const int L = min(max(seqlen_of(r), 0), p.t_max);
            seg_len = max(0, min(seg_len, L - seg_a));
        }
        const int split_j = k - row_lo / chunk;
        const bool final_out = pl_nsplit(r) == 1;
        const int slot = pl_base(r) + split_j;
        const unsigned char* seg_base = cg + ((size_t)r * p.t_max + seg_a) * kRowBytesBf16;
        const int n_tiles = (seg_len + T::N - 1) / T::N;

        int pg_blk = 0, pg_off = 0;
        if (PAGED) {
            pg_blk = seg_a / p.block_size;
            pg_off = seg_a - pg_blk * p.block_size;
        }
        // global address of the next tile (tiles are requested once each, in order)
        auto tile_ptr = [&](int tile) -> const unsigned char* {
            if (!PAGED) return seg_base + (size_t)tile * T::N * kRowBytesBf16;
            const int e = min(max(*(cint32c_t*)(p.block_table + (size_t)r * p.max_blocks + pg_blk), 0),
                              p.num_blocks - 1);
            const unsigned char* a = cg + ((size_t)e * p.block_size + pg_off) * kRowBytesBf16;
            pg_off += T::N;
            if (pg_off == p.block_size) {
                pg_off = 0;
                ++pg_blk;
            }
            return a;
        };
        // DMA instruction li of this wave's share of `tile` into stage SC;
        // rows past the segment end re-read its last row (masked scores).
        auto issue_load = [&](auto SC, const LaneOffs& lo, const unsigned char* tptr, int tile, int li) {
            const int lane = lo.lane;
            const int t0 = tile * T::N;
            const int last = min(T::N, seg_len - t0) - 1;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)tptr, (short)0, (last + 1) * kRowBytesBf16, kBufferFlags);
            lds_byte* st = stage_lds<T::TILE_BYTES, decltype(SC)::value>();
            if (li < T::LOADS_A) {
                const int row = wave + li * T::NW;
                const int srow = min(row, last);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + row * T::ROW_A + 16 * rot16c(row)), 16, (unsigned)lane << 4,
                    __builtin_amdgcn_readfirstlane(srow * kRowBytesBf16), 0, 0);
            } else {
                const int gb = wave + (li - T::LOADS_A) * T::NW;
                const int row = gb * 8 + (lane >> 3);
                const int srow = min(row, last);
                const int lc = (lane & 7) ^ xb(row & 15);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + T::A_BYTES + gb * 1024), 16,
                    (unsigned)(srow * kRowBytesBf16 + 1024 + lc * 16), 0, 0, 0);
            }
        };
        auto issue_tile = [&](auto SC, const LaneOffs& lo, int tile) {
            const unsigned char* tp = tile_ptr(tile);
#pragma unroll
            for (int li = 0; li < T::LOADS; ++li) issue_load(SC, lo, tp, tile, li);
        };

        auto k_frag = [&](const LaneOffs& lo, lds_byte* tb, int j) -> bf16x8_t {
            const lds_byte* a = (j < T::KSA) ? tb + lo.kA + 32 * j : tb + (lo.kB ^ ((j - T::KSA) << 5));
            return *(const LDS_AS bf16x8_t*)a;
        };
        // transposed V fragment: token half u, column block cb of this wave's 128
        auto v_frag = [&](const LaneOffs& lo, lds_byte* tb, int u, int cb) -> bf16x8_t {
            const int blk = 64 * cb + u * 16 * T::ROW_A;
            // this wave's 128 columns start 256 bytes in per wave (in vA)
            const i16x4_t v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + vA + blk));
            const i16x4_t v1 =
                __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + vA + blk + 8 * T::ROW_A + 32));
            return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, v0), __builtin_bit_cast(bf16x4_t, v1),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        };
        // probabilities of head group g, token half u, from buffer b
        auto p_frag = [&](const LaneOffs& lo, int b, int g, int u) -> bf16x8_t {
            return *(const LDS_AS bf16x8_t*)(pbuf + (((b * T::NW + g) * 2 + u) * 64 + lo.lane) * 16);
        };

        // Tile 0 first, then the queries (B operand; lane -> head hl,
        // channels 16j + 8grp .. +7 of step j; a lane past the last head reads
        // head 0's), then tile 1.
        const LaneOffs lo0 = lane_offs();
        if (0 < n_tiles) issue_tile(IC<0>{}, lo0, 0);
        bf16x8_t qf[T::KS];
        {
            const bf16x8_t* qrow = (const bf16x8_t*)(qg + ((size_t)r * p.h + (head_ok ? head : 0)) * kDqk);
#pragma unroll
            for (int j = 0; j < T::KS; ++j) qf[j] = qrow[2 * j + grp];
        }
        if (1 < n_tiles) issue_tile(IC<1>{}, lo0, 1);

        acc_t o[T::CB][T::G];
#pragma unroll
        for (int cb = 0; cb < T::CB; ++cb)
#pragma unroll
            for (int g = 0; g < T::G; ++g) {
                o[cb][g] = (acc_t){};
                // a distinct accumulator per block from here on (left to
                // itself the compiler feeds one shared zero block to every
                // first MFMA, which needs 16 AGPRs more than there are)
                asm volatile("" : "+a"(o[cb][g]));
            }
        float m_run = kNegBig;
        float l_run = 0.f;

        // Softmax of the score tile s (tile index t, tokens valid: tvalid),
        // in pieces 0..11 so that they can sit between MFMAs; writes the
        // probabilities (and the rescale factor and flag) of buffer b.
        // s[e]: token (e/4)*8 + 4grp + e%4, head hl.
        struct SmState {
            float tmax, mnew;
            bf16x8_t pb[2];
        };
        auto sm_piece = [&](const LaneOffs& lo, acc_t& s, SmState& st, int t, int b, int piece) {
            const int lane = lo.lane, hl = lane & 31, grp = lane >> 5;
            float& sm_tmax = st.tmax;
            float& sm_mnew = st.mnew;
            bf16x8_t(&pb)[2] = st.pb;
            if (piece == 0) {
                const int tvalid = __builtin_amdgcn_readfirstlane(seg_len - t * T::N);
                if (tvalid < T::N) {
                    const int lim = tvalid - 4 * grp;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if ((e >> 2) * 8 + (e & 3) >= lim) s[e] = -INFINITY;
                }
                float tm = fmaxf(fmaxf(s[0], s[1]), s[2]);
#pragma unroll
                for (int e = 3; e < 16; ++e) tm = fmaxf(tm, s[e]);
                sm_tmax = tm;
            } else if (piece == 1) {
                sm_tmax = max_xor32(sm_tmax) * c2;
                sm_mnew = fmaxf(m_run, sm_tmax);
            } else if (piece == 2) {
                int sm_flag = 0;
                if (t == 0) {
                    m_run = sm_mnew;  // first tile: nothing accumulated yet
                } else if (__any(sm_mnew > m_run + kRescaleThreshold)) {
                    const float alpha = exp2_fast(m_run - sm_mnew);
                    l_run *= alpha;
                    m_run = sm_mnew;
                    if (grp == 0) *(LDS_AS float*)(aux + ((b * T::G + wave) * 32 + hl) * 4) = alpha;
                    sm_flag = 1;
                }
                if (lane == 0) *(LDS_AS int*)(aux + T::A_OFF_FLAGS + (b * T::G + wave) * 4) = sm_flag;
            } else if (piece < 11) {
                // pieces 3..10: two probabilities each
                const int e0 = 2 * (piece - 3);
#pragma unroll
                for (int e = e0; e < e0 + 2; ++e) {
                    const float x = exp2_fast(__builtin_fmaf(s[e], c2, -m_run));
                    l_run += x;
                    pb[e >> 3][e & 7] = (__bf16)x;
                }
            } else {
                // piece 11: publish this wave's probabilities in the B-operand layout
#pragma unroll
                for (int u = 0; u < 2; ++u)
                    *(LDS_AS bf16x8_t*)(pbuf + (((b * T::NW + wave) * 2 + u) * 64 + lane) * 16) = pb[u];
            }
        };

        // Rescale the accumulator blocks of the head groups flagged in buffer b
        // (factor 1 for the others).
        auto apply_rescale = [&](const LaneOffs& lo, int b) {
            const int hl = lo.lane & 31;
            typedef int i32x4_t __attribute__((ext_vector_type(4)));
            const i32x4_t f = *(const LDS_AS i32x4_t*)(aux + T::A_OFF_FLAGS + b * T::G * 4);
            if (__builtin_amdgcn_readfirstlane(f[0] | f[1] | f[2] | f[3]) == 0) return;
#pragma unroll
            for (int g = 0; g < T::G; ++g) {
                const float a = f[g] ? *(const LDS_AS float*)(aux + ((b * T::G + g) * 32 + hl) * 4) : 1.0f;
#pragma unroll
                for (int cb = 0; cb < T::CB; ++cb) {
                    // the copy used for the multiply is pinned to VGPRs and the
                    // result back to AGPRs, one block at a time
                    acc_t x = o[cb][g];
                    asm volatile("" : "+v"(x));
                    x *= a;
                    asm volatile("" : "+a"(x));
                    o[cb][g] = x;
                }
            }
        };

        // ---- prologue: scores and softmax of tile 0 -------------------------
        if (n_tiles > 0) {
            if (1 < n_tiles)
                wait_vmcnt<T::LOADS>();  // tile 0 and the queries (tile 1 may still be in flight)
            else
                wait_vmcnt<0>();
            lds_exchange_barrier();
            lds_byte* tb = stage_lds<T::TILE_BYTES, 0>();
            constexpr int PF = 4;
            bf16x8_t kring[PF];
            const LaneOffs lo = lane_offs();
#pragma unroll
            for (int j = 0; j < PF; ++j) kring[j] = k_frag(lo, tb, j);
            acc_t s0;
#pragma unroll
            for (int j = 0; j < T::KS; ++j) {
                const bf16x8_t kf = kring[j % PF];
                if (j + PF < T::KS) kring[j % PF] = k_frag(lo, tb, j + PF);
                if (j == 0)
                    s0 = score_first(kf, qf[0]);
                else
                    score_acc(s0, kf, qf[j]);
                __builtin_amdgcn_sched_barrier(0);
            }
            score_wait(s0);
            SmState st;
#pragma unroll
            for (int piece = 0; piece < 12; ++piece) sm_piece(lo, s0, st, 0, 0, piece);
        }

        // ---- iteration i: scores of tile i+1, then the weighted sum of tile i
        // with the softmax of tile i+1 between its MFMAs.  On the last tile
        // the score MFMAs are skipped and the softmax sees a fully masked
        // tile, which leaves its state unchanged: every weighted-sum MFMA
        // stays on one code path (a second path would need a second
        // placement of the 256 accumulators).
        auto iter = [&](auto SC, int i) {
            constexpr int S = decltype(SC)::value;           // stage of tile i
            constexpr int SN = (S + 1) % T::STAGES;          // stage of tile i+1
            constexpr int SR = (S + 2) % T::STAGES;          // stage of tile i+2 (refill)
            lds_byte* tc = stage_lds<T::TILE_BYTES, S>();
            lds_byte* tn = stage_lds<T::TILE_BYTES, SN>();
            const bool has_next = i + 1 < n_tiles;
            const bool refill = i + 2 < n_tiles;
            const int b = i & 1;
            const unsigned char* rptr = refill ? tile_ptr(i + 2) : nullptr;
            wait_vmcnt<0>();          // tile i+1 (the only DMA in flight) has landed
            lds_exchange_barrier();   // tile i+1 and P(i) visible; tile i-1's stage free
            const LaneOffs lo = lane_offs();
            apply_rescale(lo, b);

            // scores of tile i+1 (refill DMA spread over the first steps)
            auto scores = [&](auto RF) {
                constexpr bool REFILL = decltype(RF)::value != 0;
                constexpr int PF = 4;
                bf16x8_t kring[PF];
#pragma unroll
                for (int j = 0; j < PF; ++j) kring[j] = k_frag(lo, tn, j);
                acc_t sacc;
#pragma unroll
                for (int j = 0; j < T::KS; ++j) {
                    const bf16x8_t kf = kring[j % PF];
                    if (j + PF < T::KS) kring[j % PF] = k_frag(lo, tn, j + PF);
                    if (j == 0)
                        sacc = score_first(kf, qf[j]);
                    else
                        score_acc(sacc, kf, qf[j]);
                    if (REFILL && j < T::LOADS) issue_load(IC<SR>{}, lo, rptr, i + 2, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
                score_wait(sacc);
                return sacc;
            };
            acc_t sn;
            if (refill)
                sn = scores(IC<1>{});
            else if (has_next)
                sn = scores(IC<0>{});
            // weighted sum of tile i; the softmax of tile i+1 in between
            SmState st;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                bf16x8_t pf[T::G];
#pragma unroll
                for (int g = 0; g < T::G; ++g) pf[g] = p_frag(lo, b, g, u);
                bf16x8_t vring[2] = {v_frag(lo, tc, u, 0), v_frag(lo, tc, u, 1)};
#pragma unroll
                for (int idx = 0; idx < 16; ++idx) {
                    const int cb = idx >> 2, g = idx & 3;
                    o[cb][g] = M::mma(vring[cb & 1], pf[g], o[cb][g]);
                    if (g == 3 && cb + 2 < T::CB) vring[cb & 1] = v_frag(lo, tc, u, cb + 2);
                    const int piece = u * 16 + idx - 1;   // pieces 0..11 after weighted-sum MFMAs 1..12
                    if (piece >= 0 && piece < 12) sm_piece(lo, sn, st, i + 1, b ^ 1, piece);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        };

        for (int i0 = 0; i0 < n_tiles; i0 += T::STAGES) {
            iter(IC<0>{}, i0);
            if (i0 + 1 < n_tiles) iter(IC<1>{}, i0 + 1);
            if (i0 + 2 < n_tiles) iter(IC<2>{}, i0 + 2);
        }

        // ---- segment epilogue ----------------------------------------------
        // The score waves publish 1/l and lse of their heads; every wave then
        // normalises its 128 columns of all heads and stores them through a
        // staging area in the (now idle) tile ring, 64 heads at a time, as
        // whole 256-byte pieces of the output rows.
        l_run += __shfl_xor(l_run, 32, 64);
        {
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2c : -INFINITY;
            if (grp == 0) {
                *(LDS_AS float*)(epi + (wave * 32 + hl) * 4) = inv;
                *(LDS_AS float*)(epi + (T::HG + wave * 32 + hl) * 4) = lse_v;
            }
        }
        lds_exchange_barrier();  // every wave is past the last tile; 1/l visible
        {
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int e_lane = tid & 63;
            const int e_grp = (tid >> 5) & 1;
            const int e_hl = tid & 31;
            const int head0 = hg * T::HG;
            __bf16* obase = (final_out ? (__bf16*)p.out + (size_t)r * p.h * kDc
                                       : (__bf16*)p.po + (size_t)slot * p.h * kDc) +
                            (size_t)head0 * kDc + 128 * wave;
            // two waves per ring stage (separate arrays need not be contiguous)
            lds_byte* stg = ((wave >> 1) == 0 ? stage_lds<T::TILE_BYTES, 0>() : stage_lds<T::TILE_BYTES, 1>()) +
                            (wave & 1) * 64 * T::STG_ROW;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // accumulator entry e of block (cb, g): column 32cb + (e/4)*8 + 4grp + e%4, head 32g + hl
#pragma unroll
                for (int gg = 0; gg < 2; ++gg) {
                    const int g = 2 * half + gg;
                    const float inv = *(const LDS_AS float*)(epi + (g * 32 + e_hl) * 4);
#pragma unroll
                    for (int cb = 0; cb < T::CB; ++cb)
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4) {
                            bf16x4_t v;
#pragma unroll
                            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[cb][g][q4 * 4 + e] * inv);
                            const int col = cb * 32 + q4 * 8 + e_grp * 4;
                            *(LDS_AS bf16x4_t*)(stg + (gg * 32 + e_hl) * T::STG_ROW + 2 * col) = v;
                        }
                }
                // this wave's LDS accesses complete in order: the reads see the writes
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int row = 4 * i + (e_lane >> 4);     // head inside the half
                    const int hh = half * 64 + row;
                    const bf16x8_t v = *(const LDS_AS bf16x8_t*)(stg + row * T::STG_ROW + 16 * (e_lane & 15));
                    if (head0 + hh < p.h) *(bf16x8_t*)(obase + (size_t)hh * kDc + 8 * (e_lane & 15)) = v;
                }
            }
            if (wave == 0) {
                // lse of all 128 heads from the table above, two per lane
#pragma unroll
                for (int i = 0; i < 2; ++i) {
                    const int hh = i * 64 + e_lane;
                    const float lv = *(const LDS_AS float*)(epi + (T::HG + hh) * 4);
                    if (head0 + hh < p.h)
                        (final_out ? p.lse + (size_t)r * p.h : p.plse + (size_t)slot * p.h)[head0 + hh] = lv;
                }
            }
        }

        pos = seg_end;
        if (pos >= end) break;
        wg_barrier();  // every wave is done with the ring and the tables before the next segment
        ++r;
        while (pl_cu(r + 1) <= pos) ++r;
    }
    plan_duties();
}

template <bool PAGED>
__global__ __launch_bounds__(256) void decode_colsplit_kernel(DecodeParams p)
{
    clock_stamp(p.clock_stamps, 0);
    colsplit_body<PAGED>(p);
    clock_stamp(p.clock_stamps, 1);
}

}  // namespace

hipError_t launch_decode_colsplit(const DecodeParams& p, hipStream_t stream)
{
    if (p.plan_in_kernel && (p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks))
        return hipErrorInvalidValue;  // no room for the plan in this kernel's LDS
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    if (p.block_table != nullptr)
        decode_colsplit_kernel<true><<<grid, ColTiling::THREADS, 0, stream>>>(p);
    else
        decode_colsplit_kernel<false><<<grid, ColTiling::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

}  // namespace mla355
