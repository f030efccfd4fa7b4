// Split-KV absorbed-MLA decode, bf16 in / fp32 accumulate: the wide-wave
// kernel for 32 or more heads.
//
// Same operation, plan and partial format as the other bf16 kernels (the
// glossary page "Multi-head Latent Attention", section on why decode absorbs
// the matrices: absorbed query heads score directly against the shared latent
// rows, and the softmax-weighted sum of the c_KV parts is the output).
//
// Layout of the work:
//  * One workgroup = NW waves = one token chunk x 32*NW heads.  Every wave owns
//    32 heads outright: their 576-wide queries stay in VGPRs for the whole
//    chunk (the B operand of every score MFMA) and their 512-wide fp32 output
//    accumulators stay in AGPRs.  No wave needs anything from another except
//    the shared latent tile, so one barrier per tile is the only
//    synchronisation.
//  * With 128 heads a single workgroup covers every head, so each latent row
//    is fetched from HBM exactly once.
//  * Tiles of 32 latent rows stream HBM -> LDS with direct-to-LDS 16-byte DMA
//    (STAGES-deep ring, STAGES-1 tiles in flight).  A tile is stored as
//    region A = the first 1024 B of each row (one DMA instruction per row,
//    rows padded to 1152 B) and region B = the last 128 B (8 rows per
//    instruction); see the per-lane offsets below for the swizzles.  The
//    refill DMA of a tile is spread over the first score MFMAs rather than
//    issued as one burst.
//  * Per tile and wave (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//      S^T[32 tok x 32 heads] = K . Q'^T   36 MFMAs, A = latent rows read from
//                                          LDS (ds_read_b128), B = queries;
//      online softmax on S^T (each lane holds one head: lane-local running
//      max/sum, one cross-lane step for the tile max);
//      O^T[512 x 32 heads] += V^T . P^T    32 MFMAs, A = latent rows read
//                                          transposed (ds_read_b64_tr_b16),
//                                          B = P^T straight from the S^T
//                                          accumulator layout.
//  * Online softmax in base 2, lazy rescale (only when the running max grows
//    by more than 2^8), exact final normalisation.
#include "bf16_common.h"
#include "plan_build.h"

#include <math.h>

namespace mla355 {
namespace {

constexpr float kLn2 = 0.69314718055994531f;

// Chunk rotation of region-A row r (see the per-lane offsets in the kernel).
__device__ __forceinline__ int rot16(int r) { return 4 * ((r >> 1) & 1) + ((r >> 2) & 3); }

template <int NW, int STAGES>
struct WideTiling {
    static constexpr int THREADS = NW * 64;
    static constexpr int HG = 32 * NW;                 // heads per workgroup
    static constexpr int N = 32;                       // tokens per tile
    static constexpr int ROW_A = 1024 + 128;              // LDS stride of a region-A row (rotated)
    static constexpr int A_BYTES = N * ROW_A;
    static constexpr int TILE_BYTES = A_BYTES + N * 128;  // + region B
    static constexpr int LOADS_A = N / NW;             // region-A DMA instructions per wave
    static constexpr int GROUPS_B = N / 8;             // region-B DMA instructions per tile
    static constexpr int LOADS_B = GROUPS_B / NW > 0 ? GROUPS_B / NW : 1;
    static constexpr int LOADS = LOADS_A + LOADS_B;    // DMA instructions per wave per tile
    static constexpr int KS = kDqk / 16;               // 36 score k-steps
    static constexpr int KSA = kDc / 16;               // 32 of them in region A
    static constexpr int MBLK = kDc / 32;              // 16 output blocks of 32 columns
    // Epilogue staging: 32 rows of 256 outputs (bf16) per wave, rows padded
    // by 16 B so that the rows of one accumulator write start in distinct
    // bank groups; two waves per ring stage.
    static constexpr int STG_ROW = 512 + 16;
    static_assert(2 * 32 * STG_ROW <= TILE_BYTES && NW <= 2 * STAGES, "epilogue staging fits the ring");
    static_assert(NW == 1 || NW == 2 || NW == 4, "waves per workgroup");
    static_assert(GROUPS_B % NW == 0, "region-B groups split evenly over waves");
    static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");
    static_assert(STAGES * TILE_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 2) * LOADS <= 63, "vmcnt range");
    static_assert(LOADS <= KS, "refill spread over the score steps");
    // room in LDS for the workgroup's own copy of the split plan
    static constexpr bool PLANS = STAGES * TILE_BYTES + kPlanLdsInts * 4 <= 160 * 1024;
};

// Scalar (constant address space) view of device data that no kernel writes
// while this one runs: a uniform index loads through the scalar cache.
typedef const __attribute__((address_space(4))) int32_t cint32_t;

// Kernel body.  CAUSAL: the "heads" are q_len new tokens x heads_per_token
// heads (q' [b, q_len, h, 576] read as [b, q_len*h, 576]), and new token i of
// a row of L cached rows (the new ones last) attends to its first
// L - q_len + 1 + i rows only.
template <int NW, int STAGES, bool PAGED, bool CAUSAL>
__device__ __forceinline__ void decode_wide_body(const DecodeParams& p)
{
    using T = WideTiling<NW, STAGES>;
    using M = Mfma<32>;
    typedef f32x16_t acc_t;

    const int lane = threadIdx.x & 63;
    // wave index is uniform: keep it (and all DMA arithmetic built on it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hl = lane & 31;    // head inside the wave's 32
    const int grp = lane >> 5;   // k-slot group (0/1) of the MFMA operand layouts

    int k, hg;
    block_work(p.n_chunks, p.n_hg, k, hg);
    // The split plan: plan_kernel's copy in the workspace or, with
    // plan_in_kernel, this workgroup's own copy in LDS, built by wave 0 from
    // seqlens (one load of the lengths instead of a kernel launch and two
    // dependent plan loads).  Entries are the same for every lane: they are
    // kept in scalar registers.
    __shared__ int32_t lplan[T::PLANS ? kPlanLdsInts : 1];
    const bool lds_plan = p.plan_in_kernel != 0;
    if (lds_plan) {
        if (!T::PLANS) return;  // the launcher refuses this combination
        if (wave == 0)
            build_plan(p.seqlens, p.b, p.t_max, p.n_chunks, p.plan_min_chunk, p.plan_align,
                       (LDS_AS int32_t*)lplan);
        __syncthreads();
        // The combine reads the plan from the workspace: workgroup 0 leaves it
        // there.  These stores go out before any tile DMA, so they only make
        // the tile waits below (which count outstanding vector-memory
        // operations) more conservative.
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
    // With its own plan, every workgroup also takes its share of the plan
    // kernel's other duty once its segments are done: rows with no tokens
    // (lengths read from the plan) get out = 0, lse = -inf.
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
    // Region A: row r of the tile at r * ROW_A (ROW_A = 1152 B = 72 16-byte
    // bank quads, so row r starts at quad 8 (r & 1) of the 16 quads of a
    // 256-byte bank cycle); its 16-byte chunk c sits at chunk position
    // c + g(r), g(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3) (inside the row's
    // 128 bytes of padding, no wrap-around).  Row r's chunk c then starts at
    // quad 8 (r & 1) + 4 ((r >> 1) & 1) + ((r >> 2) & 3) + c (mod 16), distinct
    // over any 16 consecutive rows for a 16-byte read, and the transposed reads
    // (4 rows x 4 chunks per 32 lanes) cover all 64 banks once.  Every read is
    // a per-lane base plus a compile-time offset.
    // Score step j < 32 reads row rr = lane & 31, chunk 2j + grp:
    //   rr * ROW_A + 16 (grp + g(rr)) + 32 j.
    // Region B (last 128 B of each row): rows of 128 B, chunk c of row r at
    // position c ^ xb(r); step 32 + j reads chunk 2j + grp:
    //   kB ^ (j << 5) (the swizzle only touches bits 5-6 of the address).
    const int rr = lane & 31;
    const int kA = rr * T::ROW_A + 16 * (grp + rot16(rr));
    int kB;
    {
        const int xbv = xb(rr & 15);
        kB = T::A_BYTES + rr * 128 + 32 * (xbv >> 1) + 16 * (grp ^ (xbv & 1));
    }
    // Transposed reads of 16 tokens x 32 columns: this lane supplies 4 columns
    // (16((lane>>4)&1) + 4(lane&3) .. +3 of the block) of token row0 (+8); the
    // instruction hands every lane one column and 4 tokens.  Block (u, mb):
    //   vA + 16u ROW_A + 64 mb, and the rows 8 further on at
    //   + 8 ROW_A + 32 (g(row0 + 8) = g(row0) + 2 for row0 < 8).
    int vA;
    {
        const int row0 = grp * 4 + ((lane & 15) >> 2);
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        vA = row0 * T::ROW_A + 16 * (cc + rot16(row0)) + ((lane & 1) << 3);
    }

    while (true) {
        const int row_lo = pl_cu(r);
        const int row_hi = pl_cu(r + 1);
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        int seg_len = seg_end - pos;
        if (PAGED) {
            // the plan covers lengths rounded up to whole tiles: mask the rest
            const int L = min(max(seqlen_of(r), 0), p.t_max);
            seg_len = max(0, min(seg_len, L - seg_a));
        }
        // CAUSAL: tokens of this segment the lane's query row may see (any
        // value: <= 0 none, >= seg_len all)
        int c_lim = 0;
        if constexpr (CAUSAL) {
            const int L = PAGED ? min(max(seqlen_of(r), 0), p.t_max) : row_hi - row_lo;
            c_lim = L - p.q_len + 1 + head / p.heads_per_token - seg_a;
        }
        const int split_j = k - row_lo / chunk;
        const bool final_out = pl_nsplit(r) == 1;
        const int slot = pl_base(r) + split_j;
        const unsigned char* seg_base = cg + ((size_t)r * p.t_max + seg_a) * kRowBytesBf16;
        int n_tiles = (seg_len + T::N - 1) / T::N;
        if constexpr (CAUSAL) {
            // Tiles past the causal limit of every query row of this
            // workgroup hold nothing any of its rows may see: the segment
            // stops at the last tile the latest row can reach.
            const int last_row = min(hg * T::HG + T::HG, p.h) - 1;
            const int L = PAGED ? min(max(seqlen_of(r), 0), p.t_max) : row_hi - row_lo;
            const int lim_max = L - p.q_len + 1 + last_row / p.heads_per_token - seg_a;
            n_tiles = max(0, min(n_tiles, (lim_max + T::N - 1) / T::N));
        }

        // Global address of the first row of `tile`.  Paged: tiles are issued
        // once each, in increasing order, so the block-table position of the
        // next one is tracked (segments start at multiples of the tile, and
        // the block size is a multiple of it: a tile never straddles blocks).
        int pg_blk = 0, pg_off = 0;
        if (PAGED) {
            pg_blk = seg_a / p.block_size;
            pg_off = seg_a - pg_blk * p.block_size;
        }
        auto tile_ptr = [&](int tile) -> const unsigned char* {
            if (!PAGED) return seg_base + (size_t)tile * T::N * kRowBytesBf16;
            if (tile >= n_tiles) return cg;  // an empty refill: no block-table read
            // a scalar load: its wait does not queue behind the tile DMAs in flight
            const int e = min(max(*(cint32_t*)(p.block_table + (size_t)r * p.max_blocks + pg_blk), 0),
                              p.num_blocks - 1);
            const unsigned char* a = cg + ((size_t)e * p.block_size + pg_off) * kRowBytesBf16;
            pg_off += T::N;
            if (pg_off == p.block_size) {
                pg_off = 0;
                ++pg_blk;
            }
            return a;
        };

        // DMA instruction `li` (0 .. LOADS-1) of this wave's share of `tile`
        // (first row at tptr) into stage SC.  Rows past the segment end
        // re-read its last row (the scores of those slots are masked), so
        // every access stays inside the rows of this segment.  A tile at or
        // past n_tiles gets an empty resource: the instructions still issue
        // (a free stage receives zeros, no memory is read), so every step
        // issues the same DMA count, the waits below are constants and the
        // compiler's own DMA bookkeeping adds no wait of its own.
        auto issue_load = [&](auto SC, const unsigned char* tptr, int tile, int li) {
            const int t0 = tile * T::N;
            const int last = (tile < n_tiles ? min(T::N, seg_len - t0) : 0) - 1;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)tptr, (short)0, (last + 1) * kRowBytesBf16, kBufferFlags);
            lds_byte* st = stage_lds<T::TILE_BYTES, decltype(SC)::value>();
            if (li < T::LOADS_A) {
                const int row = wave + li * NW;
                const int srow = min(row, last);
                // the row's 64 chunks land contiguously from position g(row)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + row * T::ROW_A + 16 * rot16(row)), 16, (unsigned)lane << 4,
                    __builtin_amdgcn_readfirstlane(srow * kRowBytesBf16), 0, 0);
            } else {
                const int gb = wave + (li - T::LOADS_A) * NW;
                const int row = gb * 8 + (lane >> 3);
                const int srow = min(row, last);
                const int lc = (lane & 7) ^ xb(row & 15);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + T::A_BYTES + gb * 1024), 16,
                    (unsigned)(srow * kRowBytesBf16 + 1024 + lc * 16), 0, 0, 0);
            }
        };
        auto issue_tile = [&](auto SC, int tile) {
            const unsigned char* tp = tile_ptr(tile);
#pragma unroll
            for (int li = 0; li < T::LOADS; ++li) issue_load(SC, tp, tile, li);
        };
        // Wait until this wave's share of tile t has landed.  Tile 0 goes out
        // before the queries, tiles 1 .. STAGES-2 right after them, and step i
        // refills tile i+STAGES-1 (real or empty), so the tiles issued after t
        // are always t+1 .. t+STAGES-2 (at step 0 the queries sit between tile
        // 0 and tile 1 and are waited for too, which the first MFMA needs anyway).
        auto wait_tile = [&]() { wait_vmcnt<(STAGES - 2) * T::LOADS>(); };

        // Tile 0 first: the queries are as large as a tile, and the first
        // score MFMA needs both.
        issue_tile(IC<0>{}, 0);
        // Queries (B operand): lane -> head hl, channels 16j + 8grp .. +7 of step j.
        // A lane past the last head reads head 0's query instead (finite values,
        // results never stored), so nothing waits on the loads before the
        // first score MFMA.
        bf16x8_t qf[T::KS];
        {
            const bf16x8_t* qrow =
                (const bf16x8_t*)(qg + ((size_t)r * p.h + (head_ok ? head : 0)) * kDqk);
#pragma unroll
            for (int j = 0; j < T::KS; ++j) qf[j] = qrow[2 * j + grp];
        }
        if (STAGES > 2) issue_tile(IC<(STAGES > 2 ? 1 : 0)>{}, 1);
        if (STAGES > 3) issue_tile(IC<(STAGES > 3 ? 2 : 0)>{}, 2);

        acc_t o[T::MBLK];
#pragma unroll
        for (int mb = 0; mb < T::MBLK; ++mb) o[mb] = (acc_t){};
        float m_run = kNegBig;
        float l_run = 0.f;

        auto k_frag = [&](lds_byte* tb, int j) -> bf16x8_t {
            const lds_byte* a = (j < T::KSA) ? tb + kA + 32 * j : tb + (kB ^ ((j - T::KSA) << 5));
            return *(const LDS_AS bf16x8_t*)a;
        };
        // Transposed V fragment idx: token half u = idx / MBLK, column block mb = idx % MBLK.
        auto v_frag = [&](lds_byte* tb, int idx) -> bf16x8_t {
            const int u = idx / T::MBLK, mb = idx % T::MBLK;
            const int blk = 64 * mb + u * 16 * T::ROW_A;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + vA + blk));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + vA + blk + 8 * T::ROW_A + 32));
            return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        };

        // One tile: tile index i in stage SC.
        auto step = [&](auto SC, int i) {
            constexpr int S = decltype(SC)::value;
            constexpr int SR = (S + STAGES - 1) % STAGES;  // stage of tile i-1 = refill target
            lds_byte* tb = stage_lds<T::TILE_BYTES, S>();
            // the refill's address first: a paged lookup completes during the barrier
            const unsigned char* rptr = tile_ptr(i + STAGES - 1);
            wait_tile();
            lds_exchange_barrier();  // tile i visible to all; everyone is done with tile i-1

            // ---- scores: S^T = K . Q'^T, the refill DMA of tile i+STAGES-1
            // spread over the first steps
            acc_t sacc;
            {
                constexpr int PF = 4;
                bf16x8_t kring[PF];
#pragma unroll
                for (int j = 0; j < PF; ++j) kring[j] = k_frag(tb, j);
#pragma unroll
                for (int j = 0; j < T::KS; ++j) {
                    const bf16x8_t kf = kring[j % PF];
                    if (j + PF < T::KS) kring[j % PF] = k_frag(tb, j + PF);
                    if (j == 0)
                        sacc = score_first(kf, qf[j]);
                    else
                        score_acc(sacc, kf, qf[j]);
                    if (j < T::LOADS) issue_load(IC<SR>{}, rptr, i + STAGES - 1, j);
                    __builtin_amdgcn_sched_barrier(0);
                }
                score_wait(sacc);
            }

            // ---- online softmax; sacc[e]: token (e/4)*8 + 4grp + e%4, head hl
            const int tvalid = __builtin_amdgcn_readfirstlane(seg_len - i * T::N);
            if constexpr (CAUSAL) {
                const int lim_l = min(tvalid, c_lim - i * T::N);
                if (__any(lim_l < T::N)) {
                    const int lim = lim_l - 4 * grp;
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if ((e >> 2) * 8 + (e & 3) >= lim) sacc[e] = -INFINITY;
                }
            } else if (tvalid < T::N) {
                const int lim = tvalid - 4 * grp;
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    if ((e >> 2) * 8 + (e & 3) >= lim) sacc[e] = -INFINITY;
            }
            float tm = fmaxf(fmaxf(sacc[0], sacc[1]), sacc[2]);
#pragma unroll
            for (int e = 3; e < 16; ++e) tm = fmaxf(tm, sacc[e]);
            const float tmax = max_xor32(tm) * c2;
            const float m_new = fmaxf(m_run, tmax);
            if (i == 0) {
                m_run = m_new;  // first tile: nothing accumulated yet
            } else if (__any(m_new > m_run + kRescaleThreshold)) {
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
                // The accumulators live in AGPRs; the empty asm statements pin
                // the copy used for the multiply to VGPRs and the result back
                // to AGPRs, one block at a time (left to itself the register
                // allocator moves all 256 accumulators and spills).
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
            // probabilities of the first 16 tokens now; those of the second 16
            // (needed from weighted-sum step MBLK on) between the first MFMAs
            bf16x8_t pb[2];
            auto prob = [&](int e) {
                const float x = exp2_fast(__builtin_fmaf(sacc[e], c2, -m_run));
                l_run += x;
                pb[e >> 3][e & 7] = (__bf16)x;
            };
#pragma unroll
            for (int e = 0; e < 8; ++e) prob(e);

            // ---- weighted sum: O^T += V^T . P^T
            constexpr int NPV = 2 * T::MBLK;
            constexpr int PFV = 4;
            bf16x8_t vring[PFV];
#pragma unroll
            for (int j = 0; j < PFV; ++j) vring[j] = v_frag(tb, j);
#pragma unroll
            for (int idx = 0; idx < NPV; ++idx) {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                const bf16x8_t a = vring[idx % PFV];
                if (idx + PFV < NPV) vring[idx % PFV] = v_frag(tb, idx + PFV);
                o[mb] = M::mma(a, pb[u], o[mb]);
                if (idx < 8) prob(8 + idx);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // The steps form one chain (each reachable only from the one before),
        // so every path into a step carries the same DMA queue.
        for (int i0 = 0; i0 < n_tiles; i0 += STAGES) {
            step(IC<0>{}, i0);
            if (i0 + 1 >= n_tiles) break;
            step(IC<1 % STAGES>{}, i0 + 1);
            if (i0 + 2 >= n_tiles) break;
            if constexpr (STAGES > 2) {
                step(IC<(STAGES > 2 ? 2 : 0)>{}, i0 + 2);
                if (i0 + 3 >= n_tiles) break;
            }
            if constexpr (STAGES > 3) {
                step(IC<(STAGES > 3 ? 3 : 0)>{}, i0 + 3);
                if (i0 + 4 >= n_tiles) break;
            }
        }

        // ---- segment epilogue ----------------------------------------------
        // A row finished here writes out/lse; otherwise its slot's partial
        // (normalised, bf16) and partial lse.  A store straight from the
        // accumulator layout would write 16 bytes into each of 32 head rows;
        // instead each wave stages half of its 32 x 512 outputs at a time in
        // LDS (the tile ring is free once every wave is past the last tile)
        // and stores whole 512-byte half rows.
        l_run += __shfl_xor(l_run, 32, 64);
        wait_vmcnt<0>();         // the empty refills past the last tile have landed
        lds_exchange_barrier();
        {
            // The lane's head and column group are derived again here from the
            // thread index (opaque to the compiler) instead of being kept live
            // across the tile loop, where every register is taken.
            int tid = threadIdx.x;
            asm volatile("" : "+v"(tid));
            const int e_lane = tid & 63;
            const int e_grp = (tid >> 5) & 1;
            const int e_hl = tid & 31;
            const int head0 = hg * T::HG + wave * 32;
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * kLn2 : -INFINITY;
            __bf16* obase = (final_out ? (__bf16*)p.out + (size_t)r * p.h * kDc
                                       : (__bf16*)p.po + (size_t)slot * p.h * kDc) + (size_t)head0 * kDc;
            lds_byte* stg = ((wave >> 1) == 0 ? stage_lds<T::TILE_BYTES, 0>() : stage_lds<T::TILE_BYTES, 1>()) +
                            (wave & 1) * 32 * T::STG_ROW;
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                // accumulator entry e of block mb: column 32mb + (e/4)*8 + 4grp + e%4
#pragma unroll
                for (int mb = half * T::MBLK / 2; mb < (half + 1) * T::MBLK / 2; ++mb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        bf16x4_t v;
#pragma unroll
                        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(o[mb][q4 * 4 + e] * inv);
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

template <int NW, int STAGES, bool PAGED>
__global__ __launch_bounds__(NW * 64) void decode_wide_kernel(DecodeParams p)
{
    clock_stamp(p.clock_stamps, 0);
    decode_wide_body<NW, STAGES, PAGED, false>(p);
    clock_stamp(p.clock_stamps, 1);
}

template <int NW, int STAGES, bool PAGED>
__global__ __launch_bounds__(NW * 64) void decode_wide_causal_kernel(DecodeParams p)
{
    clock_stamp(p.clock_stamps, 0);
    decode_wide_body<NW, STAGES, PAGED, true>(p);
    clock_stamp(p.clock_stamps, 1);
}

}  // namespace

template <int NW, int STAGES>
hipError_t launch_decode_wide(const DecodeParams& p, hipStream_t stream)
{
    using T = WideTiling<NW, STAGES>;
    if (p.plan_in_kernel && (!T::PLANS || p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks))
        return hipErrorInvalidValue;  // no room for the plan in this kernel's LDS
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    if (p.block_table != nullptr)
        decode_wide_kernel<NW, STAGES, true><<<grid, T::THREADS, 0, stream>>>(p);
    else
        decode_wide_kernel<NW, STAGES, false><<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

template hipError_t launch_decode_wide<4, 3>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide<4, 4>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide<4, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide<2, 3>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide<2, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide<1, 3>(const DecodeParams&, hipStream_t);

template <int NW, int STAGES>
hipError_t launch_decode_wide_causal(const DecodeParams& p, hipStream_t stream)
{
    using T = WideTiling<NW, STAGES>;
    if (p.plan_in_kernel && (!T::PLANS || p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks))
        return hipErrorInvalidValue;  // no room for the plan in this kernel's LDS
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    if (p.block_table != nullptr)
        decode_wide_causal_kernel<NW, STAGES, true><<<grid, T::THREADS, 0, stream>>>(p);
    else
        decode_wide_causal_kernel<NW, STAGES, false><<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

template hipError_t launch_decode_wide_causal<4, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide_causal<2, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide_causal<1, 3>(const DecodeParams&, hipStream_t);

}  // namespace mla355
