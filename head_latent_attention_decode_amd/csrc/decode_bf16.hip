// Split-KV absorbed-MLA decode kernel, bf16 in / fp32 accumulate, for gfx950.
//
// What it computes (glossary "Multi-head Latent Attention", section on why
// decode absorbs the matrices): every absorbed query head q'_h (576 wide:
// q^C_h (W^UK_h)^T followed by the rope query) scores directly against the
// shared latent rows [c_KV ; k_R]; the softmax-weighted sum of the c_KV parts
// is the 512-wide output.  Per-head keys and values are never formed.
//
// How (one workgroup = one token chunk x one group of HG = HS*WH heads):
//  * Tiles of N = TS*NT latent rows stream HBM -> LDS with direct-to-LDS
//    16-byte DMA loads (global_load_lds_dwordx4), STAGES deep, one copy per
//    workgroup shared by all its heads.  A tile is stored as two regions:
//      A: the first 1024 B of every row (c_KV), 1 KB per row, so one wave DMA
//         instruction moves one row;
//      B: the last 128 B of every row (k_R), 8 rows per DMA instruction.
//    16-byte chunks are XOR-swizzled inside each row (chunk c of row r sits at
//    c ^ xA(r) in region A, c ^ xB(r) in region B) so that the MFMA operand
//    reads of consecutive rows fall in distinct LDS banks.
//  * Each wave owns WH heads (16 -> v_mfma_f32_16x16x32_bf16, 32 ->
//    v_mfma_f32_32x32x16_bf16) and NT tokens of each tile:
//      S^T = K . Q'^T     A = latent rows from LDS (ds_read_b128),
//                         B = the wave's queries, resident in VGPRs.
//      O^T += V^T . P^T   A = latent rows read transposed from LDS
//                         (ds_read_b64_tr_b16), B = P^T straight from the
//                         S^T accumulator layout (no data movement).
//    In both products every lane holds exactly one head, so the online
//    softmax state (running max m, running sum l, rescale) is lane-local;
//    the per-tile max needs one or two cross-lane steps.
//  * Online softmax in base 2 (scale * log2 e folded into the scores).  The
//    accumulator is only rescaled when the running max grows by more than
//    2^8 (values stay far inside fp32 range); the final normalisation uses the
//    same max for l and O, so this is exact.
//  * TS > 1: the TS waves of one head subgroup split each tile's tokens and
//    merge their (m, l, O) through LDS at the end of a segment.
//  * Segment end: a row finished inside this chunk writes out (bf16) and lse;
//    otherwise the normalised fp32 partial and its lse go to the row's slot.
#include "bf16_common.h"
#include "variants.h"

#include <array>
#include <type_traits>
#include <utility>

#include <math.h>

namespace mla355 {
namespace {


// fp8 staging layout: 16-byte chunk c of staged row r sits at chunk
// f8chunk(c, f8sw(r)) (chunks 32..35, the rope key, stay inside their group of
// four).  With the 592-byte row stride this keeps both fp8 operand reads free
// of bank conflicts: the 8-byte score reads of rows 2i + sb (i = 0..15) and
// the transposed 8-byte reads of 8 consecutive rows per 16 lanes.
__device__ __forceinline__ int f8sw(int r) { return ((r >> 4) & 1) | ((r & 1) << 1); }
__device__ __forceinline__ int f8chunk(int c, int sw) { return (c & ~3) | ((c & 3) ^ sw); }

template <int WH, int HS, int TS, int NT, int STAGES>
struct Tiling {
    static constexpr int NW = HS * TS;
    static constexpr int THREADS = NW * 64;
    static constexpr int HG = HS * WH;             // heads per workgroup
    static constexpr int N = TS * NT;              // tokens per tile
    static constexpr int A_BYTES = N * 1024;
    static constexpr int TILE_BYTES = N * kRowBytesBf16;
    static constexpr int LDS_BYTES = STAGES * TILE_BYTES;
    static constexpr int LOADS_A = N / NW;         // region-A DMA instructions per wave
    static constexpr int GROUPS_B = N / 8;         // region-B DMA instructions per tile
    static constexpr int LOADS_B_MAX = (GROUPS_B + NW - 1) / NW;
    static constexpr int LOADS = LOADS_A + LOADS_B_MAX;
    static constexpr int KSTEPS = kDqk / Mfma<WH>::kK;
    static constexpr int KSTEPS_A = kDc / Mfma<WH>::kK;   // steps inside region A
    static constexpr int MBLK = kDc / WH;          // O^T blocks (WH latent columns each)
    static constexpr int SBLK = NT / WH;           // S^T blocks per wave per tile
    static constexpr int MERGE_FLOATS = MBLK * Mfma<WH>::kAcc + 2;  // per lane
    // fp8 cache: a stage holds the tile's raw rows (576 B each) and per-token
    // scales; the conversion pass writes the bf16 tile above into one buffer
    static constexpr int ROW8 = kDqk;                      // fp8 row bytes in HBM
    static constexpr int LROW8 = kDqk + 16;                // LDS stride of a staged fp8 row
    static constexpr int STG8_BYTES = N * LROW8 + N * 4;   // rows + per-token scales
    static constexpr int SCL8 = N * LROW8;                 // scales offset
    static constexpr int DMA8 = N / NW;                    // one row per DMA instruction
    static_assert(N % NW == 0, "region A rows split evenly over waves");
    static_assert(STAGES >= 2 && STAGES <= 4, "pipeline depth");
    static_assert(STAGES == 2 || GROUPS_B % NW == 0, "exact vmcnt accounting needs even B split");
    static_assert(NT % 32 == 0 && NT % WH == 0, "wave token slice must be whole MFMA blocks");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 1) * LOADS <= 63, "vmcnt range");
    static_assert(TS == 1 || (TS - 1) * HS * 64 * MERGE_FLOATS * 4 <= TILE_BYTES, "merge area");
};

template <int WH, int HS, int TS, int NT, int STAGES, bool FP8>
__device__ __forceinline__ void decode_bf16_body(const DecodeParams& p)
{
    using T = Tiling<WH, HS, TS, NT, STAGES>;
    static_assert(!FP8 || (STAGES == 2 && T::N % T::NW == 0 && T::N <= 64 && WH == 16 && NT == 32 &&
                           HS == 1),
                  "fp8 form: two stages, 16-head waves of 32 tokens, one scale per lane");
    static_assert(!FP8 || 2 * STAGES * T::STG8_BYTES <= 160 * 1024, "fp8: two workgroups per CU");
    static_assert(!FP8 || TS == 1 || (TS - 1) * HS * 64 * T::MERGE_FLOATS * 4 <= T::STG8_BYTES,
                  "fp8 merge area");
    using M = Mfma<WH>;
    typedef typename M::acc_t acc_t;
    // An operand fragment as read from LDS: 8 bf16, or (fp8) 8 e4m3 codes.
    typedef std::conditional_t<FP8, unsigned long long, bf16x8_t> kraw_t;
    auto to_bf16x8 = [](kraw_t f) -> bf16x8_t {
        if constexpr (FP8)
            return cvt8_e4m3(f);
        else
            return f;
    };

    const int lane = threadIdx.x & 63;
    // wave index is uniform: keep it (and the DMA row arithmetic built on it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int hs = wave % HS;
    const int ts = wave / HS;
    const int hl = lane & (WH - 1);   // this lane's head inside the wave's WH heads
    const int grp = lane / WH;        // lane group sharing that head (0..64/WH-1)

    int k, hg;
    block_work(p.n_chunks, p.n_hg, k, hg);
    const PlanView pv{const_cast<int32_t*>(p.plan), p.b};
    const int total = p.plan[0];
    const int chunk = p.plan[1];
    int r = pv.chunk_row()[k];
    if (r < 0) return;
    int pos = k * chunk;
    const int end = pos + min(chunk, total - pos);  // no int overflow near 2^31 tokens

    const __bf16* __restrict__ qg = (const __bf16*)p.q;
    const unsigned char* __restrict__ cg = (const unsigned char*)p.cache;
    const int head = hg * T::HG + hs * WH + hl;
    const bool head_ok = head < p.h;
    const int tok0 = ts * NT;  // this wave's first token in every tile

    // ---- per-lane LDS byte offsets (relative to a stage base) --------------
    // K reads (S^T A operand): lane -> token row tok0 + sb*WH + rr, logical
    // chunk ks*(kK/8) + grp.  rr & 15 == lane & 15 for every sb.
    const int rr = lane & (WH - 1);
    constexpr int CPK = M::kK / 8;                    // chunks per k-step per lane group
    constexpr int NQA = 16 / CPK;                     // distinct (c & 15) patterns in region A
    constexpr int KSTEPS_B = T::KSTEPS - T::KSTEPS_A; // steps inside region B
    int koffA[NQA], koffB[KSTEPS_B];
    {
        const int xa = M::xa(rr & 15);
        const int xbv = xb(rr & 15);
#pragma unroll
        for (int q = 0; q < NQA; ++q) koffA[q] = (tok0 + rr) * 1024 + (((q * CPK + grp) ^ xa) << 4);
#pragma unroll
        for (int q = 0; q < KSTEPS_B; ++q)
            koffB[q] = T::A_BYTES + (tok0 + rr) * 128 + (((q * CPK + grp) ^ xbv) << 4);
    }
    // V^T reads (transposed, region A).  See the ds_read_b64_tr_b16 mapping:
    // inside each 16-lane group, source lane s supplies 4 consecutive columns
    // of one row; output lane i, element e receives source lane 4e + i/4,
    // element i%4.
    constexpr int NQV = (WH == 16) ? 8 : 4;           // distinct column patterns
    int voff0[NQV], voff1[NQV];
    {
        if (WH == 16) {
            const int row0 = tok0 + grp * 4 + ((lane & 15) >> 2);  // + u*32, hi rows +16
            const int x = M::xa(row0 & 15);
            const int hb = (lane & 3) >> 1;
#pragma unroll
            for (int q = 0; q < NQV; ++q) {
                voff0[q] = row0 * 1024 + (((2 * q + hb) ^ x) << 4) + ((lane & 1) << 3);
                voff1[q] = 0;  // hi rows are row0 + 16: same swizzle, immediate offset
            }
        } else {
            const int row0 = tok0 + (lane >> 5) * 4 + ((lane & 15) >> 2);  // + u*16, hi rows +8
            const int x0 = M::xa(row0 & 15), x1 = M::xa((row0 + 8) & 15);
            const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
            for (int q = 0; q < NQV; ++q) {
                voff0[q] = row0 * 1024 + (((4 * q + cc) ^ x0) << 4) + ((lane & 1) << 3);
                voff1[q] = (row0 + 8) * 1024 + (((4 * q + cc) ^ x1) << 4) + ((lane & 1) << 3);
            }
        }
    }

    // fp8 operand reads (16-head waves, 32 tokens per wave and tile).
    //  * scores: S block sb row i is token 2i + sb of the wave's 32 (so that the
    //    weighted sum's k slots below are 8 consecutive tokens per 16 lanes).
    //    Lane -> row 2 (lane & 15) + sb; at k step ks it reads logical chunk
    //    2 ks + (g >> 1), byte 8 (g & 1), g = lane >> 4:
    //    k8off[sb] + k8x[sb][ks & 1] + 64 (ks >> 1).
    //  * weighted sum: ds_read_b64_tr_b8 hands output lane i (of 16) byte i % 8
    //    of source lanes 2e + i / 8, e = 0..7.  Source lane (g, s) supplies
    //    token 8g + perm(s >> 1) (perm = 0,2,4,6,1,3,5,7: the P^T slot order
    //    the S layout above gives), bytes 16 mb + 8 (s & 1) .. +7, so output
    //    lane i gets column 16 mb + i of the 8 tokens in slot order:
    //    v8off + v8x[mb & 3] + 64 (mb >> 2).
    int k8off[2] = {0, 0}, k8x[2][2] = {{0, 0}, {0, 0}}, v8off = 0, v8x[4] = {0, 0, 0, 0};
    if (FP8) {
        const int g = lane >> 4;
#pragma unroll
        for (int sb = 0; sb < 2; ++sb) {
            const int row = tok0 + 2 * (lane & 15) + sb;
            k8off[sb] = row * T::LROW8 + 8 * (g & 1);
            const int sw = f8sw(row);
#pragma unroll
            for (int par = 0; par < 2; ++par) k8x[sb][par] = ((2 * par + (g >> 1)) ^ sw) << 4;
        }
        const int e = (lane & 15) >> 1;
        const int row = tok0 + 8 * g + (e < 4 ? 2 * e : 2 * (e - 4) + 1);
        v8off = row * T::LROW8 + 8 * (lane & 1);
        const int sw = f8sw(row);
#pragma unroll
        for (int q = 0; q < 4; ++q) v8x[q] = (q ^ sw) << 4;
    }

    while (true) {
        const int row_lo = pv.cu()[r];
        const int row_hi = pv.cu()[r + 1];
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        const int seg_len = seg_end - pos;
        const int split_j = k - row_lo / chunk;
        const bool final_out = pv.nsplit()[r] == 1;
        const int slot = pv.base()[r] + split_j;
        const unsigned char* seg_base = cg + ((size_t)r * p.t_max + seg_a) * (FP8 ? T::ROW8 : kRowBytesBf16);
        const float* seg_scale = FP8 ? p.cache_scale + (size_t)r * p.t_max + seg_a : nullptr;
        const int n_tiles = (seg_len + T::N - 1) / T::N;

        // Queries: B operand of S^T = K . Q^T.  Lane -> head hl, k-slots
        // grp*8 .. +7 of contraction step ks (k = ks*kK + grp*8 + j).
        bf16x8_t qf[T::KSTEPS];
        {
            const bf16x8_t* qrow =
                (const bf16x8_t*)(qg + ((size_t)r * p.h + (head_ok ? head : 0)) * kDqk);
#pragma unroll
            for (int ks = 0; ks < T::KSTEPS; ++ks) {
                bf16x8_t v = qrow[ks * CPK + grp];
                if (!head_ok) v = (bf16x8_t){};
                qf[ks] = v;
            }
        }

        // fp8 staging: one DMA instruction per row (36 lanes x 16 bytes), row r
        // at r * LROW8 with its 16-byte chunks XOR-swizzled by f8sw(r) (chunks
        // 32..35, the rope key, inside their group of 4).  The buffer resource
        // spans the valid rows only and the whole offset is in the
        // bounds-checked per-lane part, so rows past the segment end read as
        // zero codes (finite; those tokens are masked).  Wave 0 also copies
        // the N scales, 4 bytes per lane (zero past the valid rows too).
        auto issue_tile8 = [&](auto SC, int tile) {
            const int t0 = tile * T::N;
            const int last = min(T::N, seg_len - t0) - 1;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(seg_base + (size_t)t0 * T::ROW8), (short)0, (last + 1) * T::ROW8, kBufferFlags);
            lds_byte* st = stage_lds<T::STG8_BYTES, decltype(SC)::value>();
            if (lane < kDqk / 16) {
#pragma unroll
                for (int j = 0; j < T::DMA8; ++j) {
                    const int row = wave + j * T::NW;
                    const int c = f8chunk(lane, f8sw(row));
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (LDS_AS void*)(st + row * T::LROW8), 16,
                                                             (unsigned)(row * T::ROW8 + c * 16), 0, 0, 0);
                }
            }
            if (wave == 0 && lane < T::N) {  // one 4-byte scale per lane
                const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(seg_scale + t0), (short)0, (last + 1) * 4, kBufferFlags);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(st + T::SCL8), 4,
                                                         (unsigned)(lane * 4), 0, 0, 0);
            }
        };

        auto issue_tile = [&](auto SC, int tile) {
            if (FP8) {
                issue_tile8(SC, tile);
                return;
            }
            const int t0 = tile * T::N;
            const int last = min(T::N, seg_len - t0) - 1;  // last valid tile row
            // Buffer resource over this tile's valid rows.  Rows past the end of
            // the segment are clamped to the last valid row (finite data; their
            // scores are masked), so no access leaves [t0, seg_len).
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(seg_base + (size_t)t0 * kRowBytesBf16), (short)0,
                (last + 1) * kRowBytesBf16, kBufferFlags);
            lds_byte* st = stage_lds<T::TILE_BYTES, decltype(SC)::value>();
            // region A: one row per instruction; lane l fetches logical chunk l ^ xA(row).
#pragma unroll
            for (int j = 0; j < T::LOADS_A; ++j) {
                const int row = wave + j * T::NW;
                const int srow = min(row, last);   // rows past the end re-read a valid row
                const unsigned voff = (unsigned)((lane ^ M::xa(row & 15)) << 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + row * 1024), 16, voff,
                    __builtin_amdgcn_readfirstlane(srow * kRowBytesBf16), 0, 0);
            }
            // region B: 8 rows per instruction; lane l -> row 8*gb + l/8, slot l%8.
#pragma unroll
            for (int j = 0; j < T::LOADS_B_MAX; ++j) {
                const int gb = wave + j * T::NW;
                if (T::GROUPS_B % T::NW == 0 || gb < T::GROUPS_B) {
                    const int row = gb * 8 + (lane >> 3);
                    const int srow = min(row, last);
                    const int lc = (lane & 7) ^ xb(row & 15);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rsrc, (LDS_AS void*)(st + T::A_BYTES + gb * 1024), 16,
                        (unsigned)(srow * kRowBytesBf16 + 1024 + lc * 16), 0, 0, 0);
                }
            }
        };

        acc_t o[T::MBLK];
#pragma unroll
        for (int mb = 0; mb < T::MBLK; ++mb) o[mb] = (acc_t){};
        float m_run = kNegBig;  // running max (base-2 scaled scores)
        float l_run = 0.f;      // this lane's share of the running sum

        if (0 < n_tiles) issue_tile(IC<0>{}, 0);
        if (STAGES > 2 && 1 < n_tiles) issue_tile(IC<(STAGES > 2 ? 1 : 0)>{}, 1);
        if (STAGES > 3 && 2 < n_tiles) issue_tile(IC<(STAGES > 3 ? 2 : 0)>{}, 2);

        auto tile_body = [&](auto SC, int it) {
            constexpr int S = decltype(SC)::value;
            // Tiles issued after `it` so far: it+1 .. min(it+STAGES-2, n_tiles-1).
            if (STAGES > 2 && n_tiles - 1 - it >= STAGES - 2)
                wait_vmcnt<(STAGES > 2 ? (STAGES - 2) * T::LOADS : 0)>();
            else
                wait_vmcnt<0>();
            // DMA of tile `it` complete (vmcnt above); after the barrier every wave
            // sees it, and every wave has consumed its reads of tile it-1.
            lds_exchange_barrier();
            if (it + STAGES - 1 < n_tiles) issue_tile(IC<(S + STAGES - 1) % STAGES>{}, it + STAGES - 1);

            lds_byte* tb = stage_lds<T::TILE_BYTES, S>();
            const lds_byte* sg = stage_lds<T::STG8_BYTES, S>();
            const int tvalid = seg_len - it * T::N - tok0;  // valid tokens for this wave (may be <= 0)

            // ---- S^T = K . Q^T -------------------------------------------------
            // K fragments stream through a small register ring, PF steps ahead
            // of the MFMA that consumes them; the scheduling fence after every
            // step keeps the compiler from hoisting all of a tile's LDS reads
            // (which would exhaust the register file).  Two accumulator chains
            // per S block (even / odd k steps) keep dependent MFMAs apart.
            constexpr int NSTEP = T::KSTEPS * T::SBLK;
            constexpr int PF = 4;
            auto k_addr = [&](int idx) -> const lds_byte* {
                const int ks = idx / T::SBLK, sb = idx % T::SBLK;
                if (ks < T::KSTEPS_A) return tb + koffA[ks % NQA] + (ks / NQA) * 256 + sb * WH * 1024;
                return tb + koffB[ks - T::KSTEPS_A] + sb * WH * 128;
            };
            // The ring holds fragments as read (fp8: raw codes); an fp8
            // fragment is converted only where its MFMA takes it, so the
            // conversion does not wait for a read issued in the same step.
            auto k_frag = [&](int idx) -> kraw_t {
                if constexpr (!FP8) {
                    return *(const LDS_AS bf16x8_t*)k_addr(idx);
                } else {
                    const int ks = idx / T::SBLK, sb = idx % T::SBLK;
                    return *(const LDS_AS unsigned long long*)(sg + k8off[sb] + k8x[sb][ks & 1] + 64 * (ks >> 1));
                }
            };
            acc_t sacc[T::SBLK][2];
#pragma unroll
            for (int sb = 0; sb < T::SBLK; ++sb) sacc[sb][0] = sacc[sb][1] = (acc_t){};
            kraw_t kring[PF];
#pragma unroll
            for (int i = 0; i < PF; ++i) kring[i] = k_frag(i);
#pragma unroll
            for (int idx = 0; idx < NSTEP; ++idx) {
                const int ks = idx / T::SBLK, sb = idx % T::SBLK;
                const bf16x8_t kf = to_bf16x8(kring[idx % PF]);
                if (idx + PF < NSTEP) kring[idx % PF] = k_frag(idx + PF);
                sacc[sb][ks & 1] = M::mma(kf, qf[ks], sacc[sb][ks & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            acc_t sfin[T::SBLK];
#pragma unroll
            for (int sb = 0; sb < T::SBLK; ++sb) sfin[sb] = sacc[sb][0] + sacc[sb][1];

            // ---- online softmax (lane-local head) ------------------------------
            // sfin[sb][i] is the score of token tok0 + sb*WH + toff(i), head hl.
            float tmax = -INFINITY;
            const bool full = tvalid >= NT;
            // fp8: per-token scale of every accumulator entry's token
            float tsc[T::SBLK][M::kAcc];
#pragma unroll
            for (int sb = 0; sb < T::SBLK; ++sb)
#pragma unroll
                for (int i = 0; i < M::kAcc; ++i) {
                    // fp8: entry (sb, i) is token 2 (4 grp + i) + sb of the wave's 32
                    tsc[sb][i] = FP8 ? *(const LDS_AS float*)(sg + T::SCL8 + (tok0 + 2 * (grp * 4 + i) + sb) * 4)
                                     : 1.0f;
                }
#pragma unroll
            for (int sb = 0; sb < T::SBLK; ++sb) {
#pragma unroll
                for (int i = 0; i < M::kAcc; ++i) {
                    const int toff = (WH == 16) ? (grp * 4 + i) : ((i >> 2) * 8 + grp * 4 + (i & 3));
                    const int tok = FP8 ? 2 * (grp * 4 + i) + sb : sb * WH + toff;
                    float v = sfin[sb][i] * (FP8 ? p.scale_log2 * tsc[sb][i] : p.scale_log2);
                    if (!full && tok >= tvalid) v = -INFINITY;
                    sfin[sb][i] = v;
                    tmax = fmaxf(tmax, v);
                }
            }
            if (WH == 16) tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float m_new = fmaxf(m_run, tmax);
            if (__any(m_new > m_run + kRescaleThreshold)) {
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int mb = 0; mb < T::MBLK; ++mb) o[mb] *= alpha;
                m_run = m_new;
            }
            // P^T as the B operand of O^T += V^T . P^T.  WH = 16: slots 0..3 are
            // block 2u's tokens grp*4+i, slots 4..7 block 2u+1's.  WH = 32: MFMA
            // u = 2sb + v of block sb uses accumulator entries 8v .. 8v+7.
            constexpr int NPB = NT / 32 * (WH == 16 ? 1 : 2);
            bf16x8_t pb[NPB];
#pragma unroll
            for (int sb = 0; sb < T::SBLK; ++sb) {
#pragma unroll
                for (int i = 0; i < M::kAcc; ++i) {
                    const float e = exp2_fast(sfin[sb][i] - m_run);
                    l_run += e;
                    const float pe = FP8 ? e * tsc[sb][i] : e;  // fp8: dequantising scale of V
                    if (WH == 16)
                        pb[sb >> 1][(sb & 1) * 4 + i] = (__bf16)pe;
                    else
                        pb[sb * 2 + (i >> 3)][i & 7] = (__bf16)pe;
                }
            }

            // ---- O^T += V^T . P^T ------------------------------------------------
            // MFMA u covers 32 (WH=16) or 16 (WH=32) tokens starting at tok0 + u*TPU.
            // Transposed V fragments stream through a register ring like K above.
            constexpr int TPU = (WH == 16) ? 32 : 16;
            constexpr int NPV = NPB * T::MBLK;
            constexpr int PFV = 4;
            auto v_frag = [&](int idx) -> kraw_t {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                if constexpr (FP8) {
                    typedef int v2i_t __attribute__((ext_vector_type(2)));
                    const v2i_t c = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                        (LDS_AS v2i_t*)(sg + v8off + v8x[mb & 3] + 64 * (mb >> 2)));
                    return __builtin_bit_cast(unsigned long long, c);
                } else {
                    const int q = mb % NQV;
                    const int blk = (mb / NQV) * 256 + u * TPU * 1024;
                    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (LDS_AS i16x4_t*)(tb + voff0[q] + blk));
                    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (LDS_AS i16x4_t*)(tb + (WH == 16 ? voff0[q] + 16 * 1024 : voff1[q]) + blk));
                    return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo),
                                                   __builtin_bit_cast(bf16x4_t, hi), 0, 1, 2, 3, 4, 5, 6, 7);
                }
            };
            kraw_t vring[PFV];
#pragma unroll
            for (int i = 0; i < PFV; ++i) vring[i] = v_frag(i);
#pragma unroll
            for (int idx = 0; idx < NPV; ++idx) {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                const bf16x8_t a = to_bf16x8(vring[idx % PFV]);
                if (idx + PFV < NPV) vring[idx % PFV] = v_frag(idx + PFV);
                o[mb] = M::mma(a, pb[u], o[mb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        for (int it0 = 0; it0 < n_tiles; it0 += STAGES) {
            tile_body(IC<0>{}, it0);
            if (STAGES > 1 && it0 + 1 < n_tiles) tile_body(IC<(STAGES > 1 ? 1 : 0)>{}, it0 + 1);
            if (STAGES > 2 && it0 + 2 < n_tiles) tile_body(IC<(STAGES > 2 ? 2 : 0)>{}, it0 + 2);
            if (STAGES > 3 && it0 + 3 < n_tiles) tile_body(IC<(STAGES > 3 ? 3 : 0)>{}, it0 + 3);
        }

        // ---- segment epilogue ------------------------------------------------
        if (WH == 16) l_run += __shfl_xor(l_run, 16, 64);
        l_run += __shfl_xor(l_run, 32, 64);

        bool writer = true;
        if (TS > 1) {
            // Waves ts >= 1 publish (m, l, O); wave ts == 0 of the same head
            // subgroup merges them.  The merge area overlays the tile stages,
            // so first every wave must have finished reading the last tile.
            wg_barrier();
            float* area = (float*)(FP8 ? stage_lds<T::STG8_BYTES, 0>() : stage_lds<T::TILE_BYTES, 0>());
            if (ts > 0) {
                float* dst = area + ((size_t)((ts - 1) * HS + hs) * T::MERGE_FLOATS) * 64;
                dst[lane] = m_run;
                dst[64 + lane] = l_run;
#pragma unroll
                for (int mb = 0; mb < T::MBLK; ++mb)
#pragma unroll
                    for (int i = 0; i < M::kAcc; ++i) dst[(2 + mb * M::kAcc + i) * 64 + lane] = o[mb][i];
                writer = false;
            }
            wg_barrier();
            if (ts == 0) {
#pragma unroll
                for (int t2 = 1; t2 < TS; ++t2) {
                    const float* src = area + ((size_t)((t2 - 1) * HS + hs) * T::MERGE_FLOATS) * 64;
                    const float m2 = src[lane];
                    const float l2 = src[64 + lane];
                    const float mm = fmaxf(m_run, m2);
                    const float a1 = exp2_fast(m_run - mm);
                    const float a2 = exp2_fast(m2 - mm);
                    l_run = l_run * a1 + l2 * a2;
#pragma unroll
                    for (int mb = 0; mb < T::MBLK; ++mb)
#pragma unroll
                        for (int i = 0; i < M::kAcc; ++i)
                            o[mb][i] = o[mb][i] * a1 + src[(2 + mb * M::kAcc + i) * 64 + lane] * a2;
                    m_run = mm;
                }
            }
        }

        if (writer && head_ok) {
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
            // O^T accumulator entry i of block mb is latent column
            //   WH=16: mb*16 + grp*4 + i       WH=32: mb*32 + (i/4)*8 + grp*4 + i%4
            // a row finished here writes out/lse; otherwise its slot's partial
            // (normalised, in the input dtype) and partial lse
            __bf16* orow = (final_out ? (__bf16*)p.out + (size_t)r * p.h * kDc
                                      : (__bf16*)p.po + (size_t)slot * p.h * kDc) + (size_t)head * kDc;
#pragma unroll
            for (int mb = 0; mb < T::MBLK; ++mb)
#pragma unroll
                for (int q4 = 0; q4 < M::kAcc / 4; ++q4) {
                    const int c = mb * WH + q4 * 8 + grp * 4;
                    bf16x4_t v;
                    v[0] = (__bf16)(o[mb][q4 * 4 + 0] * inv);
                    v[1] = (__bf16)(o[mb][q4 * 4 + 1] * inv);
                    v[2] = (__bf16)(o[mb][q4 * 4 + 2] * inv);
                    v[3] = (__bf16)(o[mb][q4 * 4 + 3] * inv);
                    *(bf16x4_t*)(orow + c) = v;
                }
            if (grp == 0) (final_out ? p.lse + (size_t)r * p.h : p.plse + (size_t)slot * p.h)[head] = lse_v;
        }

        pos = seg_end;
        if (pos >= end) break;
        // The next segment reuses the LDS stages: every wave must be done.
        wg_barrier();
        ++r;
        while (pv.cu()[r + 1] <= pos) ++r;  // skip empty rows
    }
}

template <int WH, int HS, int TS, int NT, int STAGES, bool FP8>
__global__ __launch_bounds__(HS * TS * 64) void decode_bf16_kernel(DecodeParams p)
{
    clock_stamp(p.clock_stamps, 0);
    decode_bf16_body<WH, HS, TS, NT, STAGES, FP8>(p);
    clock_stamp(p.clock_stamps, 1);
}


// ---------------------------------------------------------------------------
// Paired-wave, software-pipelined variant for many heads
// (v_mfma_f32_32x32x16_bf16 throughout).
//
// A wave that owned 32 heads outright would hold 144 VGPRs of queries and
// 256 accumulator registers of output, leaving no room for the score tile.
// Here the two waves of a pair share 32 heads:
//   * scores: wave q (0/1) contracts half of the 576 latent dims -- region-A
//     chunks [32q, 32q+32) (latent columns 256q .. 256q+255) and region-B
//     chunks [4q, 4q+4) (rope columns 32q .. 32q+31) -- so it keeps only 72
//     VGPRs of queries.  The two fp32 partial score tiles are exchanged
//     through LDS and summed (fp addition is commutative, so both waves derive
//     bit-identical softmax state);
//   * weighted sum: wave q accumulates latent columns 256q .. 256q+255 only
//     (128 accumulator registers).
// With one wave per SIMD, the matrix unit would idle while the wave does
// softmax arithmetic and LDS exchange, so each iteration overlaps work of two
// tiles: while the score MFMAs of tile i+1 run, the vector ALU computes the
// softmax of tile i; while the weighted-sum MFMAs of tile i run, the partial
// scores of tile i+1 go to the partner.  Tiles are 32 tokens; a STAGES-deep
// ring of LDS stages is refilled by DMA as soon as every wave has finished a
// tile (two tiles are in use at any time, STAGES-2 are in flight).
// ---------------------------------------------------------------------------
template <int P, int STAGES>
struct PairTiling {
    static constexpr int NW = 2 * P;
    static constexpr int THREADS = NW * 64;
    static constexpr int HG = 32 * P;
    static constexpr int N = 32;
    static constexpr int A_BYTES = N * 1024;
    static constexpr int TILE_BYTES = N * kRowBytesBf16;
    static constexpr int XBUF_BYTES = NW * 64 * 16 * 4;   // one 32x32 fp32 tile per wave
    static constexpr int LOADS_A = N / NW;
    static constexpr int GROUPS_B = N / 8;
    static constexpr int LOADS_B_MAX = (GROUPS_B + NW - 1) / NW;
    static constexpr int LOADS = LOADS_A + LOADS_B_MAX;
    static constexpr int KA = 16;   // k steps (of 16) in region A per wave
    static constexpr int KB = 2;    // k steps in region B per wave
    static constexpr int KS = KA + KB;
    static constexpr int MBLK = 8;  // 32-column output blocks per wave
    static_assert(N % NW == 0, "region A rows split evenly over waves");
    static_assert(STAGES >= 3 && STAGES <= 4, "pipeline depth");
    static_assert(GROUPS_B % NW == 0, "exact vmcnt accounting needs even B split");
    static_assert(STAGES * TILE_BYTES + XBUF_BYTES <= 160 * 1024, "LDS budget");
    static_assert((STAGES - 1) * LOADS <= 63, "vmcnt range");
};

template <int P, int STAGES>
__global__ __launch_bounds__(P * 128) void decode_pair_kernel(DecodeParams p)
{
    using T = PairTiling<P, STAGES>;
    using M = Mfma<32>;
    typedef f32x16_t acc_t;

    const int lane = threadIdx.x & 63;
    // wave index is uniform: keep it (and all row/DMA arithmetic built on it) scalar
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pr = wave >> 1;          // pair inside the workgroup
    const int q = wave & 1;            // contraction half / output-column half
    const int hl = lane & 31;          // head inside the pair's 32
    const int grp = lane >> 5;         // k-slot group (0/1)

    int k, hg;
    block_work(p.n_chunks, p.n_hg, k, hg);
    const PlanView pv{const_cast<int32_t*>(p.plan), p.b};
    const int total = p.plan[0];
    const int chunk = p.plan[1];
    int r = pv.chunk_row()[k];
    if (r < 0) return;
    int pos = k * chunk;
    const int end = pos + min(chunk, total - pos);

    const __bf16* __restrict__ qg = (const __bf16*)p.q;
    const unsigned char* __restrict__ cg = (const unsigned char*)p.cache;
    const int head = hg * T::HG + pr * 32 + hl;
    const bool head_ok = head < p.h;
    lds_byte* const xbuf = stage_lds<T::XBUF_BYTES, 7>();
    const float c2 = p.scale_log2;

    // ---- per-lane LDS offsets --------------------------------------------
    // K reads: token row rr = lane & 31, k step j of region A -> logical chunk
    // 32q + 2j + grp;  region B step j -> chunk 4q + 2j + grp.
    const int rr = lane & 31;
    int koffA[8], koffB[T::KB];
    {
        const int x = M::xa(rr & 15);
        const int xbv = xb(rr & 15);
#pragma unroll
        for (int j = 0; j < 8; ++j) koffA[j] = rr * 1024 + (((2 * j + grp) ^ x) << 4) + q * 512;
#pragma unroll
        for (int j = 0; j < T::KB; ++j) koffB[j] = T::A_BYTES + rr * 128 + (((4 * q + 2 * j + grp) ^ xbv) << 4);
    }
    // V^T reads (transposed, region A): rows u*16 + grp*4 + (lane&15)/4 (+8),
    // columns 256q + 32mb + 16*((lane>>4)&1) + 4*(lane&3).
    int voff0[4], voff1[4];
    {
        const int row0 = (lane >> 5) * 4 + ((lane & 15) >> 2);
        const int x0 = M::xa(row0 & 15), x1 = M::xa((row0 + 8) & 15);
        const int cc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            voff0[j] = row0 * 1024 + (((4 * j + cc) ^ x0) << 4) + ((lane & 1) << 3) + q * 512;
            voff1[j] = (row0 + 8) * 1024 + (((4 * j + cc) ^ x1) << 4) + ((lane & 1) << 3) + q * 512;
        }
    }

    while (true) {
        const int row_lo = pv.cu()[r];
        const int row_hi = pv.cu()[r + 1];
        const int seg_end = min(end, row_hi);
        const int seg_a = pos - row_lo;
        const int seg_len = seg_end - pos;
        const int split_j = k - row_lo / chunk;
        const bool final_out = pv.nsplit()[r] == 1;
        const int slot = pv.base()[r] + split_j;
        const unsigned char* seg_base = cg + ((size_t)r * p.t_max + seg_a) * kRowBytesBf16;
        const int n_tiles = (seg_len + T::N - 1) / T::N;

        // Queries for this wave's contraction half: B operand, lane -> head hl,
        // k-slots grp*8 .. +7 of each 16-wide step.
        bf16x8_t qf[T::KS];
        {
            const bf16x8_t* qrow =
                (const bf16x8_t*)(qg + ((size_t)r * p.h + (head_ok ? head : 0)) * kDqk);
#pragma unroll
            for (int j = 0; j < T::KA; ++j) {
                bf16x8_t v = qrow[(256 * q + 16 * j) / 8 + grp];
                if (!head_ok) v = (bf16x8_t){};
                qf[j] = v;
            }
#pragma unroll
            for (int j = 0; j < T::KB; ++j) {
                bf16x8_t v = qrow[(512 + 32 * q + 16 * j) / 8 + grp];
                if (!head_ok) v = (bf16x8_t){};
                qf[T::KA + j] = v;
            }
        }

        auto issue_tile = [&](auto SC, int tile) {
            const int t0 = tile * T::N;
            const int last = min(T::N, seg_len - t0) - 1;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(seg_base + (size_t)t0 * kRowBytesBf16), (short)0,
                (last + 1) * kRowBytesBf16, kBufferFlags);
            lds_byte* st = stage_lds<T::TILE_BYTES, decltype(SC)::value>();
#pragma unroll
            for (int j = 0; j < T::LOADS_A; ++j) {
                const int row = wave + j * T::NW;
                const int srow = min(row, last);
                const unsigned voff = (unsigned)((lane ^ M::xa(row & 15)) << 4);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + row * 1024), 16, voff,
                    __builtin_amdgcn_readfirstlane(srow * kRowBytesBf16), 0, 0);
            }
#pragma unroll
            for (int j = 0; j < T::LOADS_B_MAX; ++j) {
                const int gb = wave + j * T::NW;
                const int row = gb * 8 + (lane >> 3);
                const int srow = min(row, last);
                const int lc = (lane & 7) ^ xb(row & 15);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rsrc, (LDS_AS void*)(st + T::A_BYTES + gb * 1024), 16,
                    (unsigned)(srow * kRowBytesBf16 + 1024 + lc * 16), 0, 0, 0);
            }
        };
        // Wait until tile `t` has landed: tiles issued after it are t+1 ..
        // min(t+STAGES-2, n_tiles-1) (the ring never holds more than that).
        auto wait_tile = [&](int t) {
            const int after = min(STAGES - 2, n_tiles - 1 - t);
            if (after >= 2)
                wait_vmcnt<(STAGES > 3 ? 2 : 0) * T::LOADS>();
            else if (after == 1)
                wait_vmcnt<T::LOADS>();
            else
                wait_vmcnt<0>();
        };

        acc_t o[T::MBLK];
#pragma unroll
        for (int mb = 0; mb < T::MBLK; ++mb) o[mb] = (acc_t){};
        float m_run = kNegBig;
        float l_run = 0.f;

        // K fragment j of the tile in stage SB.
        auto k_frag = [&](lds_byte* tb, int j) -> bf16x8_t {
            const lds_byte* a = (j < T::KA) ? tb + koffA[j % 8] + (j / 8) * 256 : tb + koffB[j - T::KA];
            return *(const LDS_AS bf16x8_t*)a;
        };
        // Transposed V fragment idx (u = idx / MBLK token half, mb = idx % MBLK).
        auto v_frag = [&](lds_byte* tb, int idx) -> bf16x8_t {
            const int u = idx / T::MBLK, mb = idx % T::MBLK;
            const int blk = (mb / 4) * 256 + u * 16 * 1024;
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + voff0[mb % 4] + blk));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4_t*)(tb + voff1[mb % 4] + blk));
            return __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                           0, 1, 2, 3, 4, 5, 6, 7);
        };
        // Exchange this wave's partial score tile with the partner's: returns the sum.
        auto exchange = [&](const acc_t& part) -> acc_t {
            LDS_AS f32x4_t* mine = (LDS_AS f32x4_t*)(xbuf + wave * 4096);
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4)
                mine[i4 * 64 + lane] = (f32x4_t){part[4 * i4], part[4 * i4 + 1], part[4 * i4 + 2], part[4 * i4 + 3]};
            lds_exchange_barrier();
            const LDS_AS f32x4_t* other = (const LDS_AS f32x4_t*)(xbuf + (wave ^ 1) * 4096);
            f32x4_t ov[4];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) ov[i4] = other[i4 * 64 + lane];
            acc_t sum;
#pragma unroll
            for (int i = 0; i < 16; ++i) sum[i] = part[i] + ov[i >> 2][i & 3];
            return sum;
        };

        // Softmax pieces on the (raw) score tile sc of tile t; see the header.
        // sc[i]: token (i/4)*8 + grp*4 + i%4 of the tile, head hl.
        float sm_tmax = 0.f;
        auto sm_max = [&](acc_t& sc, int t) {
            const int tvalid = __builtin_amdgcn_readfirstlane(seg_len - t * T::N);
            if (tvalid < T::N) {  // tail tile: scores of missing tokens -> -inf
                // token of entry i is (i/4)*8 + i%4 + 4*grp: compare the constant
                // part against one per-lane limit
                const int lim = tvalid - 4 * grp;
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if ((i >> 2) * 8 + (i & 3) >= lim) sc[i] = -INFINITY;
            }
            float tm = fmaxf(fmaxf(sc[0], sc[1]), sc[2]);
#pragma unroll
            for (int i = 3; i < 16; ++i) tm = fmaxf(tm, sc[i]);
            // the head's other lane group is lane ^ 32
            sm_tmax = max_xor32(tm) * c2;
        };
        auto sm_rescale = [&]() {
            const float m_new = fmaxf(m_run, sm_tmax);
            if (__any(m_new > m_run + kRescaleThreshold)) {
                const float alpha = exp2_fast(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int mb = 0; mb < T::MBLK; ++mb) o[mb] *= alpha;
                m_run = m_new;
            }
        };
        auto sm_exp = [&](const acc_t& sc, bf16x8_t* pb, int i0) {
#pragma unroll
            for (int i = i0; i < i0 + 4; ++i) {
                const float e = exp2_fast(__builtin_fmaf(sc[i], c2, -m_run));
                l_run += e;
                pb[i >> 3][i & 7] = (__bf16)e;
            }
        };

        // ---- prologue: fill the ring, scores of tile 0 ----------------------
        if (0 < n_tiles) issue_tile(IC<0>{}, 0);
        if (1 < n_tiles) issue_tile(IC<1>{}, 1);
        if (2 < n_tiles) issue_tile(IC<2>{}, 2);
        if (STAGES > 3 && 3 < n_tiles) issue_tile(IC<(STAGES > 3 ? 3 : 0)>{}, 3);
        acc_t scur;  // summed scores of the tile about to be consumed
        if (n_tiles > 0) {
            wait_tile(0);
            lds_exchange_barrier();
            lds_byte* tb = stage_lds<T::TILE_BYTES, 0>();
            acc_t sacc[2] = {(acc_t){}, (acc_t){}};
#pragma unroll
            for (int j = 0; j < T::KS; ++j) sacc[j & 1] = M::mma(k_frag(tb, j), qf[j], sacc[j & 1]);
            scur = exchange(sacc[0] + sacc[1]);
        }

        // Weighted-sum MFMAs of the tile in stage tc with probabilities pb;
        // mid() runs half way through (publishing the next tile's partial scores).
        auto pv_phase = [&](lds_byte* tc, const bf16x8_t (&pb)[2], auto&& mid) {
            constexpr int NPV = 2 * T::MBLK;
            constexpr int PFV = 4;
            bf16x8_t vring[PFV];
#pragma unroll
            for (int j = 0; j < PFV; ++j) vring[j] = v_frag(tc, j);
#pragma unroll
            for (int idx = 0; idx < NPV; ++idx) {
                const int u = idx / T::MBLK, mb = idx % T::MBLK;
                const bf16x8_t a = vring[idx % PFV];
                if (idx + PFV < NPV) vring[idx % PFV] = v_frag(tc, idx + PFV);
                o[mb] = M::mma(a, pb[u], o[mb]);
                if (idx == 8) mid();
                __builtin_amdgcn_sched_barrier(0);
            }
        };

        // ---- steady state: iteration i consumes tile i (PV) and scores tile i+1
        auto iter = [&](auto SC, int i) {
            constexpr int SI = decltype(SC)::value;              // stage of tile i
            constexpr int SN = (SI + 1) % STAGES;                // stage of tile i+1
            lds_byte* tc = stage_lds<T::TILE_BYTES, SI>();
            lds_byte* tn = stage_lds<T::TILE_BYTES, SN>();
            wait_tile(i + 1);
            lds_exchange_barrier();  // tile i+1 visible to all waves
            // Phase A: score MFMAs of tile i+1 interleaved with the softmax of tile i.
            acc_t sacc[2] = {(acc_t){}, (acc_t){}};
            bf16x8_t pb[2];
            constexpr int PF = 4;
            bf16x8_t kring[PF];
#pragma unroll
            for (int j = 0; j < PF; ++j) kring[j] = k_frag(tn, j);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < T::KS; ++j) {
                const bf16x8_t kf = kring[j % PF];
                if (j + PF < T::KS) kring[j % PF] = k_frag(tn, j + PF);
                sacc[j & 1] = M::mma(kf, qf[j], sacc[j & 1]);
                if (j == 0) sm_max(scur, i);
                if (j == 3) sm_rescale();
                if (j == 5) sm_exp(scur, pb, 0);
                if (j == 7) sm_exp(scur, pb, 4);
                if (j == 9) sm_exp(scur, pb, 8);
                if (j == 11) sm_exp(scur, pb, 12);
                __builtin_amdgcn_sched_barrier(0);
            }
            // Phase B: weighted-sum MFMAs of tile i; partial scores of tile i+1
            // go to the partner half way through.
            acc_t part;
            pv_phase(tc, pb, [&]() {
                part = sacc[0] + sacc[1];
                LDS_AS f32x4_t* mine = (LDS_AS f32x4_t*)(xbuf + wave * 4096);
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4)
                    mine[i4 * 64 + lane] = (f32x4_t){part[4 * i4], part[4 * i4 + 1], part[4 * i4 + 2], part[4 * i4 + 3]};
            });
            // Every wave is done with tile i and has published its partial
            // scores of tile i+1: refill stage SI, then finish the exchange.
            lds_exchange_barrier();
            if (i + STAGES < n_tiles) issue_tile(IC<SI>{}, i + STAGES);
            const LDS_AS f32x4_t* other = (const LDS_AS f32x4_t*)(xbuf + (wave ^ 1) * 4096);
            f32x4_t ov[4];
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) ov[i4] = other[i4 * 64 + lane];
#pragma unroll
            for (int i2 = 0; i2 < 16; ++i2) scur[i2] = part[i2] + ov[i2 >> 2][i2 & 3];
        };
        // Last tile: softmax and weighted sum only.  Every DMA has completed by
        // now (the last wait was vmcnt(0)), so a runtime-selected stage is fine.
        auto last_iter = [&](int i) {
            const int st = i % STAGES;
            lds_byte* tc = st == 0 ? stage_lds<T::TILE_BYTES, 0>()
                         : st == 1 ? stage_lds<T::TILE_BYTES, 1>()
                         : st == 2 ? stage_lds<T::TILE_BYTES, 2>()
                                   : stage_lds<T::TILE_BYTES, (STAGES > 3 ? 3 : 0)>();
            bf16x8_t pb[2];
            sm_max(scur, i);
            sm_rescale();
            sm_exp(scur, pb, 0);
            sm_exp(scur, pb, 4);
            sm_exp(scur, pb, 8);
            sm_exp(scur, pb, 12);
            pv_phase(tc, pb, []() {});
        };

        const int n_full = n_tiles - 1;  // iterations that also score a next tile
        for (int i0 = 0; i0 < n_full; i0 += STAGES) {
            iter(IC<0>{}, i0);
            if (i0 + 1 < n_full) iter(IC<1>{}, i0 + 1);
            if (i0 + 2 < n_full) iter(IC<2>{}, i0 + 2);
            if (STAGES > 3 && i0 + 3 < n_full) iter(IC<(STAGES > 3 ? 3 : 0)>{}, i0 + 3);
        }
        if (n_tiles > 0) last_iter(n_full);

        // ---- segment epilogue ----------------------------------------------
        l_run += __shfl_xor(l_run, 32, 64);
        if (head_ok) {
            const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
            const float lse_v = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
            // accumulator entry i of block mb: column 256q + 32mb + (i/4)*8 + grp*4 + i%4
            __bf16* orow = (final_out ? (__bf16*)p.out + (size_t)r * p.h * kDc
                                      : (__bf16*)p.po + (size_t)slot * p.h * kDc) + (size_t)head * kDc + 256 * q;
#pragma unroll
            for (int mb = 0; mb < T::MBLK; ++mb)
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) {
                    bf16x4_t v;
                    v[0] = (__bf16)(o[mb][q4 * 4 + 0] * inv);
                    v[1] = (__bf16)(o[mb][q4 * 4 + 1] * inv);
                    v[2] = (__bf16)(o[mb][q4 * 4 + 2] * inv);
                    v[3] = (__bf16)(o[mb][q4 * 4 + 3] * inv);
                    *(bf16x4_t*)(orow + mb * 32 + q4 * 8 + grp * 4) = v;
                }
            if (q == 0 && grp == 0) (final_out ? p.lse + (size_t)r * p.h : p.plse + (size_t)slot * p.h)[head] = lse_v;
        }

        pos = seg_end;
        if (pos >= end) break;
        wg_barrier();
        ++r;
        while (pv.cu()[r + 1] <= pos) ++r;
    }
}

template <int P, int STAGES>
hipError_t launch_pair_variant(const DecodeParams& p, hipStream_t stream)
{
    using T = PairTiling<P, STAGES>;
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    decode_pair_kernel<P, STAGES><<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

template <int WH, int HS, int TS, int NT, int STAGES>
hipError_t launch_variant(const DecodeParams& p, hipStream_t stream)
{
    using T = Tiling<WH, HS, TS, NT, STAGES>;
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    decode_bf16_kernel<WH, HS, TS, NT, STAGES, false><<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

// fp8 latent cache (p.cache holds e4m3 codes, p.cache_scale per-token scales)
template <int WH, int HS, int TS, int NT, int STAGES>
hipError_t launch_variant_fp8(const DecodeParams& p, hipStream_t stream)
{
    using T = Tiling<WH, HS, TS, NT, STAGES>;
    const unsigned grid = (unsigned)p.n_chunks * (unsigned)p.n_hg;
    decode_bf16_kernel<WH, HS, TS, NT, STAGES, true><<<grid, T::THREADS, 0, stream>>>(p);
    return hipGetLastError();
}

typedef hipError_t (*LaunchFn)(const DecodeParams&, hipStream_t);

// The launcher of variant I (fp8: its fp8-cache form, nullptr if it has none),
// instantiated from the template arguments the table lists.
template <int I, bool FP8>
constexpr LaunchFn variant_launcher()
{
    constexpr VariantInfo v = kVariantInfo[I];
    if constexpr (FP8) {
        if constexpr (v.family == KernelFamily::Tiled && v.fp8_name != nullptr)
            return &launch_variant_fp8<v.targs[0], v.targs[1], v.targs[2], v.targs[3], v.targs[4]>;
        else if constexpr (v.family == KernelFamily::Wide && v.fp8_name != nullptr)
            return &launch_decode_wide_fp8;
        else
            return nullptr;
    } else if constexpr (v.family == KernelFamily::Tiled) {
        return &launch_variant<v.targs[0], v.targs[1], v.targs[2], v.targs[3], v.targs[4]>;
    } else if constexpr (v.family == KernelFamily::Pair) {
        return &launch_pair_variant<v.targs[0], v.targs[1]>;
    } else if constexpr (v.family == KernelFamily::Split) {
        return &launch_decode_colsplit;
    } else {
        return &launch_decode_wide<v.targs[0], v.targs[1]>;
    }
}

struct Launchers {
    LaunchFn launch, launch_fp8;
};

template <int... I>
constexpr auto make_launchers(std::integer_sequence<int, I...>)
{
    return std::array<Launchers, sizeof...(I)>{Launchers{variant_launcher<I, false>(), variant_launcher<I, true>()}...};
}

const auto kLaunchers = make_launchers(std::make_integer_sequence<int, kNumVariants>{});

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int heads_per_group, int variant,
                              hipStream_t stream)
{
    const int i = find_variant_index(heads_per_group, variant);
    if (i < 0) return hipErrorInvalidValue;
    if (p.cache_scale != nullptr) {
        if (kLaunchers[i].launch_fp8 == nullptr) return hipErrorInvalidValue;
        return kLaunchers[i].launch_fp8(p, stream);
    }
    return kLaunchers[i].launch(p, stream);
}

}  // namespace mla355
