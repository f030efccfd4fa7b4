// Internal declarations shared by the libmla355 host layer and its kernels.
// Not installed; the public ABI is include/mla355.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace mla355 {

constexpr int kDc = 512;       // latent width
constexpr int kDr = 64;        // RoPE key width
constexpr int kDqk = 576;      // latent row width
constexpr int kDk = 128;       // per-head query width (absorb q)
constexpr int kDv = 128;       // per-head value width (absorb o)
constexpr int kRowBytesBf16 = kDqk * 2;  // 1152 B: 72 chunks of 16 B

// ---------------------------------------------------------------------------
// Split plan, built on the device from seqlens (plan_build.h): by plan_kernel
// into the workspace, or by each wide attention workgroup into its own LDS.
// The batch is viewed as one concatenated token sequence (row 0's tokens,
// then row 1's, ...).  It is cut into n_chunks equal chunks of `chunk`
// tokens; each chunk (per head group) is one workgroup's work.  A chunk may
// cover the tail of one row and the head of the next; each (row, chunk)
// intersection is a "segment" with its own softmax state.  A row cut into
// several segments writes partials (normalised output in the dtype of the
// call, fp32 lse) into numbered slots, merged afterwards by the log-sum-exp
// combine kernel; a row that lies inside one chunk writes its final output
// directly.
//
// int32 layout (offsets in elements):
//   [0] total tokens  [1] chunk  [2] n_chunks  [3] unused
//   cu[b+1]        at 4              prefix sums of clamped lengths
//   base[b]        at 4 + (b+1)      first partial slot of each row
//   nsplit[b]      at 4 + (b+1) + b  segments per row (0 for an empty row)
//   chunk_row[n]   at 4 + (b+1) + 2b first row touched by chunk k (-1: idle)
// ---------------------------------------------------------------------------
struct PlanView {
    int32_t* p;
    int b;
    __host__ __device__ int32_t* cu() const { return p + 4; }
    __host__ __device__ int32_t* base() const { return p + 4 + (b + 1); }
    __host__ __device__ int32_t* nsplit() const { return p + 4 + (b + 1) + b; }
    __host__ __device__ int32_t* chunk_row() const { return p + 4 + (b + 1) + 2 * b; }
};

struct WorkspaceLayout {
    size_t plan_ints;   // int32 elements of the plan
    size_t plse_off;    // byte offset of partial lse  [slots, h] fp32
    size_t po_off;      // byte offset of partial out  [slots, h, 512] (dtype of the call)
    size_t clock_off;   // byte offset of the engine-clock stamps (the last kClockBytes)
    size_t total;       // bytes
    int max_slots;
};

// Engine-clock stamps (opt-in: config reserved[0] bit 0): the attention
// kernel's workgroup 0 writes four uint64 at clock_off: the shader clock
// (s_memtime) and the 100 MHz real-time counter (s_memrealtime) at its start,
// then both again at its end.
constexpr size_t kClockBytes = 256;
constexpr int kConfigRecordClock = 1;

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// part_bytes: bytes per partial-output element (2 for bf16 calls, 4 for fp32).
inline WorkspaceLayout workspace_layout(int b, int h, int n_chunks, int part_bytes)
{
    WorkspaceLayout w;
    w.plan_ints = 4 + (size_t)(b + 1) + 2 * (size_t)b + (size_t)n_chunks;
    w.max_slots = n_chunks + b;  // every chunk adds at most one cut inside a row
    w.plse_off = align_up(w.plan_ints * 4, 256);
    w.po_off = align_up(w.plse_off + (size_t)w.max_slots * h * 4, 256);
    w.clock_off = align_up(w.po_off + (size_t)w.max_slots * h * kDc * part_bytes, 256);
    w.total = w.clock_off + kClockBytes;
    return w;
}

struct DecodeParams {
    const void* q;        // [b,h,576] dtype
    const void* cache;    // [b,t_max,576] dtype
    const int32_t* plan;  // plan (see above)
    void* out;            // [b,h,512] dtype
    float* lse;           // [b,h]
    float* plse;          // [slots,h]
    void* po;             // [slots,h,512] normalised partial outputs, dtype of the call
    // paged cache (block_table != nullptr): cache is the block pool
    // [num_blocks, block_size, 576]; row r's token t sits in block
    // block_table[r * max_blocks + t / block_size] (clamped to the pool) at
    // row t % block_size; t_max = max_blocks * block_size; the plan is
    // tile-aligned and seqlens gives the true lengths.
    const int32_t* block_table;
    const int32_t* seqlens;
    // fp8 cache (cache_scale != nullptr): cache holds OCP e4m3 codes
    // [b, t_max, 576] and cache_scale [b, t_max] the per-token scales
    const float* cache_scale;
    int num_blocks, block_size, max_blocks;
    // several causal query tokens per row (causal kernels only): the h
    // "heads" are q_len tokens x heads_per_token heads
    int q_len, heads_per_token;
    int b, h, t_max;
    int n_chunks;         // chunks per head group
    int n_hg;             // head groups
    float scale_log2;     // softmax_scale * log2(e)
    // plan_in_kernel != 0 (wide kernels only): no plan kernel ran; every
    // workgroup builds the plan in LDS from seqlens (with plan_min_chunk and
    // plan_align), workgroup 0 leaves a copy at `plan` for the combine, and
    // the attention kernel gives rows with no tokens out = 0, lse = -inf.
    int plan_in_kernel, plan_min_chunk, plan_align;
    // engine-clock stamps (see kClockBytes), nullptr when not asked for
    unsigned long long* clock_stamps;
};

// Largest batch and chunk count whose plan an attention workgroup builds in
// its own LDS (11 KB); larger ones go through plan_kernel.
constexpr int kPlanLdsRows = 256;
constexpr int kPlanLdsChunks = 2048;
constexpr int kPlanLdsInts = 4 + (kPlanLdsRows + 1) + 2 * kPlanLdsRows + kPlanLdsChunks;

// Launchers (return hipGetLastError() after the launch).
// launch_plan also writes out = 0, lse = -inf for every row with no tokens
// (no decode workgroup touches such a row).  align > 1 lays the plan over
// lengths (and a chunk) rounded up to multiples of align (paged cache).
hipError_t launch_plan(const int32_t* seqlens, int b, int h, int t_max, int n_chunks, int min_chunk,
                       int align, int32_t* plan, bool bf16, void* out, float* lse, hipStream_t stream);
// n_chunks picks the combine's layout (rows with many segments get a
// workgroup per (row, head)); any value gives the same result.
hipError_t launch_combine(bool bf16, const int32_t* plan, int b, int h, int n_chunks, const float* plse,
                          const void* po, void* out, float* lse, hipStream_t stream);

// bf16 decode variants (table in variants.h, queries in variants.cpp).
// heads_per_group selects the family; variant picks a tiling inside it
// (0 = default).  launch_decode_bf16 returns hipErrorInvalidValue if absent.
bool bf16_variant_exists(int heads_per_group, int variant);
int bf16_tile_tokens(int heads_per_group, int variant);
const char* bf16_kernel_name(int heads_per_group, int variant, bool paged);
bool bf16_variant_pages(int heads_per_group, int variant);  // has a paged-cache form
// fp8 latent cache: only some variants have a form that reads e4m3 codes
bool bf16_variant_fp8(int heads_per_group, int variant);
// the variant builds its split plan itself (plan_in_kernel may be set)
bool bf16_variant_plans(int heads_per_group, int variant);
const char* fp8_kernel_name(int heads_per_group, int variant);
hipError_t launch_decode_bf16(const DecodeParams& p, int heads_per_group, int variant,
                              hipStream_t stream);

// Wide-wave bf16 kernel: NW waves of 32 heads each, STAGES-deep LDS ring.
template <int NW, int STAGES>
hipError_t launch_decode_wide(const DecodeParams& p, hipStream_t stream);

// The same with q_len causal query tokens per row (p.q_len, p.heads_per_token).
template <int NW, int STAGES>
hipError_t launch_decode_wide_causal(const DecodeParams& p, hipStream_t stream);

// Column-split, software-pipelined bf16 kernel for groups of 128 heads.
hipError_t launch_decode_colsplit(const DecodeParams& p, hipStream_t stream);

// fp8-cache form of the 128-head wide kernel: queries quantised to e4m3 per
// (batch row, head) on entry, scores on FP8 MFMAs, weighted sum on bf16 ones
// (contiguous cache, one query token per row).
hipError_t launch_decode_wide_fp8(const DecodeParams& p, hipStream_t stream);

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t stream);

hipError_t launch_quantize_fp8(long long n_rows, const void* x, void* codes, float* scale,
                               hipStream_t stream);

hipError_t launch_absorb_q(bool bf16, int b, int h, const void* q_nope, const void* w_uk,
                           const void* q_rope, void* q_prime, hipStream_t stream);
hipError_t launch_absorb_o(bool bf16, int b, int h, const void* o, const void* w_uv, void* y,
                           hipStream_t stream);

// Appending a token's latent row: the hidden dimension must be a multiple of
// append_kd(); the workspace (partial sums and a copy of the positions) takes
// append_workspace_bytes(b, d_model) (both in append_layout.h).
// block_table == nullptr: cache [b, t_max, 576]; else cache is the pool
// [num_blocks, block_size, 576] and t_max = max_blocks * block_size.
hipError_t launch_cache_append(int b, int d_model, int t_max, int n_pos, const void* x,
                               const void* w_dkv, const void* w_kr, const float* rope_cos,
                               const float* rope_sin, void* cache, const int32_t* seqlens,
                               int32_t* seqlens_out, void* workspace, hipStream_t stream,
                               const int32_t* block_table, int num_blocks, int block_size,
                               int max_blocks);

}  // namespace mla355
