// C ABI of libmla355 (declared in include/mla355.h): argument validation,
// scheduling choice, workspace carving and launch sequencing.
//
// Validation is pure host code and runs before any HIP call, so every error
// path can be exercised without a GPU.
#include "../../include/mla355.h"
#include "append_layout.h"
#include "mla355_internal.h"
#include "variants.h"

#include <math.h>
#include <stdint.h>

using namespace mla355;

namespace {

// Whole-chip compute-unit count the automatic schedule is sized for (MI355X:
// 8 XCDs x 32 CUs).  It is a constant, not a device query, so that the
// workspace size stays a pure host function of the problem size.
constexpr int kCUs = 256;
constexpr int kMaxChunks = 65536;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Schedule {
    int hpg;        // heads per workgroup group
    int variant;    // bf16 kernel variant (0 for fp32)
    int n_hg;       // head groups
    int n_chunks;   // token chunks per head group
    int min_chunk;  // smallest chunk (tokens)
};

int round_down8(int x) { return x < 8 ? 8 : x / 8 * 8; }

static_assert(kClockBytes == MLA_CLOCK_BYTES && kConfigRecordClock == MLA_CONFIG_RECORD_CLOCK,
              "the clock-stamp hook as the header states it");

mla_status_t choose_schedule(mla_dtype_t dt, int h, const mla_decode_config_t* cfg, Schedule* s)
{
    if (cfg) {
        if ((cfg->reserved[0] & ~kConfigRecordClock) != 0) return MLA_ERR_UNSUPPORTED;
        for (int i = 1; i < 5; ++i)
            if (cfg->reserved[i] != 0) return MLA_ERR_UNSUPPORTED;
        if (cfg->n_chunks < 0 || cfg->heads_per_group < 0 || cfg->variant < 0)
            return MLA_ERR_UNSUPPORTED;
        if ((cfg->profile_events[0] == nullptr) != (cfg->profile_events[1] == nullptr))
            return MLA_ERR_UNSUPPORTED;
    }
    if (dt == MLA_DTYPE_F32) {
        s->hpg = 16;
        s->variant = 0;
        if (cfg && cfg->heads_per_group != 0 && cfg->heads_per_group != 16) return MLA_ERR_UNSUPPORTED;
        if (cfg && cfg->variant != 0) return MLA_ERR_UNSUPPORTED;
        s->min_chunk = 16;
    } else {
        // <= 16 heads: 16-head workgroups of two token-splitting waves
        // (memory-bound regime); 17..32 heads: 32-head workgroups of 16x16
        // MFMA tiles; more: wide-wave workgroups (32 heads per wave) of 64 or
        // 128 heads, so every latent row is fetched once per head group.
        int hpg = h <= 16 ? 16 : h <= 32 ? 32 : h <= 64 ? 64 : 128;
        int def_variant = h <= 16 ? 1 : h <= 32 ? 1 : h <= 64 ? 6 : 4;
        if (cfg && cfg->heads_per_group != 0) {
            hpg = cfg->heads_per_group;
            def_variant = 1;
        }
        const int variant = (cfg && cfg->variant != 0) ? cfg->variant : def_variant;
        if (!bf16_variant_exists(hpg, variant)) return MLA_ERR_UNSUPPORTED;
        s->hpg = hpg;
        s->variant = variant;
        s->min_chunk = bf16_tile_tokens(hpg, variant);
    }
    s->n_hg = (h + s->hpg - 1) / s->hpg;
    if (cfg && cfg->n_chunks != 0) {
        if (cfg->n_chunks % 8 != 0 || cfg->n_chunks > kMaxChunks) return MLA_ERR_UNSUPPORTED;
        s->n_chunks = cfg->n_chunks;
    } else {
        s->n_chunks = round_down8(kCUs / s->n_hg);
    }
    return MLA_OK;
}

// Schedule for a paged cache: only the wide-wave kernels address the block
// pool, so the automatic choice is the wide kernel with the fewest heads per
// group that covers h (32, 64 or 128), and an explicit choice must be one.
mla_status_t choose_paged_schedule(int h, const mla_decode_config_t* cfg, Schedule* s)
{
    mla_decode_config_t c{};
    if (cfg) c = *cfg;
    if (c.heads_per_group == 0) c.heads_per_group = h <= 32 ? 32 : h <= 64 ? 64 : 128;
    if (c.variant == 0) c.variant = c.heads_per_group == 64 ? 6 : 4;
    const mla_status_t st = choose_schedule(MLA_DTYPE_BF16, h, &c, s);
    if (st != MLA_OK) return st;
    if (!bf16_variant_pages(s->hpg, s->variant)) return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

bool paged_dims_ok(int b, int h, int num_blocks, int block_size, int max_blocks)
{
    if (b <= 0 || h <= 0 || num_blocks <= 0 || block_size <= 0 || max_blocks <= 0) return false;
    if (block_size % 32 != 0) return false;
    const int64_t t_max = (int64_t)max_blocks * block_size;
    // the plan covers lengths rounded up to whole 32-token tiles
    if ((int64_t)b * (t_max + 32) >= ((int64_t)1 << 31)) return false;
    if ((int64_t)b * (int64_t)h >= ((int64_t)1 << 31) / kDqk) return false;
    return true;
}

// Schedule for an fp8 cache.  Up to 64 heads: the 16-head two-wave kernel
// (exact bf16 queries, bf16 MFMAs).  More: the 128-head wide kernel, which
// also quantises the queries and scores on FP8 MFMAs.
mla_status_t choose_fp8_schedule(int h, const mla_decode_config_t* cfg, Schedule* s)
{
    mla_decode_config_t c{};
    if (cfg) c = *cfg;
    if (c.heads_per_group == 0) c.heads_per_group = h <= 64 ? 16 : 128;
    if (c.variant == 0) c.variant = c.heads_per_group == 128 ? 4 : 1;
    const mla_status_t st = choose_schedule(MLA_DTYPE_BF16, h, &c, s);
    if (st != MLA_OK) return st;
    if (!bf16_variant_fp8(s->hpg, s->variant)) return MLA_ERR_UNSUPPORTED;
    // the 16-head fp8 form needs 77 KB of LDS: two workgroups fit on a CU, so
    // the automatic grid is twice as large
    if (c.n_chunks == 0 && s->hpg == 16) s->n_chunks = round_down8(2 * kCUs / s->n_hg);
    return MLA_OK;
}

// Schedule for q_len causal query tokens per row (q_len > 1): the wide-wave
// kernels, whose query rows are the q_len * h (token, head) pairs of a batch
// row, 32 per wave.
struct MtpSchedule {
    int nw;         // waves per workgroup (32 query rows each)
    int n_hg;       // groups of 32 * nw query rows
    int n_chunks;
};

MtpSchedule choose_mtp_schedule(int rows)
{
    MtpSchedule s;
    s.nw = rows > 64 ? 4 : rows > 32 ? 2 : 1;
    s.n_hg = (rows + 32 * s.nw - 1) / (32 * s.nw);
    s.n_chunks = round_down8(kCUs / s.n_hg);
    return s;
}

bool dims_ok(int b, int h, int t_max)
{
    if (b <= 0 || h <= 0 || t_max < 0) return false;
    if ((int64_t)b * (int64_t)t_max >= ((int64_t)1 << 31)) return false;
    if ((int64_t)b * (int64_t)h >= ((int64_t)1 << 31) / kDqk) return false;
    return true;
}

bool dtype_ok(mla_dtype_t dt) { return dt == MLA_DTYPE_F32 || dt == MLA_DTYPE_BF16; }

mla_status_t hip_status(hipError_t e) { return e == hipSuccess ? MLA_OK : MLA_ERR_HIP; }

// Launch parameters shared by every split-KV attention call: inputs, outputs
// and the workspace carved by `w` (plan first, then the partial lse and the
// partial outputs), for `rows` query rows per batch row.  The cache form (a
// paged pool, fp8 scales, causal query tokens) is set by the caller.
DecodeParams split_params(const void* q_prime, const void* cache, const int32_t* seqlens, void* out,
                          float* lse, void* workspace, const WorkspaceLayout& w, int b, int rows,
                          int t_max, int n_chunks, int n_hg, float softmax_scale)
{
    unsigned char* ws = (unsigned char*)workspace;
    DecodeParams p;
    p.q = q_prime;
    p.cache = cache;
    p.plan = (const int32_t*)ws;
    p.out = out;
    p.lse = lse;
    p.plse = (float*)(ws + w.plse_off);
    p.po = (void*)(ws + w.po_off);
    p.block_table = nullptr;
    p.seqlens = seqlens;
    p.cache_scale = nullptr;
    p.num_blocks = p.block_size = p.max_blocks = 0;
    p.q_len = 1;
    p.heads_per_token = rows;
    p.plan_in_kernel = p.plan_min_chunk = 0;
    p.plan_align = 1;
    p.clock_stamps = (unsigned long long*)(ws + w.clock_off);  // cleared by run_split unless asked for
    p.b = b;
    p.h = rows;
    p.t_max = t_max;
    p.n_chunks = n_chunks;
    p.n_hg = n_hg;
    p.scale_log2 = softmax_scale * 1.4426950408889634f;
    return p;
}

// plan -> attention kernel -> combine on `hs`, with the caller's profiling
// events (if any) recorded right before and after the attention kernel.
// align > 1 lays the plan over lengths rounded up to whole tiles (paged pool).
// kernel_plans: the attention kernel can build the plan itself; it does when
// the plan fits its LDS, and no plan kernel is launched.  `kernel` is called
// with the final parameters.
template <typename Kernel>
mla_status_t run_split(DecodeParams p, bool bf16, int min_chunk, int align, bool kernel_plans,
                       const mla_decode_config_t* cfg, hipStream_t hs, Kernel&& kernel)
{
    hipEvent_t ev0 = cfg ? (hipEvent_t)cfg->profile_events[0] : nullptr;
    hipEvent_t ev1 = cfg ? (hipEvent_t)cfg->profile_events[1] : nullptr;
    if (!(cfg && (cfg->reserved[0] & kConfigRecordClock))) p.clock_stamps = nullptr;
    p.plan_in_kernel = kernel_plans && p.b <= kPlanLdsRows && p.n_chunks <= kPlanLdsChunks;
    p.plan_min_chunk = min_chunk;
    p.plan_align = align;
    if (!p.plan_in_kernel) {
        hipError_t e = launch_plan(p.seqlens, p.b, p.h, p.t_max, p.n_chunks, min_chunk, align,
                                   const_cast<int32_t*>(p.plan), bf16, p.out, p.lse, hs);
        if (e != hipSuccess) return MLA_ERR_HIP;
    }
    if (ev0 && hipEventRecord(ev0, hs) != hipSuccess) return MLA_ERR_HIP;
    if (kernel(p) != hipSuccess) return MLA_ERR_HIP;
    if (ev1 && hipEventRecord(ev1, hs) != hipSuccess) return MLA_ERR_HIP;
    return hip_status(launch_combine(bf16, p.plan, p.b, p.h, p.n_chunks, p.plse, p.po, p.out, p.lse, hs));
}

}  // namespace

// Everything is built with hidden visibility; only the C ABI is exported.
#pragma GCC visibility push(default)
extern "C" {

int mla_abi_version(void) { return MLA355_ABI_VERSION; }

const char* mla_status_string(mla_status_t s)
{
    switch (s) {
    case MLA_OK: return "ok";
    case MLA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case MLA_ERR_UNSUPPORTED: return "unsupported configuration";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MLA_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

size_t mla_decode_workspace_bytes_ex(mla_dtype_t dt, int b, int h, int t_max,
                                     const mla_decode_config_t* cfg)
{
    if (!dtype_ok(dt) || !dims_ok(b, h, t_max)) return 0;
    Schedule s;
    if (choose_schedule(dt, h, cfg, &s) != MLA_OK) return 0;
    return workspace_layout(b, h, s.n_chunks, dt == MLA_DTYPE_BF16 ? 2 : 4).total;
}

const char* mla_decode_kernel_name(mla_dtype_t dt, int h, const mla_decode_config_t* cfg)
{
    if (!dtype_ok(dt) || h <= 0) return nullptr;
    Schedule s;
    if (choose_schedule(dt, h, cfg, &s) != MLA_OK) return nullptr;
    if (dt == MLA_DTYPE_F32) return "decode_f32_kernel";
    return bf16_kernel_name(s.hpg, s.variant, false);
}

size_t mla_decode_workspace_bytes(mla_dtype_t dt, int b, int h, int t_max)
{
    return mla_decode_workspace_bytes_ex(dt, b, h, t_max, nullptr);
}

mla_status_t mla_decode_ex(mla_dtype_t dt, int b, int h, int t_max, const void* q_prime,
                           const void* cache, const int32_t* seqlens, float softmax_scale,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           const mla_decode_config_t* cfg, void* stream)
{
    if (!dtype_ok(dt) || !dims_ok(b, h, t_max)) return MLA_ERR_INVALID_ARGUMENT;
    if (!q_prime || !cache || !seqlens || !out || !lse || !workspace) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_prime) || !aligned16(cache) || !aligned16(seqlens) || !aligned16(out) ||
        !aligned16(lse) || ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    Schedule s;
    const mla_status_t st = choose_schedule(dt, h, cfg, &s);
    if (st != MLA_OK) return st;
    const WorkspaceLayout w = workspace_layout(b, h, s.n_chunks, dt == MLA_DTYPE_BF16 ? 2 : 4);
    if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    const bool bf16 = dt == MLA_DTYPE_BF16;
    DecodeParams p = split_params(q_prime, cache, seqlens, out, lse, workspace, w, b, h, t_max,
                                  s.n_chunks, s.n_hg, softmax_scale);
    const bool plans = bf16 && bf16_variant_plans(s.hpg, s.variant);
    return run_split(p, bf16, s.min_chunk, 1, plans, cfg, (hipStream_t)stream, [&](const DecodeParams& q) {
        return bf16 ? launch_decode_bf16(q, s.hpg, s.variant, (hipStream_t)stream)
                    : launch_decode_f32(q, (hipStream_t)stream);
    });
}

mla_status_t mla_decode(mla_dtype_t dt, int b, int h, int t_max, const void* q_prime,
                        const void* cache, const int32_t* seqlens, float softmax_scale, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    return mla_decode_ex(dt, b, h, t_max, q_prime, cache, seqlens, softmax_scale, out, lse,
                         workspace, workspace_bytes, nullptr, stream);
}

static bool mtp_dims_ok(int b, int q_len, int h, int t_max)
{
    if (q_len <= 0 || h <= 0 || (int64_t)q_len * h > ((int64_t)1 << 20)) return false;
    return dims_ok(b, q_len * h, t_max);
}

// The causal kernel for `nw` waves of 32 query rows.
static hipError_t launch_mtp(const DecodeParams& p, int nw, hipStream_t hs)
{
    return nw == 4 ? launch_decode_wide_causal<4, 2>(p, hs)
           : nw == 2 ? launch_decode_wide_causal<2, 2>(p, hs)
                     : launch_decode_wide_causal<1, 3>(p, hs);
}

// Config of the multi-token call: only n_chunks and the profiling events may be set.
static mla_status_t check_mtp_config(const mla_decode_config_t* cfg)
{
    if (!cfg) return MLA_OK;
    if ((cfg->reserved[0] & ~kConfigRecordClock) != 0) return MLA_ERR_UNSUPPORTED;
    for (int i = 1; i < 5; ++i)
        if (cfg->reserved[i] != 0) return MLA_ERR_UNSUPPORTED;
    if (cfg->heads_per_group != 0 || cfg->variant != 0) return MLA_ERR_UNSUPPORTED;
    if (cfg->n_chunks < 0 || cfg->n_chunks % 8 != 0 || cfg->n_chunks > kMaxChunks) return MLA_ERR_UNSUPPORTED;
    if ((cfg->profile_events[0] == nullptr) != (cfg->profile_events[1] == nullptr))
        return MLA_ERR_UNSUPPORTED;
    return MLA_OK;
}

static MtpSchedule mtp_schedule(int rows, const mla_decode_config_t* cfg)
{
    MtpSchedule s = choose_mtp_schedule(rows);
    if (cfg && cfg->n_chunks != 0) s.n_chunks = cfg->n_chunks;
    return s;
}

size_t mla_decode_mtp_workspace_bytes_ex(mla_dtype_t dt, int b, int q_len, int h, int t_max,
                                         const mla_decode_config_t* cfg)
{
    if (dt != MLA_DTYPE_BF16 || !mtp_dims_ok(b, q_len, h, t_max)) return 0;
    if (check_mtp_config(cfg) != MLA_OK) return 0;
    if (q_len == 1) return mla_decode_workspace_bytes_ex(dt, b, h, t_max, cfg);
    const MtpSchedule s = mtp_schedule(q_len * h, cfg);
    return workspace_layout(b, q_len * h, s.n_chunks, 2).total;
}

size_t mla_decode_mtp_workspace_bytes(mla_dtype_t dt, int b, int q_len, int h, int t_max)
{
    return mla_decode_mtp_workspace_bytes_ex(dt, b, q_len, h, t_max, nullptr);
}

const char* mla_decode_mtp_kernel_name(mla_dtype_t dt, int q_len, int h)
{
    if (dt != MLA_DTYPE_BF16 || q_len <= 0 || h <= 0 || (int64_t)q_len * h > ((int64_t)1 << 20))
        return nullptr;
    if (q_len == 1) return mla_decode_kernel_name(dt, h, nullptr);
    switch (choose_mtp_schedule(q_len * h).nw) {
    case 4: return "decode_wide_causal_kernel<4, 2, false>";
    case 2: return "decode_wide_causal_kernel<2, 2, false>";
    default: return "decode_wide_causal_kernel<1, 3, false>";
    }
}

mla_status_t mla_decode_mtp_ex(mla_dtype_t dt, int b, int q_len, int h, int t_max,
                               const void* q_prime, const void* cache, const int32_t* seqlens,
                               float softmax_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, const mla_decode_config_t* cfg, void* stream)
{
    if (!dtype_ok(dt)) return MLA_ERR_INVALID_ARGUMENT;
    if (dt != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
    if (!mtp_dims_ok(b, q_len, h, t_max)) return MLA_ERR_INVALID_ARGUMENT;
    const mla_status_t cst = check_mtp_config(cfg);
    if (cst != MLA_OK) return cst;
    if (q_len == 1)
        return mla_decode_ex(dt, b, h, t_max, q_prime, cache, seqlens, softmax_scale, out, lse,
                             workspace, workspace_bytes, cfg, stream);
    if (!q_prime || !cache || !seqlens || !out || !lse || !workspace) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_prime) || !aligned16(cache) || !aligned16(seqlens) || !aligned16(out) ||
        !aligned16(lse) || ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    const int rows = q_len * h;
    const MtpSchedule s = mtp_schedule(rows, cfg);
    const WorkspaceLayout w = workspace_layout(b, rows, s.n_chunks, 2);
    if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    DecodeParams p = split_params(q_prime, cache, seqlens, out, lse, workspace, w, b, rows, t_max,
                                  s.n_chunks, s.n_hg, softmax_scale);
    p.q_len = q_len;
    p.heads_per_token = h;
    return run_split(p, true, 32, 1, true, cfg, (hipStream_t)stream,
                     [&](const DecodeParams& q) { return launch_mtp(q, s.nw, (hipStream_t)stream); });
}

mla_status_t mla_decode_mtp(mla_dtype_t dt, int b, int q_len, int h, int t_max, const void* q_prime,
                            const void* cache, const int32_t* seqlens, float softmax_scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream)
{
    return mla_decode_mtp_ex(dt, b, q_len, h, t_max, q_prime, cache, seqlens, softmax_scale, out,
                             lse, workspace, workspace_bytes, nullptr, stream);
}

size_t mla_decode_paged_workspace_bytes(mla_dtype_t dt, int b, int h, int num_blocks,
                                        int block_size, int max_blocks,
                                        const mla_decode_config_t* cfg)
{
    if (dt != MLA_DTYPE_BF16 || !paged_dims_ok(b, h, num_blocks, block_size, max_blocks)) return 0;
    Schedule s;
    if (choose_paged_schedule(h, cfg, &s) != MLA_OK) return 0;
    return workspace_layout(b, h, s.n_chunks, 2).total;
}

const char* mla_decode_paged_kernel_name(mla_dtype_t dt, int h, const mla_decode_config_t* cfg)
{
    if (dt != MLA_DTYPE_BF16 || h <= 0) return nullptr;
    Schedule s;
    if (choose_paged_schedule(h, cfg, &s) != MLA_OK) return nullptr;
    return bf16_kernel_name(s.hpg, s.variant, true);
}

mla_status_t mla_decode_paged_ex(mla_dtype_t dt, int b, int h, const void* q_prime,
                                 const void* kv_pool, int num_blocks, int block_size,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* seqlens, float softmax_scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 const mla_decode_config_t* cfg, void* stream)
{
    if (!dtype_ok(dt)) return MLA_ERR_INVALID_ARGUMENT;
    if (dt != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
    if (!paged_dims_ok(b, h, num_blocks, block_size, max_blocks)) return MLA_ERR_INVALID_ARGUMENT;
    if (!q_prime || !kv_pool || !block_table || !seqlens || !out || !lse || !workspace)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_prime) || !aligned16(kv_pool) || !aligned16(block_table) ||
        !aligned16(seqlens) || !aligned16(out) || !aligned16(lse) ||
        ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    Schedule s;
    const mla_status_t st = choose_paged_schedule(h, cfg, &s);
    if (st != MLA_OK) return st;
    const WorkspaceLayout w = workspace_layout(b, h, s.n_chunks, 2);
    if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    const int t_max = max_blocks * block_size;

    DecodeParams p = split_params(q_prime, kv_pool, seqlens, out, lse, workspace, w, b, h, t_max,
                                  s.n_chunks, s.n_hg, softmax_scale);
    p.block_table = block_table;
    p.num_blocks = num_blocks;
    p.block_size = block_size;
    p.max_blocks = max_blocks;
    // tile-aligned plan: every segment starts at a multiple of 32 tokens
    return run_split(p, true, 32, 32, bf16_variant_plans(s.hpg, s.variant), cfg, (hipStream_t)stream,
                     [&](const DecodeParams& q) { return launch_decode_bf16(q, s.hpg, s.variant, (hipStream_t)stream); });
}

mla_status_t mla_decode_paged(mla_dtype_t dt, int b, int h, const void* q_prime, const void* kv_pool,
                              int num_blocks, int block_size, const int32_t* block_table,
                              int max_blocks, const int32_t* seqlens, float softmax_scale, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream)
{
    return mla_decode_paged_ex(dt, b, h, q_prime, kv_pool, num_blocks, block_size, block_table,
                               max_blocks, seqlens, softmax_scale, out, lse, workspace,
                               workspace_bytes, nullptr, stream);
}

mla_status_t mla_quantize_cache_fp8(long long n_rows, const void* x, void* codes, float* scale,
                                    void* stream)
{
    if (n_rows <= 0 || n_rows > ((long long)1 << 37)) return MLA_ERR_INVALID_ARGUMENT;
    if (!x || !codes || !scale) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(codes) || ((uintptr_t)scale & 3u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_quantize_fp8(n_rows, x, codes, scale, (hipStream_t)stream));
}

size_t mla_decode_fp8_workspace_bytes(int b, int h, int t_max, const mla_decode_config_t* cfg)
{
    if (!dims_ok(b, h, t_max)) return 0;
    Schedule s;
    if (choose_fp8_schedule(h, cfg, &s) != MLA_OK) return 0;
    return workspace_layout(b, h, s.n_chunks, 2).total;
}

const char* mla_decode_fp8_kernel_name(int h, const mla_decode_config_t* cfg)
{
    if (h <= 0) return nullptr;
    Schedule s;
    if (choose_fp8_schedule(h, cfg, &s) != MLA_OK) return nullptr;
    return fp8_kernel_name(s.hpg, s.variant);
}

mla_status_t mla_decode_fp8_ex(int b, int h, int t_max, const void* q_prime, const void* cache_codes,
                               const float* cache_scale, const int32_t* seqlens, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               const mla_decode_config_t* cfg, void* stream)
{
    if (!dims_ok(b, h, t_max)) return MLA_ERR_INVALID_ARGUMENT;
    if (!q_prime || !cache_codes || !cache_scale || !seqlens || !out || !lse || !workspace)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_prime) || !aligned16(cache_codes) || ((uintptr_t)cache_scale & 3u) != 0 ||
        !aligned16(seqlens) || !aligned16(out) || !aligned16(lse) ||
        ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    Schedule s;
    const mla_status_t st = choose_fp8_schedule(h, cfg, &s);
    if (st != MLA_OK) return st;
    const WorkspaceLayout w = workspace_layout(b, h, s.n_chunks, 2);
    if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;

    DecodeParams p = split_params(q_prime, cache_codes, seqlens, out, lse, workspace, w, b, h, t_max,
                                  s.n_chunks, s.n_hg, softmax_scale);
    p.cache_scale = cache_scale;
    return run_split(p, true, s.min_chunk, 1, bf16_variant_plans(s.hpg, s.variant), cfg, (hipStream_t)stream,
                     [&](const DecodeParams& q) { return launch_decode_bf16(q, s.hpg, s.variant, (hipStream_t)stream); });
}

mla_status_t mla_decode_fp8(int b, int h, int t_max, const void* q_prime, const void* cache_codes,
                            const float* cache_scale, const int32_t* seqlens, float softmax_scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream)
{
    return mla_decode_fp8_ex(b, h, t_max, q_prime, cache_codes, cache_scale, seqlens, softmax_scale,
                             out, lse, workspace, workspace_bytes, nullptr, stream);
}

mla_status_t mla_absorb_q(mla_dtype_t dt, int b, int h, const void* q_nope, const void* w_uk,
                          const void* q_rope, void* q_prime, void* stream)
{
    if (!dtype_ok(dt) || !dims_ok(b, h, 0)) return MLA_ERR_INVALID_ARGUMENT;
    if (!q_nope || !w_uk || !q_rope || !q_prime) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_nope) || !aligned16(w_uk) || !aligned16(q_rope) || !aligned16(q_prime))
        return MLA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_absorb_q(dt == MLA_DTYPE_BF16, b, h, q_nope, w_uk, q_rope, q_prime,
                                      (hipStream_t)stream));
}

size_t mla_cache_append_workspace_bytes(int b, int d_model)
{
    if (b <= 0 || d_model <= 0 || d_model % append_kd() != 0) return 0;
    return append_workspace_bytes(b, d_model);
}

mla_status_t mla_cache_append(mla_dtype_t dt, int b, int d_model, int t_max, const void* x,
                              const void* w_dkv, const void* w_kr, const float* rope_cos,
                              const float* rope_sin, int n_pos, void* cache, const int32_t* seqlens,
                              int32_t* seqlens_out, void* workspace, size_t workspace_bytes,
                              void* stream)
{
    if (!dtype_ok(dt)) return MLA_ERR_INVALID_ARGUMENT;
    if (dt != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
    if (b <= 0 || d_model <= 0 || d_model % append_kd() != 0 || t_max <= 0 || n_pos <= 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if ((int64_t)b * t_max >= ((int64_t)1 << 31) || (int64_t)b * d_model >= ((int64_t)1 << 31))
        return MLA_ERR_INVALID_ARGUMENT;
    if (!x || !w_dkv || !w_kr || !rope_cos || !rope_sin || !cache || !seqlens || !workspace)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(cache) ||
        ((uintptr_t)rope_cos & 3u) != 0 || ((uintptr_t)rope_sin & 3u) != 0 ||
        ((uintptr_t)seqlens & 3u) != 0 || ((uintptr_t)seqlens_out & 3u) != 0 ||
        ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < mla_cache_append_workspace_bytes(b, d_model)) return MLA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_cache_append(b, d_model, t_max, n_pos, x, w_dkv, w_kr, rope_cos, rope_sin,
                                          cache, seqlens, seqlens_out, workspace, (hipStream_t)stream,
                                          nullptr, 0, 0, 0));
}

mla_status_t mla_cache_append_paged(mla_dtype_t dt, int b, int d_model, const void* x,
                                    const void* w_dkv, const void* w_kr, const float* rope_cos,
                                    const float* rope_sin, int n_pos, void* kv_pool, int num_blocks,
                                    int block_size, const int32_t* block_table, int max_blocks,
                                    const int32_t* seqlens, int32_t* seqlens_out, void* workspace,
                                    size_t workspace_bytes, void* stream)
{
    if (!dtype_ok(dt)) return MLA_ERR_INVALID_ARGUMENT;
    if (dt != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
    if (d_model <= 0 || d_model % append_kd() != 0 || n_pos <= 0) return MLA_ERR_INVALID_ARGUMENT;
    if (!paged_dims_ok(b, 1, num_blocks, block_size, max_blocks)) return MLA_ERR_INVALID_ARGUMENT;
    if ((int64_t)b * d_model >= ((int64_t)1 << 31)) return MLA_ERR_INVALID_ARGUMENT;
    if (!x || !w_dkv || !w_kr || !rope_cos || !rope_sin || !kv_pool || !block_table || !seqlens ||
        !workspace)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(x) || !aligned16(w_dkv) || !aligned16(w_kr) || !aligned16(kv_pool) ||
        ((uintptr_t)rope_cos & 3u) != 0 || ((uintptr_t)rope_sin & 3u) != 0 ||
        ((uintptr_t)block_table & 3u) != 0 || ((uintptr_t)seqlens & 3u) != 0 ||
        ((uintptr_t)seqlens_out & 3u) != 0 || ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < mla_cache_append_workspace_bytes(b, d_model)) return MLA_ERR_WORKSPACE_TOO_SMALL;
    return hip_status(launch_cache_append(b, d_model, max_blocks * block_size, n_pos, x, w_dkv, w_kr,
                                          rope_cos, rope_sin, kv_pool, seqlens, seqlens_out, workspace,
                                          (hipStream_t)stream, block_table, num_blocks, block_size,
                                          max_blocks));
}

size_t mla_decode_mtp_paged_workspace_bytes(mla_dtype_t dt, int b, int q_len, int h, int num_blocks,
                                            int block_size, int max_blocks)
{
    if (dt != MLA_DTYPE_BF16 || q_len <= 0 || h <= 0 || (int64_t)q_len * h > ((int64_t)1 << 20)) return 0;
    if (!paged_dims_ok(b, q_len * h, num_blocks, block_size, max_blocks)) return 0;
    if (q_len == 1) return mla_decode_paged_workspace_bytes(dt, b, h, num_blocks, block_size, max_blocks, nullptr);
    const MtpSchedule s = choose_mtp_schedule(q_len * h);
    return workspace_layout(b, q_len * h, s.n_chunks, 2).total;
}

mla_status_t mla_decode_mtp_paged(mla_dtype_t dt, int b, int q_len, int h, const void* q_prime,
                                  const void* kv_pool, int num_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream)
{
    if (!dtype_ok(dt)) return MLA_ERR_INVALID_ARGUMENT;
    if (dt != MLA_DTYPE_BF16) return MLA_ERR_UNSUPPORTED;
    if (q_len <= 0 || h <= 0 || (int64_t)q_len * h > ((int64_t)1 << 20)) return MLA_ERR_INVALID_ARGUMENT;
    if (q_len == 1)
        return mla_decode_paged_ex(dt, b, h, q_prime, kv_pool, num_blocks, block_size, block_table,
                                   max_blocks, seqlens, softmax_scale, out, lse, workspace,
                                   workspace_bytes, nullptr, stream);
    const int rows = q_len * h;
    if (!paged_dims_ok(b, rows, num_blocks, block_size, max_blocks)) return MLA_ERR_INVALID_ARGUMENT;
    if (!q_prime || !kv_pool || !block_table || !seqlens || !out || !lse || !workspace)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(q_prime) || !aligned16(kv_pool) || !aligned16(block_table) ||
        !aligned16(seqlens) || !aligned16(out) || !aligned16(lse) ||
        ((uintptr_t)workspace & 255u) != 0)
        return MLA_ERR_INVALID_ARGUMENT;
    if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return MLA_ERR_INVALID_ARGUMENT;
    const MtpSchedule s = choose_mtp_schedule(rows);
    const WorkspaceLayout w = workspace_layout(b, rows, s.n_chunks, 2);
    if (workspace_bytes < w.total) return MLA_ERR_WORKSPACE_TOO_SMALL;
    const int t_max = max_blocks * block_size;

    DecodeParams p = split_params(q_prime, kv_pool, seqlens, out, lse, workspace, w, b, rows, t_max,
                                  s.n_chunks, s.n_hg, softmax_scale);
    p.block_table = block_table;
    p.num_blocks = num_blocks;
    p.block_size = block_size;
    p.max_blocks = max_blocks;
    p.q_len = q_len;
    p.heads_per_token = h;
    // tile-aligned plan: every segment starts at a multiple of 32 tokens
    return run_split(p, true, 32, 32, true, nullptr, (hipStream_t)stream,
                     [&](const DecodeParams& q) { return launch_mtp(q, s.nw, (hipStream_t)stream); });
}

mla_status_t mla_absorb_o(mla_dtype_t dt, int b, int h, const void* o, const void* w_uv, void* y,
                          void* stream)
{
    if (!dtype_ok(dt) || !dims_ok(b, h, 0)) return MLA_ERR_INVALID_ARGUMENT;
    if (!o || !w_uv || !y) return MLA_ERR_INVALID_ARGUMENT;
    if (!aligned16(o) || !aligned16(w_uv) || !aligned16(y)) return MLA_ERR_INVALID_ARGUMENT;
    return hip_status(launch_absorb_o(dt == MLA_DTYPE_BF16, b, h, o, w_uv, y, (hipStream_t)stream));
}

}  // extern "C"
#pragma GCC visibility pop
