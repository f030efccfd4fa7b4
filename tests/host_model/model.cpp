// Stand-in launchers for the CPU build of the host layer: each one replays
// its kernel's memory accesses (see model.h).  The split plan comes from the
// device's own builder (plan_build.h) run on 64 emulated lanes, into the
// caller's workspace (host memory here, left uninitialised by the driver), so
// every walk below reads the plan exactly as the device would write it.
#include "model.h"

#include "append_layout.h"
#include "mla355_internal.h"
#include "plan_build.h"
#include "variants.h"

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>

namespace model {
namespace {

struct Region {
    uintptr_t base;
    size_t bytes;
    std::string name;
    bool real;
};
std::vector<Region> regions;
std::vector<std::string> fails;
std::string context;
long long n_launches = 0;
long planted_index = -1;
int planted_value = 0;

void fail(const std::string& what)
{
    if (fails.size() < 16) fails.push_back(context + ": " + what);
}

// [p, p + bytes) lies inside one registered buffer.
bool check(const void* p, size_t bytes, const char* what)
{
    const uintptr_t a = (uintptr_t)p;
    for (const Region& r : regions)
        if (a >= r.base && bytes <= r.bytes && a - r.base <= r.bytes - bytes) return true;
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %zu bytes at %#lx lie outside every buffer", what, bytes,
                  (unsigned long)a);
    fail(buf);
    return false;
}

}  // namespace

void clear_regions() { regions.clear(); }
void add_region(const void* base, size_t bytes, const char* name, bool real)
{
    regions.push_back({(uintptr_t)base, bytes, name, real});
}
void set_context(const std::string& ctx) { context = ctx; }
std::vector<std::string> take_failures()
{
    std::vector<std::string> f;
    f.swap(fails);
    return f;
}
long long launches() { return n_launches; }
void plant_plan_entry(long index, int value)
{
    planted_index = index;
    planted_value = value;
}
// Applies (once) a planted plan entry.
void apply_plant(int32_t* plan)
{
    if (planted_index >= 0) plan[planted_index] = planted_value;
    planted_index = -1;
}

}  // namespace model

using model::check;
using model::fail;

namespace mla355 {
namespace {

size_t plan_ints(int b, int n_chunks) { return 4 + (size_t)(b + 1) + 2 * (size_t)b + (size_t)n_chunks; }

// The device's plan builder on 64 emulated lanes.
void build_plan_on_cpu(const int32_t* seqlens, int b, int t_max, int n_chunks, int min_chunk, int align,
                       int32_t* plan)
{
    run_wave([&] { build_plan(seqlens, b, t_max, n_chunks, min_chunk, align, plan); });
    model::apply_plant(plan);
}

// Kernel geometry the walk needs.
struct Shape {
    int HG;             // heads per workgroup
    int N;              // tokens per tile
    bool xcd_map;       // workgroup -> (chunk, head group) through block_work
    bool q_clamp;       // lanes past the last head read head 0's query
    size_t elem;        // bytes per element of q, cache (bf16 path), out and partials
    size_t row_bytes;   // bytes per cache row in HBM
};

// Replays one split-KV attention launch.
void walk_split(const DecodeParams& p, const Shape& s)
{
    ++model::n_launches;
    const size_t nints = plan_ints(p.b, p.n_chunks);
    std::vector<int32_t> lds;
    const int32_t* plan = p.plan;
    if (p.plan_in_kernel) {
        // every workgroup builds the plan in its LDS; workgroup 0 copies it out
        lds.assign(kPlanLdsInts, (int32_t)0xABABABAB);
        build_plan_on_cpu(p.seqlens, p.b, p.t_max, p.n_chunks, p.plan_min_chunk, p.plan_align, lds.data());
        if (check(p.plan, nints * 4, "plan copy to the workspace"))
            std::memcpy(const_cast<int32_t*>(p.plan), lds.data(), nints * 4);
        plan = lds.data();
    }
    bool bad = false;
    auto P = [&](long i) -> int32_t {
        if (i < 0 || (size_t)i >= nints) {
            fail("plan index " + std::to_string(i) + " outside the plan");
            bad = true;
            return 0;
        }
        if (!p.plan_in_kernel && !check(plan + i, 4, "plan read")) {
            bad = true;
            return 0;
        }
        return plan[i];
    };
    const long cu0 = 4, base0 = 4 + (p.b + 1), ns0 = base0 + p.b, cr0 = ns0 + p.b;
    const int total = P(0), chunk = P(1);
    if (chunk <= 0) {
        fail("chunk " + std::to_string(chunk) + " is not positive");
        return;
    }
    const WorkspaceLayout wl = workspace_layout(p.b, p.h, p.n_chunks, (int)s.elem);
    const unsigned char* qg = (const unsigned char*)p.q;
    const unsigned char* cg = (const unsigned char*)p.cache;
    const size_t qrow = (size_t)kDqk * s.elem, orow = (size_t)kDc * s.elem;
    const int grid = p.n_chunks * p.n_hg;
    for (int wg = 0; wg < grid && !bad; ++wg) {
        int k, hg;
        if (s.xcd_map) {
            const int xcd = wg & 7, slot8 = wg >> 3;
            k = xcd * (p.n_chunks >> 3) + slot8 / p.n_hg;
            hg = slot8 % p.n_hg;
        } else {
            k = wg / p.n_hg;
            hg = wg % p.n_hg;
        }
        int r = P(cr0 + k);
        if (r < 0) continue;
        int pos = k * chunk;
        const int end = pos + std::min(chunk, total - pos);
        for (int guard = 0;; ++guard) {
            if (r >= p.b || guard > p.b) {
                fail("segment walk left the batch (row " + std::to_string(r) + ")");
                bad = true;
                break;
            }
            const int row_lo = P(cu0 + r), row_hi = P(cu0 + r + 1);
            const int seg_end = std::min(end, row_hi);
            const int seg_a = pos - row_lo;
            int seg_len = seg_end - pos;
            if (seg_a < 0 || seg_len <= 0) {
                fail("empty or negative segment: row " + std::to_string(r) + " seg_a " + std::to_string(seg_a) +
                     " len " + std::to_string(seg_len));
                bad = true;
                break;
            }
            int L = row_hi - row_lo;
            if (p.block_table != nullptr) {
                if (!check(p.seqlens + r, 4, "seqlens read")) break;
                L = std::min(std::max(p.seqlens[r], 0), p.t_max);
                seg_len = std::max(0, std::min(seg_len, L - seg_a));
            }
            if (seg_a + seg_len > p.t_max) fail("segment past t_max");
            const int split_j = k - row_lo / chunk;
            const bool final_out = P(ns0 + r) == 1;
            const int slot = P(base0 + r) + split_j;
            if (!final_out && (slot < 0 || slot >= wl.max_slots)) fail("partial slot out of range");
            // cache rows, one tile at a time (rows past the segment end are never fetched)
            int pg_blk = 0, pg_off = 0;
            if (p.block_table != nullptr) {
                pg_blk = seg_a / p.block_size;
                pg_off = seg_a - pg_blk * p.block_size;
            }
            for (int t0 = 0; t0 < seg_len; t0 += s.N) {
                const int cnt = std::min(s.N, seg_len - t0);
                const unsigned char* a;
                if (p.block_table != nullptr) {
                    const int32_t* be = p.block_table + (size_t)r * p.max_blocks + pg_blk;
                    if (!check(be, 4, "block table read")) break;
                    const int e = std::min(std::max(*be, 0), p.num_blocks - 1);
                    a = cg + ((size_t)e * p.block_size + pg_off) * s.row_bytes;
                    pg_off += s.N;
                    if (pg_off == p.block_size) {
                        pg_off = 0;
                        ++pg_blk;
                    }
                } else {
                    a = cg + ((size_t)r * p.t_max + seg_a + t0) * s.row_bytes;
                }
                check(a, (size_t)cnt * s.row_bytes, "cache tile");
                if (p.cache_scale != nullptr)
                    check(p.cache_scale + (size_t)r * p.t_max + seg_a + t0, (size_t)cnt * 4, "fp8 scales");
            }
            for (int i = 0; i < s.HG; ++i) {
                const int head = hg * s.HG + i;
                const bool ok = head < p.h;
                if (ok || s.q_clamp) check(qg + ((size_t)r * p.h + (ok ? head : 0)) * qrow, qrow, "query row");
                if (!ok) continue;
                if (final_out) {
                    check((const unsigned char*)p.out + ((size_t)r * p.h + head) * orow, orow, "output row");
                    check(p.lse + (size_t)r * p.h + head, 4, "lse");
                } else {
                    check((const unsigned char*)p.po + ((size_t)slot * p.h + head) * orow, orow, "partial row");
                    check(p.plse + (size_t)slot * p.h + head, 4, "partial lse");
                }
            }
            pos = seg_end;
            if (pos >= end) break;
            ++r;
            while (!bad && P(cu0 + r + 1) <= pos) ++r;
        }
    }
    if (p.plan_in_kernel) {
        // the attention kernel also writes out = 0, lse = -inf for empty rows
        for (int r = 0; r < p.b; ++r)
            if (lds[cu0 + r + 1] == lds[cu0 + r]) {
                check((const unsigned char*)p.out + (size_t)r * p.h * orow, (size_t)p.h * orow, "empty row out");
                check(p.lse + (size_t)r * p.h, (size_t)p.h * 4, "empty row lse");
            }
    }
}

template <typename F>
hipError_t wide_launch(const DecodeParams& p, int nw, int stages, F&& walk)
{
    const bool plans = stages * (32 * 1152 + 32 * 128) + kPlanLdsInts * 4 <= 160 * 1024;
    if (p.plan_in_kernel && (!plans || p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks)) return hipErrorInvalidValue;
    walk(Shape{32 * nw, 32, true, true, 2, (size_t)kRowBytesBf16});
    return hipSuccess;
}

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, int b, int h, int t_max, int n_chunks, int min_chunk, int align,
                       int32_t* plan, bool bf16, void* out, float* lse, hipStream_t)
{
    ++model::n_launches;
    if (!check(plan, plan_ints(b, n_chunks) * 4, "plan in the workspace")) return hipSuccess;
    if (!check(seqlens, (size_t)b * 4, "seqlens")) return hipSuccess;
    build_plan_on_cpu(seqlens, b, t_max, n_chunks, min_chunk, align, plan);
    const size_t orow = (size_t)kDc * (bf16 ? 2 : 4);
    for (int r = 0; r < b; ++r)
        if (clamped_len(seqlens, r, t_max) == 0) {
            check((const unsigned char*)out + (size_t)r * h * orow, (size_t)h * orow, "empty row out");
            check(lse + (size_t)r * h, (size_t)h * 4, "empty row lse");
        }
    return hipSuccess;
}

hipError_t launch_combine(bool bf16, const int32_t* plan, int b, int h, int n_chunks, const float* plse,
                          const void* po, void* out, float* lse, hipStream_t)
{
    ++model::n_launches;
    if (!check(plan, plan_ints(b, n_chunks) * 4, "plan read by the combine")) return hipSuccess;
    const PlanView v{const_cast<int32_t*>(plan), b};
    const size_t orow = (size_t)kDc * (bf16 ? 2 : 4);
    const int max_slots = n_chunks + b;
    for (int r = 0; r < b; ++r) {
        const int ns = v.nsplit()[r];
        if (ns <= 1) continue;
        const int s0 = v.base()[r];
        if (s0 < 0 || s0 + ns > max_slots) {
            fail("combine slots out of range");
            continue;
        }
        for (int head = 0; head < h; ++head) {
            check(plse + (size_t)s0 * h + head, 4, "combine partial lse (first)");
            check(plse + (size_t)(s0 + ns - 1) * h + head, 4, "combine partial lse (last)");
            check((const unsigned char*)po + ((size_t)s0 * h + head) * orow, orow, "combine partial (first)");
            check((const unsigned char*)po + ((size_t)(s0 + ns - 1) * h + head) * orow, orow,
                  "combine partial (last)");
            check((const unsigned char*)out + ((size_t)r * h + head) * orow, orow, "combine output");
            check(lse + (size_t)r * h + head, 4, "combine lse");
        }
    }
    return hipSuccess;
}

hipError_t launch_decode_bf16(const DecodeParams& p, int heads_per_group, int variant, hipStream_t)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    if (v == nullptr) return hipErrorInvalidValue;
    const bool fp8 = p.cache_scale != nullptr;
    if (fp8 && v->fp8_name == nullptr) return hipErrorInvalidValue;
    if (p.block_table != nullptr && v->paged_name == nullptr) return hipErrorInvalidValue;
    const size_t row_bytes = fp8 ? (size_t)kDqk : (size_t)kRowBytesBf16;
    switch (v->family) {
    case KernelFamily::Tiled:
        walk_split(p, Shape{v->targs[1] * v->targs[0], v->targs[2] * v->targs[3], true, true, 2, row_bytes});
        return hipSuccess;
    case KernelFamily::Pair:
        walk_split(p, Shape{32 * v->targs[0], 32, true, true, 2, row_bytes});
        return hipSuccess;
    case KernelFamily::Wide:
        if (fp8) {
            // decode_wide_fp8_kernel: 128 heads, 32-token tiles of e4m3 rows
            // and their scales, plan in LDS when it fits; contiguous cache only
            if (p.plan_in_kernel && (p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks))
                return hipErrorInvalidValue;
            if (p.block_table != nullptr || p.q_len != 1) return hipErrorInvalidValue;
            walk_split(p, Shape{128, 32, true, true, 2, row_bytes});
            return hipSuccess;
        }
        return wide_launch(p, v->targs[0], v->targs[1], [&](const Shape& s) { walk_split(p, s); });
    case KernelFamily::Split:
        if (p.plan_in_kernel && (p.b > kPlanLdsRows || p.n_chunks > kPlanLdsChunks)) return hipErrorInvalidValue;
        walk_split(p, Shape{128, 32, true, true, 2, row_bytes});
        return hipSuccess;
    }
    return hipErrorInvalidValue;
}

template <int NW, int STAGES>
hipError_t launch_decode_wide(const DecodeParams& p, hipStream_t)
{
    return wide_launch(p, NW, STAGES, [&](const Shape& s) { walk_split(p, s); });
}

template <int NW, int STAGES>
hipError_t launch_decode_wide_causal(const DecodeParams& p, hipStream_t)
{
    return wide_launch(p, NW, STAGES, [&](const Shape& s) { walk_split(p, s); });
}

template hipError_t launch_decode_wide_causal<4, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide_causal<2, 2>(const DecodeParams&, hipStream_t);
template hipError_t launch_decode_wide_causal<1, 3>(const DecodeParams&, hipStream_t);

hipError_t launch_decode_f32(const DecodeParams& p, hipStream_t)
{
    walk_split(p, Shape{16, 16, false, false, 4, (size_t)kDqk * 4});
    return hipSuccess;
}

hipError_t launch_quantize_fp8(long long n_rows, const void* x, void* codes, float* scale, hipStream_t)
{
    ++model::n_launches;
    check(x, (size_t)n_rows * kRowBytesBf16, "quantiser input");
    check(codes, (size_t)n_rows * kDqk, "quantiser codes");
    check(scale, (size_t)n_rows * 4, "quantiser scales");
    return hipSuccess;
}

hipError_t launch_absorb_q(bool bf16, int b, int h, const void* q_nope, const void* w_uk, const void* q_rope,
                           void* q_prime, hipStream_t)
{
    ++model::n_launches;
    const size_t e = bf16 ? 2 : 4;
    check(q_nope, (size_t)b * h * kDk * e, "q_nope");
    check(w_uk, (size_t)h * kDk * kDc * e, "W_UK");
    check(q_rope, (size_t)b * h * kDr * e, "q_rope");
    check(q_prime, (size_t)b * h * kDqk * e, "q'");
    return hipSuccess;
}

hipError_t launch_absorb_o(bool bf16, int b, int h, const void* o, const void* w_uv, void* y, hipStream_t)
{
    ++model::n_launches;
    const size_t e = bf16 ? 2 : 4;
    check(o, (size_t)b * h * kDc * e, "o");
    check(w_uv, (size_t)h * kDc * kDv * e, "W_UV");
    check(y, (size_t)b * h * kDv * e, "y");
    return hipSuccess;
}

hipError_t launch_cache_append(int b, int d_model, int t_max, int n_pos, const void* x, const void* w_dkv,
                               const void* w_kr, const float* rope_cos, const float* rope_sin, void* cache,
                               const int32_t* seqlens, int32_t* seqlens_out, void* workspace, hipStream_t,
                               const int32_t* block_table, int num_blocks, int block_size, int max_blocks)
{
    ++model::n_launches;
    check(x, (size_t)b * d_model * 2, "x");
    check(w_dkv, (size_t)d_model * kDc * 2, "W_DKV");
    check(w_kr, (size_t)d_model * kDr * 2, "W_KR");
    check(rope_cos, (size_t)n_pos * (kDr / 2) * 4, "cos table");
    check(rope_sin, (size_t)n_pos * (kDr / 2) * 4, "sin table");
    check(workspace, append_workspace_bytes(b, d_model), "append workspace");
    if (!check(seqlens, (size_t)b * 4, "seqlens")) return hipSuccess;
    if (seqlens_out) check(seqlens_out, (size_t)b * 4, "seqlens_out");
    for (int i = 0; i < b; ++i) {
        const int pos = seqlens[i];
        if (pos < 0 || pos >= std::min(t_max, n_pos)) continue;  // no write
        if (block_table != nullptr) {
            const int32_t* be = block_table + (size_t)i * max_blocks + pos / block_size;
            if (!check(be, 4, "block table read")) continue;
            if (*be < 0 || *be >= num_blocks) continue;
            check((unsigned char*)cache + ((size_t)*be * block_size + pos % block_size) * kRowBytesBf16,
                  kRowBytesBf16, "appended row");
        } else {
            check((unsigned char*)cache + ((size_t)i * t_max + pos) * kRowBytesBf16, kRowBytesBf16,
                  "appended row");
        }
    }
    return hipSuccess;
}

}  // namespace mla355
