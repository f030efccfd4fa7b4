// Driver of the CPU build of the host layer (api.cpp and variants.cpp, with
// the stand-in launchers of model.cpp), run under AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_host_model.py.
//
// Part 1 calls every entry point with one bad argument at a time and checks
// the status (nothing may reach a launcher).  Part 2 runs the schedules the
// GPU tests use -- every kernel variant, the edge-length batch, automatic
// and forced chunk counts, paged pools, fp8 caches, several query tokens,
// the full-size configurations -- through the model, which checks every
// address each kernel would form against the buffers the call was given.
// Device buffers are address ranges reserved without access rights, so the
// model can only compare addresses, never touch them; seqlens, block tables
// and the workspace are real host memory, the workspace filled with a
// garbage pattern before every call.
#include "../../include/mla355.h"
#include "model.h"

#include <sys/mman.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <string>
#include <vector>

namespace {

int failures = 0;
long long calls = 0;
bool expecting_failures = false;  // self-check: failures are the point, not errors

void expect(bool ok, const std::string& what)
{
    if (!ok) {
        ++failures;
        if (!expecting_failures) std::fprintf(stderr, "FAIL %s\n", what.c_str());
    }
}

void drain(const std::string& what)
{
    for (const std::string& f : model::take_failures()) {
        ++failures;
        if (!expecting_failures) std::fprintf(stderr, "FAIL %s: %s\n", what.c_str(), f.c_str());
    }
}

// A device buffer stand-in: reserved address space, no access rights.
struct Fake {
    void* p = nullptr;
    size_t bytes = 0, mapped = 0;
    Fake(size_t n, const char* name) : bytes(n)
    {
        mapped = (n + 4095) / 4096 * 4096 + 4096;
        p = mmap(nullptr, mapped, PROT_NONE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
        if (p == MAP_FAILED) {
            std::perror("mmap");
            std::exit(2);
        }
        model::add_region(p, n, name, false);
    }
    ~Fake() { munmap(p, mapped); }
    Fake(const Fake&) = delete;
    Fake& operator=(const Fake&) = delete;
};

// Host memory the model reads or writes, registered with its exact size.
struct Real {
    void* p = nullptr;
    size_t bytes = 0;
    Real(size_t n, const char* name, int fill) : bytes(n)
    {
        const size_t alloc = (n + 255) / 256 * 256;
        p = std::aligned_alloc(256, alloc ? alloc : 256);
        std::memset(p, fill, alloc ? alloc : 256);
        model::add_region(p, n, name, true);
    }
    ~Real() { std::free(p); }
    Real(const Real&) = delete;
    Real& operator=(const Real&) = delete;
};

Real* ints(const std::vector<int32_t>& v, const char* name)
{
    Real* r = new Real(v.size() * 4, name, 0);
    std::memcpy(r->p, v.data(), v.size() * 4);
    return r;
}

mla_decode_config_t cfg_of(int n_chunks, int hpg, int variant)
{
    mla_decode_config_t c;
    std::memset(&c, 0, sizeof c);
    c.n_chunks = n_chunks;
    c.heads_per_group = hpg;
    c.variant = variant;
    return c;
}

std::string desc(const char* what, int b, int h, const mla_decode_config_t* c)
{
    char buf[200];
    std::snprintf(buf, sizeof buf, "%s b=%d h=%d chunks=%d hpg=%d variant=%d", what, b, h, c ? c->n_chunks : 0,
                  c ? c->heads_per_group : 0, c ? c->variant : 0);
    return buf;
}

// One mla_decode_ex call through the model.
void run_decode(mla_dtype_t dt, const std::vector<int32_t>& lens, int t_max, int h, const mla_decode_config_t* c,
                const char* what)
{
    const int b = (int)lens.size();
    const size_t e = dt == MLA_DTYPE_BF16 ? 2 : 4;
    const size_t ws = mla_decode_workspace_bytes_ex(dt, b, h, t_max, c);
    const std::string d = desc(what, b, h, c);
    expect(ws > 0, d + ": workspace size");
    if (ws == 0) return;
    model::clear_regions();
    Fake q((size_t)b * h * 576 * e, "q'"), cache((size_t)b * t_max * 576 * e, "cache"),
        out((size_t)b * h * 512 * e, "out"), lse((size_t)b * h * 4, "lse");
    Real* sl = ints(lens, "seqlens");
    Real w(ws, "workspace", 0xAB);
    model::set_context(d);
    const mla_status_t st = mla_decode_ex(dt, b, h, t_max, q.p, cache.p, (const int32_t*)sl->p, 0.0721688f, out.p,
                                          (float*)lse.p, w.p, ws, c, nullptr);
    ++calls;
    expect(st == MLA_OK, d + ": status " + std::to_string(st));
    drain(d);
    delete sl;
}

void run_paged(const std::vector<int32_t>& lens, int h, int bs, int max_blocks, int spare, int bad_entry,
               const mla_decode_config_t* c, int q_len, const char* what)
{
    const int b = (int)lens.size();
    const int nb = b * max_blocks + spare;
    const std::string d = desc(what, b, h, c) + " bs=" + std::to_string(bs) + " q_len=" + std::to_string(q_len);
    const size_t ws = q_len == 1 ? mla_decode_paged_workspace_bytes(MLA_DTYPE_BF16, b, h, nb, bs, max_blocks, c)
                                 : mla_decode_mtp_paged_workspace_bytes(MLA_DTYPE_BF16, b, q_len, h, nb, bs,
                                                                        max_blocks);
    expect(ws > 0, d + ": workspace size");
    if (ws == 0) return;
    std::mt19937 g(b * 131 + h + bs);
    std::vector<int32_t> perm(nb);
    for (int i = 0; i < nb; ++i) perm[i] = i;
    std::shuffle(perm.begin(), perm.end(), g);
    std::vector<int32_t> bt((size_t)b * max_blocks);
    for (size_t i = 0; i < bt.size(); ++i) bt[i] = perm[i];
    for (int i = 0; i < b; ++i)  // entries past a sequence's last block are never read
        for (int k = (std::max(lens[i], 0) + bs - 1) / bs; k < max_blocks; ++k) bt[(size_t)i * max_blocks + k] = bad_entry;
    model::clear_regions();
    const int rows = q_len * h;
    Fake q((size_t)b * rows * 1152, "q'"), pool((size_t)nb * bs * 1152, "pool"), out((size_t)b * rows * 1024, "out"),
        lse((size_t)b * rows * 4, "lse");
    Real* sl = ints(lens, "seqlens");
    Real* table = ints(bt, "block table");
    Real w(ws, "workspace", 0xAB);
    model::set_context(d);
    mla_status_t st;
    if (q_len == 1)
        st = mla_decode_paged_ex(MLA_DTYPE_BF16, b, h, q.p, pool.p, nb, bs, (const int32_t*)table->p, max_blocks,
                                 (const int32_t*)sl->p, 0.0721688f, out.p, (float*)lse.p, w.p, ws, c, nullptr);
    else
        st = mla_decode_mtp_paged(MLA_DTYPE_BF16, b, q_len, h, q.p, pool.p, nb, bs, (const int32_t*)table->p,
                                  max_blocks, (const int32_t*)sl->p, 0.0721688f, out.p, (float*)lse.p, w.p, ws,
                                  nullptr);
    ++calls;
    expect(st == MLA_OK, d + ": status " + std::to_string(st));
    drain(d);
    delete sl;
    delete table;
}

void run_mtp(const std::vector<int32_t>& lens, int q_len, int h, const mla_decode_config_t* c)
{
    const int b = (int)lens.size();
    int t_max = 1;
    for (int L : lens) t_max = std::max(t_max, L);
    const std::string d = desc("mtp", b, h, c) + " q_len=" + std::to_string(q_len);
    const size_t ws = mla_decode_mtp_workspace_bytes_ex(MLA_DTYPE_BF16, b, q_len, h, t_max, c);
    expect(ws > 0, d + ": workspace size");
    if (ws == 0) return;
    model::clear_regions();
    const int rows = q_len * h;
    Fake q((size_t)b * rows * 1152, "q'"), cache((size_t)b * t_max * 1152, "cache"), out((size_t)b * rows * 1024, "out"),
        lse((size_t)b * rows * 4, "lse");
    Real* sl = ints(lens, "seqlens");
    Real w(ws, "workspace", 0xAB);
    model::set_context(d);
    const mla_status_t st = mla_decode_mtp_ex(MLA_DTYPE_BF16, b, q_len, h, t_max, q.p, cache.p,
                                              (const int32_t*)sl->p, 0.0721688f, out.p, (float*)lse.p, w.p, ws, c,
                                              nullptr);
    ++calls;
    expect(st == MLA_OK, d + ": status " + std::to_string(st));
    drain(d);
    delete sl;
}

void run_fp8(const std::vector<int32_t>& lens, int h, const mla_decode_config_t* c)
{
    const int b = (int)lens.size();
    int t_max = 1;
    for (int L : lens) t_max = std::max(t_max, L);
    const std::string d = desc("fp8", b, h, c);
    const size_t ws = mla_decode_fp8_workspace_bytes(b, h, t_max, c);
    expect(ws > 0, d + ": workspace size");
    if (ws == 0) return;
    model::clear_regions();
    Fake q((size_t)b * h * 1152, "q'"), codes((size_t)b * t_max * 576, "codes"), scale((size_t)b * t_max * 4, "scales"),
        out((size_t)b * h * 1024, "out"), lse((size_t)b * h * 4, "lse");
    Real* sl = ints(lens, "seqlens");
    Real w(ws, "workspace", 0xAB);
    model::set_context(d);
    const mla_status_t st = mla_decode_fp8_ex(b, h, t_max, q.p, codes.p, (const float*)scale.p,
                                              (const int32_t*)sl->p, 0.0721688f, out.p, (float*)lse.p, w.p, ws, c,
                                              nullptr);
    ++calls;
    expect(st == MLA_OK, d + ": status " + std::to_string(st));
    drain(d);
    delete sl;
}

const std::vector<int32_t> kEdge = {1, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 0, 700};

// ---------------------------------------------------------------- part 1

void validation()
{
    model::clear_regions();
    const long long launches_before = model::launches();
    void* A = (void*)0x10000;        // aligned, never dereferenced
    void* M = (void*)0x10008;        // misaligned
    const int32_t* S = (const int32_t*)0x20000;
    float* F = (float*)0x30000;
    const size_t ws = mla_decode_workspace_bytes(MLA_DTYPE_BF16, 4, 16, 100);
    expect(ws > 0, "workspace query");
    struct Case {
        const char* name;
        mla_status_t want;
        mla_status_t got;
    };
    mla_decode_config_t bad_chunks = cfg_of(12, 0, 0), bad_hpg = cfg_of(0, 48, 0), bad_var = cfg_of(0, 16, 9);
    mla_decode_config_t bad_res = cfg_of(0, 0, 0);
    bad_res.reserved[2] = 1;
    const Case cases[] = {
        {"null q'", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 4, 16, 100, nullptr, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"misaligned cache", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 4, 16, 100, A, M, S, 0.07f, A, F, A, ws, nullptr)},
        {"b = 0", MLA_ERR_INVALID_ARGUMENT, mla_decode(MLA_DTYPE_BF16, 0, 16, 100, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"h < 0", MLA_ERR_INVALID_ARGUMENT, mla_decode(MLA_DTYPE_BF16, 4, -1, 100, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"t_max < 0", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 4, 16, -5, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"b * t_max >= 2^31", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 1 << 16, 16, 1 << 15, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"unknown dtype", MLA_ERR_INVALID_ARGUMENT,
         mla_decode((mla_dtype_t)7, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"scale NaN", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, NAN, A, F, A, ws, nullptr)},
        {"scale 0", MLA_ERR_INVALID_ARGUMENT, mla_decode(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.f, A, F, A, ws, nullptr)},
        {"workspace misaligned", MLA_ERR_INVALID_ARGUMENT,
         mla_decode(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, (char*)A + 16, ws, nullptr)},
        {"workspace small", MLA_ERR_WORKSPACE_TOO_SMALL,
         mla_decode(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws - 1, nullptr)},
        {"chunks not a multiple of 8", MLA_ERR_UNSUPPORTED,
         mla_decode_ex(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws << 4, &bad_chunks, nullptr)},
        {"heads per group 48", MLA_ERR_UNSUPPORTED,
         mla_decode_ex(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws << 4, &bad_hpg, nullptr)},
        {"unknown variant", MLA_ERR_UNSUPPORTED,
         mla_decode_ex(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws << 4, &bad_var, nullptr)},
        {"reserved field set", MLA_ERR_UNSUPPORTED,
         mla_decode_ex(MLA_DTYPE_BF16, 4, 16, 100, A, A, S, 0.07f, A, F, A, ws << 4, &bad_res, nullptr)},
        {"absorb_q null", MLA_ERR_INVALID_ARGUMENT, mla_absorb_q(MLA_DTYPE_BF16, 4, 16, A, nullptr, A, A, nullptr)},
        {"absorb_q misaligned", MLA_ERR_INVALID_ARGUMENT, mla_absorb_q(MLA_DTYPE_BF16, 4, 16, A, A, M, A, nullptr)},
        {"absorb_o b = 0", MLA_ERR_INVALID_ARGUMENT, mla_absorb_o(MLA_DTYPE_F32, 0, 16, A, A, A, nullptr)},
        {"paged block size 48", MLA_ERR_INVALID_ARGUMENT,
         mla_decode_paged(MLA_DTYPE_BF16, 4, 16, A, A, 8, 48, S, 2, S, 0.07f, A, F, A, ws, nullptr)},
        {"paged fp32", MLA_ERR_UNSUPPORTED,
         mla_decode_paged(MLA_DTYPE_F32, 4, 16, A, A, 8, 64, S, 2, S, 0.07f, A, F, A, ws, nullptr)},
        {"quantise 0 rows", MLA_ERR_INVALID_ARGUMENT, mla_quantize_cache_fp8(0, A, A, F, nullptr)},
        {"fp8 null scales", MLA_ERR_INVALID_ARGUMENT,
         mla_decode_fp8(4, 16, 100, A, A, nullptr, S, 0.07f, A, F, A, ws, nullptr)},
        {"mtp fp32", MLA_ERR_UNSUPPORTED,
         mla_decode_mtp(MLA_DTYPE_F32, 4, 2, 16, 100, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"mtp q_len 0", MLA_ERR_INVALID_ARGUMENT,
         mla_decode_mtp(MLA_DTYPE_BF16, 4, 0, 16, 100, A, A, S, 0.07f, A, F, A, ws, nullptr)},
        {"append d_model 100", MLA_ERR_INVALID_ARGUMENT,
         mla_cache_append(MLA_DTYPE_BF16, 4, 100, 64, A, A, A, F, F, 64, A, S, nullptr, A, 1 << 20, nullptr)},
        {"append small workspace", MLA_ERR_WORKSPACE_TOO_SMALL,
         mla_cache_append(MLA_DTYPE_BF16, 4, 256, 64, A, A, A, F, F, 64, A, S, nullptr, A, 16, nullptr)},
    };
    for (const Case& c : cases) expect(c.got == c.want, std::string("validation: ") + c.name);
    expect(model::launches() == launches_before, "validation: a rejected call reached a launcher");
    expect(mla_decode_workspace_bytes(MLA_DTYPE_BF16, 0, 16, 100) == 0, "workspace query b = 0");
    expect(mla_decode_kernel_name(MLA_DTYPE_BF16, 128, nullptr) != nullptr, "kernel name");
    expect(std::strcmp(mla_status_string(MLA_ERR_HIP), "HIP launch error") == 0, "status string");
    drain("validation");
}

// ---------------------------------------------------------------- part 2

void schedules()
{
    // every kernel variant on the edge-length batch, automatic and forced chunk counts
    struct V {
        int h, hpg, variant;
    };
    const V variants[] = {{1, 0, 0},    {3, 0, 0},    {16, 0, 0},   {16, 16, 2},  {32, 0, 0},   {32, 32, 2},
                          {64, 0, 0},   {64, 64, 2},  {128, 0, 0},  {128, 128, 2}, {128, 64, 0}, {128, 16, 0},
                          {40, 16, 0},  {64, 64, 3},  {32, 32, 3},  {100, 0, 0},  {16, 16, 1},  {128, 128, 3},
                          {128, 128, 4}, {128, 128, 5}, {100, 128, 3}, {64, 64, 5}, {64, 64, 6},  {32, 32, 4},
                          {20, 32, 4},  {48, 0, 0},   {33, 0, 0},   {256, 0, 0},  {128, 128, 6},
                          {100, 128, 6}, {256, 128, 6}};
    for (const V& v : variants)
        for (int n : {0, 8, 64, 256, 2560}) {
            mla_decode_config_t c = cfg_of(n, v.hpg, v.variant);
            run_decode(MLA_DTYPE_BF16, kEdge, 700, v.h, &c, "edge lengths");
        }
    // fp32 kernels: partial head groups
    for (int h : {3, 16, 20, 40})
        for (int n : {0, 8, 64, 256}) {
            mla_decode_config_t c = cfg_of(n, 0, 0);
            run_decode(MLA_DTYPE_F32, {1, 15, 16, 17, 33, 0, 257}, 257, h, &c, "fp32");
        }
    // out-of-range lengths are clamped, empty batches
    for (int h : {16, 64, 128}) {
        run_decode(MLA_DTYPE_BF16, {-3, 1000000000, 40}, 64, h, nullptr, "clamped lengths");
        run_decode(MLA_DTYPE_BF16, {0, 0, 0}, 1, h, nullptr, "all empty");
    }
    // long rows cut into many segments (both combine forms)
    for (int n : {96, 256, 2048}) {
        mla_decode_config_t c = cfg_of(n, 0, 0);
        run_decode(MLA_DTYPE_BF16, {20000, 13001, 5}, 20000, 100, &c, "many segments");
    }
    // in-LDS plan limits and the plan kernel past them; many short rows
    {
        std::mt19937 g(7);
        for (int b : {256, 257, 3000}) {
            std::vector<int32_t> lens(b);
            for (int i = 0; i < b; ++i) lens[i] = i % 7 == 0 ? 0 : (int)(g() % 300);
            for (int n : {0, 2048, 2056}) {
                mla_decode_config_t c = cfg_of(n, 0, 0);
                run_decode(MLA_DTYPE_BF16, lens, 300, 128, &c, "plan limits");
            }
            run_decode(MLA_DTYPE_BF16, lens, 300, 16, nullptr, "short rows, 16 heads");
        }
    }
    // the full-size configurations (automatic schedule, as the benchmark runs them)
    run_decode(MLA_DTYPE_BF16, std::vector<int32_t>(64, 4096), 4096, 128, nullptr, "dsv3 decode b64 h128 T4096");
    run_decode(MLA_DTYPE_BF16, std::vector<int32_t>(128, 8192), 8192, 16, nullptr, "few heads b128 h16 T8192");
    {
        std::mt19937 g(1004);
        std::vector<int32_t> lens(132);
        for (auto& L : lens) L = 1 + (int)(g() % 32768);
        run_decode(MLA_DTYPE_BF16, lens, 32768, 128, nullptr, "ragged b132 h128");
    }
    run_decode(MLA_DTYPE_BF16, std::vector<int32_t>(4, 131072), 131072, 128, nullptr, "long b4 h128 T131072");
    run_decode(MLA_DTYPE_F32, {128, 257}, 257, 16, nullptr, "tiny fp32");
    // paged pools: block sizes, head counts, unused table entries out of range
    for (int bs : {32, 64, 128, 256})
        for (int h : {16, 20, 64, 100, 128})
            for (int n : {0, 8, 64, 256}) {
                mla_decode_config_t c = cfg_of(n, 0, 0);
                run_paged(kEdge, h, bs, (700 + bs - 1) / bs, 3, -12345, &c, 1, "paged");
            }
    run_paged(std::vector<int32_t>(64, 4096), 128, 64, 64, 0, 0, nullptr, 1, "paged dsv3 decode");
    // several causal query tokens per row, contiguous and paged
    run_mtp({700, 257, 1000, 33, 2}, 2, 128, nullptr);
    run_mtp({100, 3, 1, 0, 64}, 3, 16, nullptr);
    run_mtp({129, 32, 31, 5}, 4, 8, nullptr);
    run_mtp({513, 96}, 2, 100, nullptr);
    run_mtp({300, 40, 8}, 8, 16, nullptr);
    {
        mla_decode_config_t c = cfg_of(2560, 0, 0);
        run_mtp({700, 257, 1000, 33, 2}, 2, 128, &c);
    }
    run_mtp(std::vector<int32_t>(64, 4096), 2, 128, nullptr);
    run_paged({700, 257, 1000, 33, 2}, 128, 64, 16, 2, -777, nullptr, 2, "mtp paged");
    run_paged({100, 3, 1, 0, 64}, 16, 32, 4, 2, -777, nullptr, 3, "mtp paged");
    // fp8 cache
    for (int h : {1, 3, 16, 20, 128})
        for (int n : {0, 8, 64, 256}) {
            mla_decode_config_t c = cfg_of(n, 0, 0);
            run_fp8(kEdge, h, &c);
        }
    run_fp8(std::vector<int32_t>(128, 8192), 16, nullptr);
}

void other_calls()
{
    for (int bf16 : {0, 1})
        for (int b : {3, 17, 40, 64, 100})
            for (int h : {3, 16, 20, 128}) {
                model::clear_regions();
                const mla_dtype_t dt = bf16 ? MLA_DTYPE_BF16 : MLA_DTYPE_F32;
                const size_t e = bf16 ? 2 : 4;
                Fake qn((size_t)b * h * 128 * e, "q_nope"), wk((size_t)h * 128 * 512 * e, "W_UK"),
                    qr((size_t)b * h * 64 * e, "q_rope"), qp((size_t)b * h * 576 * e, "q'"),
                    o((size_t)b * h * 512 * e, "o"), wv((size_t)h * 512 * 128 * e, "W_UV"),
                    y((size_t)b * h * 128 * e, "y");
                const std::string d = desc(bf16 ? "absorbs bf16" : "absorbs fp32", b, h, nullptr);
                model::set_context(d);
                expect(mla_absorb_q(dt, b, h, qn.p, wk.p, qr.p, qp.p, nullptr) == MLA_OK, d + " absorb_q");
                expect(mla_absorb_o(dt, b, h, o.p, wv.p, y.p, nullptr) == MLA_OK, d + " absorb_o");
                calls += 2;
                drain(d);
            }
    {
        model::clear_regions();
        const long long n = 128LL * 8192;
        Fake x((size_t)n * 1152, "x"), codes((size_t)n * 576, "codes"), scale((size_t)n * 4, "scales");
        model::set_context("quantise");
        expect(mla_quantize_cache_fp8(n, x.p, codes.p, (float*)scale.p, nullptr) == MLA_OK, "quantise");
        ++calls;
        drain("quantise");
    }
    for (int d_model : {256, 7168}) {
        const std::vector<int32_t> lens = {0, 7, 47, 48, -3, 20};
        const int b = (int)lens.size(), t_max = 48, n_pos = 48;
        model::clear_regions();
        Fake x((size_t)b * d_model * 2, "x"), wd((size_t)d_model * 512 * 2, "W_DKV"), wr((size_t)d_model * 64 * 2, "W_KR"),
            cs((size_t)n_pos * 32 * 4, "cos"), sn((size_t)n_pos * 32 * 4, "sin"),
            cache((size_t)b * t_max * 1152, "cache");
        Real* sl = ints(lens, "seqlens");
        Real* so = ints(std::vector<int32_t>(b, 0), "seqlens_out");
        const size_t ws = mla_cache_append_workspace_bytes(b, d_model);
        Real w(ws, "workspace", 0xAB);
        const std::string d = "append d_model=" + std::to_string(d_model);
        model::set_context(d);
        expect(mla_cache_append(MLA_DTYPE_BF16, b, d_model, t_max, x.p, wd.p, wr.p, (const float*)cs.p,
                                (const float*)sn.p, n_pos, cache.p, (const int32_t*)sl->p, (int32_t*)so->p, w.p, ws,
                                nullptr) == MLA_OK,
               d);
        ++calls;
        drain(d);
        delete sl;
        delete so;
    }
    {
        const std::vector<int32_t> lens = {0, 70, 127, 128, 200, 63};
        const int b = (int)lens.size(), bs = 64, mb = 4, nb = b * mb + 2, d_model = 512;
        std::vector<int32_t> bt((size_t)b * mb);
        for (size_t i = 0; i < bt.size(); ++i) bt[i] = (int32_t)((i * 7) % nb);
        bt[5 * mb + 0] = nb + 3;  // outside the pool: no write
        model::clear_regions();
        Fake x((size_t)b * d_model * 2, "x"), wd((size_t)d_model * 512 * 2, "W_DKV"), wr((size_t)d_model * 64 * 2, "W_KR"),
            cs((size_t)256 * 32 * 4, "cos"), sn((size_t)256 * 32 * 4, "sin"), pool((size_t)nb * bs * 1152, "pool");
        Real* sl = ints(lens, "seqlens");
        Real* table = ints(bt, "block table");
        const size_t ws = mla_cache_append_workspace_bytes(b, d_model);
        Real w(ws, "workspace", 0xAB);
        model::set_context("append paged");
        expect(mla_cache_append_paged(MLA_DTYPE_BF16, b, d_model, x.p, wd.p, wr.p, (const float*)cs.p,
                                      (const float*)sn.p, 256, pool.p, nb, bs, (const int32_t*)table->p, mb,
                                      (const int32_t*)sl->p, nullptr, w.p, ws, nullptr) == MLA_OK,
               "append paged");
        ++calls;
        drain("append paged");
        delete sl;
        delete table;
    }
}

// The model must catch what it exists to catch: a plan entry pointing past the
// batch, a workgroup started in the wrong row, and a buffer one row short.
void self_check()
{
    const std::vector<int32_t> lens = {300, 0, 45};
    const int b = 3, cr0 = 4 + (b + 1) + 2 * b;
    struct Plant {
        long index;
        int value;
        const char* what;
    };
    const Plant plants[] = {{cr0 + 0, 7, "chunk starts in row 7 of 3"},
                            {cr0 + 1, 2, "chunk 1 starts in the wrong row"},
                            {4 + 1, -40, "prefix sum negative"}};
    for (const Plant& pl : plants) {
        model::plant_plan_entry(pl.index, pl.value);
        mla_decode_config_t c = cfg_of(8, 0, 0);
        expecting_failures = true;
        run_decode(MLA_DTYPE_BF16, lens, 300, 128, &c, "self-check");
        expecting_failures = false;
        const bool caught = failures > 0;
        failures = 0;
        expect(caught, std::string("self-check: planted '") + pl.what + "' not caught");
        if (caught) std::printf("self-check caught: %s\n", pl.what);
    }
    // a query buffer one row short (the last head of the last batch row)
    model::clear_regions();
    const int h = 128;
    const size_t ws = mla_decode_workspace_bytes(MLA_DTYPE_BF16, b, h, 300);
    Fake q((size_t)b * h * 1152 - 1152, "q'"), cache((size_t)b * 300 * 1152, "cache"), out((size_t)b * h * 1024, "out"),
        lse((size_t)b * h * 4, "lse");
    Real* sl = ints(lens, "seqlens");
    Real w(ws, "workspace", 0xAB);
    model::set_context("self-check short q'");
    mla_decode(MLA_DTYPE_BF16, b, h, 300, q.p, cache.p, (const int32_t*)sl->p, 0.07f, out.p, (float*)lse.p, w.p, ws,
               nullptr);
    const std::vector<std::string> f = model::take_failures();
    expect(!f.empty(), "self-check: a query buffer one row short was not caught");
    if (!f.empty()) std::printf("self-check caught: %s\n", f[0].c_str());
    delete sl;
}

}  // namespace

int main()
{
    self_check();
    validation();
    schedules();
    other_calls();
    std::printf("host model: %lld calls, %lld modelled launches, %d failures\n", calls, model::launches(), failures);
    return failures == 0 ? 0 : 1;
}
