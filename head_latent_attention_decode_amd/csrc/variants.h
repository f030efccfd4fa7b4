// Host-side table of the bf16 split-KV attention kernel variants: which
// kernel family and template arguments serve a (heads per group, variant)
// pair, the names profilers print for them, and what each form supports.
// No device code: the launchers in decode_bf16.hip are generated from this
// table at compile time, and host code (the scheduler in api.cpp, CPU builds
// of the host layer) reads it directly.
#pragma once

namespace mla355 {

enum class KernelFamily {
    Tiled,  // decode_bf16_kernel<WH, HS, TS, NT, STAGES, FP8>
    Pair,   // decode_pair_kernel<P, STAGES>
    Wide,   // decode_wide_kernel<NW, STAGES, PAGED>; fp8 cache: decode_wide_fp8_kernel (128 heads)
    Split,  // decode_colsplit_kernel<PAGED>: 128 heads, weighted sum split by columns
};

struct VariantInfo {
    int heads_per_group;
    int variant;
    int tile_tokens;         // tokens per LDS tile (the plan's smallest chunk)
    KernelFamily family;
    int targs[5];            // template arguments, in the family's order
    const char* name;        // kernel name as profilers print it
    const char* paged_name;  // the same for a paged cache; nullptr: not supported
    const char* fp8_name;    // the same for an fp8 cache; nullptr: not supported
    bool plans;              // builds its own split plan in LDS
};

// The three-stage pair kernel (<2, 3>) is not listed: it took a GPU memory
// fault on the edge-length batch (lengths 0..700, 64 heads) whose cause has
// not been found; every listed variant passes the same tests.
inline constexpr VariantInfo kVariantInfo[] = {
    {16, 1, 64, KernelFamily::Tiled, {16, 1, 2, 32, 2}, "decode_bf16_kernel<16, 1, 2, 32, 2, false>", nullptr,
     "decode_bf16_kernel<16, 1, 2, 32, 2, true>", false},
    {16, 2, 32, KernelFamily::Tiled, {16, 1, 1, 32, 2}, "decode_bf16_kernel<16, 1, 1, 32, 2, false>", nullptr,
     nullptr, false},
    {32, 1, 64, KernelFamily::Tiled, {16, 2, 2, 32, 2}, "decode_bf16_kernel<16, 2, 2, 32, 2, false>", nullptr,
     nullptr, false},
    {32, 2, 32, KernelFamily::Tiled, {32, 1, 1, 32, 2}, "decode_bf16_kernel<32, 1, 1, 32, 2, false>", nullptr,
     nullptr, false},
    {64, 1, 64, KernelFamily::Tiled, {16, 4, 1, 64, 2}, "decode_bf16_kernel<16, 4, 1, 64, 2, false>", nullptr,
     nullptr, false},
    {64, 2, 32, KernelFamily::Tiled, {32, 2, 1, 32, 4}, "decode_bf16_kernel<32, 2, 1, 32, 4, false>", nullptr,
     nullptr, false},
    {128, 1, 32, KernelFamily::Tiled, {32, 4, 1, 32, 4}, "decode_bf16_kernel<32, 4, 1, 32, 4, false>", nullptr,
     nullptr, false},
    {128, 2, 32, KernelFamily::Tiled, {16, 8, 1, 32, 2}, "decode_bf16_kernel<16, 8, 1, 32, 2, false>", nullptr,
     nullptr, false},
    {64, 3, 32, KernelFamily::Pair, {2, 4}, "decode_pair_kernel<2, 4>", nullptr, nullptr, false},
    {32, 3, 32, KernelFamily::Pair, {1, 4}, "decode_pair_kernel<1, 4>", nullptr, nullptr, false},
    {128, 3, 32, KernelFamily::Wide, {4, 3}, "decode_wide_kernel<4, 3, false>", "decode_wide_kernel<4, 3, true>",
     nullptr, true},
    {128, 4, 32, KernelFamily::Wide, {4, 2}, "decode_wide_kernel<4, 2, false>", "decode_wide_kernel<4, 2, true>",
     "decode_wide_fp8_kernel", true},
    {128, 5, 32, KernelFamily::Wide, {4, 4}, "decode_wide_kernel<4, 4, false>", "decode_wide_kernel<4, 4, true>",
     nullptr, false},
    {64, 5, 32, KernelFamily::Wide, {2, 3}, "decode_wide_kernel<2, 3, false>", "decode_wide_kernel<2, 3, true>",
     nullptr, true},
    {64, 6, 32, KernelFamily::Wide, {2, 2}, "decode_wide_kernel<2, 2, false>", "decode_wide_kernel<2, 2, true>",
     nullptr, true},
    {32, 4, 32, KernelFamily::Wide, {1, 3}, "decode_wide_kernel<1, 3, false>", "decode_wide_kernel<1, 3, true>",
     nullptr, true},
    {128, 6, 32, KernelFamily::Split, {}, "decode_colsplit_kernel<false>", "decode_colsplit_kernel<true>", nullptr,
     true},
};
inline constexpr int kNumVariants = (int)(sizeof(kVariantInfo) / sizeof(kVariantInfo[0]));

// Index of (heads_per_group, variant) in kVariantInfo (variant 0 means 1), or -1.
inline int find_variant_index(int heads_per_group, int variant)
{
    if (variant == 0) variant = 1;
    for (int i = 0; i < kNumVariants; ++i)
        if (kVariantInfo[i].heads_per_group == heads_per_group && kVariantInfo[i].variant == variant) return i;
    return -1;
}

inline const VariantInfo* find_variant_info(int heads_per_group, int variant)
{
    const int i = find_variant_index(heads_per_group, variant);
    return i < 0 ? nullptr : &kVariantInfo[i];
}

}  // namespace mla355
