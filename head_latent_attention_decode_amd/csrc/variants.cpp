// Host-side queries on the bf16 attention kernel variants (the table in
// variants.h): which exist, their names, tiles and supported cache forms.
#include "variants.h"

#include "mla355_internal.h"

namespace mla355 {

bool bf16_variant_exists(int heads_per_group, int variant)
{
    return find_variant_info(heads_per_group, variant) != nullptr;
}

const char* bf16_kernel_name(int heads_per_group, int variant, bool paged)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v == nullptr ? nullptr : (paged ? v->paged_name : v->name);
}

bool bf16_variant_fp8(int heads_per_group, int variant)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v != nullptr && v->fp8_name != nullptr;
}

const char* fp8_kernel_name(int heads_per_group, int variant)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v == nullptr ? nullptr : v->fp8_name;
}

bool bf16_variant_plans(int heads_per_group, int variant)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v != nullptr && v->plans;
}

bool bf16_variant_pages(int heads_per_group, int variant)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v != nullptr && v->paged_name != nullptr;
}

int bf16_tile_tokens(int heads_per_group, int variant)
{
    const VariantInfo* v = find_variant_info(heads_per_group, variant);
    return v ? v->tile_tokens : 0;
}

}  // namespace mla355
