// Host-side layout of the cache-append workspace, shared by the append
// launcher and host code that sizes or checks it.
#pragma once

#include "mla355_internal.h"

namespace mla355 {

// The projection cuts the hidden dimension into chunks of this many columns.
constexpr int kAppendKD = 256;

// Workspace: fp32 partial sums [b][d_model / kAppendKD][576], then a copy of
// the b positions.
inline size_t append_part_bytes(int b, int d_model)
{
    return align_up((size_t)b * (size_t)(d_model / kAppendKD) * kDqk * sizeof(float), 256);
}

inline size_t append_workspace_bytes(int b, int d_model)
{
    return append_part_bytes(b, d_model) + align_up((size_t)b * sizeof(int32_t), 256);
}

inline int append_kd() { return kAppendKD; }

}  // namespace mla355
