// CPU model of the library's kernels for the host-layer build under the
// sanitizers (tests/host_model).  Device buffers are address ranges the
// driver registers; the model's stand-in launchers replay each kernel's
// addressing (the split plan built by the device's own plan code on emulated
// lanes, each workgroup's walk over its segments, every query row, cache row,
// partial and output it reads or writes) and record any access that falls
// outside every registered range.
#pragma once

#include <cstddef>
#include <functional>
#include <string>
#include <vector>

namespace model {

// A registered buffer.  `real` buffers are host memory the model reads or
// writes (seqlens, block tables, the workspace); the others are address
// ranges only (queries, cache, outputs), never dereferenced.
void clear_regions();
void add_region(const void* base, size_t bytes, const char* name, bool real);
void set_context(const std::string& ctx);
// Out-of-range accesses and broken invariants since the last call (cleared).
std::vector<std::string> take_failures();
long long launches();
// Self-check hooks: after the next plan build, plan entry `index` is set to
// `value` (index < 0: off).
void plant_plan_entry(long index, int value);

}  // namespace model

void run_wave(const std::function<void()>& fn);
