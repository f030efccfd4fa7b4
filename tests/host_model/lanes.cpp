// 64 host threads as the lanes of one wave, for running wave-level device
// code (the split-plan builder) on the CPU.  Shuffles and ballots exchange
// values through a shared array between two barriers; a lane that waits more
// than a few seconds at a barrier means the lanes' calls diverged, which is
// reported and aborts the run.
#include <hip/hip_runtime.h>

#include <chrono>
#include <condition_variable>
#include <cstdio>
#include <cstdlib>
#include <functional>
#include <mutex>
#include <thread>
#include <vector>

thread_local HostThreadIdx threadIdx = {0, 0, 0};

hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }

namespace {

constexpr int kLanes = 64;
std::mutex mu;
std::condition_variable cv;
int arrived = 0;
unsigned long long generation = 0;
long long slots[kLanes];

void lane_barrier()
{
    std::unique_lock<std::mutex> lk(mu);
    const unsigned long long g = generation;
    if (++arrived == kLanes) {
        arrived = 0;
        ++generation;
        cv.notify_all();
        return;
    }
    if (!cv.wait_for(lk, std::chrono::seconds(20), [&] { return generation != g; })) {
        std::fprintf(stderr, "lane barrier timed out: the emulated lanes took different paths\n");
        std::abort();
    }
}

long long exchange(long long v, int src)
{
    const int lane = threadIdx.x & 63;
    slots[lane] = v;
    lane_barrier();
    const long long r = slots[src];
    lane_barrier();
    return r;
}

}  // namespace

int __shfl_up(int v, unsigned delta, int)
{
    const int lane = threadIdx.x & 63;
    return (int)exchange(v, lane >= (int)delta ? lane - (int)delta : lane);
}

int __shfl(int v, int src_lane, int) { return (int)exchange(v, src_lane & 63); }

unsigned long long __ballot(int pred)
{
    const int lane = threadIdx.x & 63;
    slots[lane] = pred != 0;
    lane_barrier();
    unsigned long long m = 0;
    for (int i = 0; i < kLanes; ++i)
        if (slots[i]) m |= 1ull << i;
    lane_barrier();
    return m;
}

// Runs fn on 64 lanes (threadIdx.x = 0..63) and waits for all of them.
void run_wave(const std::function<void()>& fn)
{
    std::vector<std::thread> lanes;
    lanes.reserve(kLanes);
    for (int l = 0; l < kLanes; ++l)
        lanes.emplace_back([l, &fn] {
            threadIdx.x = (unsigned)l;
            fn();
        });
    for (auto& t : lanes) t.join();
}
