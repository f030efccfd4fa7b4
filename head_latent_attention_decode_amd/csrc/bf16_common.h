// Device-side building blocks shared by the bf16 decode kernels: vector
// types, LDS-DMA wait and barrier helpers, per-stage LDS arrays, the MFMA
// wrappers with their tile swizzles.  Everything sits in an anonymous
// namespace, so each kernel file gets its own copies.
#pragma once

#include "mla355_internal.h"

namespace mla355 {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

#define LDS_AS __attribute__((address_space(3)))
typedef LDS_AS unsigned char lds_byte;

constexpr float kRescaleThreshold = 8.0f;  // log2 of the largest tolerated growth
constexpr float kNegBig = -1.0e30f;        // finite "minus infinity" for the running max
// Buffer resource word 3 for raw (untyped, unswizzled) buffer access on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (expcnt and lgkmcnt left at their maxima).  Issued
// through the builtin so that the compiler's own wait insertion sees it.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8); }

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
}

// Workgroup barrier ordering LDS only: the fences make every LDS access
// before the barrier complete (lgkmcnt) and keep the compiler from moving LDS
// accesses across it, without waiting for outstanding global loads.  Tile
// data arrives by DMA, so its completion is awaited separately (vmcnt) by
// the issuing wave before the barrier.
__device__ __forceinline__ void wg_barrier()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Barrier for data exchanged through ordinary LDS stores (not DMA): waits for
// this wave's LDS accesses (lgkmcnt) only.  A release fence on LDS would also
// wait for every DMA still landing in other stages (the compiler counts those
// as LDS writes), which would serialise the tile prefetch with compute.  The
// empty asm statements keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_exchange_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Orders this wave's own LDS traffic: its earlier LDS accesses complete
// before its later ones issue (for data a wave stages through LDS for itself).
__device__ __forceinline__ void lds_wave_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt((0xF) | (0x3 << 14) | (0x7 << 4));  // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

// One LDS array per pipeline stage.  Distinct objects let the compiler prove
// that reads of one stage do not alias DMA still landing in another, so it
// does not insert conservative vmcnt(0) waits before them.
template <int BYTES, int S>
__device__ __forceinline__ lds_byte* stage_lds()
{
    __shared__ __attribute__((aligned(1024))) unsigned char buf[BYTES];
    return (lds_byte*)buf;
}

template <int V>
struct IC {
    static constexpr int value = V;
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x of lane l, x of lane l ^ 32): lanes l and l + 32 hold the two halves
// of one head in the 32-wide MFMA layouts.  v_permlane32_swap exchanges the
// upper 32 lanes of its first operand with the lower 32 lanes of its second,
// so with x in both, each lane ends with its own value in one register and
// its partner's in the other.  Written as inline asm because the compiler's
// builtin returns its first result for both (the second result is lost); the
// nops give the wait states around a permlane that the hazard recognizer
// cannot see inside asm.
__device__ __forceinline__ float max_xor32(float x)
{
    unsigned a = __builtin_bit_cast(unsigned, x), b = a;
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
    return fmaxf(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

template <int WH>
struct Mfma;

template <>
struct Mfma<16> {
    typedef f32x4_t acc_t;
    static constexpr int kK = 32;      // contraction per instruction
    static constexpr int kAcc = 4;     // fp32 accumulators per lane
    __device__ __forceinline__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // Region-A swizzle (4 bits), chunk position c ^ xa(r & 15).  On gfx950 a
    // ds_read_b128 serves its 64 lanes in four cycles of 16 lanes; lane l
    // goes to cycle (l >> 5, bit2 ^ bit3 ^ bit4 of l), which is not 16
    // consecutive lanes (a b64 read, transposed or not, serves lanes 0..31
    // then 32..63).  Score reads: lane (g = l >> 4, rr = l & 15) reads chunk
    // (4k + g) ^ xa(rr) of row rr, so one cycle holds rows {b2 ^ b3 = p} with
    // g even and rows {b2 ^ b3 = p ^ 1} with g odd; both sets of positions are
    // disjoint and cover all 16 bank quads when xa of the rows with
    // b2 ^ b3 = 1 (rows 4..11) is closed under ^1.  Transposed reads of 8
    // rows (0..7 or 8..15) by a 16-column strip need xa >> 1 distinct over
    // each of those runs of 8.  Rows 0..7 -> 2r, rows 8..15 -> 2((r & 7) ^ 4) + 1.
    __device__ __forceinline__ static int xa(int r) { return (((r & 7) << 1) ^ (r & 8)) | ((r >> 3) & 1); }
};

template <>
struct Mfma<32> {
    typedef f32x16_t acc_t;
    static constexpr int kK = 16;
    static constexpr int kAcc = 16;
    __device__ __forceinline__ static acc_t mma(bf16x8_t a, bf16x8_t b, acc_t c)
    {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // rows 0..15 distinct, and each run of 4 rows lands in distinct 64-byte
    // quads (b64 transposed reads of a 32-column strip by 4 rows).
    __device__ __forceinline__ static int xa(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
};

// Workgroup -> (chunk k, head group hg).  Workgroups are dispatched
// round-robin over the 8 XCDs (block i -> XCD i % 8), each with its own L2.
// XCD x takes a contiguous run of n_chunks / 8 chunks with all their head
// groups: the head groups of a chunk share that L2's copy of its latent tiles,
// and the consecutive chunks of one batch row share its query rows.
// n_chunks is a multiple of 8.
__device__ __forceinline__ void block_work(int n_chunks, int n_hg, int& k, int& hg)
{
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    k = xcd * (n_chunks >> 3) + slot / n_hg;
    hg = slot % n_hg;
}

// Opt-in engine-clock stamps (DecodeParams::clock_stamps): the first thread
// of workgroup 0 records the shader clock and the 100 MHz real-time counter,
// pair `which` (0: start, 1: end).  A vector store (the thread condition makes
// the data a per-lane value).
__device__ __forceinline__ void clock_stamp(unsigned long long* st, int which)
{
    if (st != nullptr && blockIdx.x == 0 && threadIdx.x == 0) {
        const unsigned long long c = __builtin_amdgcn_s_memtime();
        const unsigned long long r = __builtin_amdgcn_s_memrealtime();
        st[2 * which] = c;
        st[2 * which + 1] = r;
    }
}

// Eight OCP e4m3 codes (first in the low byte) -> eight bf16, exact: every
// e4m3 value is a bf16 value.
__device__ __forceinline__ bf16x8_t cvt8_e4m3(unsigned long long codes)
{
    const unsigned lo = (unsigned)codes, hi = (unsigned)(codes >> 32);
    const bf16x2_t a0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    const bf16x2_t a1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    const bf16x2_t a2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    const bf16x2_t a3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    return (bf16x8_t){a0[0], a0[1], a1[0], a1[1], a2[0], a2[1], a3[0], a3[1]};
}

// 32x32x16 score MFMAs with the accumulator in VGPRs, for kernels whose
// output sums take all 256 AGPRs: given the builtin, the compiler picks one
// register form for every MFMA of a kernel, places the score accumulator in
// AGPRs as well and parks an output block in VGPRs around every score chain.
// The hazard recognizer does not look inside asm: score_wait() supplies the
// wait states between the last MFMA of a chain and the first vector-ALU
// access to its result (more than the 12 that a dependent read of an 8-pass
// result needs).
__device__ __forceinline__ f32x16_t score_first(bf16x8_t a, bf16x8_t b)
{
    f32x16_t d;
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
    return d;
}
__device__ __forceinline__ void score_acc(f32x16_t& acc, bf16x8_t a, bf16x8_t b)
{
    asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_wait(f32x16_t& acc)
{
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(acc));
}

// Region-B swizzle (3 bits, 128-byte rows): rows of equal parity distinct.
__device__ __forceinline__ int xb(int r) { return (r >> 1) & 7; }

}  // namespace
}  // namespace mla355
