// Query and output absorption (per-head batched matrix products).
//
// Glossary "Multi-head Latent Attention", section on why decode absorbs:
//   q absorb: qbar_h = q^C_h (W^UK_h)^T, a 512-wide latent-space query, which
//             the FlashMLA issue-16 answer concatenates with the 64-wide rope
//             query into the 576-wide attention input;
//   o absorb: (sum_t p_t c_t) W^UV_h, the value up-projection applied once to
//             the 512-wide attention output.
// Both are per-head products with a 128 x 512 weight block used by only b
// query rows, so they are weight-read bound at small b.  bf16: one workgroup
// per (head, 64 or 256 output columns) DMAs its weight slabs and the head's
// input rows (64 at a time) into LDS in 16 KB parts, all requested at once
// and each multiplied as it lands, reads the slab transposed
// (ds_read_b64_tr_b16) as the A operand of v_mfma_f32_16x16x32_bf16 and the
// input rows as the B operand, fp32 accumulation.  fp32: the vector-ALU
// kernels below (IEEE fp32 FMAs), one workgroup per (head, block of 16 batch
// rows).
#include "append_layout.h"
#include "bf16_common.h"

#include <utility>

namespace mla355 {
namespace {

constexpr int kRows = 16;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }
template <typename T>
__device__ __forceinline__ T from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

template <typename T>
struct Vec4;
template <>
struct Vec4<float> {
    typedef float type __attribute__((ext_vector_type(4)));
};
template <>
struct Vec4<__bf16> {
    typedef __bf16 type __attribute__((ext_vector_type(4)));
};

// q'[r,h,0:512] = q_nope[r,h,:] . W_UK[h] ;  q'[r,h,512:576] = q_rope[r,h,:]
// 128 threads; thread t owns latent columns 4t .. 4t+3 for the 16 rows.
template <typename T>
__global__ __launch_bounds__(128) void absorb_q_kernel(int b, int h, const T* __restrict__ q_nope,
                                                       const T* __restrict__ w_uk,
                                                       const T* __restrict__ q_rope,
                                                       T* __restrict__ q_prime)
{
    typedef typename Vec4<T>::type v4;
    __shared__ float qs[kRows][kDk];
    const int head = blockIdx.x % h;
    const int r0 = (blockIdx.x / h) * kRows;
    const int nrows = min(kRows, b - r0);
    const int t = threadIdx.x;
    for (int i = t; i < kRows * kDk; i += 128) {
        const int rr = i / kDk, j = i % kDk;
        qs[rr][j] = rr < nrows ? to_f32(q_nope[((size_t)(r0 + rr) * h + head) * kDk + j]) : 0.f;
    }
    __syncthreads();
    float acc[kRows][4];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[rr][e] = 0.f;
    const T* w = w_uk + (size_t)head * kDk * kDc + 4 * t;
    for (int j = 0; j < kDk; ++j) {
        const v4 wv = *(const v4*)(w + (size_t)j * kDc);
        const float w0 = to_f32(wv[0]), w1 = to_f32(wv[1]), w2 = to_f32(wv[2]), w3 = to_f32(wv[3]);
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) {
            const float q = qs[rr][j];
            acc[rr][0] = fmaf(q, w0, acc[rr][0]);
            acc[rr][1] = fmaf(q, w1, acc[rr][1]);
            acc[rr][2] = fmaf(q, w2, acc[rr][2]);
            acc[rr][3] = fmaf(q, w3, acc[rr][3]);
        }
    }
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) {
        if (rr < nrows) {
            v4 o;
#pragma unroll
            for (int e = 0; e < 4; ++e) o[e] = from_f32<T>(acc[rr][e]);
            *(v4*)(q_prime + ((size_t)(r0 + rr) * h + head) * kDqk + 4 * t) = o;
        }
    }
    for (int i = t; i < nrows * kDr; i += 128) {
        const int rr = i / kDr, j = i % kDr;
        q_prime[((size_t)(r0 + rr) * h + head) * kDqk + kDc + j] =
            q_rope[((size_t)(r0 + rr) * h + head) * kDr + j];
    }
}

// y[r,h,:] = o[r,h,:] . W_UV[h]
// 128 threads; thread t owns output column t for the 16 rows.
template <typename T>
__global__ __launch_bounds__(128) void absorb_o_kernel(int b, int h, const T* __restrict__ o,
                                                       const T* __restrict__ w_uv,
                                                       T* __restrict__ y)
{
    __shared__ float os[kRows][kDc];
    const int head = blockIdx.x % h;
    const int r0 = (blockIdx.x / h) * kRows;
    const int nrows = min(kRows, b - r0);
    const int t = threadIdx.x;
    for (int i = t; i < kRows * kDc; i += 128) {
        const int rr = i / kDc, c = i % kDc;
        os[rr][c] = rr < nrows ? to_f32(o[((size_t)(r0 + rr) * h + head) * kDc + c]) : 0.f;
    }
    __syncthreads();
    float acc[kRows];
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr) acc[rr] = 0.f;
    const T* w = w_uv + (size_t)head * kDc * kDv + t;
    for (int c = 0; c < kDc; ++c) {
        const float wv = to_f32(w[(size_t)c * kDv]);
#pragma unroll
        for (int rr = 0; rr < kRows; ++rr) acc[rr] = fmaf(os[rr][c], wv, acc[rr]);
    }
#pragma unroll
    for (int rr = 0; rr < kRows; ++rr)
        if (rr < nrows) y[((size_t)(r0 + rr) * h + head) * kDv + t] = from_f32<T>(acc[rr]);
}


// Weight slab [KD][64] bf16 in LDS, 128-byte rows.  16-byte chunk c of row r is
// stored at c ^ (2 * f(r)), f(r) = ((r >> 1) & 1) | (((r >> 3) & 1) << 1), so the
// transposed reads of 4-row groups spread over distinct 32-byte bank windows.
__device__ __forceinline__ int slab_chunk(int r, int c)
{
    const int f = ((r >> 1) & 1) | (((r >> 3) & 1) << 1);
    return c ^ (2 * f);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>)
{
    (f(IC<I>{}), ...);
}
// f(IC<0>{}), ..., f(IC<N - 1>{}): a loop whose index is a compile-time constant.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Block index for workgroup id `id` of `count` when each head has NB blocks
// that read the same input rows.  Workgroups go to the 8 XCDs round-robin by
// id, so ids that are equal mod 8 share one XCD and its L2: head 8a + x gets
// the ids 8 NB a + 8 j + x (its block j), and its input rows come from HBM
// once rather than NB times.  Ids past the last whole group of 8 heads keep
// their own index.
template <int NB>
__device__ __forceinline__ int xcd_head_block(int id, int count)
{
    constexpr int kSpan = 8 * NB;
    const int full = count / kSpan * kSpan;
    if (id >= full) return id;
    const int a = id / kSpan, rem = id % kSpan;
    return (8 * a + rem % 8) * NB + rem / 8;
}

// Y^T[n, m] = sum_k W[h][k][n] X[m][h][k] for 64 NCB columns n0.. of head h.
//   W  [H][KD][ND] (n contiguous)      X  row m of head h at x + m*x_rs + h*KD
//   Y  row m of head h at y + m*y_rs + h*y_hs + n
// Both operands go HBM -> LDS by direct-to-LDS DMA (the product is bound by
// reading the weights), in parts of 16 KB: a part is 128 contraction rows of
// one 64-column weight slab (NCB > 1: slab p, all of KD = 128; NCB = 1: rows
// 128p .. of the one slab) and, for NCB = 1, the same 128 columns of the
// head's 64 input rows (NCB > 1: all input columns with part 0).  Every part
// of row block 0 is requested at once, each into its own LDS object, and each
// is multiplied as soon as it has landed, while the later parts still stream.
// Staged input rows are 256 bytes, 16-byte chunk c of row m at c ^ (m & 15),
// so 16 consecutive rows read at one k offset hit 16 distinct bank quads.
// 4 waves; wave w owns columns 16w .. +15 of a slab (v_mfma_f32_16x16x32_bf16
// A rows, read transposed with ds_read_b64_tr_b16); batch rows are the B
// columns, 16 per block.  Each 64 x 64 output block goes out through LDS as
// whole 16-byte pieces of its rows.  When rope != nullptr (q absorb), the
// workgroups of column block 0 also copy rope[m][h][0:64] to y[...][ND:ND+64].
// blk: this workgroup's index among the product's H * ND / (64 NCB) blocks;
// OutT: type of Y (bf16, or fp32 for partial sums that are added up later).
template <int KD, int ND, int NCB, typename OutT>
__device__ __forceinline__ void absorb_mfma_body(int blk, int M, int H, const __bf16* __restrict__ x,
                                                 long x_rs, const __bf16* __restrict__ w,
                                                 OutT* __restrict__ y, long y_rs, int y_hs,
                                                 const __bf16* __restrict__ rope)
{
    static_assert(NCB == 1 ? KD % 128 == 0 : KD == 128, "parts of 128 contraction rows");
    constexpr int NB = ND / (64 * NCB);       // workgroups per head
    constexpr int P = NCB > 1 ? NCB : KD / 128;
    constexpr int KSP = 4;                    // k steps (of 32) per part
    constexpr int XP = NCB > 1 ? 1 : P;       // staged input parts
    constexpr int PART = 16384;               // bytes of a weight part, and of an input part
    constexpr int DMA_W = PART / 4096;        // 1 KB DMA instructions per wave and part
    constexpr int DMA_X = PART / 4096;
    constexpr int STG_ROW = 64 * (int)sizeof(OutT) + 16;  // output staging row (padded)
    static_assert(ND % (64 * NCB) == 0, "whole slabs per workgroup");
    const int h = blk / NB;
    const int n0 = (blk % NB) * 64 * NCB;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, s = lane & 15;

    // One LDS object per part (and per staged input part): the compiler then
    // tracks the DMA of each separately and waits only for the part it reads.
    auto wpart = [&](auto PI) -> lds_byte* { return stage_lds<PART, 10 + decltype(PI)::value>(); };
    auto xpart = [&](auto PI) -> lds_byte* { return stage_lds<PART, 20 + decltype(PI)::value>(); };
    lds_byte* stg = stage_lds<64 * STG_ROW, 30>();

    const __bf16* wh = w + (size_t)h * KD * ND + n0;
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        (void*)wh, (short)0, ((KD - 1) * ND + 64 * NCB) * 2, kBufferFlags);
    const __bf16* xh = x + (size_t)h * KD;
    const unsigned x_bytes = (unsigned)(((size_t)(M - 1) * x_rs + KD) * 2);
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc((void*)xh, (short)0, x_bytes, kBufferFlags);

    // weight part p: 128 contraction rows (of slab p, or rows 128p.. of the
    // one slab) x 64 columns; DMA block j = rows 8j .. +7, lane -> row
    // 8j + lane/8, slot lane%8.
    auto stage_w = [&](auto PI) {
        constexpr int p = decltype(PI)::value;
        lds_byte* dst = wpart(PI);
#pragma unroll
        for (int i = 0; i < DMA_W; ++i) {
            const int j = wave * DMA_W + i;
            const int r = j * 8 + (lane >> 3);
            const int c = slab_chunk(r, lane & 7);
            const int k = NCB > 1 ? r : p * 128 + r;
            const int cb = NCB > 1 ? p : 0;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (LDS_AS void*)(dst + j * 1024), 16,
                                                     (unsigned)((k * ND + cb * 64 + c * 8) * 2), 0, 0, 0);
        }
    };
    // input part p of row block mb0: rows mb0*64 .. +63 (rows past M re-read
    // row M-1; never stored), contraction columns 128p .. +127 as 256-byte rows,
    // 16-byte chunk c of row m at c ^ (m & 15).
    auto stage_x = [&](auto PI, int mb0) {
        constexpr int p = decltype(PI)::value;
        lds_byte* dst = xpart(PI);
#pragma unroll
        for (int i = 0; i < DMA_X; ++i) {
            const int j = wave * DMA_X + i;
            const int m = j * 4 + (lane >> 4);
            const int c = (lane & 15) ^ (m & 15);
            const int mg = min(mb0 * 64 + m, M - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (LDS_AS void*)(dst + j * 1024), 16,
                                                     (unsigned)(((size_t)mg * x_rs + p * 128 + c * 8) * 2), 0, 0, 0);
        }
    };

    // A operand (W^T rows n, k-slots g*8 .. +7) for the 4 k steps of a part.
    // tr16 mapping: source lane s of a 16-lane group supplies row k0 + g*8 + s/4
    // (+4 for the upper half), columns 4*(s%4) .. +3 of the wave's 16 columns.
    const int col = wave * 16 + 4 * (s & 3);
    auto read_a = [&](const lds_byte* sl, bf16x8_t (&a)[KSP]) {
#pragma unroll
        for (int ks = 0; ks < KSP; ++ks) {
            const int r0 = ks * 32 + g * 8 + (s >> 2);
            const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS i16x4_t*)(sl + r0 * 128 + (slab_chunk(r0, col >> 3) << 4) + (col & 7) * 2));
            const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (LDS_AS i16x4_t*)(sl + (r0 + 4) * 128 + (slab_chunk(r0 + 4, col >> 3) << 4) + (col & 7) * 2));
            a[ks] = __builtin_shufflevector(__builtin_bit_cast(bf16x4_t, lo), __builtin_bit_cast(bf16x4_t, hi),
                                            0, 1, 2, 3, 4, 5, 6, 7);
        }
    };
    // acc[mb] += W-part^T . X-part^T for batch rows mb*16 + s (B operand:
    // staged row mb*16 + s, k-slots g*8 .. +7 of each step).
    auto mma_part = [&](const lds_byte* wl, const lds_byte* xl, f32x4_t (&acc)[4]) {
        bf16x8_t a[KSP];
        read_a(wl, a);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const lds_byte* xr = xl + (mb * 16 + s) * 256;
#pragma unroll
            for (int ks = 0; ks < KSP; ++ks) {
                const bf16x8_t b = *(const LDS_AS bf16x8_t*)(xr + (((ks * 4 + g) ^ s) << 4));
                acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b, acc[mb], 0, 0, 0);
            }
        }
    };
    // Output block (64 batch rows x 64 columns n0 + 64cb ..) through LDS, so
    // that each row goes out as whole 16-byte pieces of one 128-byte (bf16) or
    // 256-byte (fp32) run.  acc[mb][i]: row mb*16 + s, column 16 wave + 4g + i.
    auto store_block = [&](const f32x4_t (&acc)[4], int mb0, int cb) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            lds_byte* d = stg + (mb * 16 + s) * STG_ROW + (wave * 16 + g * 4) * (int)sizeof(OutT);
            if constexpr (sizeof(OutT) == 2) {
                bf16x4_t o;
                o[0] = (__bf16)acc[mb][0];
                o[1] = (__bf16)acc[mb][1];
                o[2] = (__bf16)acc[mb][2];
                o[3] = (__bf16)acc[mb][3];
                *(LDS_AS bf16x4_t*)d = o;
            } else {
                *(LDS_AS f32x4_t*)d = acc[mb];
            }
        }
        lds_exchange_barrier();
        constexpr int PIECES = 64 * (int)sizeof(OutT) / 16;  // 16-byte pieces per row
        constexpr int ROWS_PER_PASS = 256 / PIECES;
#pragma unroll
        for (int r0 = 0; r0 < 64; r0 += ROWS_PER_PASS) {
            const int rr = r0 + threadIdx.x / PIECES, pc = threadIdx.x % PIECES;
            const int m = mb0 * 64 + rr;
            const bf16x8_t v = *(const LDS_AS bf16x8_t*)(stg + rr * STG_ROW + pc * 16);
            if (m < M)
                *(bf16x8_t*)(y + (size_t)m * y_rs + (size_t)h * y_hs + n0 + cb * 64 +
                             pc * (16 / (int)sizeof(OutT))) = v;
        }
        lds_exchange_barrier();  // staging free for the next block
    };
    // q absorb: rope[m][h][0:64] -> y[...][ND:ND+64] for the rows of block mb0
    // (workgroups of column block 0; two 16-byte pieces per thread).  Loaded
    // before the DMAs (rows past M re-read row M-1, unconditionally: a
    // per-lane branch around the load makes the compiler wait for it at once)
    // and stored at the end of the block.
    bf16x8_t rv[2];
    auto rope_load = [&](int mb0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = threadIdx.x + 256 * u;
            const int m = min(mb0 * 64 + (i >> 3), M - 1), c = i & 7;
            rv[u] = *(const bf16x8_t*)(rope + ((size_t)m * H + h) * 64 + c * 8);
        }
    };
    auto rope_store = [&](int mb0) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = threadIdx.x + 256 * u;
            const int m = mb0 * 64 + (i >> 3), c = i & 7;
            if (m < M) *(bf16x8_t*)(y + (size_t)m * y_rs + (size_t)h * y_hs + ND + c * 8) = rv[u];
        }
    };
    const bool do_rope = rope != nullptr && n0 == 0;

    // ---- row block 0: every part in flight at once, each consumed as it lands
    auto zero = [](f32x4_t (&acc)[4]) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) acc[mb] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    };

    // ---- row block 0: every part in flight at once, each consumed as it lands
    if (do_rope) rope_load(0);
    static_for<P>([&](auto PI) {
        constexpr int p = decltype(PI)::value;
        if constexpr (NCB == 1 || p == 0) stage_x(PI, 0);
        stage_w(PI);
    });
    {
        f32x4_t acc[4];
        zero(acc);
        static_for<P>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            // this wave's DMAs of the later parts may stay in flight; the
            // barrier then makes part p of every wave visible
            wait_vmcnt<(P - 1 - p) * (DMA_W + (NCB == 1 ? DMA_X : 0))>();
            lds_exchange_barrier();
            mma_part(wpart(PI), xpart(IC<NCB == 1 ? p : 0>{}), acc);
            if constexpr (NCB > 1) {
                store_block(acc, 0, p);
                zero(acc);
            }
        });
        if constexpr (NCB == 1) store_block(acc, 0, 0);
    }
    if (do_rope) rope_store(0);

    // ---- further row blocks (more than 64 batch rows): restage the input
    for (int mb0 = 1; mb0 * 64 < M; ++mb0) {
        if (do_rope) rope_load(mb0);
        lds_exchange_barrier();  // every wave is done with the previous block's input
        static_for<XP>([&](auto PI) { stage_x(PI, mb0); });
        wait_vmcnt<0>();
        lds_exchange_barrier();
        f32x4_t acc[4];
        zero(acc);
        static_for<P>([&](auto PI) {
            constexpr int p = decltype(PI)::value;
            mma_part(wpart(PI), xpart(IC<NCB == 1 ? p : 0>{}), acc);
            if constexpr (NCB > 1) {
                store_block(acc, mb0, p);
                zero(acc);
            }
        });
        if constexpr (NCB == 1) store_block(acc, mb0, 0);
        if (do_rope) rope_store(mb0);
    }
}

template <int KD, int ND, int NCB>
__global__ __launch_bounds__(256) void absorb_mfma_kernel(int M, int H, const __bf16* __restrict__ x,
                                                          long x_rs, const __bf16* __restrict__ w,
                                                          __bf16* __restrict__ y, long y_rs, int y_hs,
                                                          const __bf16* __restrict__ rope)
{
    absorb_mfma_body<KD, ND, NCB, __bf16>(xcd_head_block<ND / (64 * NCB)>(blockIdx.x, gridDim.x), M, H, x,
                                          x_rs, w, y, y_rs, y_hs, rope);
}

// ---- appending a token's latent row ------------------------------------------
// Glossary "Multi-head Latent Attention", layout difference from MHA/GQA: the
// cached row of token t is [c_t ; k^R_t] with c_t = x_t W^DKV (d_c = 512) and
// k^R_t = RoPE(x_t W^KR) (d_r = 64); Lesson 28: x_t is the d_model-wide
// hidden state (7168 in its example).  The projection is the per-head product
// above with the hidden dimension cut into d_model / kAppendKD chunks taking
// the place of heads: chunk h of every x row times rows h*kAppendKD.. of
// W_DKV (512 columns, 8 blocks of 64) and of W_KR (64 columns, 1 block), into
// fp32 partial sums P[m][h][0:576].  One launch covers both weights.
__global__ __launch_bounds__(256) void append_proj_kernel(int M, int H, const __bf16* __restrict__ x,
                                                          const __bf16* __restrict__ w_dkv,
                                                          const __bf16* __restrict__ w_kr,
                                                          float* __restrict__ part,
                                                          const int32_t* __restrict__ seqlens,
                                                          int32_t* __restrict__ wpos)
{
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < M; i += 256) wpos[i] = seqlens[i];
    const long x_rs = (long)H * kAppendKD;
    const int dkv_blocks = H * (kDc / 64);
    if ((int)blockIdx.x < dkv_blocks)
        absorb_mfma_body<kAppendKD, kDc, 1, float>(xcd_head_block<kDc / 64>(blockIdx.x, dkv_blocks), M, H, x,
                                                   x_rs, w_dkv, part, (long)H * kDqk, kDqk, nullptr);
    else
        absorb_mfma_body<kAppendKD, kDr, 1, float>(blockIdx.x - dkv_blocks, M, H, x, x_rs, w_kr,
                                                   part + kDc, (long)H * kDqk, kDqk, nullptr);
}

// One workgroup per (batch row m, block of 64 of the 576 columns): sum the H
// partials of its columns (thread t: column t % 64, every fourth chunk from
// t / 64, loads issued eight at a time), then write them as bf16 at cache row
// pos; the block of the 64 RoPE columns first turns each adjacent pair (2j,
// 2j+1) by the table entry (pos, j).  pos is the copy of seqlens[m] the
// projection kernel took (so that an in-place length update by block 0 cannot
// race with the other blocks' reads); nothing is written when pos is outside
// [0, min(t_max, n_pos)).  Block 0 writes seqlens_out[m] (may be null or equal
// to seqlens): pos + 1 for a written row, pos otherwise.
//
// Paged pool (block_table != null): cache is the pool [num_blocks,
// block_size, 576]; row pos of batch row m is row pos % block_size of block
// block_table[m * max_blocks + pos / block_size] (t_max = max_blocks *
// block_size); an entry outside [0, num_blocks) means no write.
__global__ __launch_bounds__(256) void append_finish_kernel(int H, int t_max, int n_pos,
                                                            const float* __restrict__ part,
                                                            const int32_t* __restrict__ wpos,
                                                            const float* __restrict__ rope_cos,
                                                            const float* __restrict__ rope_sin,
                                                            __bf16* __restrict__ cache,
                                                            int32_t* seqlens_out,
                                                            const int32_t* __restrict__ block_table,
                                                            int num_blocks, int block_size, int max_blocks)
{
    __shared__ float red[4][64];
    constexpr int NCB = kDqk / 64;
    const int m = blockIdx.x / NCB, cb = blockIdx.x % NCB;
    const int t = threadIdx.x;
    const int pos = wpos[m];
    bool write = pos >= 0 && pos < t_max && pos < n_pos;
    size_t row_off = (size_t)m * t_max + pos;  // destination row (contiguous cache)
    if (write && block_table != nullptr) {
        const int blk = block_table[(size_t)m * max_blocks + pos / block_size];
        write = blk >= 0 && blk < num_blocks;
        row_off = (size_t)blk * block_size + pos % block_size;
    }
    if (cb == 0 && t == 0 && seqlens_out != nullptr) seqlens_out[m] = write ? pos + 1 : pos;
    if (!write) return;
    const int col = cb * 64 + (t & 63);
    const float* pm = part + (size_t)m * H * kDqk + col;
    float acc = 0.f;
    for (int h0 = t >> 6; h0 < H; h0 += 32) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int h = h0 + 4 * u;
            v[u] = h < H ? pm[(size_t)h * kDqk] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += v[u];
    }
    red[t >> 6][t & 63] = acc;
    __syncthreads();
    if (t >= 64) return;
    const float val = (red[0][t] + red[1][t]) + (red[2][t] + red[3][t]);
    __bf16* dst = cache + row_off * kDqk + cb * 64;
    if (cb < NCB - 1) {
        dst[t] = (__bf16)val;
    } else {
        // RoPE block: lanes 2j and 2j+1 (of the one wave left) hold the pair
        const float other = __shfl_xor(val, 1, 64);
        const int j = t >> 1;
        const float r0 = (t & 1) ? other : val, r1 = (t & 1) ? val : other;
        const float cs = rope_cos[(size_t)pos * (kDr / 2) + j];
        const float sn = rope_sin[(size_t)pos * (kDr / 2) + j];
        dst[t] = (__bf16)((t & 1) ? r0 * sn + r1 * cs : r0 * cs - r1 * sn);
    }
}

constexpr int kAbsorbQSlabs = 4;  // 64-column weight slabs per q-absorb workgroup

}  // namespace

hipError_t launch_absorb_q(bool bf16, int b, int h, const void* q_nope, const void* w_uk,
                           const void* q_rope, void* q_prime, hipStream_t stream)
{
    const unsigned grid = (unsigned)h * (unsigned)((b + kRows - 1) / kRows);
    if (bf16)
        absorb_mfma_kernel<kDk, kDc, kAbsorbQSlabs><<<h * (kDc / (64 * kAbsorbQSlabs)), 256, 0, stream>>>(
            b, h, (const __bf16*)q_nope, (long)h * kDk, (const __bf16*)w_uk, (__bf16*)q_prime,
            (long)h * kDqk, kDqk, (const __bf16*)q_rope);
    else
        absorb_q_kernel<float><<<grid, 128, 0, stream>>>(b, h, (const float*)q_nope,
                                                         (const float*)w_uk, (const float*)q_rope,
                                                         (float*)q_prime);
    return hipGetLastError();
}


hipError_t launch_cache_append(int b, int d_model, int t_max, int n_pos, const void* x,
                               const void* w_dkv, const void* w_kr, const float* rope_cos,
                               const float* rope_sin, void* cache, const int32_t* seqlens,
                               int32_t* seqlens_out, void* workspace, hipStream_t stream,
                               const int32_t* block_table, int num_blocks, int block_size,
                               int max_blocks)
{
    const int H = d_model / kAppendKD;
    float* part = (float*)workspace;
    int32_t* wpos = (int32_t*)((unsigned char*)workspace + append_part_bytes(b, d_model));
    append_proj_kernel<<<H * (kDc / 64 + 1), 256, 0, stream>>>(b, H, (const __bf16*)x, (const __bf16*)w_dkv,
                                                               (const __bf16*)w_kr, part, seqlens, wpos);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    append_finish_kernel<<<b * (kDqk / 64), 256, 0, stream>>>(H, t_max, n_pos, part, wpos, rope_cos, rope_sin,
                                                              (__bf16*)cache, seqlens_out, block_table,
                                                              num_blocks, block_size, max_blocks);
    return hipGetLastError();
}

hipError_t launch_absorb_o(bool bf16, int b, int h, const void* o, const void* w_uv, void* y,
                           hipStream_t stream)
{
    const unsigned grid = (unsigned)h * (unsigned)((b + kRows - 1) / kRows);
    if (bf16)
        absorb_mfma_kernel<kDc, kDv, 1><<<h * (kDv / 64), 256, 0, stream>>>(
            b, h, (const __bf16*)o, (long)h * kDc, (const __bf16*)w_uv, (__bf16*)y, (long)h * kDv,
            kDv, nullptr);
    else
        absorb_o_kernel<float><<<grid, 128, 0, stream>>>(b, h, (const float*)o,
                                                         (const float*)w_uv, (float*)y);
    return hipGetLastError();
}

}  // namespace mla355
