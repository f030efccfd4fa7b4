/*
 * mla355.h -- C ABI of libmla355: absorbed Multi-head Latent Attention (MLA)
 * decode on one AMD Instinct MI355X (gfx950).
 *
 * The method (pages cited by title and section):
 *   Each cached token holds one latent row [c_KV (512) ; k_R (64)] shared by
 *   every query head ("Multi-head Latent Attention", LLM glossary, layout
 *   section; "MLA" notes, Dimensions: 512 + 64 = 576 per token).  Decode
 *   never expands per-head keys or values.  Instead the key up-projection is
 *   folded into the query (q absorb), attention scores run directly against
 *   the latent rows, and the value up-projection is applied after the
 *   softmax-weighted sum (o absorb) (glossary, section on why decode absorbs
 *   the matrices).  FlashMLA issue 16 ("up matrix is not involved?") gives
 *   the interface split: q absorb and o absorb are separate calls; attention
 *   takes the 576-wide absorbed query and returns a 512-wide latent output.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to dense, row-major
 *     (C-contiguous) arrays.  The caller owns every buffer.  The library never
 *     allocates, frees or synchronises; all work is enqueued on `stream`
 *     (a hipStream_t; NULL selects the default stream) and is asynchronous.
 *   - Inputs are read only; outputs must not alias inputs.
 *   - Every tensor base pointer must be 16-byte aligned (128-bit accesses);
 *     the workspace must be 256-byte aligned.
 *   - Errors: argument checks run on the host before anything is enqueued and
 *     return a status; nothing is launched then.  A failed launch returns
 *     MLA_ERR_HIP.  Nothing is printed, no exception or errno crosses the ABI.
 *   - The library holds no mutable state: calls are thread-safe (two calls
 *     that share output or workspace buffers must not overlap in time).
 *   - dtype selects the element type of q_nope, q_rope, w_uk, w_uv, q_prime,
 *     cache, out and y: MLA_DTYPE_BF16 (compute: bf16 MFMA, fp32
 *     accumulation) or MLA_DTYPE_F32 (compute: fp32 throughout).  lse is
 *     always fp32.
 */
#ifndef MLA355_H
#define MLA355_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA355_ABI_VERSION 1

#define MLA_D_C 512  /* latent width c_KV                         */
#define MLA_D_R 64   /* decoupled RoPE key width k_R              */
#define MLA_D_QK 576 /* latent row / absorbed query width         */
#define MLA_D_K 128  /* per-head query (no-RoPE part) width       */
#define MLA_D_V 128  /* per-head value width after o absorb       */

typedef enum {
    MLA_OK = 0,
    MLA_ERR_INVALID_ARGUMENT = 1,
    MLA_ERR_UNSUPPORTED = 2,
    MLA_ERR_WORKSPACE_TOO_SMALL = 3,
    MLA_ERR_HIP = 4
} mla_status_t;

typedef enum { MLA_DTYPE_F32 = 0, MLA_DTYPE_BF16 = 1 } mla_dtype_t;

/* Scheduling overrides and profiling hooks for mla_decode_ex.  Zero / NULL in
 * a field means "choose automatically" / "none".  Results are the same
 * function of the inputs for every valid setting (up to floating-point
 * rounding order). */
typedef struct {
    int n_chunks;       /* token chunks the whole batch is cut into (the split-KV
                           grid size per head group); multiple of 8, <= 65536 */
    int heads_per_group;/* heads one workgroup scores against a shared tile:
                           16, 32, 64 or 128 (bf16), 16 (fp32) */
    int variant;        /* kernel variant index for the chosen head group (0 = auto) */
    int reserved[5];    /* reserved[0]: MLA_CONFIG_RECORD_CLOCK or 0; the
                           others must be zero */
    void* profile_events[2]; /* optional hipEvent_t pair, recorded on `stream`
                                right before and right after the split-KV
                                attention kernel (both or neither) */
} mla_decode_config_t;

/* Measurement hook.  With reserved[0] = MLA_CONFIG_RECORD_CLOCK the split-KV
 * attention kernel's workgroup 0 writes four uint64 into the last
 * MLA_CLOCK_BYTES of the workspace size the library reports for the call
 * (mla_*_workspace_bytes*, same arguments and config): the shader clock
 * (s_memtime) and the 100 MHz real-time counter (s_memrealtime) at its start,
 * then both again at its end, so the engine clock during the launch is
 * 100 MHz x (clock difference) / (real-time difference).  The bf16 kernels of
 * 16 heads per group, the wide-wave, column-split and fp8 kernels write them;
 * the pair and fp32 kernels write nothing.  Every workspace size includes the
 * area. */
#define MLA_CONFIG_RECORD_CLOCK 1
#define MLA_CLOCK_BYTES 256

int mla_abi_version(void);
const char* mla_status_string(mla_status_t status);

/*
 * mla_absorb_q -- query absorption.
 *   q_prime[b,h,0:512]   = q_nope[b,h,:] . W_UK[h]   (contracts d_k = 128)
 *   q_prime[b,h,512:576] = q_rope[b,h,:]
 * Glossary, section on why decode absorbs: qbar_h = q^C_h (W^UK_h)^T is a
 * latent-width query; FlashMLA issue 16 answer: it is concatenated with the
 * 64-wide rope query.  Layouts:
 *   q_nope [b,h,128], w_uk [h,128,512] (row j of head h is the j-th query
 *   dimension's weights over the 512 latent channels), q_rope [b,h,64],
 *   q_prime [b,h,576] (written).
 * fp32 accumulation; the result is rounded once to dtype.
 * Errors: MLA_ERR_INVALID_ARGUMENT for a null or misaligned pointer,
 * b <= 0, h <= 0 or an unknown dtype.
 */
mla_status_t mla_absorb_q(mla_dtype_t dtype, int b, int h, const void* q_nope, const void* w_uk,
                          const void* q_rope, void* q_prime, void* stream);

/*
 * mla_decode_workspace_bytes -- bytes of device workspace mla_decode needs for
 * this problem size.  Pure host function: it makes no HIP call and needs no GPU.
 * Returns 0 for invalid arguments.
 */
size_t mla_decode_workspace_bytes(mla_dtype_t dtype, int b, int h, int t_max);

/*
 * mla_decode -- attention of every absorbed query head against the shared
 * latent cache (the latent form of MLA decode).  For each batch row i and head
 * j, over the first L = seqlens[i] cached rows t:
 *   s_t      = softmax_scale * sum_{k<576} q_prime[i,j,k] * cache[i,t,k]
 *   p_t      = exp(s_t) / sum_u exp(s_u)
 *   out[i,j,c] = sum_t p_t * cache[i,t,c]        (c < 512; k_R is a key only)
 *   lse[i,j] = log(sum_t exp(s_t))                (natural log)
 * Glossary, section on why decode absorbs (scores against the cached latent,
 * value up-projection moved after the weighted sum), and its runnable check
 * (softmax of the summed content + RoPE score, scaled by 1/sqrt(d_k + d_r)).
 * Layouts: q_prime [b,h,576]; cache [b,t_max,576] (row t of batch i at
 * ((i*t_max)+t)*576); seqlens [b] int32 on the device; out [b,h,512] dtype
 * (written); lse [b,h] fp32 (written).
 * Tokens attended: exactly the first seqlens[i] rows, no causal mask.  A
 * device-side seqlens value outside [0, t_max] is clamped into it.  A row with
 * L = 0 yields out = 0 and lse = -inf.  Rows at or past L are never read.
 * workspace: device scratch of at least mla_decode_workspace_bytes(dtype, b, h,
 * t_max) bytes, 256-byte aligned, contents need not be initialised; it holds
 * the split plan and the split-KV partial results (each partial output is
 * normalised and stored in dtype, its log-sum-exp in fp32; the combine
 * accumulates in fp32).
 * Errors (host side, before any launch): MLA_ERR_INVALID_ARGUMENT for a null
 * or misaligned pointer, b <= 0, h <= 0, t_max < 0, b*t_max >= 2^31, unknown
 * dtype, or softmax_scale not finite or <= 0; MLA_ERR_WORKSPACE_TOO_SMALL.
 */
mla_status_t mla_decode(mla_dtype_t dtype, int b, int h, int t_max, const void* q_prime,
                        const void* cache, const int32_t* seqlens, float softmax_scale, void* out,
                        float* lse, void* workspace, size_t workspace_bytes, void* stream);

/* As mla_decode_workspace_bytes / mla_decode with explicit scheduling
 * overrides (config may be NULL: automatic).  Additional error:
 * MLA_ERR_UNSUPPORTED for a config field outside its documented range. */
size_t mla_decode_workspace_bytes_ex(mla_dtype_t dtype, int b, int h, int t_max,
                                     const mla_decode_config_t* config);
mla_status_t mla_decode_ex(mla_dtype_t dtype, int b, int h, int t_max, const void* q_prime,
                           const void* cache, const int32_t* seqlens, float softmax_scale,
                           void* out, float* lse, void* workspace, size_t workspace_bytes,
                           const mla_decode_config_t* config, void* stream);

/*
 * mla_decode_kernel_name -- name of the split-KV attention kernel that
 * mla_decode_ex would launch for this dtype, head count and config (config
 * may be NULL: automatic), as profilers list it (for example
 * "decode_wide_kernel<4, 3, false>").  Pure host function: no HIP call, no GPU
 * needed.  The string is static and owned by the library.  Returns NULL for
 * an unknown dtype, h <= 0 or a config mla_decode_ex would reject.
 */
const char* mla_decode_kernel_name(mla_dtype_t dtype, int h, const mla_decode_config_t* config);

/*
 * mla_decode_mtp -- mla_decode with q_len new query tokens per batch row
 * (several tokens decoded at once, e.g. speculative or multi-token
 * prediction steps).  The glossary's production notes say prefill and decode
 * take different paths; the Polish overview gives attention's cost over
 * every (token, earlier token) pair.  Neither spells out a mask; the reading
 * taken here is the standard causal one: the q_len new tokens are the last
 * q_len of the L = seqlens[i] cached rows of row i (already appended), and new
 * token n (0-based) attends to the first L - q_len + 1 + n rows, its own
 * included.  For each (i, n, j):
 *   s_t = softmax_scale * q_prime[i,n,j,:] . cache[i,t,:],  t < L - q_len + 1 + n
 *   out[i,n,j,:] = sum_t softmax(s)_t cache[i,t,0:512],  lse[i,n,j] = log sum_t exp(s_t)
 * A token with no row to attend to (L < q_len - n) gets out = 0, lse = -inf.
 * q_len = 1 is exactly mla_decode (same kernels, same results).
 * Layouts: q_prime [b,q_len,h,576] bf16; cache [b,t_max,576] bf16; seqlens [b]
 * int32 on the device, clamped to [0, t_max]; out [b,q_len,h,512] bf16
 * (written); lse [b,q_len,h] fp32 (written).
 * workspace: device scratch of at least mla_decode_mtp_workspace_bytes(...)
 * bytes, 256-byte aligned, contents need not be initialised.
 * Errors (host side, before any launch): MLA_ERR_UNSUPPORTED for dtype
 * MLA_DTYPE_F32; MLA_ERR_INVALID_ARGUMENT for an unknown dtype, a null or
 * misaligned pointer, b <= 0, q_len <= 0, h <= 0, q_len*h > 2^20, t_max < 0,
 * b*t_max >= 2^31, or softmax_scale not finite or <= 0;
 * MLA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t mla_decode_mtp_workspace_bytes(mla_dtype_t dtype, int b, int q_len, int h, int t_max);
mla_status_t mla_decode_mtp(mla_dtype_t dtype, int b, int q_len, int h, int t_max,
                            const void* q_prime, const void* cache, const int32_t* seqlens,
                            float softmax_scale, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);
/* As mla_decode_mtp_workspace_bytes / mla_decode_mtp with a config (may be
 * NULL): only n_chunks (the split count, a multiple of 8, 0 = automatic) and
 * profile_events may be set; any other field non-zero, or an n_chunks outside
 * its range, gives MLA_ERR_UNSUPPORTED (workspace query: 0). */
size_t mla_decode_mtp_workspace_bytes_ex(mla_dtype_t dtype, int b, int q_len, int h, int t_max,
                                         const mla_decode_config_t* config);
mla_status_t mla_decode_mtp_ex(mla_dtype_t dtype, int b, int q_len, int h, int t_max,
                               const void* q_prime, const void* cache, const int32_t* seqlens,
                               float softmax_scale, void* out, float* lse, void* workspace,
                               size_t workspace_bytes, const mla_decode_config_t* config,
                               void* stream);
/* Name of the attention kernel mla_decode_mtp launches (pure host function;
 * NULL for arguments it would reject). */
const char* mla_decode_mtp_kernel_name(mla_dtype_t dtype, int q_len, int h);

/*
 * mla_cache_append -- write the new token's latent row into the cache (the
 * step before attention).  Glossary "Multi-head Latent Attention", layout
 * difference from MHA/GQA: the cached row of token t is [c_t ; k^R_t] with
 * c_t = x_t W^DKV and k^R_t = RoPE(x_t W^KR), one RoPE key shared by all heads;
 * Lesson 28 ("Down-projection and On-the-Fly Up-projection in MLA"): x_t is the
 * d_model-wide hidden state (7168 in its example).  The pages give no RoPE base
 * or pairing: the caller supplies the rotation as tables rope_cos/rope_sin
 * [n_pos, 32] (fp32, entry (p, j) = cos/sin of the angle of pair j at position
 * p), and RoPE turns each adjacent pair (2j, 2j+1) of x W^KR:
 *   k[2j] = r[2j] cos - r[2j+1] sin,   k[2j+1] = r[2j] sin + r[2j+1] cos.
 * Batch row i's token goes to cache row pos = seqlens[i] (its position), in
 * bf16 after fp32 accumulation; a row with pos outside [0, min(t_max, n_pos))
 * is not written.  seqlens_out (may be NULL, may equal seqlens) receives pos + 1
 * for a written row and pos otherwise, so that the following attention call
 * sees the new token.
 * Layouts: x [b, d_model] bf16; w_dkv [d_model, 512] bf16; w_kr [d_model, 64]
 * bf16 (row-major); cache [b, t_max, 576] bf16 (updated in place).
 * workspace: device scratch of at least mla_cache_append_workspace_bytes(b,
 * d_model) bytes (fp32 partial sums and a copy of seqlens), 256-byte aligned.
 * Errors (host side, before any launch): MLA_ERR_UNSUPPORTED for dtype
 * MLA_DTYPE_F32; MLA_ERR_INVALID_ARGUMENT for an unknown dtype, a null pointer
 * (seqlens_out excepted), x / w_dkv / w_kr / cache not 16-byte aligned, the
 * tables or seqlens not 4-byte aligned, b <= 0, t_max <= 0, n_pos <= 0, d_model
 * not a positive multiple of 256, b*t_max >= 2^31 or b*d_model >= 2^31;
 * MLA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t mla_cache_append_workspace_bytes(int b, int d_model);
mla_status_t mla_cache_append(mla_dtype_t dtype, int b, int d_model, int t_max, const void* x,
                              const void* w_dkv, const void* w_kr, const float* rope_cos,
                              const float* rope_sin, int n_pos, void* cache, const int32_t* seqlens,
                              int32_t* seqlens_out, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * mla_cache_append_paged -- mla_cache_append into a paged latent cache (the
 * pool and block table of mla_decode_paged).  Batch row i's new row pos =
 * seqlens[i] goes to row pos % block_size of block
 * block_table[i * max_blocks + pos / block_size]; nothing is written when pos
 * is outside [0, min(max_blocks * block_size, n_pos)) or that table entry is
 * outside [0, num_blocks) (a write is never redirected into another block).
 * seqlens_out as in mla_cache_append (pos + 1 only for a written row).
 * kv_pool [num_blocks, block_size, 576] bf16 (updated in place); block_table
 * [b, max_blocks] int32; other arguments as in mla_cache_append.
 * Errors: those of mla_cache_append, with the pool checks of mla_decode_paged
 * (block_size a positive multiple of 32, num_blocks > 0, max_blocks > 0, the
 * table 4-byte aligned) in place of the t_max checks.
 */
mla_status_t mla_cache_append_paged(mla_dtype_t dtype, int b, int d_model, const void* x,
                                    const void* w_dkv, const void* w_kr, const float* rope_cos,
                                    const float* rope_sin, int n_pos, void* kv_pool, int num_blocks,
                                    int block_size, const int32_t* block_table, int max_blocks,
                                    const int32_t* seqlens, int32_t* seqlens_out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * mla_decode_mtp_paged -- mla_decode_mtp over a paged latent cache (pool and
 * block table as in mla_decode_paged; the q_len new tokens are the last q_len
 * rows of each sequence).  q_len = 1 is exactly mla_decode_paged.
 * Errors: those of mla_decode_mtp with the pool checks of mla_decode_paged.
 */
size_t mla_decode_mtp_paged_workspace_bytes(mla_dtype_t dtype, int b, int q_len, int h,
                                            int num_blocks, int block_size, int max_blocks);
mla_status_t mla_decode_mtp_paged(mla_dtype_t dtype, int b, int q_len, int h, const void* q_prime,
                                  const void* kv_pool, int num_blocks, int block_size,
                                  const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                                  float softmax_scale, void* out, float* lse, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * mla_decode_paged -- mla_decode over a paged latent cache.  The cached rows
 * of every sequence live in fixed-size blocks of a shared pool, found through
 * a block table (glossary, capacity and cost section: MLA leaves dynamic
 * allocation to a paged scheme and the latent cache can still be split into
 * blocks; relations section: such an allocator manages the physical latent
 * blocks).  The operation on the rows is exactly mla_decode's.  For batch
 * row i, cached token t (t < seqlens[i]) is row (t % block_size) of block
 * block_table[i * max_blocks + t / block_size] of the pool.  Output, lse and
 * the definition are those of mla_decode over the rows gathered that way.
 * Layouts: q_prime [b,h,576] bf16; kv_pool [num_blocks, block_size, 576] bf16
 * (row-major); block_table [b, max_blocks] int32 on the device; seqlens [b]
 * int32 on the device, clamped to [0, max_blocks * block_size]; out
 * [b,h,512] bf16 (written); lse [b,h] fp32 (written).  A block-table entry
 * outside [0, num_blocks) is clamped into it (entries past a sequence's last
 * block are never read).  block_size must be a positive multiple of 32 (a
 * 32-token tile never straddles two blocks).
 * workspace: device scratch of at least mla_decode_paged_workspace_bytes(...)
 * bytes, 256-byte aligned, contents need not be initialised.
 * Errors (host side, before any launch): MLA_ERR_UNSUPPORTED for dtype
 * MLA_DTYPE_F32 or a config naming a kernel without a paged form;
 * MLA_ERR_INVALID_ARGUMENT for a null or misaligned pointer, b, h,
 * num_blocks, block_size or max_blocks <= 0, block_size not a multiple of 32,
 * b * (max_blocks * block_size + 32) >= 2^31, or softmax_scale not finite or
 * <= 0; MLA_ERR_WORKSPACE_TOO_SMALL.
 */
size_t mla_decode_paged_workspace_bytes(mla_dtype_t dtype, int b, int h, int num_blocks,
                                        int block_size, int max_blocks,
                                        const mla_decode_config_t* config);
mla_status_t mla_decode_paged(mla_dtype_t dtype, int b, int h, const void* q_prime,
                              const void* kv_pool, int num_blocks, int block_size,
                              const int32_t* block_table, int max_blocks, const int32_t* seqlens,
                              float softmax_scale, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);
mla_status_t mla_decode_paged_ex(mla_dtype_t dtype, int b, int h, const void* q_prime,
                                 const void* kv_pool, int num_blocks, int block_size,
                                 const int32_t* block_table, int max_blocks,
                                 const int32_t* seqlens, float softmax_scale, void* out,
                                 float* lse, void* workspace, size_t workspace_bytes,
                                 const mla_decode_config_t* config, void* stream);
/* Name of the attention kernel mla_decode_paged_ex would launch (pure host;
 * NULL for a rejected dtype, h or config). */
const char* mla_decode_paged_kernel_name(mla_dtype_t dtype, int h, const mla_decode_config_t* config);

/*
 * mla_quantize_cache_fp8 -- per-token fp8 form of latent rows for
 * mla_decode_fp8.  The pages define no quantised cache; this is the plainest
 * form that keeps the scales out of the inner products.  For each row
 * x[0:576] (bf16) of the n_rows rows:
 *   scale    = max_i |x_i| / 448            (fp32, IEEE division; 448 is the
 *                                           largest finite OCP e4m3 value)
 *   codes[i] = e4m3(clamp(x_i / scale, -448, 448))   (fp32 quotient, rounded
 *              to the nearest e4m3 value, ties to even; 0 when scale = 0)
 * so that x_i ~ e4m3_value(codes[i]) * scale.  Codes are OCP FP8 E4M3 bytes
 * (bias 7, no infinities, 0x7F/0xFF NaN).  Layouts: x [n_rows, 576] bf16,
 * codes [n_rows, 576] uint8 (written), scale [n_rows] fp32 (written).
 * A latent cache [b, t_max, 576] is n_rows = b * t_max rows.
 * Errors: MLA_ERR_INVALID_ARGUMENT for n_rows <= 0 or > 2^37, a null pointer,
 * x or codes not 16-byte aligned, or scale not 4-byte aligned.
 */
mla_status_t mla_quantize_cache_fp8(long long n_rows, const void* x, void* codes, float* scale,
                                    void* stream);

/*
 * mla_decode_fp8 -- mla_decode over an fp8 latent cache: the same operation
 * with each cached row replaced by its dequantised value
 * e4m3_value(cache_codes[i, t, :]) * cache_scale[i, t] (the form written by
 * mla_quantize_cache_fp8).  The cache streams at 580 bytes per token instead
 * of 1152.  q_prime [b,h,576] bf16; cache_codes [b,t_max,576] uint8 (OCP e4m3);
 * cache_scale [b,t_max] fp32; seqlens [b] int32 on the device (clamped to
 * [0, t_max]); out [b,h,512] bf16 and lse [b,h] fp32 (written).  Scores and
 * weighted sums run on bf16 MFMA with fp32 accumulation (e4m3 values are
 * exact in bf16; each token's scale multiplies its score and probability).
 * workspace: at least mla_decode_fp8_workspace_bytes(...) bytes, 256-byte
 * aligned, contents need not be initialised.  config: as for mla_decode_ex;
 * only the 16-heads-per-group kernel has an fp8 form (other choices give
 * MLA_ERR_UNSUPPORTED).
 * Errors (host side, before any launch): MLA_ERR_INVALID_ARGUMENT for a null
 * or misaligned pointer (cache_scale: 4-byte alignment), b <= 0, h <= 0,
 * t_max < 0, b*t_max >= 2^31, or softmax_scale not finite or <= 0;
 * MLA_ERR_WORKSPACE_TOO_SMALL; MLA_ERR_UNSUPPORTED as above.
 */
size_t mla_decode_fp8_workspace_bytes(int b, int h, int t_max, const mla_decode_config_t* config);
mla_status_t mla_decode_fp8(int b, int h, int t_max, const void* q_prime, const void* cache_codes,
                            const float* cache_scale, const int32_t* seqlens, float softmax_scale,
                            void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream);
mla_status_t mla_decode_fp8_ex(int b, int h, int t_max, const void* q_prime, const void* cache_codes,
                               const float* cache_scale, const int32_t* seqlens, float softmax_scale,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               const mla_decode_config_t* config, void* stream);
/* Name of the attention kernel mla_decode_fp8_ex would launch (pure host;
 * NULL for a rejected h or config). */
const char* mla_decode_fp8_kernel_name(int h, const mla_decode_config_t* config);

/*
 * mla_decode_noalloc -- mla_decode without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  It computes exactly what
 * mla_decode computes (same kernels, same automatic schedule, bit-identical
 * results), with the split plan and partial results kept in a fixed device
 * array of MLA_NOALLOC_SCRATCH_BYTES inside the library.  Each GPU the
 * library runs on holds its own copy of that array until the process ends;
 * its address is looked up on the first call on each device.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams or threads) race on it and must be serialised by
 * the caller.  Arguments as mla_decode without workspace / workspace_bytes.
 * Errors: those of mla_decode; MLA_ERR_WORKSPACE_TOO_SMALL when the problem
 * needs more than MLA_NOALLOC_SCRATCH_BYTES of workspace
 * (mla_decode_workspace_bytes(dtype, b, h, t_max) > the constant; at 128
 * heads in bf16, batches of up to 250 rows fit); MLA_ERR_HIP if the array's
 * device address cannot be found.
 */
#define MLA_NOALLOC_SCRATCH_BYTES (64u << 20)
mla_status_t mla_decode_noalloc(mla_dtype_t dtype, int b, int h, int t_max, const void* q_prime,
                                const void* cache, const int32_t* seqlens, float softmax_scale,
                                void* out, float* lse, void* stream);

/*
 * mla_absorb_o -- output absorption.
 *   y[b,h,:] = o[b,h,:] . W_UV[h]   (contracts d_c = 512)
 * Glossary, section on why decode absorbs: sum_t p_t (c_t W^UV_h) equals
 * (sum_t p_t c_t) W^UV_h, so the up-projection runs once on the 512-wide
 * decode output.  Layouts: o [b,h,512], w_uv [h,512,128], y [b,h,128]
 * (written).  fp32 accumulation, one rounding to dtype.
 * Errors: as mla_absorb_q.
 */
mla_status_t mla_absorb_o(mla_dtype_t dtype, int b, int h, const void* o, const void* w_uv,
                          void* y, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA355_H */
