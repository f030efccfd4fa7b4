/*
 * mla_oracle.c -- plain fp64 CPU oracle for absorbed Multi-head Latent
 * Attention (MLA) decode.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library calls, links or
 * loads this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code with the HIP path.
 *
 * Every routine is the textbook definition written out as straight loops in
 * double precision: no blocking, no tiling, no online softmax, no split.
 * Inputs arrive as doubles (bf16 or fp32 values widened exactly).
 *
 * Sources (cited by page title and section):
 *  - "Multi-head Latent Attention" (LLM glossary, tokens-kit):
 *      section on the layout difference from MHA/GQA -- per-head content key
 *        k_{t,h} = c_t W^UK_h, value v_{t,h} = c_t W^UV_h, one RoPE key k^R_t
 *        shared by all heads, and the two-part score
 *        s = q^C_h (k^C_{t,h})^T + q^R_h (k^R_t)^T;
 *      section on why decode absorbs the matrices -- query absorption
 *        qbar_h = q^C_h (W^UK_h)^T and value absorption
 *        sum_t p_t (c_t W^UV_h) = (sum_t p_t c_t) W^UV_h;
 *      runnable expanded-vs-absorbed check -- softmax of the summed score
 *        scaled by 1/sqrt(d_k + d_r).
 *  - "up matrix is not involved?" (FlashMLA issue 16), the answer that splits
 *      q-absorb / attention / o-absorb: attention takes [qbar ; q_rope]
 *      (512 + 64) against the latent rows and returns a 512-wide output.
 *
 * Weight layouts (a reading of the pages, which disagree on transposes):
 *   w_uk[h][j][c]  (d_k x d_c per head): k_{t,h}[j] = sum_c c_t[c] w_uk[h][j][c]
 *                  and qbar[c] = sum_j q_nope[j] w_uk[h][j][c]
 *   w_uv[h][c][j]  (d_c x d_v per head): v_{t,h}[j] = sum_c c_t[c] w_uv[h][c][j]
 * A latent cache row is [c_KV (d_c) ; k_R (d_r)], d_c + d_r wide.
 *
 * Which tokens are attended: exactly the first seqlens[b] cached rows, no
 * causal mask (the glossary's check attends only to the earlier tokens).
 * seqlens[b] == 0 yields out = 0, lse = -inf.
 *
 * Several query tokens per row (oracle_decode_latent_causal): the glossary's
 * production notes say prefill and decode take different paths, and the
 * Polish overview gives attention's O(n^2 d) cost (every token against every
 * earlier one) without spelling out a mask.  Reading: the q_len new tokens
 * are the last q_len of the seqlens[b] cached rows, and new token i (0-based)
 * attends to the rows up to and including its own, i.e. the first
 * seqlens[b] - q_len + 1 + i rows (none if that is not positive).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>

#define IDX2(i, j, n1) ((size_t)(i) * (size_t)(n1) + (size_t)(j))
#define IDX3(i, j, k, n1, n2) (((size_t)(i) * (size_t)(n1) + (size_t)(j)) * (size_t)(n2) + (size_t)(k))

int oracle_abi_version(void) { return 1; }

/* Threads the OpenMP loops use (reported with CPU timings). */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        n = omp_get_num_threads();
    }
    return n;
}

/*
 * Softmax of s[0..n) (natural exponent), written into p, returning
 * log(sum_t exp(s_t)).  The maximum is subtracted before exponentiating,
 * which changes nothing mathematically (softmax is shift invariant) and
 * keeps exp() in range.  n == 0 returns -inf and writes nothing.
 */
static double softmax_f64(const double* s, int n, double* p)
{
    if (n <= 0) return -INFINITY;
    double m = s[0];
    for (int t = 1; t < n; ++t)
        if (s[t] > m) m = s[t];
    double l = 0.0;
    for (int t = 0; t < n; ++t) {
        p[t] = exp(s[t] - m);
        l += p[t];
    }
    for (int t = 0; t < n; ++t) p[t] /= l;
    return m + log(l);
}

static int clamp_len(int32_t L, int t_max)
{
    if (L < 0) return 0;
    if (L > t_max) return t_max;
    return (int)L;
}

/*
 * Latent (absorbed) form: the operation mla_decode performs.
 *   s_t = scale * sum_{i < d_c + d_r} q'[b,h,i] * row_t[i]
 *   p   = softmax(s over t < L_b)
 *   out[b,h,c] = sum_t p_t * row_t[c]    (c < d_c: the RoPE columns are keys only)
 *   lse[b,h]   = log sum_t exp(s_t)
 * Glossary "Multi-head Latent Attention": the absorbed query scores the cached
 * latent directly; the value up-projection moves after the weighted sum.
 * scores (optional, may be NULL) receives s_t at [b,h,t] for t < L_b.
 */
void oracle_decode_latent(int b, int h, int t_max, int d_c, int d_r,
                          const double* q_prime, const double* cache,
                          const int32_t* seqlens, double scale,
                          double* out, double* lse, double* scores)
{
    const int d = d_c + d_r;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < (long)b * h; ++bh) {
        const int bi = (int)(bh / h), hi = (int)(bh % h);
        const int L = clamp_len(seqlens[bi], t_max);
        const double* q = q_prime + IDX2(bh, 0, d);
        double* o = out + IDX2(bh, 0, d_c);
        double* s = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        double* p = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        for (int t = 0; t < L; ++t) {
            const double* row = cache + IDX3(bi, t, 0, t_max, d);
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += q[i] * row[i];
            s[t] = scale * acc;
            if (scores) scores[IDX3(bi, hi, t, h, t_max)] = s[t];
        }
        lse[bh] = softmax_f64(s, L, p);
        for (int c = 0; c < d_c; ++c) o[c] = 0.0;
        for (int t = 0; t < L; ++t) {
            const double* row = cache + IDX3(bi, t, 0, t_max, d);
            for (int c = 0; c < d_c; ++c) o[c] += p[t] * row[c];
        }
        free(s);
        free(p);
    }
}

/*
 * Un-absorbed (expanded) form, the method's own definition before any
 * absorption.  For each (b, h) and each cached token t < L_b:
 *   k_{t,h}[j] = sum_c c_t[c] * w_uk[h][j][c]          (j < d_k)
 *   v_{t,h}[j] = sum_c c_t[c] * w_uv[h][c][j]          (j < d_v)
 *   s_t = scale * ( sum_j q_nope[b,h,j] k_{t,h}[j] + sum_r q_rope[b,h,r] kR_t[r] )
 *   p   = softmax(s),  y[b,h,j] = sum_t p_t v_{t,h}[j],  lse = log sum_t exp(s_t)
 * Glossary "Multi-head Latent Attention", layout section (per-head up-projection
 * of the shared latent, shared RoPE key, two-part score); the runnable check
 * scales the summed score by 1/sqrt(d_k + d_r).
 * heads (optional, may be NULL) restricts the work to n_sel listed heads; y,
 * lse, scores and probs are then indexed by the position in that list
 * ([b, n_sel, ...]).  With heads == NULL, n_sel must equal h.
 * scores / probs (optional) receive s_t and p_t at [b, sel, t] for t < L_b.
 */
void oracle_decode_unabsorbed(int b, int h, int t_max, int d_c, int d_r, int d_k, int d_v,
                              const double* q_nope, const double* q_rope,
                              const double* w_uk, const double* w_uv,
                              const double* cache, const int32_t* seqlens, double scale,
                              const int32_t* heads, int n_sel,
                              double* y, double* lse, double* scores, double* probs)
{
    const int d = d_c + d_r;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bs = 0; bs < (long)b * n_sel; ++bs) {
        const int bi = (int)(bs / n_sel), si = (int)(bs % n_sel);
        const int hi = heads ? heads[si] : si;
        const int L = clamp_len(seqlens[bi], t_max);
        const double* qn = q_nope + IDX3(bi, hi, 0, h, d_k);
        const double* qr = q_rope + IDX3(bi, hi, 0, h, d_r);
        double* s = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        double* p = (double*)malloc(sizeof(double) * (L > 0 ? L : 1));
        double* kv = (double*)malloc(sizeof(double) * (d_k > d_v ? d_k : d_v));
        for (int t = 0; t < L; ++t) {
            const double* c_t = cache + IDX3(bi, t, 0, t_max, d);
            const double* kR = c_t + d_c;
            for (int j = 0; j < d_k; ++j) {
                double acc = 0.0;
                for (int c = 0; c < d_c; ++c) acc += c_t[c] * w_uk[IDX3(hi, j, c, d_k, d_c)];
                kv[j] = acc;
            }
            double content = 0.0, rope = 0.0;
            for (int j = 0; j < d_k; ++j) content += qn[j] * kv[j];
            for (int r = 0; r < d_r; ++r) rope += qr[r] * kR[r];
            s[t] = scale * (content + rope);
            if (scores) scores[IDX3(bi, si, t, n_sel, t_max)] = s[t];
        }
        lse[bs] = softmax_f64(s, L, p);
        double* yo = y + IDX2(bs, 0, d_v);
        for (int j = 0; j < d_v; ++j) yo[j] = 0.0;
        for (int t = 0; t < L; ++t) {
            const double* c_t = cache + IDX3(bi, t, 0, t_max, d);
            for (int j = 0; j < d_v; ++j) {
                double acc = 0.0;
                for (int c = 0; c < d_c; ++c) acc += c_t[c] * w_uv[IDX3(hi, c, j, d_c, d_v)];
                kv[j] = acc;
            }
            for (int j = 0; j < d_v; ++j) yo[j] += p[t] * kv[j];
            if (probs) probs[IDX3(bi, si, t, n_sel, t_max)] = p[t];
        }
        free(s);
        free(p);
        free(kv);
    }
}

/*
 * Latent form with q_len query tokens per row and the causal reading above.
 * q_prime [b, q_len, h, d_c + d_r], out [b, q_len, h, d_c], lse [b, q_len, h]:
 *   n_i = seqlens[b] - q_len + 1 + i   (clamped to [0, seqlens[b]])
 *   s_t = scale * sum_i q'[b,i,h,:] . row_t,  t < n_i
 *   p   = softmax(s),  out = sum_t p_t row_t[0:d_c],  lse = log sum_t exp(s_t)
 */
void oracle_decode_latent_causal(int b, int q_len, int h, int t_max, int d_c, int d_r,
                                 const double* q_prime, const double* cache,
                                 const int32_t* seqlens, double scale,
                                 double* out, double* lse)
{
    const int d = d_c + d_r;
    const long rows = (long)b * q_len * h;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < rows; ++r) {
        const int bi = (int)(r / ((long)q_len * h));
        const int qi = (int)((r / h) % q_len);
        const int L = clamp_len(seqlens[bi], t_max);
        int n = L - q_len + 1 + qi;
        if (n < 0) n = 0;
        if (n > L) n = L;
        const double* q = q_prime + IDX2(r, 0, d);
        double* o = out + IDX2(r, 0, d_c);
        double* s = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
        double* p = (double*)malloc(sizeof(double) * (n > 0 ? n : 1));
        for (int t = 0; t < n; ++t) {
            const double* row = cache + IDX3(bi, t, 0, t_max, d);
            double acc = 0.0;
            for (int i = 0; i < d; ++i) acc += q[i] * row[i];
            s[t] = scale * acc;
        }
        lse[r] = softmax_f64(s, n, p);
        for (int c = 0; c < d_c; ++c) o[c] = 0.0;
        for (int t = 0; t < n; ++t) {
            const double* row = cache + IDX3(bi, t, 0, t_max, d);
            for (int c = 0; c < d_c; ++c) o[c] += p[t] * row[c];
        }
        free(s);
        free(p);
    }
}

/*
 * Appending the new token's latent row (the step before attention).
 * Glossary "Multi-head Latent Attention", layout difference from MHA/GQA: the
 * cached content part is c_t = x_t W^DKV and the cached RoPE key is
 * k^R_t = RoPE(x_t W^KR), one per token, shared by all heads; Lesson 28 shows
 * the hidden state (width d_model, e.g. 7168) down-projected to the 512-wide
 * latent that is cached.  The pages fix no RoPE base or pairing; reading: the
 * caller supplies the rotation as tables cos_tab/sin_tab [n_pos, d_r/2] and
 * RoPE turns each adjacent pair (2j, 2j+1) of x W^KR by the angle of entry
 * (pos, j):
 *   k[2j]   = r[2j] cos - r[2j+1] sin,   k[2j+1] = r[2j] sin + r[2j+1] cos.
 * The new token of batch row i is written at row pos = seqlens[i] (its
 * position); a row with pos outside [0, min(t_max, n_pos)) is not written.
 * x [b, d_model], w_dkv [d_model, d_c], w_kr [d_model, d_r], cache
 * [b, t_max, d_c + d_r] (updated in place).
 */
void oracle_cache_append(int b, int d_model, int d_c, int d_r, int t_max, int n_pos,
                         const double* x, const double* w_dkv, const double* w_kr,
                         const double* cos_tab, const double* sin_tab,
                         const int32_t* seqlens, double* cache)
{
    const int d = d_c + d_r;
#pragma omp parallel for schedule(static)
    for (int bi = 0; bi < b; ++bi) {
        const int pos = seqlens[bi];
        if (pos < 0 || pos >= t_max || pos >= n_pos) continue;
        const double* xr = x + IDX2(bi, 0, d_model);
        double* row = cache + IDX3(bi, pos, 0, t_max, d);
        for (int c = 0; c < d_c; ++c) {
            double acc = 0.0;
            for (int k = 0; k < d_model; ++k) acc += xr[k] * w_dkv[IDX2(k, c, d_c)];
            row[c] = acc;
        }
        for (int j = 0; j < d_r / 2; ++j) {
            double r0 = 0.0, r1 = 0.0;
            for (int k = 0; k < d_model; ++k) {
                r0 += xr[k] * w_kr[IDX2(k, 2 * j, d_r)];
                r1 += xr[k] * w_kr[IDX2(k, 2 * j + 1, d_r)];
            }
            const double cs = cos_tab[IDX2(pos, j, d_r / 2)], sn = sin_tab[IDX2(pos, j, d_r / 2)];
            row[d_c + 2 * j] = r0 * cs - r1 * sn;
            row[d_c + 2 * j + 1] = r0 * sn + r1 * cs;
        }
    }
}

/*
 * Query absorption: q'[b,h,0:d_c] = q_nope[b,h,:] (W^UK_h)^T and
 * q'[b,h,d_c:d_c+d_r] = q_rope[b,h,:].
 * Glossary "Multi-head Latent Attention", why decode absorbs: qbar_h =
 * q^C_h (W^UK_h)^T lives in the latent width; FlashMLA issue 16 answer: the
 * absorbed 512-wide query is concatenated with the 64-wide rope query.
 *   q'[b,h,c] = sum_j q_nope[b,h,j] * w_uk[h][j][c]
 */
void oracle_absorb_q(int b, int h, int d_k, int d_c, int d_r,
                     const double* q_nope, const double* w_uk, const double* q_rope,
                     double* q_prime)
{
    const int d = d_c + d_r;
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < (long)b * h; ++bh) {
        const int hi = (int)(bh % h);
        const double* qn = q_nope + IDX2(bh, 0, d_k);
        double* qp = q_prime + IDX2(bh, 0, d);
        for (int c = 0; c < d_c; ++c) {
            double acc = 0.0;
            for (int j = 0; j < d_k; ++j) acc += qn[j] * w_uk[IDX3(hi, j, c, d_k, d_c)];
            qp[c] = acc;
        }
        for (int r = 0; r < d_r; ++r) qp[d_c + r] = q_rope[IDX2(bh, r, d_r)];
    }
}

/*
 * Output absorption: y[b,h,j] = sum_c o[b,h,c] * w_uv[h][c][j].
 * Glossary "Multi-head Latent Attention", why decode absorbs: the value
 * up-projection applies once to the weighted latent sum.
 */
void oracle_absorb_o(int b, int h, int d_c, int d_v,
                     const double* o, const double* w_uv, double* y)
{
#pragma omp parallel for schedule(static)
    for (long bh = 0; bh < (long)b * h; ++bh) {
        const int hi = (int)(bh % h);
        const double* oo = o + IDX2(bh, 0, d_c);
        double* yo = y + IDX2(bh, 0, d_v);
        for (int j = 0; j < d_v; ++j) {
            double acc = 0.0;
            for (int c = 0; c < d_c; ++c) acc += oo[c] * w_uv[IDX3(hi, c, j, d_c, d_v)];
            yo[j] = acc;
        }
    }
}
