/*
 * Exact-attention oracle: plain, slow, fp64 CPU reference.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this file; only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code, header, table or
 * constant with the HIP library.
 *
 * What it computes is the plain definition of attention, not the tiled method:
 *   s_ij = scale * sum_c q_ic k_jc                       (similarity step,
 *          "FlashAttention v1 / attention implementation" section of the
 *          91haoming.cn page; the johneyzheng.top code listing with scale 1)
 *   causal: key j is visible to query i iff j <= pos_i  (the mask is only named
 *          as "optional masking" on the 91haoming.cn page; this is the reading
 *          taken for it: top-left aligned, diagonal visible)
 *   m_i = max_j s_ij ; e_ij = exp(s_ij - m_i) ; l_i = sum_j e_ij
 *          (3-pass safe softmax, "safe softmax" part of the jibinghu.github.io
 *          page)
 *   o_ic = sum_j e_ij v_jc / l_i                         (weighted sum step)
 *   L_i  = m_i + ln l_i                                  (logsumexp kept by the
 *          forward pass, "forward pass improvements" of FlashAttention v2 on the
 *          91haoming.cn page; natural log, units of the scaled scores)
 * A row with no visible key gets O = 0 and L = -inf (the pages do not cover it;
 * this is the reading exp(-inf - (-inf)) := 0).
 *
 * Input decoders (exact): bf16 bit patterns, and OCP E4M3FN bytes from the OCP
 * 8-bit floating point specification (bias 7, no infinities, S.1111.111 is NaN,
 * largest finite 448), plus the per-(head, 128-token) block dequantisation that
 * the FlashAttention-3 "block quantization" description implies: x = decode(x8)
 * times the block's fp32 scale.
 *
 * Paged decode: the keys/values of sequence s are token t = 0..ctx_s-1 at
 * physical page block_table[s][t / page_size], slot t mod page_size (block table
 * of the PagedAttention section of the johneyzheng.top page), the query attends
 * to all of them, no mask.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* One query row against n_vis visible keys. Pure definition, fp64. */
static void attend_row(const double *q, const double *k, const double *v,
                       long n_vis, int d, double scale, double *s_buf,
                       double *o, double *lse)
{
    if (n_vis <= 0) {
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        *lse = -INFINITY;
        return;
    }
    /* pass 1: scores and their maximum */
    double m = -INFINITY;
    for (long j = 0; j < n_vis; ++j) {
        double acc = 0.0;
        const double *kj = k + j * (long)d;
        for (int c = 0; c < d; ++c) acc += q[c] * kj[c];
        s_buf[j] = scale * acc;
        if (s_buf[j] > m) m = s_buf[j];
    }
    /* pass 2: exponentials and their sum */
    double l = 0.0;
    for (long j = 0; j < n_vis; ++j) {
        s_buf[j] = exp(s_buf[j] - m);
        l += s_buf[j];
    }
    /* pass 3: normalised weighted sum of values */
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    for (long j = 0; j < n_vis; ++j) {
        const double *vj = v + j * (long)d;
        double w = s_buf[j];
        for (int c = 0; c < d; ++c) o[c] += w * vj[c];
    }
    for (int c = 0; c < d; ++c) o[c] /= l;
    *lse = m + log(l);
}

/*
 * Batched attention over BH independent heads.
 * q [BH, n_q, d], k/v [BH, n_k, d], o [BH, n_q, d], lse [BH, n_q]  (fp64, contiguous)
 * causal: query i sees keys j <= i (n_q == n_k in every use).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention(const double *q, const double *k, const double *v,
                     double *o, double *lse, long BH, long n_q, long n_k, int d,
                     double scale, int causal)
{
    if (!q || !k || !v || !o || !lse || BH < 0 || n_q < 0 || n_k < 0 || d <= 0)
        return -1;
    int err = 0;
    long total = BH * n_q;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        if (!s_buf) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(dynamic, 16)
            for (long r = 0; r < total; ++r) {
                long bh = r / n_q, i = r % n_q;
                long n_vis = causal ? (i + 1 < n_k ? i + 1 : n_k) : n_k;
                attend_row(q + r * d, k + bh * n_k * d, v + bh * n_k * d, n_vis, d,
                           scale, s_buf, o + r * d, lse + r);
            }
            free(s_buf);
        }
    }
    return err;
}

/*
 * Selected rows of one head: q_rows [n_rows, d] with positions pos[n_rows]
 * (causal: key j visible iff j <= pos[r]), k/v [n_k, d].
 */
int oracle_attention_rows(const double *q_rows, const long *pos, long n_rows,
                          const double *k, const double *v, long n_k, int d,
                          double scale, int causal, double *o, double *lse)
{
    if (!q_rows || !k || !v || !o || !lse || n_rows < 0 || n_k < 0 || d <= 0)
        return -1;
    if (causal && !pos) return -1;
    int err = 0;
#pragma omp parallel
    {
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(n_k > 0 ? n_k : 1));
        if (!s_buf) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < n_rows; ++r) {
                long n_vis = n_k;
                if (causal) n_vis = pos[r] + 1 < n_k ? pos[r] + 1 : n_k;
                attend_row(q_rows + r * d, k, v, n_vis, d, scale, s_buf, o + r * d, lse + r);
            }
            free(s_buf);
        }
    }
    return err;
}

/* bf16 bit pattern -> fp64 (exact: the bf16 bits are the top half of an fp32). */
void oracle_bf16_to_f64(const uint16_t *x, double *out, long n)
{
    for (long i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)x[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        out[i] = (double)f;
    }
}

/* OCP E4M3FN byte -> fp64, from the format definition. */
static double e4m3_value(uint8_t b)
{
    int sign = b >> 7;
    int e = (b >> 3) & 0xF;
    int m = b & 0x7;
    double mag;
    if (e == 0xF && m == 0x7) return NAN;          /* S.1111.111 */
    if (e == 0) mag = ldexp((double)m, -9);        /* subnormal: m/8 * 2^(1-7) */
    else mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

void oracle_e4m3_to_f64(const uint8_t *x, double *out, long n)
{
    for (long i = 0; i < n; ++i) out[i] = e4m3_value(x[i]);
}

/*
 * Block dequantisation: x8 [BH, N, d] bytes, scales [BH, ceil(N/block)] fp32,
 * out [BH, N, d] = decode(x8) * scale of the token's block.
 */
void oracle_dequant_e4m3(const uint8_t *x8, const float *scales, double *out,
                         long BH, long N, int d, int block)
{
    long nblk = (N + block - 1) / block;
    for (long bh = 0; bh < BH; ++bh)
        for (long t = 0; t < N; ++t) {
            double sc = (double)scales[bh * nblk + t / block];
            const uint8_t *src = x8 + (bh * N + t) * d;
            double *dst = out + (bh * N + t) * d;
            for (int c = 0; c < d; ++c) dst[c] = e4m3_value(src[c]) * sc;
        }
}

/*
 * Paged decode. q [S, H, d] fp64; kcache/vcache bf16 bits [num_pages, H, page_size, d];
 * block_table int32 [S, max_blocks]; ctx_lens int32 [S].
 * o [S, H, d], lse [S, H]. Returns 0, -1 bad argument, -2 table entry out of range.
 */
int oracle_paged_decode(const double *q, const uint16_t *kcache, const uint16_t *vcache,
                        const int32_t *block_table, const int32_t *ctx_lens,
                        long S, int H, int d, int page_size, long max_blocks,
                        long num_pages, double scale, double *o, double *lse)
{
    if (!q || !kcache || !vcache || !block_table || !ctx_lens || !o || !lse)
        return -1;
    if (S < 0 || H <= 0 || d <= 0 || page_size <= 0 || max_blocks < 0) return -1;
    for (long s = 0; s < S; ++s) {
        long ctx = ctx_lens[s];
        if (ctx < 0 || ctx > max_blocks * page_size) return -1;
        for (long b = 0; b < (ctx + page_size - 1) / page_size; ++b) {
            int32_t p = block_table[s * max_blocks + b];
            if (p < 0 || p >= num_pages) return -2;
        }
    }
    int err = 0;
    long total = S * H;
#pragma omp parallel
    {
        long max_ctx = max_blocks * page_size;
        double *kg = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1) * d);
        double *vg = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1) * d);
        double *s_buf = (double *)malloc(sizeof(double) * (size_t)(max_ctx > 0 ? max_ctx : 1));
        if (!kg || !vg || !s_buf) {
#pragma omp atomic write
            err = -1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (long r = 0; r < total; ++r) {
                long s = r / H, h = r % H;
                long ctx = ctx_lens[s];
                /* gather the sequence's keys and values through the block table */
                for (long t = 0; t < ctx; ++t) {
                    long page = block_table[s * max_blocks + t / page_size];
                    long slot = t % page_size;
                    long base = ((page * H + h) * page_size + slot) * d;
                    oracle_bf16_to_f64(kcache + base, kg + t * d, d);
                    oracle_bf16_to_f64(vcache + base, vg + t * d, d);
                }
                attend_row(q + r * d, kg, vg, ctx, d, scale, s_buf, o + r * d, lse + r);
            }
        }
        free(kg);
        free(vg);
        free(s_buf);
    }
    return err;
}

/*
 * Backward pass of the same definition (gradients of a loss that reaches the
 * attention only through O). The pages describe the backward pass by what it
 * stores and recomputes, not by formulas (FlashAttention v1 recomputation and
 * v2 "store only L" on the 91haoming.cn page; the backward part of the
 * jibinghu.github.io page), so this is the plain chain rule through the three
 * steps of the forward definition, per head:
 *   weighted sum o_i = sum_j p_ij v_j :  dv_j  = sum_i p_ij do_i,
 *                                        dp_ij = do_i . v_j
 *   softmax p_i = softmax_j(s_ij) over the visible keys (Jacobian
 *   diag(p) - p p^T):                    ds_ij = p_ij (dp_ij - sum_k p_ik dp_ik)
 *   similarity s_ij = scale q_i . k_j :  dq_i  = scale sum_j ds_ij k_j,
 *                                        dk_j  = scale sum_i ds_ij q_i
 * p is recomputed here from the scores (3-pass safe softmax). A row with no
 * visible key contributes nothing.
 * q, k, v, dout [BH, n, d]; dq, dk, dv [BH, n, d] (fp64, contiguous).
 * Returns 0, or -1 on a bad argument or allocation failure.
 */
int oracle_attention_bwd(const double *q, const double *k, const double *v,
                         const double *dout, double *dq, double *dk, double *dv,
                         long BH, long n, int d, double scale, int causal)
{
    if (!q || !k || !v || !dout || !dq || !dk || !dv || BH < 0 || n < 0 || d <= 0)
        return -1;
    int err = 0;
#pragma omp parallel
    {
        double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        double *dp = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
        if (!p || !dp) {
#pragma omp atomic write
            err = -1;
        } else {
            /* one head per iteration: dk and dv of a head are sums over its rows */
#pragma omp for schedule(dynamic, 1)
            for (long bh = 0; bh < BH; ++bh) {
                const long off = bh * n * d;
                const double *qh = q + off, *kh = k + off, *vh = v + off, *gh = dout + off;
                double *dqh = dq + off, *dkh = dk + off, *dvh = dv + off;
                for (long x = 0; x < n * d; ++x) dqh[x] = dkh[x] = dvh[x] = 0.0;
                for (long i = 0; i < n; ++i) {
                    const long n_vis = causal ? i + 1 : n;
                    const double *qi = qh + i * d, *gi = gh + i * d;
                    /* recompute p_i: scores, max, exponentials, sum, normalise */
                    double m = -INFINITY;
                    for (long j = 0; j < n_vis; ++j) {
                        double acc = 0.0;
                        for (int c = 0; c < d; ++c) acc += qi[c] * kh[j * d + c];
                        p[j] = scale * acc;
                        if (p[j] > m) m = p[j];
                    }
                    double l = 0.0;
                    for (long j = 0; j < n_vis; ++j) {
                        p[j] = exp(p[j] - m);
                        l += p[j];
                    }
                    for (long j = 0; j < n_vis; ++j) p[j] /= l;
                    /* through the weighted sum */
                    double pdp = 0.0;
                    for (long j = 0; j < n_vis; ++j) {
                        double acc = 0.0;
                        for (int c = 0; c < d; ++c) {
                            dvh[j * d + c] += p[j] * gi[c];
                            acc += gi[c] * vh[j * d + c];
                        }
                        dp[j] = acc;
                        pdp += p[j] * acc;
                    }
                    /* through the softmax, then the similarity */
                    for (long j = 0; j < n_vis; ++j) {
                        const double ds = p[j] * (dp[j] - pdp);
                        for (int c = 0; c < d; ++c) {
                            dqh[i * d + c] += scale * ds * kh[j * d + c];
                            dkh[j * d + c] += scale * ds * qi[c];
                        }
                    }
                }
            }
        }
        free(p);
        free(dp);
    }
    return err;
}
