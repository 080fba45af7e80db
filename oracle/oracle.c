/*
 * oracle.c -- plain CPU reference for paged GQA attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or
 * calls this file; only the tests, the smoke check and the benchmark's CPU
 * baseline do.  It shares no code, header or table with the HIP library.
 *
 * Every input element (bf16, OCP e4m3fn, bf16 scale) is widened exactly to
 * double and every step is done in double.  The method is exact softmax
 * attention, out = softmax(scale * q K^T + mask) V, so each entry point is
 * that definition written out over an explicitly gathered K/V sequence:
 *
 *   decode (paged / contiguous)  AstrAI "CUDA Kernels" doc, Overview table
 *                                (attn_decode, attn_paged_decode) and the
 *                                Python Wrappers interface note (mask keeps
 *                                True entries; scale 1/sqrt(D) by default).
 *   split partials + combine     AstrAI csrc commit history, the commit that
 *                                partitions KV across gridDim.z into
 *                                unnormalised (O, m, l) partials reduced by a
 *                                combine kernel.
 *   ragged paged prefill         AstrAI "CUDA Kernels" doc, section
 *                                "Q Scheduling and KV Addressing" (packed Q,
 *                                qo_indptr, 64-row tiles) and the csrc commit
 *                                that unifies causal_offset (-1 off, >=0 the
 *                                absolute position of the first query row)
 *                                and lets causal and mask coexist.
 *   fp8 sliding-window decode    native_swa_decode.py, _fallback_batched_sdp:
 *                                slot -> (block, offset) gather, e4m3fn view,
 *                                multiply by the per-slot inverse scale,
 *                                mask (position >= len or index < 0), SDPA
 *                                with K = V.
 *   ragged work map              AstrAI "CUDA Kernels" doc, section
 *                                "Q Scheduling and KV Addressing" (worked
 *                                example with q lengths 70, 10, 130).
 *   paged KV append, rotary,     the cache write the backend layer owns, the
 *   fp8 quantize-on-write        rotary kernel's complex-product rotation,
 *                                and the FP8 multiplier convention (see each
 *                                function below).
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - query head h uses KV head h / (Hq / Hkv) (consecutive heads share);
 *   - a row with no admissible key yields out = 0 and lse = -inf;
 *   - causal admits key j for query row i iff j <= causal_offset + i;
 *   - the 3D mask is indexed [b, local query row, absolute key position];
 *   - fp8 dequantisation is the exact product e4m3(x) * inv_scale, unless
 *     emulate_bf16_dequant asks for the fallback's rounding to bf16.
 *
 * Return value of every entry point: 0 on success, -1 on a bad argument.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- scalars */

/* bf16 is the upper half of an IEEE binary32: widening is a shift. */
double orc_bf16_to_f64(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* OCP FP8 E4M3 ("fn": no infinities): sign, 4 exponent bits with bias 7,
 * 3 mantissa bits; exponent field 0 is subnormal; S.1111.111 is NaN. */
double orc_e4m3fn_to_f64(uint8_t bits)
{
    int s = bits >> 7, e = (bits >> 3) & 15, m = bits & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m / 8.0, -6);
    else v = ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

/* Round a double (exactly representable in binary32) to bf16, nearest-even. */
static double round_to_bf16(double x)
{
    float f = (float)x;
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u) return x;     /* inf / nan */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7fffu + lsb;
    u &= 0xffff0000u;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------- attention core */

/*
 * One query row against a dense gathered key/value sequence.
 * allow[j] != 0 admits key j.  Writes out[0..D) and *lse (natural log).
 */
static void attend(const double *qrow, const double *K, const double *V,
                   const unsigned char *allow, int n, int D, double scale,
                   double *out, double *lse, double *s /* scratch [n] */)
{
    double mx = -INFINITY;
    for (int j = 0; j < n; ++j) {
        if (!allow[j]) continue;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += qrow[d] * K[(size_t)j * D + d];
        s[j] = scale * dot;
        if (s[j] > mx) mx = s[j];
    }
    for (int d = 0; d < D; ++d) out[d] = 0.0;
    if (mx == -INFINITY) {          /* nothing admissible */
        *lse = -INFINITY;
        return;
    }
    double z = 0.0;
    for (int j = 0; j < n; ++j) {
        if (!allow[j]) continue;
        double w = exp(s[j] - mx);
        z += w;
        for (int d = 0; d < D; ++d) out[d] += w * V[(size_t)j * D + d];
    }
    for (int d = 0; d < D; ++d) out[d] /= z;
    *lse = mx + log(z);
}

/* Gather logical positions [0, n) of KV head g through a block table. */
static void gather_paged(const uint16_t *pool, int64_t s_page, int64_t s_slot,
                         int64_t s_head, const int32_t *bt_row, int ps, int g,
                         int n, int D, double *dst)
{
    for (int j = 0; j < n; ++j) {
        int64_t page = bt_row[j / ps];
        int64_t slot = j % ps;
        const uint16_t *src = pool + page * s_page + slot * s_slot + (int64_t)g * s_head;
        for (int d = 0; d < D; ++d) dst[(size_t)j * D + d] = orc_bf16_to_f64(src[d]);
    }
}

static void load_q(const uint16_t *q, int D, double *dst)
{
    for (int d = 0; d < D; ++d) dst[d] = orc_bf16_to_f64(q[d]);
}

static int check_heads(int Hq, int Hkv, int D)
{
    return Hq > 0 && Hkv > 0 && D > 0 && Hq % Hkv == 0;
}

/* ------------------------------------------------------------- decode */

/*
 * Paged decode.  q [B, Hq, D] (strides q_sb, q_sh); K/V pools addressed as
 * page * s_page + slot * s_slot + head * s_head; block_table row b at
 * bt + b * bt_sb; kv_lens [B].  Optional 2D keep-mask [B, *] with stride m_sb.
 * out [B, Hq, D] and lse [B, Hq], dense.
 */
int orc_paged_decode(const uint16_t *q, int64_t q_sb, int64_t q_sh,
                     const uint16_t *k_pool, const uint16_t *v_pool,
                     int64_t s_page, int64_t s_slot, int64_t s_head,
                     const int32_t *bt, int64_t bt_sb, const int32_t *kv_lens,
                     const uint8_t *mask, int64_t m_sb,
                     int B, int Hq, int Hkv, int D, int ps, double scale,
                     double *out, double *lse)
{
    if (!check_heads(Hq, Hkv, D) || B < 0 || ps <= 0) return -1;
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            int n = kv_lens[b];
            double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *s = malloc(sizeof(double) * ((size_t)n + 1));
            double *qr = malloc(sizeof(double) * (size_t)D);
            unsigned char *allow = malloc((size_t)n + 1);
            gather_paged(k_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, K);
            gather_paged(v_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, V);
            for (int j = 0; j < n; ++j) allow[j] = mask ? (mask[b * m_sb + j] != 0) : 1;
            for (int h = g * G; h < (g + 1) * G; ++h) {
                load_q(q + b * q_sb + h * q_sh, D, qr);
                attend(qr, K, V, allow, n, D, scale,
                       out + ((size_t)b * Hq + h) * D, lse + (size_t)b * Hq + h, s);
            }
            free(K); free(V); free(s); free(qr); free(allow);
        }
    }
    return 0;
}

/*
 * Contiguous decode.  K/V element (b, g, j, d) at b*sb + g*sh + j*sl + d.
 * kv_lens may be NULL, meaning every sequence has kv_len keys.
 */
int orc_decode(const uint16_t *q, int64_t q_sb, int64_t q_sh,
               const uint16_t *k, int64_t k_sb, int64_t k_sh, int64_t k_sl,
               const uint16_t *v, int64_t v_sb, int64_t v_sh, int64_t v_sl,
               const int32_t *kv_lens, int kv_len,
               int B, int Hq, int Hkv, int D, double scale,
               double *out, double *lse)
{
    if (!check_heads(Hq, Hkv, D) || B < 0) return -1;
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            int n = kv_lens ? kv_lens[b] : kv_len;
            double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *s = malloc(sizeof(double) * ((size_t)n + 1));
            double *qr = malloc(sizeof(double) * (size_t)D);
            unsigned char *allow = malloc((size_t)n + 1);
            for (int j = 0; j < n; ++j) {
                allow[j] = 1;
                for (int d = 0; d < D; ++d) {
                    K[(size_t)j * D + d] = orc_bf16_to_f64(k[b * k_sb + g * k_sh + j * k_sl + d]);
                    V[(size_t)j * D + d] = orc_bf16_to_f64(v[b * v_sb + g * v_sh + j * v_sl + d]);
                }
            }
            for (int h = g * G; h < (g + 1) * G; ++h) {
                load_q(q + b * q_sb + h * q_sh, D, qr);
                attend(qr, K, V, allow, n, D, scale,
                       out + ((size_t)b * Hq + h) * D, lse + (size_t)b * Hq + h, s);
            }
            free(K); free(V); free(s); free(qr); free(allow);
        }
    }
    return 0;
}

/* ------------------------------------------------------ split / combine */

/*
 * Split-KV partials of paged decode for caller-chosen chunk boundaries:
 * bounds[b * (S + 1) + s] .. bounds[b * (S + 1) + s + 1] is chunk s of
 * sequence b (clipped to [0, kv_lens[b])).  Per chunk and head:
 *   m = max score, l = sum exp(score - m), o = sum exp(score - m) V.
 * An empty chunk gives m = -inf, l = 0, o = 0.
 * o_part [S, B, Hq, D], m_part / l_part [S, B, Hq].
 */
int orc_paged_decode_partials(const uint16_t *q, int64_t q_sb, int64_t q_sh,
                              const uint16_t *k_pool, const uint16_t *v_pool,
                              int64_t s_page, int64_t s_slot, int64_t s_head,
                              const int32_t *bt, int64_t bt_sb, const int32_t *kv_lens,
                              const int32_t *bounds, int S,
                              int B, int Hq, int Hkv, int D, int ps, double scale,
                              double *o_part, double *m_part, double *l_part)
{
    if (!check_heads(Hq, Hkv, D) || B < 0 || ps <= 0 || S <= 0) return -1;
    int G = Hq / Hkv;
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            int n = kv_lens[b];
            double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *qr = malloc(sizeof(double) * (size_t)D);
            gather_paged(k_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, K);
            gather_paged(v_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, V);
            for (int h = g * G; h < (g + 1) * G; ++h) {
                load_q(q + b * q_sb + h * q_sh, D, qr);
                for (int s = 0; s < S; ++s) {
                    int lo = bounds[b * (S + 1) + s], hi = bounds[b * (S + 1) + s + 1];
                    if (lo < 0) lo = 0;
                    if (hi > n) hi = n;
                    size_t r = ((size_t)s * B + b) * Hq + h;
                    double *o = o_part + r * D;
                    double mx = -INFINITY, l = 0.0;
                    for (int d = 0; d < D; ++d) o[d] = 0.0;
                    for (int j = lo; j < hi; ++j) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += qr[d] * K[(size_t)j * D + d];
                        if (scale * dot > mx) mx = scale * dot;
                    }
                    for (int j = lo; j < hi; ++j) {
                        double dot = 0.0;
                        for (int d = 0; d < D; ++d) dot += qr[d] * K[(size_t)j * D + d];
                        double w = exp(scale * dot - mx);
                        l += w;
                        for (int d = 0; d < D; ++d) o[d] += w * V[(size_t)j * D + d];
                    }
                    m_part[r] = mx;
                    l_part[r] = l;
                }
            }
            free(K); free(V); free(qr);
        }
    }
    return 0;
}

/*
 * Log-sum-exp combine of S partials per row (natural-log m):
 *   M = max_s m_s, w_s = exp(m_s - M),
 *   out = sum_s w_s o_s / sum_s w_s l_s,  lse = M + log(sum_s w_s l_s).
 * Rows whose partials are all empty give out = 0, lse = -inf.
 * o_part [S, R, D]; m_part, l_part [S, R]; out [R, D]; lse [R].
 */
int orc_combine(const double *o_part, const double *m_part, const double *l_part,
                int S, int R, int D, double *out, double *lse)
{
    if (S <= 0 || R < 0 || D <= 0) return -1;
    for (int r = 0; r < R; ++r) {
        double M = -INFINITY;
        for (int s = 0; s < S; ++s)
            if (m_part[(size_t)s * R + r] > M) M = m_part[(size_t)s * R + r];
        double *o = out + (size_t)r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        if (M == -INFINITY) { lse[r] = -INFINITY; continue; }
        double L = 0.0;
        for (int s = 0; s < S; ++s) {
            double ms = m_part[(size_t)s * R + r];
            if (ms == -INFINITY) continue;
            double w = exp(ms - M);
            L += w * l_part[(size_t)s * R + r];
            for (int d = 0; d < D; ++d) o[d] += w * o_part[((size_t)s * R + r) * D + d];
        }
        for (int d = 0; d < D; ++d) o[d] /= L;
        lse[r] = M + log(L);
    }
    return 0;
}

/*
 * The same combine over single-precision partials as the GPU library lays
 * them out: o_part [S, R, D] float, ml_part [S, R, 2] float holding (m, l).
 */
int orc_combine_f32(const float *o_part, const float *ml_part, int S, int R, int D,
                    double *out, double *lse)
{
    if (S <= 0 || R < 0 || D <= 0) return -1;
    size_t no = (size_t)S * R * D, nm = (size_t)S * R;
    double *o = malloc(sizeof(double) * (no + 1));
    double *m = malloc(sizeof(double) * (nm + 1));
    double *l = malloc(sizeof(double) * (nm + 1));
    for (size_t i = 0; i < no; ++i) o[i] = (double)o_part[i];
    for (size_t i = 0; i < nm; ++i) {
        m[i] = (double)ml_part[2 * i];
        l[i] = (double)ml_part[2 * i + 1];
    }
    int rc = orc_combine(o, m, l, S, R, D, out, lse);
    free(o); free(m); free(l);
    return rc;
}

/* ------------------------------------------------------------ prefill */

/*
 * Ragged paged prefill.  Packed q [total_q, Hq, D] (strides q_st, q_sh);
 * sequence b owns rows qo_indptr[b] .. qo_indptr[b+1] and has kv_lens[b]
 * keys in the paged pool.  causal_offset may be NULL (non-causal); an entry
 * of -1 turns causality off for that sequence.  mask may be NULL; mask_ndim
 * 2 means keep = mask[b*m_sb + j], 3 means keep = mask[b*m_sb + i*m_sq + j]
 * with i the row index inside the sequence.  out [total_q, Hq, D], lse
 * [total_q, Hq].
 */
int orc_paged_prefill(const uint16_t *q, int64_t q_st, int64_t q_sh, const int32_t *qo_indptr,
                      const uint16_t *k_pool, const uint16_t *v_pool,
                      int64_t s_page, int64_t s_slot, int64_t s_head,
                      const int32_t *bt, int64_t bt_sb, const int32_t *kv_lens,
                      const int32_t *causal_offset,
                      const uint8_t *mask, int mask_ndim, int64_t m_sb, int64_t m_sq,
                      int B, int Hq, int Hkv, int D, int ps, double scale,
                      double *out, double *lse)
{
    if (!check_heads(Hq, Hkv, D) || B < 0 || ps <= 0) return -1;
    if (mask && mask_ndim != 2 && mask_ndim != 3) return -1;
    int G = Hq / Hkv;
#pragma omp parallel for collapse(2) schedule(dynamic)
    for (int b = 0; b < B; ++b) {
        for (int g = 0; g < Hkv; ++g) {
            int n = kv_lens[b];
            int r0 = qo_indptr[b], qn = qo_indptr[b + 1] - qo_indptr[b];
            int c = causal_offset ? causal_offset[b] : -1;
            double *K = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *V = malloc(sizeof(double) * ((size_t)n * D + 1));
            double *s = malloc(sizeof(double) * ((size_t)n + 1));
            double *qr = malloc(sizeof(double) * (size_t)D);
            unsigned char *allow = malloc((size_t)n + 1);
            gather_paged(k_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, K);
            gather_paged(v_pool, s_page, s_slot, s_head, bt + b * bt_sb, ps, g, n, D, V);
            for (int i = 0; i < qn; ++i) {
                for (int j = 0; j < n; ++j) {
                    int keep = 1;
                    if (c >= 0 && j > c + i) keep = 0;
                    if (mask && mask_ndim == 2 && !mask[b * m_sb + j]) keep = 0;
                    if (mask && mask_ndim == 3 && !mask[b * m_sb + (int64_t)i * m_sq + j]) keep = 0;
                    allow[j] = (unsigned char)keep;
                }
                for (int h = g * G; h < (g + 1) * G; ++h) {
                    size_t row = (size_t)(r0 + i);
                    load_q(q + (int64_t)row * q_st + h * q_sh, D, qr);
                    attend(qr, K, V, allow, n, D, scale,
                           out + (row * Hq + h) * D, lse + row * Hq + h, s);
                }
            }
            free(K); free(V); free(s); free(qr); free(allow);
        }
    }
    return 0;
}

/*
 * Ragged work map: qo_indptr is the prefix sum of q_lens; each sequence is
 * cut into ceil(q_len / tile_rows) tiles, listed in sequence order.
 * Returns the number of tiles, or -1 if it exceeds cap or an argument is bad.
 */
int orc_prefill_plan(const int32_t *q_lens, int B, int tile_rows,
                     int32_t *qo_indptr, int32_t *tile_to_batch, int32_t *tile_to_index,
                     int cap)
{
    if (B < 0 || tile_rows <= 0) return -1;
    int t = 0;
    qo_indptr[0] = 0;
    for (int b = 0; b < B; ++b) {
        if (q_lens[b] < 0) return -1;
        qo_indptr[b + 1] = qo_indptr[b] + q_lens[b];
        for (int i = 0; i * tile_rows < q_lens[b]; ++i) {
            if (t >= cap) return -1;
            tile_to_batch[t] = b;
            tile_to_index[t] = i;
            ++t;
        }
    }
    return t;
}

/* ------------------------------------------------- fp8 sliding window */

/*
 * fp8 sliding-window decode with K = V.  q [T, NH, HD] (strides q_st, q_sh);
 * cache bytes of slot idx at (idx / bs) * c_sb + (idx % bs) * c_ss;
 * inv_scale of slot idx at inv_scale[idx * s_ss] (bf16); indices row t at
 * ind + t * i_st, W entries; lens [T].  Window position j is admitted iff
 * j < lens[t] and ind[t, j] >= 0.  Every head of token t attends the same
 * dequantised rows.  out [T, NH, HD], lse [T, NH].
 */
int orc_swa_fp8_decode(const uint16_t *q, int64_t q_st, int64_t q_sh,
                       const uint8_t *cache, int64_t c_sb, int64_t c_ss,
                       const uint16_t *inv_scale, int64_t s_ss,
                       const int64_t *ind, int64_t i_st, const int64_t *lens,
                       int T, int NH, int HD, int W, int bs, double scale,
                       int emulate_bf16_dequant, double *out, double *lse)
{
    if (T < 0 || NH <= 0 || HD <= 0 || W < 0 || bs <= 0) return -1;
#pragma omp parallel for schedule(dynamic)
    for (int t = 0; t < T; ++t) {
        double *X = malloc(sizeof(double) * ((size_t)W * HD + 1));
        double *s = malloc(sizeof(double) * ((size_t)W + 1));
        double *qr = malloc(sizeof(double) * (size_t)HD);
        unsigned char *allow = malloc((size_t)W + 1);
        for (int j = 0; j < W; ++j) {
            int64_t idx = ind[t * i_st + j];
            allow[j] = (unsigned char)(j < lens[t] && idx >= 0);
            if (!allow[j]) {
                for (int d = 0; d < HD; ++d) X[(size_t)j * HD + d] = 0.0;
                continue;
            }
            const uint8_t *row = cache + (idx / bs) * c_sb + (idx % bs) * c_ss;
            double sc = orc_bf16_to_f64(inv_scale[idx * s_ss]);
            for (int d = 0; d < HD; ++d) {
                double x = orc_e4m3fn_to_f64(row[d]) * sc;
                X[(size_t)j * HD + d] = emulate_bf16_dequant ? round_to_bf16(x) : x;
            }
        }
        for (int h = 0; h < NH; ++h) {
            load_q(q + t * q_st + h * q_sh, HD, qr);
            attend(qr, X, X, allow, W, HD, scale,
                   out + ((size_t)t * NH + h) * HD, lse + (size_t)t * NH + h, s);
        }
        free(X); free(s); free(qr); free(allow);
    }
    return 0;
}

/* ------------------------------------------------ cache writes, rotary */

/*
 * Paged KV append (AstrAI "CUDA Kernels" doc, Backend Layer: the attention
 * backend owns the KV cache writes that precede paged decode / prefill).
 * New rows are packed [N, Hkv, D] (row i at k_new + i*n_st, head g at
 * + g*n_sh); sequence b owns rows new_indptr[b] .. new_indptr[b+1] and its
 * first new token sits at position start_pos[b].  Token position p of
 * sequence b lives in page bt[b][p / ps], slot p % ps.  A pure copy: every
 * written element equals its source bit for bit.
 */
int orc_kv_append(const uint16_t *k_new, const uint16_t *v_new, int64_t n_st, int64_t n_sh,
                  const int32_t *new_indptr, const int32_t *start_pos,
                  uint16_t *k_pool, uint16_t *v_pool, int64_t s_page, int64_t s_slot, int64_t s_head,
                  const int32_t *bt, int64_t bt_sb, int B, int Hkv, int D, int ps)
{
    if (B < 0 || Hkv <= 0 || D <= 0 || ps <= 0) return -1;
    for (int b = 0; b < B; ++b) {
        for (int i = new_indptr[b]; i < new_indptr[b + 1]; ++i) {
            int64_t pos = (int64_t)start_pos[b] + (i - new_indptr[b]);
            int32_t page = bt[(int64_t)b * bt_sb + pos / ps];
            if (page < 0) return -1;
            int64_t base = (int64_t)page * s_page + (pos % ps) * s_slot;
            for (int g = 0; g < Hkv; ++g)
                for (int d = 0; d < D; ++d) {
                    k_pool[base + g * s_head + d] = k_new[(int64_t)i * n_st + g * n_sh + d];
                    v_pool[base + g * s_head + d] = v_new[(int64_t)i * n_st + g * n_sh + d];
                }
        }
    }
    return 0;
}

/* Round a double to the nearest bf16 (ties to even), once. */
static double round_f64_to_bf16(double x)
{
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    frexp(x, &e);                        /* |x| = m * 2^e, 0.5 <= m < 1 */
    int q = e - 8;                       /* bf16 keeps 8 significant bits */
    if (q < -133) q = -133;              /* subnormal quantum 2^-133 */
    return ldexp(nearbyint(ldexp(x, -q)), q);
}

/*
 * Rotary embedding (AstrAI "CUDA Kernels" doc, Rotary Embedding Kernel and
 * Rotary Backend): the cos / sin rows of each token's position are looked up
 * in fp32 tables [rows, D/2] (row p at + p*tab_st) and every adjacent pair
 * (x[2i], x[2i+1]) of a head is multiplied, as a complex number, by
 * cos_i + i sin_i (the torch fallback's view_as_complex product).  x, out are
 * [T, H, D] bf16; the product is exact here and rounded to bf16 once.
 */
int orc_rotary(const uint16_t *x, int64_t x_st, int64_t x_sh, int T, int H, int D,
               const float *cos_tab, const float *sin_tab, int64_t tab_st, const int32_t *pos,
               uint16_t *out, int64_t o_st, int64_t o_sh)
{
    if (T < 0 || H <= 0 || D <= 0 || (D & 1)) return -1;
    for (int t = 0; t < T; ++t)
        for (int h = 0; h < H; ++h)
            for (int i = 0; i < D / 2; ++i) {
                double c = cos_tab[(int64_t)pos[t] * tab_st + i];
                double s = sin_tab[(int64_t)pos[t] * tab_st + i];
                double a = orc_bf16_to_f64(x[(int64_t)t * x_st + (int64_t)h * x_sh + 2 * i]);
                double b = orc_bf16_to_f64(x[(int64_t)t * x_st + (int64_t)h * x_sh + 2 * i + 1]);
                double re = round_f64_to_bf16(a * c - b * s), im = round_f64_to_bf16(a * s + b * c);
                float fr = (float)re, fi = (float)im;   /* exact: bf16 values */
                uint32_t ur, ui;
                memcpy(&ur, &fr, 4);
                memcpy(&ui, &fi, 4);
                out[(int64_t)t * o_st + (int64_t)h * o_sh + 2 * i] = (uint16_t)(ur >> 16);
                out[(int64_t)t * o_st + (int64_t)h * o_sh + 2 * i + 1] = (uint16_t)(ui >> 16);
            }
    return 0;
}

/* Nearest OCP e4m3fn code to a binary32 value: ties to the even code
 * (mantissa bit 0 clear), magnitudes at or above 448 saturate to 448, NaN
 * gives the NaN code, the sign bit is kept (so -0 gives 0x80).  Found by
 * comparing against every finite magnitude. */
static uint8_t nearest_e4m3fn(float p)
{
    if (isnan(p)) return 0x7F;
    uint32_t u;
    memcpy(&u, &p, 4);
    uint8_t sign = (u >> 31) ? 0x80 : 0x00;
    double a = fabs((double)p);
    if (a >= 448.0) return sign | 0x7E;
    int best = 0;
    double best_err = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double err = fabs(orc_e4m3fn_to_f64((uint8_t)c) - a);
        if (err < best_err || (err == best_err && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_err = err;
        }
    }
    return sign | (uint8_t)best;
}

/*
 * fp8 quantize-on-write of sliding-window cache rows (native_swa_decode.py:
 * the cache holds e4m3fn codes and a per-slot inverse scale; AstrAI "CUDA
 * Kernels" doc, FP8 section: quantize takes the multiplier and multiplies
 * by it, and amax is reported in the input domain).  Row n of x [N, HD]:
 *   amax = max |x|;  m = mult[n], or 448 / amax (1 when amax is 0) when
 *   mult is NULL;  code = nearest_e4m3fn(x * m) with the product taken in
 *   binary32 (the precision the decision is made in);  inv = bf16(1 / m)
 *   (binary32 division, then nearest-even to bf16).
 */
int orc_fp8_quantize(const uint16_t *x, int64_t x_st, int N, int HD, const float *mult,
                     uint8_t *codes, int64_t c_st, uint16_t *inv_out, float *amax_out)
{
    if (N < 0 || HD <= 0) return -1;
    for (int n = 0; n < N; ++n) {
        float amax = 0.f;
        for (int d = 0; d < HD; ++d) {
            float v = fabsf((float)orc_bf16_to_f64(x[(int64_t)n * x_st + d]));
            if (v > amax) amax = v;
        }
        float m = mult ? mult[n] : (amax > 0.f ? 448.0f / amax : 1.0f);
        for (int d = 0; d < HD; ++d) {
            float p = (float)orc_bf16_to_f64(x[(int64_t)n * x_st + d]) * m;
            codes[(int64_t)n * c_st + d] = nearest_e4m3fn(p);
        }
        float inv = 1.0f / m;
        double r = round_f64_to_bf16((double)inv);
        float rf = (float)r;
        uint32_t ur;
        memcpy(&ur, &rf, 4);
        inv_out[n] = (uint16_t)(ur >> 16);
        if (amax_out) amax_out[n] = amax;
    }
    return 0;
}

/* Number of OpenMP threads the parallel entry points use. */
int orc_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}
