/*
 * CPU oracle of the KPool-indexed DeepSeek Sparse Attention forward.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline leg of the benchmark, never by the product path. Shares no code
 * with the HIP library. Built with -ffp-contract=off so that no multiply-add
 * is fused behind the reader's back. Citations ([P4-S3] ...) are defined in
 * kpool_oracle.h.
 */
#include "kpool_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* ---------------------------------------------------------------- layout -- */

/* Pools are cut per document, in groups of kpool tokens starting at the
 * document's first token; a trailing group shorter than kpool is not a pool
 * [P4-S3]. Documents never share a pool. */
int32_t kpo_layout(const int32_t* cu, int32_t num_docs, int32_t num_tokens, int32_t kpool,
                   int32_t* cu_pools, int32_t* pool_start) {
    if (kpool < 1 || num_docs < 0 || cu[0] != 0 || cu[num_docs] != num_tokens) return -1;
    for (int32_t d = 0; d < num_docs; ++d)
        if (cu[d + 1] < cu[d]) return -1;
    int32_t p = 0;
    cu_pools[0] = 0;
    for (int32_t d = 0; d < num_docs; ++d) {
        int32_t len = cu[d + 1] - cu[d];
        for (int32_t j = 0; j + kpool <= len; j += kpool) pool_start[p++] = cu[d] + j;
        cu_pools[d + 1] = p;
    }
    return p;
}

/* The document holding t is the d with cu[d] <= t < cu[d+1]. With local
 * position l = t - cu[d], the complete pools ending at or before t are the
 * first (l+1)/kpool pools of the document; the rest of the query's own group
 * (its incomplete pool, possibly empty) starts at cu[d] + kpool*n_vis [P4-S3]. */
int32_t kpo_query_info(const int32_t* cu, int32_t num_docs, const int32_t* cu_pools, int32_t kpool,
                       int32_t t, int32_t* pool_lo, int32_t* n_vis, int32_t* tail_start) {
    for (int32_t d = 0; d < num_docs; ++d) {
        if (t >= cu[d] && t < cu[d + 1]) {
            int32_t l = t - cu[d];
            *pool_lo = cu_pools[d];
            *n_vis = (l + 1) / kpool;
            *tail_start = cu[d] + kpool * (*n_vis);
            return d;
        }
    }
    return -1;
}

/* --------------------------------------------------------------- pooling -- */

/* Per channel c of pool p (tokens s..s+kpool-1): logits a_i = gate + ape_i,
 * weights softmax over the kpool tokens, pooled key = weighted sum of the
 * tokens' keys [P4-S3]. Evaluated in float64, rounded once to float32. */
void kpo_pool(const uint16_t* k_idx, const uint16_t* gate, const float* ape,
              const int32_t* pool_start, int32_t num_pools, int32_t d_idx, int32_t kpool,
              float* out) {
#pragma omp parallel for schedule(static)
    for (int32_t p = 0; p < num_pools; ++p) {
        int64_t s = pool_start[p];
        double a[64];
        for (int32_t c = 0; c < d_idx; ++c) {
            double amax = -INFINITY;
            for (int32_t i = 0; i < kpool; ++i) {
                a[i] = bf16_value(gate[(s + i) * d_idx + c]) + (double)ape[i * d_idx + c];
                if (a[i] > amax) amax = a[i];
            }
            double den = 0.0, num = 0.0;
            for (int32_t i = 0; i < kpool; ++i) {
                double e = exp(a[i] - amax);
                den += e;
                num += e * bf16_value(k_idx[(s + i) * d_idx + c]);
            }
            out[(int64_t)p * d_idx + c] = (float)(num / den);
        }
    }
}

/* ---------------------------------------------------------------- FWHT ---- */

/* Sylvester-ordered butterflies in fp32, stride 1, 2, 4, ... n/2: each pair
 * (x_j, x_{j+h}) becomes (x_j + x_{j+h}, x_j - x_{j+h}); then one multiply by
 * fp32(1/sqrt(n)) makes the transform orthonormal [P4-S3]. */
void kpo_fwht(float* x, int32_t n) {
    for (int32_t h = 1; h < n; h <<= 1) {
        for (int32_t i = 0; i < n; i += 2 * h) {
            for (int32_t j = i; j < i + h; ++j) {
                float a = x[j], b = x[j + h];
                x[j] = a + b;
                x[j + h] = a - b;
            }
        }
    }
    float norm = (float)(1.0 / sqrt((double)n));
    for (int32_t j = 0; j < n; ++j) x[j] = x[j] * norm;
}

/* --------------------------------------------------------------- E4M3FN --- */

/* OCP 8-bit E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; S.1111.111 is NaN; largest finite 448 = 1.75 * 2^8; subnormals
 * m * 2^-9. Encoding rounds to the nearest representable value, ties to the
 * even mantissa, and saturates magnitudes above 448 to 448. */
float kpo_e4m3_decode(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 0xF, m = code & 7;
    double v;
    if (e == 0xF && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return (float)(sign ? -v : v);
}

uint8_t kpo_e4m3_encode(float vf) {
    double v = (double)vf;
    if (isnan(v)) return 0x7F;
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0) return sign | 0x7E;
    if (a == 0.0) return sign;
    int e2;
    frexp(a, &e2);                      /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                     /* floor(log2 a) */
    if (E < -6) E = -6;                 /* below the normal range the spacing is 2^-9 */
    double quantum = ldexp(1.0, E - 3); /* spacing of representable values near a */
    double n = rint(a / quantum);       /* exact division; rint rounds half to even */
    double r = n * quantum;             /* the rounded magnitude, exactly */
    if (r == 0.0) return sign;
    frexp(r, &e2);
    E = e2 - 1;
    if (E < -6) return sign | (uint8_t)ldexp(r, 9); /* subnormal: r = m * 2^-9 */
    int mant = (int)((ldexp(r, -E) - 1.0) * 8.0);
    return sign | (uint8_t)((E + 7) << 3) | (uint8_t)mant;
}

void kpo_quant_rows(const float* x, int64_t rows, int32_t n, uint8_t* codes, float* scales) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float* v = x + r * n;
        float amax = 0.0f;
        for (int32_t c = 0; c < n; ++c) {
            float m = fabsf(v[c]);
            if (m > amax) amax = m;
        }
        float s = amax > 0.0f ? amax / 448.0f : 1.0f;
        scales[r] = s;
        for (int32_t c = 0; c < n; ++c) codes[r * n + c] = kpo_e4m3_encode(v[c] / s);
    }
}

/* ------------------------------------------------------------ keys/queries */

void kpo_keys(const uint16_t* k_idx, const uint16_t* gate, const float* ape,
              const int32_t* pool_start, int32_t num_pools, int32_t d_idx, int32_t kpool,
              uint8_t* codes, float* scales, float* pooled_f32) {
    float* pooled = (float*)malloc(sizeof(float) * (size_t)num_pools * (size_t)d_idx + 1);
    kpo_pool(k_idx, gate, ape, pool_start, num_pools, d_idx, kpool, pooled);
    if (pooled_f32) memcpy(pooled_f32, pooled, sizeof(float) * (size_t)num_pools * (size_t)d_idx);
#pragma omp parallel for schedule(static)
    for (int32_t p = 0; p < num_pools; ++p) kpo_fwht(pooled + (int64_t)p * d_idx, d_idx);
    kpo_quant_rows(pooled, num_pools, d_idx, codes, scales);
    free(pooled);
}

void kpo_queries(const uint16_t* q_idx, int32_t num_q, int32_t h_idx, int32_t d_idx,
                 uint8_t* codes, float* scales) {
    int64_t rows = (int64_t)num_q * h_idx;
    float* rot = (float*)malloc(sizeof(float) * (size_t)rows * (size_t)d_idx + 1);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int32_t c = 0; c < d_idx; ++c) rot[r * d_idx + c] = (float)bf16_value(q_idx[r * d_idx + c]);
        kpo_fwht(rot + r * d_idx, d_idx);
    }
    kpo_quant_rows(rot, rows, d_idx, codes, scales);
    free(rot);
}

/* ---------------------------------------------------------------- scores -- */

/* Lightning-indexer score of query t against pool p [P4-S3]:
 *   I = sum_h w[t,h] * ReLU(sq[t,h] * sk[p] * <q8[t,h], k8[p]>).
 * Every E4M3 value is a multiple of 2^-9 below 2^9 in magnitude, so the
 * float64 dot of decoded codes is exact. Pools of other documents and pools
 * that end after t are not visible and score -inf. */
void kpo_scores(const int32_t* cu, int32_t num_docs, const int32_t* cu_pools, int32_t kpool,
                const int32_t* q_pos, int32_t num_q, int32_t max_pools,
                const uint8_t* q_codes, const float* q_scales,
                const uint8_t* k_codes, const float* k_scales,
                const float* q_rot, const float* k_rot, int32_t mode,
                const float* w, int32_t h_idx, int32_t d_idx, float* scores) {
    double dec[256];                    /* the value of every E4M3 code */
    for (int c = 0; c < 256; ++c) dec[c] = (double)kpo_e4m3_decode((uint8_t)c);
    int32_t* lo = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_q + 1));
    int32_t* nv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(num_q + 1));
    for (int32_t i = 0; i < num_q; ++i) {
        int32_t ts = 0;
        int32_t t = q_pos ? q_pos[i] : i;
        lo[i] = 0;
        nv[i] = 0;
        kpo_query_info(cu, num_docs, cu_pools, kpool, t, &lo[i], &nv[i], &ts);
    }
#pragma omp parallel for collapse(2) schedule(static)
    for (int32_t i = 0; i < num_q; ++i) {
        for (int32_t p = 0; p < max_pools; ++p) {
            float* out = scores + (int64_t)i * max_pools + p;
            if (p < lo[i] || p >= lo[i] + nv[i]) { *out = -INFINITY; continue; }
            double acc = 0.0;
            for (int32_t h = 0; h < h_idx; ++h) {
                int64_t qo = ((int64_t)i * h_idx + h) * d_idx, ko = (int64_t)p * d_idx;
                double v, dot = 0.0;
                if (mode == 0) {
                    for (int32_t c = 0; c < d_idx; ++c) dot += dec[q_codes[qo + c]] * dec[k_codes[ko + c]];
                    v = (double)q_scales[(int64_t)i * h_idx + h] * (double)k_scales[p] * dot;
                } else {
                    for (int32_t c = 0; c < d_idx; ++c) dot += (double)q_rot[qo + c] * (double)k_rot[ko + c];
                    v = dot;
                }
                if (v < 0.0) v = 0.0;
                acc += (double)w[(int64_t)i * h_idx + h] * v;
            }
            *out = (float)acc;
        }
    }
    free(lo);
    free(nv);
}

/* ----------------------------------------------------------------- top-k -- */

typedef struct { float score; int32_t pool; } cand_t;

/* Order: larger score first; equal scores (IEEE equality, so -0 == +0) by
 * lower pool index; a NaN ranks below every number. */
static int cand_cmp(const void* pa, const void* pb) {
    const cand_t* a = (const cand_t*)pa;
    const cand_t* b = (const cand_t*)pb;
    int an = isnan(a->score), bn = isnan(b->score);
    if (an != bn) return an ? 1 : -1;
    if (!an && a->score > b->score) return -1;
    if (!an && a->score < b->score) return 1;
    return (a->pool > b->pool) - (a->pool < b->pool);
}

void kpo_topk(const int32_t* cu, int32_t num_docs, const int32_t* cu_pools, int32_t kpool,
              const int32_t* q_pos, int32_t num_q, int32_t max_pools, const float* scores,
              int32_t topk, int32_t row_width, int32_t* indices, int32_t* num_valid) {
#pragma omp parallel for schedule(dynamic, 1)
    for (int32_t i = 0; i < num_q; ++i) {
        int32_t t = q_pos ? q_pos[i] : i;
        int32_t* row = indices + (int64_t)i * row_width;
        int32_t pool_lo = 0, n_vis = 0, tail_start = 0, pos = 0;
        int32_t d = kpo_query_info(cu, num_docs, cu_pools, kpool, t, &pool_lo, &n_vis, &tail_start);
        if (d >= 0) {
            int32_t k = n_vis < topk ? n_vis : topk;
            cand_t* c = (cand_t*)malloc(sizeof(cand_t) * (size_t)(n_vis + 1));
            unsigned char* keep = (unsigned char*)calloc((size_t)n_vis + 1, 1);
            for (int32_t j = 0; j < n_vis; ++j) {
                c[j].score = scores[(int64_t)i * max_pools + pool_lo + j];
                c[j].pool = j;
            }
            qsort(c, (size_t)n_vis, sizeof(cand_t), cand_cmp);
            for (int32_t r = 0; r < k; ++r) keep[c[r].pool] = 1;
            for (int32_t j = 0; j < n_vis; ++j)
                if (keep[j])
                    for (int32_t r = 0; r < kpool; ++r) row[pos++] = cu[d] + kpool * j + r;
            for (int32_t u = tail_start; u <= t; ++u) row[pos++] = u;
            free(c);
            free(keep);
        }
        if (num_valid) num_valid[i] = pos;
        for (int32_t j = pos; j < row_width; ++j) row[j] = -1;
    }
}

/* ------------------------------------------------------------ sparse MLA -- */

/* Dense attention restricted to the named rows, in float64: the dense SDPA
 * reference path of [P1-AB] with the index row as its mask. Keys are the whole
 * d_qk-wide latent rows; values are their first d_v columns (d_v == d_qk is the
 * NoPE form of [P4-S2]; d_qk = 576, d_v = 512 the RoPE-tail contract of [P2-CL]). */
void kpo_sparse_mla_dv(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int32_t num_q,
                       int32_t num_kv, int32_t heads, int32_t d_qk, int32_t d_v, int32_t row_width,
                       float scale, float* out, float* lse, float* out_abs) {
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int32_t i = 0; i < num_q; ++i) {
        for (int32_t h = 0; h < heads; ++h) {
            const int32_t* row = indices + (int64_t)i * row_width;
            const uint16_t* qh = q + ((int64_t)i * heads + h) * d_qk;
            double* s = (double*)malloc(sizeof(double) * (size_t)row_width + 1);
            double* o = (double*)calloc((size_t)d_v, sizeof(double));
            double* oa = (double*)calloc((size_t)d_v, sizeof(double));
            double m = -INFINITY;
            for (int32_t j = 0; j < row_width; ++j) {
                int32_t r = row[j];
                if (r < 0 || r >= num_kv) { s[j] = -INFINITY; continue; }
                double dot = 0.0;
                for (int32_t c = 0; c < d_qk; ++c)
                    dot += bf16_value(qh[c]) * bf16_value(kv[(int64_t)r * d_qk + c]);
                s[j] = (double)scale * dot;
                if (s[j] > m) m = s[j];
            }
            float* oh = out + ((int64_t)i * heads + h) * d_v;
            float* oah = out_abs ? out_abs + ((int64_t)i * heads + h) * d_v : NULL;
            if (m == -INFINITY) {
                for (int32_t c = 0; c < d_v; ++c) oh[c] = 0.0f;
                if (oah) for (int32_t c = 0; c < d_v; ++c) oah[c] = 0.0f;
                if (lse) lse[(int64_t)i * heads + h] = -INFINITY;
            } else {
                double den = 0.0;
                for (int32_t j = 0; j < row_width; ++j) {
                    int32_t r = row[j];
                    if (r < 0 || r >= num_kv) continue;
                    double p = exp(s[j] - m);
                    den += p;
                    for (int32_t c = 0; c < d_v; ++c) {
                        double v = bf16_value(kv[(int64_t)r * d_qk + c]);
                        o[c] += p * v;
                        oa[c] += p * fabs(v);
                    }
                }
                for (int32_t c = 0; c < d_v; ++c) oh[c] = (float)(o[c] / den);
                if (oah) for (int32_t c = 0; c < d_v; ++c) oah[c] = (float)(oa[c] / den);
                if (lse) lse[(int64_t)i * heads + h] = (float)(m + log(den));
            }
            free(s);
            free(o);
            free(oa);
        }
    }
}

void kpo_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int32_t num_q,
                    int32_t num_kv, int32_t heads, int32_t d_latent, int32_t row_width,
                    float scale, float* out, float* lse, float* out_abs) {
    kpo_sparse_mla_dv(q, kv, indices, num_q, num_kv, heads, d_latent, d_latent, row_width, scale, out, lse,
                      out_abs);
}

/* Gradients of kpo_sparse_mla_dv for a loss whose gradient with respect to the
 * output is d_out (the training path of [P1-AB]: the sparse kernel's backward,
 * with the indexer frozen and its index rows fixed [P4-S3]). For query i, head
 * h and the valid entries j of its row (latent row r_j, key k_j = kv[r_j],
 * value v_j = its first d_v columns):
 *   p_j   = softmax_j(scale <q, k_j>)             (the forward's weights)
 *   dp_j  = <d_out, v_j>,   delta = sum_j p_j dp_j
 *   ds_j  = p_j (dp_j - delta)                    (the softmax's Jacobian)
 *   dq    = scale sum_j ds_j k_j
 *   dkv[r_j] += scale ds_j q  (all d_qk columns: the key)
 *             + p_j d_out     (first d_v columns: the value)
 * Repeated entries contribute once per occurrence; rows of queries with no valid
 * entry contribute nothing and get dq = 0. float64 throughout; each thread
 * accumulates its own copy of dkv, summed in thread order at the end. */
void kpo_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* d_out,
                        int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_qk, int32_t d_v,
                        int32_t row_width, float scale, float* d_q, float* d_kv) {
    int nt = 1;
#ifdef _OPENMP
    nt = omp_get_max_threads();
#endif
    const size_t kvn = (size_t)num_kv * (size_t)d_qk;
    double* part = (double*)calloc((size_t)nt * kvn + 1, sizeof(double));
#pragma omp parallel
    {
        int tid = 0;
#ifdef _OPENMP
        tid = omp_get_thread_num();
#endif
        double* acc = part + (size_t)tid * kvn;
        double* p = (double*)malloc(sizeof(double) * (size_t)row_width + 1);
        double* dp = (double*)malloc(sizeof(double) * (size_t)row_width + 1);
        double* dq = (double*)malloc(sizeof(double) * (size_t)d_qk + 1);
#pragma omp for collapse(2) schedule(dynamic, 1)
        for (int32_t i = 0; i < num_q; ++i) {
            for (int32_t h = 0; h < heads; ++h) {
                const int32_t* row = indices + (int64_t)i * row_width;
                const uint16_t* qh = q + ((int64_t)i * heads + h) * d_qk;
                const uint16_t* gh = d_out + ((int64_t)i * heads + h) * d_v;
                double m = -INFINITY;
                for (int32_t j = 0; j < row_width; ++j) {
                    int32_t r = row[j];
                    if (r < 0 || r >= num_kv) { p[j] = -INFINITY; continue; }
                    double dot = 0.0;
                    for (int32_t c = 0; c < d_qk; ++c)
                        dot += bf16_value(qh[c]) * bf16_value(kv[(int64_t)r * d_qk + c]);
                    p[j] = (double)scale * dot;
                    if (p[j] > m) m = p[j];
                }
                float* dqo = d_q + ((int64_t)i * heads + h) * d_qk;
                if (m == -INFINITY) {
                    for (int32_t c = 0; c < d_qk; ++c) dqo[c] = 0.0f;
                    continue;
                }
                double den = 0.0;
                for (int32_t j = 0; j < row_width; ++j) {
                    int32_t r = row[j];
                    if (r < 0 || r >= num_kv) continue;
                    p[j] = exp(p[j] - m);
                    den += p[j];
                }
                double delta = 0.0;
                for (int32_t j = 0; j < row_width; ++j) {
                    int32_t r = row[j];
                    if (r < 0 || r >= num_kv) continue;
                    p[j] /= den;
                    double d = 0.0;
                    for (int32_t c = 0; c < d_v; ++c)
                        d += bf16_value(gh[c]) * bf16_value(kv[(int64_t)r * d_qk + c]);
                    dp[j] = d;
                    delta += p[j] * d;
                }
                for (int32_t c = 0; c < d_qk; ++c) dq[c] = 0.0;
                for (int32_t j = 0; j < row_width; ++j) {
                    int32_t r = row[j];
                    if (r < 0 || r >= num_kv) continue;
                    double ds = p[j] * (dp[j] - delta);
                    double* ar = acc + (int64_t)r * d_qk;
                    for (int32_t c = 0; c < d_qk; ++c) {
                        dq[c] += ds * bf16_value(kv[(int64_t)r * d_qk + c]);
                        ar[c] += (double)scale * ds * bf16_value(qh[c]);
                    }
                    for (int32_t c = 0; c < d_v; ++c) ar[c] += p[j] * bf16_value(gh[c]);
                }
                for (int32_t c = 0; c < d_qk; ++c) dqo[c] = (float)((double)scale * dq[c]);
            }
        }
        free(p);
        free(dp);
        free(dq);
    }
    for (size_t e = 0; e < kvn; ++e) {
        double sum = 0.0;
        for (int t = 0; t < nt; ++t) sum += part[(size_t)t * kvn + e];
        d_kv[e] = (float)sum;
    }
    free(part);
}

int32_t kpo_num_threads(void) {
#ifdef _OPENMP
    return (int32_t)omp_get_max_threads();
#else
    return 1;
#endif
}
