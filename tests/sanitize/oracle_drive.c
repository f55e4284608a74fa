/* Drives every function of the CPU oracle through small inputs and their edge
 * cases (empty and short documents, a malformed layout, special E4M3 values,
 * zero vectors, ties and NaN scores, top-k 0, masked and empty index rows,
 * 576-wide keys with 512-wide values, the backward), so that a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer sees every code path. Prints
 * "oracle drive ok" and returns 0 when every sanity check holds; the sanitizers
 * abort the run on the first error they find. Test infrastructure only. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "kpool_oracle.h"

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static double urand(void) {   /* splitmix64, uniform in [0, 1) */
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    return (double)(z >> 11) * (1.0 / 9007199254740992.0);
}
static uint16_t bf16(float f) {   /* truncation is enough for driving inputs */
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}
static void fill_bf16(uint16_t* x, size_t n, float scale) {
    for (size_t i = 0; i < n; ++i) x[i] = bf16((float)((urand() * 2.0 - 1.0) * scale));
}
static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}
#define CHECK(c)                                                          \
    do {                                                                  \
        if (!(c)) { fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); return 1; } \
    } while (0)

static int drive_layout_and_encode(void) {
    /* documents of 10, 0, 3, 17 and 1 tokens: empty and sub-pool documents */
    const int32_t cu[6] = {0, 10, 10, 13, 30, 31};
    int32_t cu_pools[6], pool_start[8];
    const int32_t P = kpo_layout(cu, 5, 31, 4, cu_pools, pool_start);
    CHECK(P == 2 + 0 + 0 + 4 + 0);
    CHECK(cu_pools[5] == P);
    for (int t = 0; t < 31; ++t) {
        int32_t lo, nv, ts;
        CHECK(kpo_query_info(cu, 5, cu_pools, 4, t, &lo, &nv, &ts) >= 0);
        CHECK(nv >= 0 && ts <= t + 1);
    }
    const int32_t bad[3] = {0, 8, 4};   /* descending: malformed */
    CHECK(kpo_layout(bad, 2, 8, 4, cu_pools, pool_start) == -1);
    CHECK(kpo_layout(cu, 5, 31, 0, cu_pools, pool_start) == -1);

    /* E4M3 on special values, and a round trip over every code */
    const float specials[] = {0.0f, -0.0f, 448.0f, 449.0f, 1e9f, -1e9f, INFINITY, -INFINITY, NAN, 1e-10f,
                              -1e-10f, 0.001953125f, 240.0f};
    for (size_t i = 0; i < sizeof specials / sizeof specials[0]; ++i)
        (void)kpo_e4m3_decode(kpo_e4m3_encode(specials[i]));
    for (int c = 0; c < 256; ++c) {
        const float v = kpo_e4m3_decode((uint8_t)c);
        if (isfinite(v)) CHECK(kpo_e4m3_decode(kpo_e4m3_encode(v)) == v);
    }
    /* FWHT sizes, a zero row and a random row through the quantiser */
    for (int n = 1; n <= 128; n *= 2) {
        float x[128];
        for (int i = 0; i < n; ++i) x[i] = (float)(urand() - 0.5);
        kpo_fwht(x, n);
    }
    float rows[2 * 32];
    memset(rows, 0, sizeof rows);
    for (int i = 32; i < 64; ++i) rows[i] = (float)(urand() * 4.0 - 2.0);
    uint8_t codes[64];
    float scales[2];
    kpo_quant_rows(rows, 2, 32, codes, scales);
    CHECK(scales[0] == 1.0f && scales[1] > 0.0f);
    return 0;
}

static int drive_indexer(void) {
    const int T = 40, B = 3, D = 32, H = 2, KP = 4;
    const int32_t cu[4] = {0, 7, 7, 40};
    int32_t cu_pools[4], pool_start[10];
    const int32_t P = kpo_layout(cu, B, T, KP, cu_pools, pool_start);
    CHECK(P == 1 + 0 + 8);
    uint16_t* k_idx = xmalloc(sizeof(uint16_t) * T * D);
    uint16_t* gate = xmalloc(sizeof(uint16_t) * T * D);
    uint16_t* q_idx = xmalloc(sizeof(uint16_t) * T * H * D);
    float ape[4 * 32], w[40 * 2];
    fill_bf16(k_idx, (size_t)T * D, 2.0f);
    fill_bf16(gate, (size_t)T * D, 1.0f);
    fill_bf16(q_idx, (size_t)T * H * D, 2.0f);
    for (int i = 0; i < KP * D; ++i) ape[i] = (float)(urand() - 0.5);
    for (int i = 0; i < T * H; ++i) w[i] = (float)(urand() - 0.3);
    uint8_t* k8 = xmalloc((size_t)P * D);
    float* ks = xmalloc(sizeof(float) * P);
    float* kf = xmalloc(sizeof(float) * P * D);
    kpo_keys(k_idx, gate, ape, pool_start, P, D, KP, k8, ks, kf);
    kpo_keys(k_idx, gate, ape, pool_start, P, D, KP, k8, ks, NULL);
    uint8_t* q8 = xmalloc((size_t)T * H * D);
    float* qs = xmalloc(sizeof(float) * T * H);
    kpo_queries(q_idx, T, H, D, q8, qs);
    /* the unquantised operands for the debug mode */
    float* q_rot = xmalloc(sizeof(float) * T * H * D);
    for (int i = 0; i < T * H; ++i)
        for (int c = 0; c < D; ++c) q_rot[i * D + c] = kpo_e4m3_decode(q8[i * D + c]) * qs[i];
    float* scores = xmalloc(sizeof(float) * T * P);
    for (int mode = 0; mode < 2; ++mode)
        kpo_scores(cu, B, cu_pools, KP, NULL, T, P, q8, qs, k8, ks, q_rot, kf, mode, w, H, D, scores);
    /* ties, a NaN and -0 in the scores of the last query */
    scores[(size_t)(T - 1) * P + cu_pools[2]] = NAN;
    scores[(size_t)(T - 1) * P + cu_pools[2] + 1] = -0.0f;
    scores[(size_t)(T - 1) * P + cu_pools[2] + 2] = 0.0f;
    const int W = 128;
    int32_t* idx = xmalloc(sizeof(int32_t) * T * W);
    int32_t* nv = xmalloc(sizeof(int32_t) * T);
    for (int topk = 0; topk <= 9; topk += 3) {
        kpo_topk(cu, B, cu_pools, KP, NULL, T, P, scores, topk, W, idx, nv);
        for (int t = 0; t < T; ++t) CHECK(nv[t] >= 0 && nv[t] <= W);
    }
    /* a subset of queries through q_pos */
    const int32_t q_pos[3] = {0, 6, 39};
    kpo_scores(cu, B, cu_pools, KP, q_pos, 3, P, q8, qs, k8, ks, NULL, NULL, 0, w, H, D, scores);
    kpo_topk(cu, B, cu_pools, KP, q_pos, 3, P, scores, 2, W, idx, nv);
    free(k_idx); free(gate); free(q_idx); free(k8); free(ks); free(kf); free(q8); free(qs); free(q_rot);
    free(scores); free(idx); free(nv);
    return 0;
}

static int drive_attention(void) {
    const int NQ = 5, NKV = 24, H = 3, W = 12;
    for (int pass = 0; pass < 2; ++pass) {
        const int DQK = pass ? 576 : 64, DV = pass ? 512 : 64;
        uint16_t* q = xmalloc(sizeof(uint16_t) * NQ * H * DQK);
        uint16_t* kv = xmalloc(sizeof(uint16_t) * NKV * DQK);
        uint16_t* d_out = xmalloc(sizeof(uint16_t) * NQ * H * DV);
        fill_bf16(q, (size_t)NQ * H * DQK, 1.0f);
        fill_bf16(kv, (size_t)NKV * DQK, 1.0f);
        fill_bf16(d_out, (size_t)NQ * H * DV, 1.0f);
        int32_t idx[5 * 12];
        for (int i = 0; i < NQ; ++i)
            for (int j = 0; j < W; ++j) idx[i * W + j] = (int32_t)(urand() * (NKV + 6)) - 3;   /* some masked */
        for (int j = 0; j < W; ++j) idx[2 * W + j] = -1;                                     /* an empty row */
        idx[3 * W + 0] = NKV;                                                                 /* past the end */
        float* out = xmalloc(sizeof(float) * NQ * H * DV);
        float* oabs = xmalloc(sizeof(float) * NQ * H * DV);
        float lse[5 * 3];
        const float scale = 1.0f / sqrtf((float)DQK);
        if (DQK == DV) {
            kpo_sparse_mla(q, kv, idx, NQ, NKV, H, DQK, W, scale, out, lse, oabs);
            kpo_sparse_mla(q, kv, idx, NQ, NKV, H, DQK, W, scale, out, lse, NULL);
        }
        kpo_sparse_mla_dv(q, kv, idx, NQ, NKV, H, DQK, DV, W, scale, out, lse, oabs);
        for (int h = 0; h < H; ++h) CHECK(isinf(lse[2 * H + h]) && lse[2 * H + h] < 0);   /* empty row */
        for (int e = 0; e < H * DV; ++e) CHECK(out[2 * H * DV + e] == 0.0f);
        float* d_q = xmalloc(sizeof(float) * NQ * H * DQK);
        float* d_kv = xmalloc(sizeof(float) * NKV * DQK);
        kpo_sparse_mla_bwd(q, kv, idx, d_out, NQ, NKV, H, DQK, DV, W, scale, d_q, d_kv);
        for (int e = 0; e < NKV * DQK; ++e) CHECK(isfinite(d_kv[e]));
        free(q); free(kv); free(d_out); free(out); free(oabs); free(d_q); free(d_kv);
    }
    return 0;
}

int main(void) {
    if (drive_layout_and_encode() || drive_indexer() || drive_attention()) return 1;
    printf("oracle drive ok (threads %d)\n", (int)kpo_num_threads());
    return 0;
}
