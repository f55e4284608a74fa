/*
 * CPU oracle of the KPool-indexed DeepSeek Sparse Attention forward.
 *
 * TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this library. It shares no code, header
 * or constant with the HIP library, and nothing in the product path calls it.
 *
 * Plain, slow, obviously correct loops. Floating point is float64 wherever the
 * pages fix no precision; the Hadamard rotation is float32 (the pages say the
 * butterfly runs in fp32) and the indexer operands are OCP FP8 E4M3FN.
 *
 * Sources (the pages, by title and section):
 *   [P4-S3] prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet:
 *           pools of 4 per document from the document's first token; per-channel
 *           softmax(gate + ape)-weighted mean; a query scores the complete pools
 *           ending at or before it, keeps the top 512 and attends to its own
 *           incomplete pool; fp32 butterfly Hadamard of queries and pooled keys
 *           before FP8 scoring; index rows padded to a multiple of 128.
 *   [P4-S2] same page, Summary, second bullet: NoPE sparse MLA in absorbed
 *           form, the 512-wide latent is both key and value.
 *   [P2-CL] NeMo AutoModel PR "add GLM-5.3-Flash training support", Changelog:
 *           K projection absorbed into the query, shared 512-wide latent K/V;
 *           packed DSA with document isolation.
 *   [P2-MLA] same page, "cuDNN sparse MLA parity and performance": 64 heads,
 *           512 latent, index_topk 2048, index_kpool 4 -> 2051 raw slots.
 *   [P1-AB] NeMo AutoModel "GLM-5.3-Flash" page, Attention Backends: a dense
 *           SDPA path serves as the numerical reference.
 *
 * Conventions: bf16 tensors are uint16 bit patterns; row-major; cu_seqlens has
 * num_docs+1 entries; positions are global token indices of the packed row.
 */
#ifndef KPOOL_ORACLE_H
#define KPOOL_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Pool layout [P4-S3]. Writes cu_pools[num_docs+1] and pool_start[P]; returns
 * P, or -1 when cu_seqlens is malformed or kpool < 1. */
int32_t kpo_layout(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens, int32_t kpool,
                   int32_t* cu_pools, int32_t* pool_start);

/* Per-query quantities [P4-S3]: first pool of the document, number of complete
 * pools ending at or before t, first token of the incomplete own pool. */
int32_t kpo_query_info(const int32_t* cu_seqlens, int32_t num_docs, const int32_t* cu_pools,
                       int32_t kpool, int32_t t, int32_t* pool_lo, int32_t* n_vis,
                       int32_t* tail_start);

/* K-pool compression [P4-S3]: out[p, c] = sum_i softmax_i(gate[s+i,c] + ape[i,c]) k[s+i,c]. */
void kpo_pool(const uint16_t* k_idx, const uint16_t* gate, const float* ape,
              const int32_t* pool_start, int32_t num_pools, int32_t d_idx, int32_t kpool,
              float* out);

/* In-place orthonormal fast Walsh-Hadamard transform in fp32 [P4-S3]. */
void kpo_fwht(float* x, int32_t n);

/* OCP FP8 E4M3FN: round to nearest even, saturate to +-448, NaN -> 0x7F. */
uint8_t kpo_e4m3_encode(float v);
float kpo_e4m3_decode(uint8_t code);

/* Per-vector quantisation: s = amax/448 (1 if amax == 0); code = e4m3(x/s). */
void kpo_quant_rows(const float* x, int64_t rows, int32_t n, uint8_t* codes, float* scales);

/* Keys: pool, rotate, quantise. pooled_f32 may be NULL. */
void kpo_keys(const uint16_t* k_idx, const uint16_t* gate, const float* ape,
              const int32_t* pool_start, int32_t num_pools, int32_t d_idx, int32_t kpool,
              uint8_t* codes, float* scales, float* pooled_f32);

/* Queries: bf16 [num_q, h_idx, d_idx] -> rotate -> quantise. */
void kpo_queries(const uint16_t* q_idx, int32_t num_q, int32_t h_idx, int32_t d_idx,
                 uint8_t* codes, float* scales);

/* Indexer scores [num_q, max_pools], -inf where not visible [P4-S3]:
 *   I[t,p] = sum_h w[t,h] * max(0, sq[t,h] * sk[p] * <dec(q8[t,h]), dec(k8[p])>).
 * mode 0: FP8 operands. mode 1: unquantised rotated fp32 operands (debug pin). */
void kpo_scores(const int32_t* cu_seqlens, int32_t num_docs, const int32_t* cu_pools, int32_t kpool,
                const int32_t* q_pos, int32_t num_q, int32_t max_pools,
                const uint8_t* q_codes, const float* q_scales,
                const uint8_t* k_codes, const float* k_scales,
                const float* q_rot, const float* k_rot, int32_t mode,
                const float* w, int32_t h_idx, int32_t d_idx, float* scores);

/* Top-k pools and index rows [P4-S3, P2-MLA]: the min(topk, n_vis) visible
 * pools with the largest score (ties: lower pool index first), in ascending
 * order, each expanded to its kpool tokens, then the own tail tokens, then -1
 * up to row_width. */
void kpo_topk(const int32_t* cu_seqlens, int32_t num_docs, const int32_t* cu_pools, int32_t kpool,
              const int32_t* q_pos, int32_t num_q, int32_t max_pools, const float* scores,
              int32_t topk, int32_t row_width, int32_t* indices, int32_t* num_valid);

/* Sparse MLA forward [P4-S2, P2-CL, P1-AB], as dense attention of each query
 * over the rows its index row names (K = V = latent):
 *   o[t,h,:] = softmax_j(scale <q[t,h], kv[idx_j]>) . kv[idx_j],  lse natural log.
 * Entries outside [0, num_kv) are masked; an empty row gives o = 0, lse = -inf.
 * out_abs (NULLABLE) receives sum_j softmax_j |kv[idx_j]|, the magnitude of
 * the terms each output element sums (the scale of its rounding error). */
void kpo_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int32_t num_q,
                    int32_t num_kv, int32_t heads, int32_t d_latent, int32_t row_width,
                    float scale, float* out, float* lse, float* out_abs);

/* The same with values narrower than keys: keys are the d_qk-wide latent rows,
 * values their first d_v columns, out [num_q, heads, d_v] ([P2-CL]: the GLM-5.2
 * contract, d_qk = 576 with a RoPE tail, d_v = 512). */
void kpo_sparse_mla_dv(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int32_t num_q,
                       int32_t num_kv, int32_t heads, int32_t d_qk, int32_t d_v, int32_t row_width,
                       float scale, float* out, float* lse, float* out_abs);

/* Backward of kpo_sparse_mla_dv [P1-AB, P4-S3]: given d_out [num_q, heads, d_v],
 * writes d_q [num_q, heads, d_qk] and d_kv [num_kv, d_qk] (fp32; computed in
 * float64). The key and the value are the same latent rows, so d_kv holds both
 * contributions. */
void kpo_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* d_out,
                        int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_qk, int32_t d_v,
                        int32_t row_width, float scale, float* d_q, float* d_kv);

/* Threads the OpenMP runtime will use (for reporting). */
int32_t kpo_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
