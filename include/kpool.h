/*
 * kpool.h -- C ABI of the KPool-indexed DeepSeek Sparse Attention forward on
 * AMD Instinct MI355X (gfx950).
 *
 * The forward of one KPool-DSA layer, as the pages describe it:
 *   1. per-document pool layout and k-pool compression of the indexer keys;
 *   2. Hadamard rotation and FP8 (E4M3) scoring of indexer queries against the
 *      complete pools visible to them;
 *   3. top-k pool selection plus the query's own incomplete pool, as index
 *      rows padded to a multiple of 128;
 *   4. absorbed, NoPE sparse latent attention (MLA) over the selected rows of a
 *      shared latent that serves as both key and value.
 *
 * Sources (page titles and sections):
 *   [P4-S3]  prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet
 *            (pools of 4 per document starting at the document's first token;
 *            per-channel softmax(gate + ape)-weighted mean; a query scores the
 *            complete pools ending at or before it, keeps the top 512 and its own
 *            incomplete pool; fp32 butterfly Hadamard of queries and pooled keys
 *            before FP8 scoring; index rows padded to a multiple of 128; the
 *            pool layout is built once per forward).
 *   [P4-S2]  same page, Summary, second bullet (NoPE sparse MLA in absorbed
 *            form: the 512-wide latent is both key and value).
 *   [P4-S5]  same page, Summary, fifth bullet (compile-safe cu_seqlens: a
 *            one-document row must work).
 *   [P2-CL]  NeMo AutoModel PR "add GLM-5.3-Flash training support",
 *            Changelog (packed DSA with document isolation; empty local shards;
 *            K projection absorbed into the query, shared 512-wide latent K/V).
 *   [P2-MLA] same page, "cuDNN sparse MLA parity and performance" (64 query
 *            heads, 512-wide latent, index_topk 2048, index_kpool 4: 2051 raw
 *            slots before alignment).
 *   [P4-PW]  prime-rl PR "GLM-5.3-Flash text model", Patches and workarounds
 *            (serving keeps hybrid KV blocks of index_kpool x 32 tokens, and
 *            the indexer's paged-MQA kernel reads 32-pool pages).
 *
 * Conventions for every entry point:
 *   - Pointers named as device data are device pointers (hipMalloc or torch
 *     CUDA tensors), row-major and contiguous. bf16 data is passed as uint16_t
 *     bit patterns; FP8 data as uint8_t OCP E4M3FN codes.
 *   - Ownership: the caller allocates and frees every buffer, including the
 *     workspace. The library allocates no device memory and keeps no state
 *     between calls beyond a per-device cache of the device check. Inputs and
 *     outputs must not alias. Buffers must stay alive until the stream has
 *     passed the call.
 *   - Asynchrony: work is enqueued on `stream` (0 = the null stream) and the
 *     call returns without synchronising.
 *   - Errors: every argument check runs on the host before anything is
 *     launched; on failure nothing is enqueued and kp_last_error() (per host
 *     thread) describes the cause. KP_ERR_INVALID_ARG: null required pointer,
 *     negative or inconsistent size. KP_ERR_UNSUPPORTED: a shape outside what
 *     this build implements, or a device that is not gfx950. KP_ERR_HIP: a HIP
 *     runtime error while launching. A call with no work (num_tokens == 0 or
 *     num_q == 0: an empty shard, [P2-CL]) returns KP_OK and enqueues nothing.
 *   - Unchecked preconditions (checking them would need a synchronisation):
 *     cu_seqlens[0] == 0, non-decreasing, cu_seqlens[num_docs] == num_tokens;
 *     every q_pos in [0, num_tokens); bf16 inputs finite. kp_check_inputs()
 *     verifies the integer ones on demand.
 *   - Positions and index-row entries are global token indices of the packed
 *     row (rows of the latent).
 *   - Shared layers (IndexShare): a DSA layer that shares its selection with
 *     the previous full layer ("GLM-5 / GLM-5.1 / GLM-5.2 / GLM-5.3 (MoE +
 *     DSA)" page, Key Features: shared layers reuse the previous full layer's
 *     top-k sparse-attention selection) skips kpool_build and
 *     indexer_score_topk and calls sparse_mla_fwd (and sparse_mla_bwd) with
 *     its own q and latent and the index rows the full layer's
 *     indexer_score_topk wrote. Index rows depend only on the indexer inputs
 *     and the layout, never on q or the latent, so they are valid for any
 *     layer over the same packed row.
 */
#ifndef KPOOL_H
#define KPOOL_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KP_OK = 0,
    KP_ERR_INVALID_ARG = 1,
    KP_ERR_UNSUPPORTED = 2,
    KP_ERR_HIP = 3
} kp_status;

/* Text of the last non-OK status returned on this host thread ("" if none). */
const char* kp_last_error(void);

/* ABI version of this header (major * 100 + minor). */
int32_t kp_version(void);

/* Width of an index row: kpool*topk_pools pool slots plus kpool-1 slots of the
 * own incomplete pool, rounded up to a multiple of 128 [P4-S3, P2-MLA]
 * (kpool 4, topk 512 -> 2051 -> 2176). Returns -1 for kpool < 1 or topk < 0. */
int32_t kp_row_width(int32_t kpool, int32_t topk_pools);

/*
 * kpool_build -- pool layout and compressed, rotated, quantised indexer keys
 * [P4-S3].
 *
 * Layout: document d (tokens cu_seqlens[d] .. cu_seqlens[d+1]-1) holds
 * floor(len/kpool) pools; pool j of d covers tokens cu_seqlens[d] + kpool*j
 * ... + kpool-1. Pools are numbered globally in document order:
 *   cu_pools[d+1] = cu_pools[d] + floor(len_d / kpool),   cu_pools[0] = 0,
 *   pool_start[p] = first token of pool p   (p < cu_pools[num_docs]),
 *   pool_start[p] = -1                      (cu_pools[num_docs] <= p < num_tokens/kpool).
 * Keys: for pool p starting at token s and channel c,
 *   kbar[p,c] = sum_i softmax_i(gate[s+i,c] + ape[i,c]) * k_idx[s+i,c],   i < kpool,
 * then x = H_n kbar[p] (orthonormal Walsh-Hadamard, n = d_idx, fp32 butterflies
 * in Sylvester order, stride 1 first, one final multiply by fp32(1/sqrt(n))),
 * then scale = max|x| / 448 (1 if x == 0) and code[c] = e4m3(x[c] / scale),
 * round to nearest even. Rows p >= cu_pools[num_docs] get code 0, scale 0.
 *
 *   cu_seqlens      device int32 [num_docs + 1]
 *   k_idx, gate     device bf16  [num_tokens, d_idx]   indexer keys, pooling gate
 *   ape             device fp32  [kpool, d_idx]        per-position pool bias
 *   d_idx           32, 64 or 128 (Hadamard size)
 *   kpool           1 .. 16
 *   cu_pools        device int32 [num_docs + 1]        (out)
 *   pool_start      device int32 [num_tokens / kpool]  (out)
 *   pooled_k_fp8    device uint8 [num_tokens / kpool, d_idx]  (out)
 *   pooled_k_scale  device fp32  [num_tokens / kpool]  (out)
 *   pooled_k_f32    device fp32  [num_tokens / kpool, d_idx]  (out, NULLABLE):
 *                   kbar before rotation, for inspection
 */
kp_status kpool_build(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                      const uint16_t* k_idx, const uint16_t* gate, const float* ape,
                      int32_t d_idx, int32_t kpool,
                      int32_t* cu_pools, int32_t* pool_start,
                      uint8_t* pooled_k_fp8, float* pooled_k_scale, float* pooled_k_f32,
                      hipStream_t stream);

/*
 * kpool_build_from -- kpool_build for the pools that end at or after token
 * token_lo, for a pooled-key cache that grows with the context (decode): the
 * keys of a complete pool depend only on its own kpool tokens [P4-S3], so the
 * pools whose last token lies before token_lo are the caller's, from an earlier
 * kpool_build or kpool_build_from over the same documents, and are not written.
 * Every other output is written exactly as kpool_build writes it: cu_pools in
 * full, and pool_start, pooled_k_fp8, pooled_k_scale (and pooled_k_f32) of each
 * pool ending at or after token_lo and of each row past cu_pools[num_docs].
 * token_lo = 0 is kpool_build. Arguments as for kpool_build, and
 *   token_lo        0 .. num_tokens (KP_ERR_INVALID_ARG otherwise)
 */
kp_status kpool_build_from(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                           const uint16_t* k_idx, const uint16_t* gate, const float* ape,
                           int32_t d_idx, int32_t kpool, int32_t token_lo,
                           int32_t* cu_pools, int32_t* pool_start,
                           uint8_t* pooled_k_fp8, float* pooled_k_scale, float* pooled_k_f32,
                           hipStream_t stream);

/*
 * indexer_rotate_quant -- the query half of the rotation and FP8 step [P4-S3]:
 * x = H_n q_idx[i,h,:] (as in kpool_build), scale[i,h] = max|x|/448 (1 if x == 0),
 * codes[i,h,c] = e4m3(x[c] / scale[i,h]).
 *
 *   q_idx   device bf16 [num_q, h_idx, d_idx]
 *   codes   device uint8 [num_q, h_idx, d_idx]  (out)
 *   scales  device fp32  [num_q, h_idx]         (out)
 */
kp_status indexer_rotate_quant(const uint16_t* q_idx, int32_t num_q, int32_t h_idx, int32_t d_idx,
                               uint8_t* codes, float* scales, hipStream_t stream);

/*
 * Bytes of workspace indexer_score_topk needs for these sizes: the rotated
 * queries, then either the score rows (num_q x max_pools fp32) or, on the
 * fused path (max_pools >= 32768 and topk_pools <= 8192), 128 KiB of
 * candidate list per query. 0 when num_q <= 0.
 */
size_t kp_indexer_workspace_bytes(int32_t num_q, int32_t max_pools, int32_t h_idx, int32_t d_idx,
                                  int32_t topk_pools);

/*
 * indexer_score_topk -- FP8 indexer scoring and top-k index rows [P4-S3,
 * P2-MLA].
 *
 * For query i at position t = q_pos[i] (t = i when q_pos is NULL) in document
 * d, with l = t - cu_seqlens[d]: the visible pools are the n_vis = (l+1)/kpool
 * complete pools of d ending at or before t, global numbers
 * cu_pools[d] .. cu_pools[d] + n_vis - 1. Each visible pool p scores
 *   I[i,p] = sum_h w_idx[i,h] * ReLU(sq[i,h] * sk[p] * <q8[i,h,:], k8[p,:]>),
 * with q8/sq the rotated FP8 queries (indexer_rotate_quant) and k8/sk the
 * pooled keys of kpool_build. The min(topk_pools, n_vis) visible pools of
 * largest score are kept; equal scores keep the lower pool number. The index
 * row lists the kept pools in ascending order, each as its kpool tokens, then
 * the tokens cu_seqlens[d] + kpool*n_vis .. t (the own incomplete pool, 0 to
 * kpool-1 tokens; none when t closes a pool), then -1 up to row_width.
 *
 *   cu_seqlens      device int32 [num_docs + 1]
 *   cu_pools        device int32 [num_docs + 1]   (from kpool_build)
 *   max_pools       num_tokens / kpool (row stride of `scores`)
 *   pooled_k_fp8    device uint8 [max_pools, d_idx]; pooled_k_scale fp32 [max_pools]
 *   q_pos           device int32 [num_q] (NULLABLE: then num_q == num_tokens, q_pos[i] = i)
 *   q_idx           device bf16 [num_q, h_idx, d_idx], not rotated
 *   w_idx           device fp32 [num_q, h_idx]   per-head weights (any sign)
 *   h_idx           1 .. 64; d_idx 32, 64 or 128; kpool as in kpool_build
 *   topk_pools      >= 0; row_width a multiple of 128, >= kpool*topk_pools + kpool - 1
 *   indices         device int32 [num_q, row_width]  (out)
 *   num_valid       device int32 [num_q]             (out, NULLABLE) entries before the -1 padding
 *   scores          device fp32 [num_q, max_pools]   (out, NULLABLE) I[i,p] for visible
 *                   pools, -inf elsewhere
 *   workspace       device memory of kp_indexer_workspace_bytes(...) bytes, 256-byte aligned
 *
 * Rows of many pools (decode over a long context): when scores == NULL,
 * max_pools >= 32768 and topk_pools <= 8192, no score tensor is formed. Per
 * query, a threshold is taken from the scores of every s-th pool (s >= 256);
 * the scoring pass keeps only the (score, pool) pairs at or above it, at most
 * 16384 per query, and the top-k is selected among them. The kept pools are
 * the first k in the order "higher score first, then lower pool first", so
 * whenever between k and 16384 pools clear the threshold they are all among
 * the candidates; a row where that fails (adversarial score patterns only) is
 * selected exactly by rescoring its pools. Either way the index rows are the
 * ones the score-tensor path writes.
 */
kp_status indexer_score_topk(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                             const int32_t* cu_pools, int32_t max_pools,
                             const uint8_t* pooled_k_fp8, const float* pooled_k_scale,
                             const int32_t* q_pos, int32_t num_q,
                             const uint16_t* q_idx, const float* w_idx,
                             int32_t h_idx, int32_t d_idx, int32_t kpool,
                             int32_t topk_pools, int32_t row_width,
                             int32_t* indices, int32_t* num_valid, float* scores,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_score_topk_noalloc -- indexer_score_topk for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc): the same arguments without the workspace,
 * and the same outputs, bit for bit. Its workspace is a device buffer the
 * library holds, KP_NOALLOC_SCRATCH_BYTES on each GPU it runs on, from the
 * library's load until the process ends; the call itself allocates nothing.
 * Sizes whose workspace (kp_indexer_workspace_bytes) exceeds that return
 * KP_ERR_UNSUPPORTED before anything is launched: the 64 decode queries of a
 * 1,048,576-token context fit (8.3 MiB on the fused path). Every call on one GPU shares that
 * GPU's buffer, which keeps the last call's contents (no byte of it needs to
 * start at zero): calls that overlap on one GPU (on different streams, or
 * from different host threads) race and give undefined results; calls in one
 * stream are ordered and safe.
 */
#define KP_NOALLOC_SCRATCH_BYTES (72u << 20)
kp_status indexer_score_topk_noalloc(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                     const int32_t* cu_pools, int32_t max_pools,
                                     const uint8_t* pooled_k_fp8, const float* pooled_k_scale,
                                     const int32_t* q_pos, int32_t num_q,
                                     const uint16_t* q_idx, const float* w_idx,
                                     int32_t h_idx, int32_t d_idx, int32_t kpool,
                                     int32_t topk_pools, int32_t row_width,
                                     int32_t* indices, int32_t* num_valid, float* scores,
                                     hipStream_t stream);

/*
 * Paged pooled-key cache [P4-PW]: physical pages of 32 * kpool token slots
 * that also hold the 32 pools those tokens form (kpool 4: 128 tokens and 32
 * pools per page). Document d (tokens cu_seqlens[d] .. cu_seqlens[d+1]-1, its
 * length len_d) owns the pages page_table[d * max_pages + q], q = 0 ..
 * max_pages - 1: its token l lives in slot page_table[d*max_pages + l / (32
 * kpool)] * 32 kpool + l % (32 kpool) of every token-row array, and its pool j
 * (tokens kpool*j .. kpool*j + kpool - 1, as in kpool_build) in row
 * page_table[d*max_pages + j / 32] * 32 + j % 32 of every pool-row array. The
 * packed numbering of cu_seqlens only describes lengths and query positions;
 * nothing is stored in it. Pages need not be contiguous, in order, or
 * distinct between documents' unused tail entries. A page-table entry outside
 * [0, num_pages), or a token or pool past a document's max_pages pages, is a
 * missing page: nothing there is read or written, and index-row entries that
 * fall in it are -1.
 */

/*
 * kpool_update_paged -- (re)compute the pooled keys of each document's pools
 * whose last token is among its last `last_tokens` tokens [P4-S3, P4-PW]:
 * decode appends tokens to the cache (their k_idx and gate rows written into
 * their slots by the caller) and calls this with last_tokens = the number of
 * tokens appended per document (the largest, when documents grew by
 * different amounts: recomputing a pool rewrites the same bytes). Keys as in
 * kpool_build, bit for bit.
 *
 *   page_table      device int32 [num_docs, max_pages]
 *   num_pages       physical pages in the cache; num_pages * 32 * kpool < 2^31
 *   k_idx_pages, gate_pages  device bf16 [num_pages * 32 * kpool, d_idx] (token rows)
 *   ape             device fp32 [kpool, d_idx]
 *   k8_pages        device uint8 [num_pages * 32, d_idx]   (out, pool rows)
 *   sk_pages        device fp32  [num_pages * 32]          (out, pool rows)
 *   last_tokens     >= 0 (0: nothing to do)
 */
kp_status kpool_update_paged(const int32_t* cu_seqlens, int32_t num_docs,
                             const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                             const uint16_t* k_idx_pages, const uint16_t* gate_pages, const float* ape,
                             int32_t d_idx, int32_t kpool, int32_t last_tokens,
                             uint8_t* k8_pages, float* sk_pages, hipStream_t stream);

/* Bytes of workspace indexer_score_topk_paged needs for these sizes. */
size_t kp_indexer_paged_workspace_bytes(int32_t num_q, int32_t num_docs, int32_t h_idx, int32_t d_idx);

/*
 * indexer_score_topk_paged -- indexer_score_topk over a paged pooled-key cache
 * [P4-S3, P4-PW], always on the fused path (no score tensor; topk_pools <=
 * 8192). The selection is the one indexer_score_topk makes over the same keys
 * in packed order; the index row entries are the page slots of the kept
 * tokens (and of the query's own incomplete pool), so sparse_mla_fwd runs on a
 * latent in the same pages (kv of num_pages * 32 * kpool rows).
 *
 *   num_tokens      cu_seqlens[num_docs]
 *   k8_pages, sk_pages  as written by kpool_update_paged
 *   row_path        device int32 [num_q] (out, NULLABLE): 0 when the row was
 *                   selected among its candidates, 1 when it was rescored
 *   workspace       kp_indexer_paged_workspace_bytes(num_q, num_docs, h_idx, d_idx)
 *                   bytes, 256-byte aligned
 *   (other arguments as in indexer_score_topk)
 */
kp_status indexer_score_topk_paged(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                   const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                                   const uint8_t* k8_pages, const float* sk_pages,
                                   const int32_t* q_pos, int32_t num_q,
                                   const uint16_t* q_idx, const float* w_idx,
                                   int32_t h_idx, int32_t d_idx, int32_t kpool,
                                   int32_t topk_pools, int32_t row_width,
                                   int32_t* indices, int32_t* num_valid, int32_t* row_path,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * indexer_topk_from_scores -- the selection step alone, on a given score
 * tensor [P4-S3]: the same index rows indexer_score_topk builds, with
 * scores[i, p] read for the visible pools only (other entries are ignored).
 * Ranking uses IEEE order with -0 == +0; a NaN ranks below every number.
 * Bit-exact by construction; no workspace.
 *
 *   scores   device fp32 [num_q, max_pools]
 *   (other arguments as in indexer_score_topk)
 */
kp_status indexer_topk_from_scores(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                   const int32_t* cu_pools, int32_t max_pools,
                                   const int32_t* q_pos, int32_t num_q, const float* scores,
                                   int32_t kpool, int32_t topk_pools, int32_t row_width,
                                   int32_t* indices, int32_t* num_valid, hipStream_t stream);

/*
 * sparse_mla_fwd -- absorbed NoPE sparse latent attention [P4-S2, P2-CL,
 * P2-MLA]. For query i, head h and the valid entries j of row i
 * (0 <= indices[i,j] < num_kv; every other entry is masked, wherever it sits):
 *   s_j      = softmax_scale * <q[i,h,:], kv[indices[i,j],:]>
 *   out[i,h] = sum_j softmax(s)_j * kv[indices[i,j], :d_v]  (K = V = the latent)
 *   lse[i,h] = log(sum_j exp(s_j))                          (natural log)
 * with d_v = d_latent, except d_latent = 576: keys 576 wide (512 + a 64-wide
 * RoPE tail), values their first 512 columns, d_v = 512 -- the GLM-5.2 contract
 * the NeMo PR keeps (Changelog: D=576, top-k at most 2048); GLM-5.3-Flash itself
 * has no tail (d_latent 512 [P4-S2]).
 * bf16 inputs, fp32 accumulation, bf16 output (round to nearest even). A row
 * with no valid entry gives out = 0 and lse = -inf. Repeated entries count
 * repeatedly.
 *
 *   q        device bf16 [num_q, heads, d_latent]   (the K projection already absorbed)
 *   kv       device bf16 [num_kv, d_latent]
 *   indices  device int32 [num_q, row_width]
 *   heads    1 .. 64;  d_latent 64, 512 or 576;  row_width 1 .. 4096 (1 .. 2048
 *            for d_latent 576); num_kv * d_latent * 2 < 4 GiB - 4 KiB;
 *            softmax_scale finite and > 0
 *   out      device bf16 [num_q, heads, d_v]        (out)
 *   lse      device fp32 [num_q, heads]             (out, NULLABLE)
 *   workspace  device memory of kp_mla_fwd_workspace_bytes(num_q, heads,
 *            d_latent, row_width) bytes, 256-byte aligned (NULLABLE). Launches
 *            of fewer than 128 queries (decode) then split each index row into
 *            up to 16 ranges of 64-row tiles, one workgroup each, whose
 *            normalised fp32 partial outputs and lse are merged by a second
 *            kernel: out = sum over ranges of exp(lse_r - lse) out_r, rounded to
 *            bf16 once. Without a workspace (or when that size is 0) each query
 *            is one workgroup. The two agree to the bf16 rounding of out.
 */
size_t kp_mla_fwd_workspace_bytes(int32_t num_q, int32_t heads, int32_t d_latent, int32_t row_width);
kp_status sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                         int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_latent,
                         int32_t row_width, float softmax_scale,
                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* Bytes of workspace sparse_mla_bwd needs for these sizes (0 when num_q <= 0,
 * row_width < 1 or d_latent is not 64 or 512). */
size_t kp_mla_bwd_workspace_bytes(int32_t num_q, int32_t d_latent, int32_t row_width);

/*
 * sparse_mla_bwd -- backward of sparse_mla_fwd: the gradients of a loss with
 * respect to q and kv, given its gradient d_out with respect to the output
 * [P1-AB: the training path runs a sparse backward; P2-MLA: its dQ and dKV are
 * validated against a dense reference]. The index rows are constants (the
 * indexer is frozen [P4-S3]). For query i, head h and the valid entries j of
 * row i (latent row r_j, as in sparse_mla_fwd), with p_j = exp(s_j - lse[i,h]):
 *   dp_j = <d_out[i,h], kv[r_j]>,  delta = <d_out[i,h], out[i,h]>,
 *   ds_j = p_j (dp_j - delta),
 *   d_q[i,h]   = softmax_scale * sum_j ds_j kv[r_j]
 *   d_kv[r_j] += softmax_scale * ds_j q[i,h] + p_j d_out[i,h]   (key and value)
 * summed over every query, head and valid entry (repeats count each time).
 * bf16 inputs, fp32 accumulation; p and ds enter the products rounded to bf16,
 * and so does each (query, entry) term of d_kv before the sum over queries.
 * d_kv is written in full; its sum over queries runs in a fixed order (queries
 * in chunks of 8192, within a chunk by position in the index rows), so d_q and
 * d_kv are bit-reproducible. A row with no valid entry gives d_q = 0.
 *
 *   q, kv, indices  as passed to sparse_mla_fwd
 *   out, lse        the outputs of that sparse_mla_fwd call (lse required)
 *   d_out           device bf16 [num_q, heads, d_latent]
 *   heads           1 .. 64;  d_latent 64 or 512;  row_width 1 .. 4096
 *   d_q             device bf16 [num_q, heads, d_latent]   (out)
 *   d_kv            device fp32 [num_kv, d_latent]         (out)
 *   workspace       device memory of kp_mla_bwd_workspace_bytes(num_q, d_latent,
 *                   row_width) bytes, 256-byte aligned: per chunk of up to 8192
 *                   queries, the per-slot softmax coefficients, the per-slot
 *                   d_kv terms (bf16), the sort of the slots by row and the
 *                   reduction's carries (about 23.7 GB at 8192 x 2176 x 512)
 */
kp_status sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                         const uint16_t* out, const float* lse, const uint16_t* d_out,
                         int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_latent,
                         int32_t row_width, float softmax_scale,
                         uint16_t* d_q, float* d_kv, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/*
 * kp_check_inputs -- debug helper: verifies on the device that cu_seqlens is
 * well formed (starts at 0, non-decreasing, ends at num_tokens) and that
 * every q_pos lies in [0, num_tokens). Synchronises `stream`. Returns KP_OK or
 * KP_ERR_INVALID_ARG with the first violation in kp_last_error().
 */
kp_status kp_check_inputs(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                          const int32_t* q_pos, int32_t num_q, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KPOOL_H */
