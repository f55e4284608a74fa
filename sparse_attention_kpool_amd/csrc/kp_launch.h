// Host-side launchers of the gfx950 kernels (internal to libkpool; the C ABI
// in api.cpp validates arguments before calling any of these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kp {

// Pool layout (cu_pools, pool_start) and rotated FP8 pooled keys.
hipError_t launch_layout_pool(const int32_t* cu, int num_docs, int num_tokens, const uint16_t* k_idx,
                              const uint16_t* gate, const float* ape, int d_idx, int kpool,
                              float norm, int32_t* cu_pools, int32_t* pool_start, uint8_t* k8,
                              float* ks, float* kf32, int token_lo, hipStream_t stream);

// Pool layout alone (cu_pools from the document lengths).
hipError_t launch_layout(const int32_t* cu, int num_docs, int kpool, int32_t* cu_pools, hipStream_t stream);

// Rotated FP8 pooled keys of the pools whose last token is among each
// document's last `last_tokens` tokens, in a paged cache (token rows in pages of
// 32*kpool slots, pool rows in pages of 32, both through the page table).
hipError_t launch_pool_paged(const int32_t* cu, int num_docs, const int32_t* table, int max_pages, int num_pages,
                             const uint16_t* k_idx, const uint16_t* gate, const float* ape, int d_idx, int kpool,
                             float norm, uint8_t* k8, float* ks, int last_tokens, hipStream_t stream);

// Rotated FP8 indexer queries: rows = num_q * h_idx vectors of d_idx channels.
hipError_t launch_rotate_quant(const uint16_t* q_idx, long long rows, int d_idx, float norm,
                               uint8_t* codes, float* scales, hipStream_t stream);

// Fill a float buffer with a constant.
hipError_t launch_fill_f32(float* dst, size_t n, float value, hipStream_t stream);

// FP8 indexer scores of the visible (query, pool) pairs; other entries untouched.
hipError_t launch_score(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                        const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                        const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                        int max_pools, float* scores, hipStream_t stream);

// Scoring that appends (key, pool) candidates at or above a per-query
// threshold instead of storing scores (page_table == nullptr: key row = pool).
hipError_t launch_score_emit(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                             const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                             const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                             int max_pools, const int32_t* page_table, int max_pages, int num_pages,
                             const uint32_t* tau, int32_t* count, uint2* cand, int cap, hipStream_t stream);

// Candidates kept per query by the fused scoring + top-k, and sampled pools at most.
constexpr int FT_CAP = 16384;
constexpr int FT_SAMPLE_MAX = 16384;

// Workspace of the fused scoring + top-k (fused_state_bytes bytes, 256-byte
// aligned): per query the threshold, the candidate count and the candidate list.
struct FusedState {
    uint32_t* tau;     // [num_q][2]
    int32_t* count;    // [num_q]
    uint2* cand;       // [num_q][FT_CAP]
};
size_t fused_state_bytes(int num_q);
FusedState fused_state_at(void* ws, int num_q);

// Fused scoring + top-k (no score tensor): threshold, emission, selection.
// topk <= FT_CAP / 2. With a page table, index rows hold page slots.
hipError_t launch_fused_topk(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                             const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq, const float* w,
                             int h_idx, int d_idx, const uint8_t* k8, const float* sk, int max_pools,
                             const int32_t* page_table, int max_pages, int num_pages, int topk, int row_width,
                             int32_t* indices, int32_t* num_valid, int32_t* row_path, const FusedState& st,
                             hipStream_t stream);

// Top-k index rows from a score tensor (visible entries only are read).
hipError_t launch_topk(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                       const int32_t* q_pos, int num_q, const float* scores, int max_pools,
                       int topk, int row_width, int32_t* indices, int32_t* num_valid,
                       hipStream_t stream);

// Sparse latent attention over the index rows.
// With `part` (sparse_mla_part_bytes bytes), rows of few-query launches are
// split over several workgroups and merged by a second kernel.
hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int num_q,
                             int num_kv, int heads, int d_latent, int row_width, float scale_log2,
                             uint16_t* out, float* lse, void* part, hipStream_t stream);
int sparse_mla_splits(int num_q, int row_width);
size_t sparse_mla_part_bytes(int num_q, int heads, int d_latent, int row_width);

// Largest index row sparse_mla_fwd accepts for this key width.
int sparse_mla_max_row_width(int d_latent);

// Backward of the sparse latent attention: dq (bf16) and dkv (fp32, written in
// full, bit-reproducible); workspace of sparse_mla_bwd_ws_bytes bytes.
hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* out,
                                 const float* lse, const uint16_t* d_out, int num_q, int num_kv, int heads,
                                 int d_latent, int row_width, float scale, uint16_t* d_q, float* d_kv,
                                 void* workspace, hipStream_t stream);
size_t sparse_mla_bwd_ws_bytes(int num_q, int d_latent, int row_width);

}  // namespace kp
