// C ABI of libkpool (declared in include/kpool.h): host-side argument checks,
// the gfx950 device check, workspace carving, and kernel launches.
#include "kpool.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kp_launch.h"

namespace {

thread_local std::string g_err;

kp_status fail(kp_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

kp_status ok() { return KP_OK; }

kp_status hip_fail(hipError_t e, const char* where) {
    return fail(KP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
std::mutex g_dev_mu;
int g_dev_ok[64];

kp_status device_check() {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(KP_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_dev_mu);
    if (g_dev_ok[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
        g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
        if (g_dev_ok[dev] == 2) g_err = std::string("device is ") + prop.gcnArchName + ", not gfx950";
    }
    if (g_dev_ok[dev] != 1) return fail(KP_ERR_UNSUPPORTED, "libkpool runs on gfx950 (MI355X) only");
    return KP_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool pow2_idx(int d) { return d == 32 || d == 64 || d == 128; }

float hadamard_norm(int n) { return (float)(1.0 / std::sqrt((double)n)); }

}  // namespace

extern "C" {

const char* kp_last_error(void) { return g_err.c_str(); }

int32_t kp_version(void) { return 200; }

int32_t kp_row_width(int32_t kpool, int32_t topk_pools) {
    if (kpool < 1 || topk_pools < 0) return -1;
    long long raw = (long long)kpool * topk_pools + kpool - 1;
    long long w = (raw + 127) / 128 * 128;
    if (w > 0x7FFFFFFFLL) return -1;
    return (int32_t)w;
}

kp_status kpool_build_from(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                           const uint16_t* k_idx, const uint16_t* gate, const float* ape,
                           int32_t d_idx, int32_t kpool, int32_t token_lo,
                           int32_t* cu_pools, int32_t* pool_start,
                           uint8_t* pooled_k_fp8, float* pooled_k_scale, float* pooled_k_f32,
                           hipStream_t stream) {
    g_err.clear();
    if (num_docs < 0 || num_tokens < 0) return fail(KP_ERR_INVALID_ARG, "negative size");
    if (token_lo < 0 || token_lo > num_tokens)
        return fail(KP_ERR_INVALID_ARG, "token_lo must be in 0..num_tokens (got %d)", token_lo);
    if (kpool < 1 || kpool > 16) return fail(KP_ERR_UNSUPPORTED, "kpool must be in 1..16 (got %d)", kpool);
    if (!pow2_idx(d_idx)) return fail(KP_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
    if (!cu_seqlens || !cu_pools) return fail(KP_ERR_INVALID_ARG, "cu_seqlens and cu_pools are required");
    if (num_tokens == 0 && num_docs == 0) return ok();
    if (num_docs == 0) return fail(KP_ERR_INVALID_ARG, "num_tokens > 0 needs at least one document");
    const int pool_cap = num_tokens / kpool;
    if (pool_cap > 0 && (!k_idx || !gate || !ape || !pool_start || !pooled_k_fp8 || !pooled_k_scale))
        return fail(KP_ERR_INVALID_ARG, "k_idx, gate, ape, pool_start, pooled_k_fp8 and pooled_k_scale are required");
    kp_status st = device_check();
    if (st != KP_OK) return st;
    hipError_t e = kp::launch_layout_pool(cu_seqlens, num_docs, num_tokens, k_idx, gate, ape, d_idx, kpool,
                                          hadamard_norm(d_idx), cu_pools, pool_start, pooled_k_fp8,
                                          pooled_k_scale, pooled_k_f32, token_lo, stream);
    if (e != hipSuccess) return hip_fail(e, "kpool_build launch");
    return ok();
}

kp_status kpool_build(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                      const uint16_t* k_idx, const uint16_t* gate, const float* ape,
                      int32_t d_idx, int32_t kpool,
                      int32_t* cu_pools, int32_t* pool_start,
                      uint8_t* pooled_k_fp8, float* pooled_k_scale, float* pooled_k_f32,
                      hipStream_t stream) {
    return kpool_build_from(cu_seqlens, num_docs, num_tokens, k_idx, gate, ape, d_idx, kpool, 0, cu_pools,
                            pool_start, pooled_k_fp8, pooled_k_scale, pooled_k_f32, stream);
}

kp_status indexer_rotate_quant(const uint16_t* q_idx, int32_t num_q, int32_t h_idx, int32_t d_idx,
                               uint8_t* codes, float* scales, hipStream_t stream) {
    g_err.clear();
    if (num_q < 0 || h_idx < 1) return fail(KP_ERR_INVALID_ARG, "num_q must be >= 0 and h_idx >= 1");
    if (!pow2_idx(d_idx)) return fail(KP_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
    if (num_q == 0) return ok();
    if (!q_idx || !codes || !scales) return fail(KP_ERR_INVALID_ARG, "q_idx, codes and scales are required");
    kp_status st = device_check();
    if (st != KP_OK) return st;
    hipError_t e = kp::launch_rotate_quant(q_idx, (long long)num_q * h_idx, d_idx, hadamard_norm(d_idx), codes,
                                           scales, stream);
    if (e != hipSuccess) return hip_fail(e, "indexer_rotate_quant launch");
    return ok();
}

// Rows this long take the fused scoring + top-k when no scores are asked for:
// its candidate lists (FT_CAP per query) are then no larger than the score rows.
static bool fused_rows(int32_t max_pools, int32_t topk_pools) {
    return max_pools >= 2 * kp::FT_CAP && topk_pools <= kp::FT_CAP / 2;
}

static size_t fused_state_bytes(int32_t num_q) { return kp::fused_state_bytes(num_q); }

size_t kp_indexer_workspace_bytes(int32_t num_q, int32_t max_pools, int32_t h_idx, int32_t d_idx,
                                  int32_t topk_pools) {
    if (num_q <= 0 || max_pools < 0 || h_idx < 1 || d_idx < 1 || topk_pools < 0) return 0;
    size_t q8 = align256((size_t)num_q * h_idx * d_idx);
    size_t sq = align256((size_t)num_q * h_idx * sizeof(float));
    size_t rest = fused_rows(max_pools, topk_pools) ? fused_state_bytes(num_q)
                                                    : align256((size_t)num_q * (size_t)max_pools * sizeof(float));
    return q8 + sq + rest;
}

size_t kp_indexer_paged_workspace_bytes(int32_t num_q, int32_t num_docs, int32_t h_idx, int32_t d_idx) {
    if (num_q <= 0 || num_docs < 0 || h_idx < 1 || d_idx < 1) return 0;
    return align256((size_t)(num_docs + 1) * sizeof(int32_t)) + align256((size_t)num_q * h_idx * d_idx) +
           align256((size_t)num_q * h_idx * sizeof(float)) + fused_state_bytes(num_q);
}

static kp_status check_topk_args(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                 const int32_t* cu_pools, int32_t max_pools, const int32_t* q_pos,
                                 int32_t num_q, int32_t kpool, int32_t topk_pools, int32_t row_width,
                                 const int32_t* indices) {
    if (num_docs < 0 || num_tokens < 0 || num_q < 0 || max_pools < 0)
        return fail(KP_ERR_INVALID_ARG, "negative size");
    if (kpool < 1 || kpool > 16) return fail(KP_ERR_UNSUPPORTED, "kpool must be in 1..16 (got %d)", kpool);
    if (topk_pools < 0) return fail(KP_ERR_INVALID_ARG, "topk_pools must be >= 0");
    if (max_pools != num_tokens / kpool)
        return fail(KP_ERR_INVALID_ARG, "max_pools must equal num_tokens / kpool (%d)", num_tokens / kpool);
    const long long need = (long long)kpool * topk_pools + kpool - 1;
    if (row_width % 128 != 0 || row_width < need || row_width < 128)
        return fail(KP_ERR_INVALID_ARG, "row_width %d must be a multiple of 128 and >= %lld", row_width, need);
    if (num_q == 0) return KP_OK;
    if (num_docs == 0 || num_tokens == 0) return fail(KP_ERR_INVALID_ARG, "queries need a non-empty row");
    if (!q_pos && num_q != num_tokens) return fail(KP_ERR_INVALID_ARG, "q_pos == NULL requires num_q == num_tokens");
    if (!cu_seqlens || !cu_pools || !indices)
        return fail(KP_ERR_INVALID_ARG, "cu_seqlens, cu_pools and indices are required");
    return KP_OK;
}

// Argument checks of indexer_score_topk other than its workspace.
static kp_status check_score_topk_args(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                       const int32_t* cu_pools, int32_t max_pools, const uint8_t* pooled_k_fp8,
                                       const float* pooled_k_scale, const int32_t* q_pos, int32_t num_q,
                                       const uint16_t* q_idx, const float* w_idx, int32_t h_idx, int32_t d_idx,
                                       int32_t kpool, int32_t topk_pools, int32_t row_width,
                                       const int32_t* indices) {
    kp_status st = check_topk_args(cu_seqlens, num_docs, num_tokens, cu_pools, max_pools, q_pos, num_q, kpool,
                                   topk_pools, row_width, indices);
    if (st != KP_OK) return st;
    if (h_idx < 1 || h_idx > 64) return fail(KP_ERR_UNSUPPORTED, "h_idx must be in 1..64 (got %d)", h_idx);
    if (!pow2_idx(d_idx)) return fail(KP_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
    if (num_q == 0) return KP_OK;
    if (!q_idx || !w_idx) return fail(KP_ERR_INVALID_ARG, "q_idx and w_idx are required");
    if (max_pools > 0 && (!pooled_k_fp8 || !pooled_k_scale))
        return fail(KP_ERR_INVALID_ARG, "pooled_k_fp8 and pooled_k_scale are required");
    return KP_OK;
}

// The launches of indexer_score_topk on a checked workspace of at least
// kp_indexer_workspace_bytes bytes (none of it needs clearing: every byte a
// kernel reads was written by an earlier kernel of the same call). Rows of
// many pools take the fused path (no score tensor) unless scores are asked for.
static kp_status score_topk_launch(const int32_t* cu_seqlens, int32_t num_docs, const int32_t* cu_pools,
                                   int32_t max_pools, const uint8_t* pooled_k_fp8, const float* pooled_k_scale,
                                   const int32_t* q_pos, int32_t num_q, const uint16_t* q_idx, const float* w_idx,
                                   int32_t h_idx, int32_t d_idx, int32_t kpool, int32_t topk_pools,
                                   int32_t row_width, int32_t* indices, int32_t* num_valid, float* scores,
                                   uint8_t* ws, hipStream_t stream) {
    uint8_t* q8 = ws;
    float* sq = reinterpret_cast<float*>(ws + align256((size_t)num_q * h_idx * d_idx));
    uint8_t* rest = reinterpret_cast<uint8_t*>(sq) + align256((size_t)num_q * h_idx * 4);
    float* sc = scores ? scores : reinterpret_cast<float*>(rest);

    const bool fused = !scores && fused_rows(max_pools, topk_pools);
    const kp::FusedState fst = kp::fused_state_at(rest, num_q);
    hipError_t e = kp::launch_rotate_quant(q_idx, (long long)num_q * h_idx, d_idx, hadamard_norm(d_idx), q8, sq,
                                           stream);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    if (fused) {
        e = kp::launch_fused_topk(cu_seqlens, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w_idx, h_idx, d_idx,
                                  pooled_k_fp8, pooled_k_scale, max_pools, nullptr, 0, 0, topk_pools, row_width,
                                  indices, num_valid, nullptr, fst, stream);
        if (e != hipSuccess) return hip_fail(e, "fused score + top-k launch");
        return KP_OK;
    }
    if (scores) {
        e = kp::launch_fill_f32(scores, (size_t)num_q * max_pools, -INFINITY, stream);
        if (e != hipSuccess) return hip_fail(e, "score fill launch");
    }
    e = kp::launch_score(cu_seqlens, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w_idx, h_idx, d_idx,
                         pooled_k_fp8, pooled_k_scale, max_pools, sc, stream);
    if (e != hipSuccess) return hip_fail(e, "score launch");
    e = kp::launch_topk(cu_seqlens, num_docs, cu_pools, kpool, q_pos, num_q, sc, max_pools, topk_pools, row_width,
                        indices, num_valid, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return KP_OK;
}

kp_status indexer_score_topk(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                             const int32_t* cu_pools, int32_t max_pools,
                             const uint8_t* pooled_k_fp8, const float* pooled_k_scale,
                             const int32_t* q_pos, int32_t num_q,
                             const uint16_t* q_idx, const float* w_idx,
                             int32_t h_idx, int32_t d_idx, int32_t kpool,
                             int32_t topk_pools, int32_t row_width,
                             int32_t* indices, int32_t* num_valid, float* scores,
                             void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    kp_status st = check_score_topk_args(cu_seqlens, num_docs, num_tokens, cu_pools, max_pools, pooled_k_fp8,
                                         pooled_k_scale, q_pos, num_q, q_idx, w_idx, h_idx, d_idx, kpool,
                                         topk_pools, row_width, indices);
    if (st != KP_OK) return st;
    if (num_q == 0) return ok();
    const size_t need = kp_indexer_workspace_bytes(num_q, max_pools, h_idx, d_idx, topk_pools);
    if (!workspace || workspace_bytes < need)
        return fail(KP_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(KP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    st = device_check();
    if (st != KP_OK) return st;
    return score_topk_launch(cu_seqlens, num_docs, cu_pools, max_pools, pooled_k_fp8, pooled_k_scale, q_pos,
                             num_q, q_idx, w_idx, h_idx, d_idx, kpool, topk_pools, row_width, indices, num_valid,
                             scores, static_cast<uint8_t*>(workspace), stream);
}

}  // extern "C"

// ---- the allocation-free variant ---------------------------------------------
// Its workspace is this file-scope device array: each GPU the library runs on
// holds one copy, at its own address, from the code object's load until the
// process ends. Host code never passes the array's name to a kernel (on the
// host the name stands for a host-side shadow, not device memory): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and only that address is used.
static __device__ __align__(256) uint8_t scratch[KP_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];   // device address of `scratch` on each device (null until looked up)

kp_status scratch_address(uint8_t** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= 64) return fail(KP_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p) return fail(KP_ERR_HIP, "hipGetSymbolAddress(scratch) returned a null address");
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<uint8_t*>(g_scratch_ptr[dev]);
    return KP_OK;
}
}  // namespace

extern "C" {

kp_status indexer_score_topk_noalloc(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                     const int32_t* cu_pools, int32_t max_pools,
                                     const uint8_t* pooled_k_fp8, const float* pooled_k_scale,
                                     const int32_t* q_pos, int32_t num_q,
                                     const uint16_t* q_idx, const float* w_idx,
                                     int32_t h_idx, int32_t d_idx, int32_t kpool,
                                     int32_t topk_pools, int32_t row_width,
                                     int32_t* indices, int32_t* num_valid, float* scores,
                                     hipStream_t stream) {
    g_err.clear();
    kp_status st = check_score_topk_args(cu_seqlens, num_docs, num_tokens, cu_pools, max_pools, pooled_k_fp8,
                                         pooled_k_scale, q_pos, num_q, q_idx, w_idx, h_idx, d_idx, kpool,
                                         topk_pools, row_width, indices);
    if (st != KP_OK) return st;
    if (num_q == 0) return ok();
    const size_t need = kp_indexer_workspace_bytes(num_q, max_pools, h_idx, d_idx, topk_pools);
    if (need > (size_t)KP_NOALLOC_SCRATCH_BYTES)
        return fail(KP_ERR_UNSUPPORTED,
                    "indexer_score_topk_noalloc: these sizes need %zu bytes of workspace, above the library's "
                    "%zu-byte device scratch (use indexer_score_topk with a caller workspace)",
                    need, (size_t)KP_NOALLOC_SCRATCH_BYTES);
    st = device_check();
    if (st != KP_OK) return st;
    uint8_t* ws = nullptr;
    st = scratch_address(&ws);
    if (st != KP_OK) return st;
    return score_topk_launch(cu_seqlens, num_docs, cu_pools, max_pools, pooled_k_fp8, pooled_k_scale, q_pos,
                             num_q, q_idx, w_idx, h_idx, d_idx, kpool, topk_pools, row_width, indices, num_valid,
                             scores, ws, stream);
}

kp_status kpool_update_paged(const int32_t* cu_seqlens, int32_t num_docs,
                             const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                             const uint16_t* k_idx_pages, const uint16_t* gate_pages, const float* ape,
                             int32_t d_idx, int32_t kpool, int32_t last_tokens,
                             uint8_t* k8_pages, float* sk_pages, hipStream_t stream) {
    g_err.clear();
    if (num_docs < 0 || max_pages < 0 || num_pages < 0 || last_tokens < 0)
        return fail(KP_ERR_INVALID_ARG, "negative size");
    if (kpool < 1 || kpool > 16) return fail(KP_ERR_UNSUPPORTED, "kpool must be in 1..16 (got %d)", kpool);
    if (!pow2_idx(d_idx)) return fail(KP_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
    if ((long long)num_pages * 32 * kpool > 0x7FFFFFFFLL || (long long)num_docs * max_pages > 0x7FFFFFFFLL)
        return fail(KP_ERR_UNSUPPORTED, "page cache too large for 32-bit slot numbers");
    if (num_docs == 0 || last_tokens == 0 || max_pages == 0 || num_pages == 0) return ok();
    if (!cu_seqlens || !page_table || !k_idx_pages || !gate_pages || !ape || !k8_pages || !sk_pages)
        return fail(KP_ERR_INVALID_ARG, "cu_seqlens, page_table, k_idx_pages, gate_pages, ape, k8_pages and "
                                        "sk_pages are required");
    kp_status st = device_check();
    if (st != KP_OK) return st;
    hipError_t e = kp::launch_pool_paged(cu_seqlens, num_docs, page_table, max_pages, num_pages, k_idx_pages,
                                         gate_pages, ape, d_idx, kpool, hadamard_norm(d_idx), k8_pages, sk_pages,
                                         last_tokens, stream);
    if (e != hipSuccess) return hip_fail(e, "kpool_update_paged launch");
    return ok();
}

kp_status indexer_score_topk_paged(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                   const int32_t* page_table, int32_t max_pages, int32_t num_pages,
                                   const uint8_t* k8_pages, const float* sk_pages,
                                   const int32_t* q_pos, int32_t num_q,
                                   const uint16_t* q_idx, const float* w_idx,
                                   int32_t h_idx, int32_t d_idx, int32_t kpool,
                                   int32_t topk_pools, int32_t row_width,
                                   int32_t* indices, int32_t* num_valid, int32_t* row_path,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream) {
    g_err.clear();
    if (num_docs < 0 || num_tokens < 0 || num_q < 0 || max_pages < 0 || num_pages < 0)
        return fail(KP_ERR_INVALID_ARG, "negative size");
    if (kpool < 1 || kpool > 16) return fail(KP_ERR_UNSUPPORTED, "kpool must be in 1..16 (got %d)", kpool);
    if (topk_pools < 0) return fail(KP_ERR_INVALID_ARG, "topk_pools must be >= 0");
    if (topk_pools > kp::FT_CAP / 2)
        return fail(KP_ERR_UNSUPPORTED, "topk_pools must be at most %d on the paged path (got %d)", kp::FT_CAP / 2,
                    topk_pools);
    const long long need_w = (long long)kpool * topk_pools + kpool - 1;
    if (row_width % 128 != 0 || row_width < need_w || row_width < 128)
        return fail(KP_ERR_INVALID_ARG, "row_width %d must be a multiple of 128 and >= %lld", row_width, need_w);
    if (h_idx < 1 || h_idx > 64) return fail(KP_ERR_UNSUPPORTED, "h_idx must be in 1..64 (got %d)", h_idx);
    if (!pow2_idx(d_idx)) return fail(KP_ERR_UNSUPPORTED, "d_idx must be 32, 64 or 128 (got %d)", d_idx);
    if ((long long)num_pages * 32 * kpool > 0x7FFFFFFFLL || (long long)num_docs * max_pages > 0x7FFFFFFFLL)
        return fail(KP_ERR_UNSUPPORTED, "page cache too large for 32-bit slot numbers");
    if (num_q == 0) return ok();
    if (num_docs == 0 || num_tokens == 0) return fail(KP_ERR_INVALID_ARG, "queries need a non-empty row");
    if (!q_pos && num_q != num_tokens) return fail(KP_ERR_INVALID_ARG, "q_pos == NULL requires num_q == num_tokens");
    if (!cu_seqlens || !page_table || !k8_pages || !sk_pages || !q_idx || !w_idx || !indices)
        return fail(KP_ERR_INVALID_ARG, "cu_seqlens, page_table, k8_pages, sk_pages, q_idx, w_idx and indices are "
                                        "required");
    const size_t need = kp_indexer_paged_workspace_bytes(num_q, num_docs, h_idx, d_idx);
    if (!workspace || workspace_bytes < need)
        return fail(KP_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(KP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    kp_status st = device_check();
    if (st != KP_OK) return st;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    int32_t* cu_pools = reinterpret_cast<int32_t*>(ws);
    uint8_t* q8 = ws + align256((size_t)(num_docs + 1) * sizeof(int32_t));
    float* sq = reinterpret_cast<float*>(q8 + align256((size_t)num_q * h_idx * d_idx));
    uint8_t* rest = reinterpret_cast<uint8_t*>(sq) + align256((size_t)num_q * h_idx * 4);
    const kp::FusedState fst = kp::fused_state_at(rest, num_q);
    hipError_t e = kp::launch_layout(cu_seqlens, num_docs, kpool, cu_pools, stream);
    if (e != hipSuccess) return hip_fail(e, "layout launch");
    e = kp::launch_rotate_quant(q_idx, (long long)num_q * h_idx, d_idx, hadamard_norm(d_idx), q8, sq, stream);
    if (e != hipSuccess) return hip_fail(e, "rotate_quant launch");
    e = kp::launch_fused_topk(cu_seqlens, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w_idx, h_idx, d_idx,
                              k8_pages, sk_pages, num_tokens / kpool, page_table, max_pages, num_pages, topk_pools,
                              row_width, indices, num_valid, row_path, fst, stream);
    if (e != hipSuccess) return hip_fail(e, "fused score + top-k launch");
    return ok();
}

kp_status indexer_topk_from_scores(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                                   const int32_t* cu_pools, int32_t max_pools,
                                   const int32_t* q_pos, int32_t num_q, const float* scores,
                                   int32_t kpool, int32_t topk_pools, int32_t row_width,
                                   int32_t* indices, int32_t* num_valid, hipStream_t stream) {
    g_err.clear();
    kp_status st = check_topk_args(cu_seqlens, num_docs, num_tokens, cu_pools, max_pools, q_pos, num_q, kpool,
                                   topk_pools, row_width, indices);
    if (st != KP_OK) return st;
    if (num_q == 0) return ok();
    if (!scores) return fail(KP_ERR_INVALID_ARG, "scores is required");
    st = device_check();
    if (st != KP_OK) return st;
    hipError_t e = kp::launch_topk(cu_seqlens, num_docs, cu_pools, kpool, q_pos, num_q, scores, max_pools,
                                   topk_pools, row_width, indices, num_valid, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
    return ok();
}

size_t kp_mla_fwd_workspace_bytes(int32_t num_q, int32_t heads, int32_t d_latent, int32_t row_width) {
    if (num_q <= 0 || heads < 1 || heads > 64 || row_width < 1) return 0;
    if (d_latent != 512 && d_latent != 64 && d_latent != 576) return 0;
    return align256(kp::sparse_mla_part_bytes(num_q, heads, d_latent, row_width));
}

kp_status sparse_mla_fwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                         int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_latent,
                         int32_t row_width, float softmax_scale,
                         uint16_t* out, float* lse, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    g_err.clear();
    if (num_q < 0 || num_kv < 0 || row_width < 1) return fail(KP_ERR_INVALID_ARG, "bad size");
    if (heads < 1 || heads > 64) return fail(KP_ERR_UNSUPPORTED, "heads must be in 1..64 (got %d)", heads);
    if (d_latent != 512 && d_latent != 64 && d_latent != 576)
        return fail(KP_ERR_UNSUPPORTED, "d_latent must be 512, 576 or 64 (got %d)", d_latent);
    if (row_width > kp::sparse_mla_max_row_width(d_latent))
        return fail(KP_ERR_UNSUPPORTED, "row_width above %d for d_latent %d (got %d)",
                    kp::sparse_mla_max_row_width(d_latent), d_latent, row_width);
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
        return fail(KP_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
    // the row loads address the latent through a buffer descriptor based 4 KiB below
    // it, whose 32-bit record count must hold the latent's bytes plus those 4 KiB
    if ((uint64_t)num_kv * (uint64_t)d_latent * 2u + 4096u > 0xFFFFFFFFull)
        return fail(KP_ERR_UNSUPPORTED, "latent of %d rows x %d is not below 4 GiB - 4 KiB", num_kv, d_latent);
    if (num_q == 0) return ok();
    if (!q || !indices || !out || (num_kv > 0 && !kv))
        return fail(KP_ERR_INVALID_ARG, "q, kv, indices and out are required");
    const size_t need = kp_mla_fwd_workspace_bytes(num_q, heads, d_latent, row_width);
    if (workspace && need > 0) {
        if (workspace_bytes < need)
            return fail(KP_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
        if (((uintptr_t)workspace & 255) != 0) return fail(KP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }
    kp_status st = device_check();
    if (st != KP_OK) return st;
    const float scale_log2 = (float)((double)softmax_scale * 1.4426950408889634074);
    hipError_t e = kp::launch_sparse_mla(q, kv, indices, num_q, num_kv, heads, d_latent, row_width, scale_log2,
                                         out, lse, need > 0 ? workspace : nullptr, stream);
    if (e != hipSuccess) return hip_fail(e, "sparse_mla launch");
    return ok();
}

size_t kp_mla_bwd_workspace_bytes(int32_t num_q, int32_t d_latent, int32_t row_width) {
    if (num_q <= 0 || row_width < 1 || (d_latent != 512 && d_latent != 64)) return 0;
    return align256(kp::sparse_mla_bwd_ws_bytes(num_q, d_latent, row_width));
}

kp_status sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices,
                         const uint16_t* out, const float* lse, const uint16_t* d_out,
                         int32_t num_q, int32_t num_kv, int32_t heads, int32_t d_latent,
                         int32_t row_width, float softmax_scale,
                         uint16_t* d_q, float* d_kv, void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
    g_err.clear();
    if (num_q < 0 || num_kv < 0 || row_width < 1) return fail(KP_ERR_INVALID_ARG, "bad size");
    if (heads < 1 || heads > 64) return fail(KP_ERR_UNSUPPORTED, "heads must be in 1..64 (got %d)", heads);
    if (d_latent != 512 && d_latent != 64)
        return fail(KP_ERR_UNSUPPORTED, "d_latent must be 512 or 64 (got %d)", d_latent);
    if (row_width > kp::sparse_mla_max_row_width(d_latent))
        return fail(KP_ERR_UNSUPPORTED, "row_width above %d (got %d)", kp::sparse_mla_max_row_width(d_latent),
                    row_width);
    if (!std::isfinite(softmax_scale) || !(softmax_scale > 0.f))
        return fail(KP_ERR_INVALID_ARG, "softmax_scale must be finite and positive");
    if ((uint64_t)num_kv * (uint64_t)d_latent * 2u + 4096u > 0xFFFFFFFFull)
        return fail(KP_ERR_UNSUPPORTED, "latent of %d rows x %d is not below 4 GiB - 4 KiB", num_kv, d_latent);
    if (num_kv > 0 && !d_kv) return fail(KP_ERR_INVALID_ARG, "d_kv is required");
    if (num_q > 0 && (!q || !kv || !indices || !out || !lse || !d_out || !d_q))
        return fail(KP_ERR_INVALID_ARG, "q, kv, indices, out, lse, d_out and d_q are required");
    const size_t need = kp_mla_bwd_workspace_bytes(num_q, d_latent, row_width);
    if (num_q > 0 && (!workspace || workspace_bytes < need))
        return fail(KP_ERR_INVALID_ARG, "workspace of %zu bytes required (got %zu)", need, workspace_bytes);
    if (((uintptr_t)workspace & 255) != 0) return fail(KP_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    if (num_q == 0 && num_kv == 0) return ok();
    kp_status st = device_check();
    if (st != KP_OK) return st;
    hipError_t e = kp::launch_sparse_mla_bwd(q, kv, indices, out, lse, d_out, num_q, num_kv, heads, d_latent,
                                             row_width, softmax_scale, d_q, d_kv, workspace, stream);
    if (e != hipSuccess) return hip_fail(e, "sparse_mla_bwd launch");
    return ok();
}

kp_status kp_check_inputs(const int32_t* cu_seqlens, int32_t num_docs, int32_t num_tokens,
                          const int32_t* q_pos, int32_t num_q, hipStream_t stream) {
    g_err.clear();
    if (num_docs < 0 || num_tokens < 0 || num_q < 0) return fail(KP_ERR_INVALID_ARG, "negative size");
    if (!cu_seqlens) return fail(KP_ERR_INVALID_ARG, "cu_seqlens is required");
    std::vector<int32_t> cu((size_t)num_docs + 1), qp((size_t)num_q);
    hipError_t e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    e = hipMemcpy(cu.data(), cu_seqlens, cu.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy cu_seqlens");
    if (cu[0] != 0) return fail(KP_ERR_INVALID_ARG, "cu_seqlens[0] = %d, expected 0", cu[0]);
    for (int d = 0; d < num_docs; ++d)
        if (cu[d + 1] < cu[d]) return fail(KP_ERR_INVALID_ARG, "cu_seqlens decreases at %d", d + 1);
    if (cu[num_docs] != num_tokens)
        return fail(KP_ERR_INVALID_ARG, "cu_seqlens[num_docs] = %d, expected %d", cu[num_docs], num_tokens);
    if (q_pos && num_q > 0) {
        e = hipMemcpy(qp.data(), q_pos, qp.size() * sizeof(int32_t), hipMemcpyDeviceToHost);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpy q_pos");
        for (int i = 0; i < num_q; ++i)
            if (qp[i] < 0 || qp[i] >= num_tokens)
                return fail(KP_ERR_INVALID_ARG, "q_pos[%d] = %d outside [0, %d)", i, qp[i], num_tokens);
    }
    return ok();
}

}  // extern "C"
