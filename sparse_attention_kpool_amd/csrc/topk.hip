// Per-query top-k pool selection and index-row construction.
//
// prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet: a query keeps
// the top 512 of the complete pools visible to it and also attends to its own
// incomplete pool; index rows are padded to a multiple of 128. NeMo AutoModel
// PR "add GLM-5.3-Flash training support", "cuDNN sparse MLA parity and
// performance": 4*512 + 3 = 2051 raw slots. Equal scores keep the lower pool.
//
// One workgroup per query row. Scores map to order-preserving 32-bit keys
// (-0 folded onto +0; NaN below -inf). A most-significant-digit-first radix
// select (digits of 11, 11 and 10 bits, histograms in LDS) finds the key K of
// the k-th largest score and how many of the kept pools score exactly K; it
// stops early when the bin holding the k-th key is kept whole. A final pass
// over contiguous per-thread chunks, in pool order, keeps every pool above K
// and the first pools equal to K, and writes each kept pool's tokens at its
// rank: the kept pools come out ascending with no sort. The keys of a row
// short enough stay in LDS between passes; longer rows are re-read.
#include "kp_device.h"
#include "kp_launch.h"

namespace kp {

constexpr int TK_THREADS = 256;
constexpr int TK_LDS_KEYS = 8192;    // keys cached in LDS (32 KB)
constexpr int TK_BINS = 2048;        // histogram bins of the widest digit

__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;                       // -0 == +0
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return 0u;  // NaN: lowest
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive scan of one int per thread over the block; returns the prefix and
// writes the total to *total.
__device__ __forceinline__ int block_excl_scan(int v, int* wave_buf, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    if (lane == 63) wave_buf[wave] = x;
    __syncthreads();
    int add = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < TK_THREADS / 64; ++w) {
        int t = wave_buf[w];
        if (w < wave) add += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return add + x - v;
}

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices, int32_t* __restrict__ num_valid) {
    __shared__ uint32_t keys_lds[TK_LDS_KEYS];
    __shared__ int hist[TK_BINS];
    __shared__ int wave_buf[TK_THREADS / 64];
    __shared__ int sel_digit, sel_above, sel_cnt;

    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = qp.n_vis;
    const int k = n < topk ? n : topk;
    const int doc_start = cu[qp.doc];
    int32_t* row = indices + (size_t)i * row_width;
    const float* srow = scores + (size_t)i * max_pools + qp.pool_lo;
    const bool cached = n <= TK_LDS_KEYS;

    const bool all = k >= n;  // every visible pool is kept (no scores needed)
    uint32_t thresh = 0xFFFFFFFFu;  // key of the k-th largest score (k == 0: above every key)
    int take_eq = 0;                // how many pools equal to thresh are kept (lowest first)
    if (!all && k > 0) {
        if (cached) {
            // sixteen loads in flight per thread before their LDS stores
            constexpr int SB = 16;
            for (int j0 = 0; j0 < n; j0 += TK_THREADS * SB) {
                float v[SB];
#pragma unroll
                for (int q = 0; q < SB; ++q) {
                    const int j = j0 + tid + TK_THREADS * q;
                    v[q] = j < n ? srow[j] : 0.0f;
                }
#pragma unroll
                for (int q = 0; q < SB; ++q) {
                    const int j = j0 + tid + TK_THREADS * q;
                    if (j < n) keys_lds[j] = score_key(v[q]);
                }
            }
        }
        int remaining = k;  // still to choose among keys matching the prefix
        uint32_t prefix = 0u, pmask = 0u;
        take_eq = -1;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int width = pass < 2 ? 11 : 10;
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nb = 1 << width;
            for (int b = tid; b < nb; b += TK_THREADS) hist[b] = 0;
            __syncthreads();
            for (int j = tid; j < n; j += TK_THREADS) {
                uint32_t key = cached ? keys_lds[j] : score_key(srow[j]);
                if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & (uint32_t)(nb - 1)], 1);
            }
            __syncthreads();
            // thread t owns the nb/256 bins just below the top 'nb/256 * t' bins;
            // a scan over threads counts the keys in bins above each thread's
            const int per = nb / TK_THREADS;
            const int top = nb - 1 - per * tid;
            int cnt_own = 0;
            for (int e = 0; e < per; ++e) cnt_own += hist[top - e];
            int tot;
            const int before = block_excl_scan(cnt_own, wave_buf, &tot);
            if (before < remaining && before + cnt_own >= remaining) {
                int acc = before;
                for (int e = 0; e < per; ++e) {
                    const int c = hist[top - e];
                    if (acc < remaining && acc + c >= remaining) {
                        sel_digit = top - e;
                        sel_above = acc;
                        sel_cnt = c;
                    }
                    acc += c;
                }
            }
            __syncthreads();
            remaining -= sel_above;
            prefix |= (uint32_t)sel_digit << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            if (sel_cnt == remaining) {
                // the whole bin is kept: every key >= prefix (low bits zero) is selected
                take_eq = 0x7FFFFFFF;
                break;
            }
        }
        thresh = prefix;
        if (take_eq < 0) take_eq = remaining;
    }

    // final pass: contiguous chunk per thread, in pool order
    const int chunk = (n + TK_THREADS - 1) / TK_THREADS;
    const int j0 = min(n, tid * chunk), j1 = min(n, j0 + chunk);
    int n_eq = 0;
    if (!all)
        for (int j = j0; j < j1; ++j) n_eq += ((cached ? keys_lds[j] : score_key(srow[j])) == thresh);
    int tot;
    int eq_before = block_excl_scan(n_eq, wave_buf, &tot);
    int n_sel = 0;
    if (!all) {
        int e = eq_before;
        for (int j = j0; j < j1; ++j) {
            uint32_t key = cached ? keys_lds[j] : score_key(srow[j]);
            n_sel += key > thresh || (key == thresh && e++ < take_eq);
        }
    } else {
        n_sel = j1 - j0;
    }
    int sel_before = block_excl_scan(n_sel, wave_buf, &tot);
    {
        int e = eq_before, pos = sel_before;
        for (int j = j0; j < j1; ++j) {
            bool keep = true;
            if (!all) {
                uint32_t key = cached ? keys_lds[j] : score_key(srow[j]);
                keep = key > thresh || (key == thresh && e++ < take_eq);
            }
            if (keep) {
                const int tok = doc_start + kpool * j;
                for (int r = 0; r < kpool; ++r) row[pos * kpool + r] = tok + r;
                ++pos;
            }
        }
    }
    // own incomplete pool, then padding
    const int base = k * kpool;
    const int n_tail = t - qp.tail_start + 1;
    for (int r = tid; r < row_width - base; r += TK_THREADS)
        row[base + r] = r < n_tail ? qp.tail_start + r : -1;
    if (tid == 0 && num_valid) num_valid[i] = base + n_tail;
}

hipError_t launch_topk(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                       const int32_t* q_pos, int num_q, const float* scores, int max_pools,
                       int topk, int row_width, int32_t* indices, int32_t* num_valid,
                       hipStream_t stream) {
    if (num_q == 0) return hipSuccess;
    topk_kernel<<<num_q, TK_THREADS, 0, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools,
                                                  topk, row_width, indices, num_valid);
    return hipGetLastError();
}

}  // namespace kp
