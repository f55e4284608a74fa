// Pool layout, k-pool compression, and the Hadamard + FP8 encoding of pooled
// keys and indexer queries.
//
// prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet: keys pooled
// per document in groups of 4 from the document's first token, as a
// per-channel softmax(gate + ape)-weighted mean; queries and pooled keys are
// rotated by an fp32 butterfly Hadamard transform before FP8 scoring.
//
// One pooled key (or one query head vector) of n channels is handled by n/4
// lanes, four consecutive channels per lane. The butterfly stages of stride 1
// and 2 run inside a lane, the rest across lanes with xor shuffles; every
// output of a stage is the single fp32 sum or difference of the same two
// inputs as in the sequential Sylvester-order transform, so the rotated values
// do not depend on how the vector is spread over lanes.
#include "kp_device.h"
#include "kp_launch.h"

namespace kp {

// ------------------------------------------------------------- layout -------
// cu_pools[d+1] = cu_pools[d] + floor((cu[d+1] - cu[d]) / kpool); one block
// scans the documents in chunks of its size.
__global__ __launch_bounds__(1024) void layout_scan_kernel(const int32_t* __restrict__ cu,
                                                           int num_docs, int kpool,
                                                           int32_t* __restrict__ cu_pools) {
    __shared__ int wave_tot[16];
    __shared__ int carry_s;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0) { carry_s = 0; cu_pools[0] = 0; }
    __syncthreads();
    for (int base = 0; base < num_docs; base += 1024) {
        int d = base + tid;
        int v = d < num_docs ? (cu[d + 1] - cu[d]) / kpool : 0;
        // inclusive scan inside the wave
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            int u = __shfl_up(v, o, 64);
            if (lane >= o) v += u;
        }
        if (lane == 63) wave_tot[wave] = v;
        __syncthreads();
        int add = carry_s;
        for (int w = 0; w < wave; ++w) add += wave_tot[w];
        if (d < num_docs) cu_pools[d + 1] = v + add;
        __syncthreads();
        if (tid == blockDim.x - 1) carry_s = v + add;
        __syncthreads();
    }
}

// ---------------------------------------------- rotate + quantise -----------
// Butterfly stages across lanes at distances B, 2B, ... < L, in that order.
template <int L, int B>
__device__ __forceinline__ void fwht4_lanes(float (&x)[4], int lane) {
    if constexpr (B < L) {
        const bool upper = (lane & B) != 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float y = lane_xor<B>(x[e]);
            x[e] = upper ? (y - x[e]) : (x[e] + y);
        }
        fwht4_lanes<L, 2 * B>(x, lane);
    }
}

// x holds channels 4*j .. 4*j+3 of a vector of n = 4*L channels spread over L
// consecutive lanes (j = lane % L). Orthonormal Walsh-Hadamard transform in
// Sylvester order: stride 1, 2 in-lane, 4 .. n/2 across lanes; then one
// multiply by `norm` = fp32(1/sqrt(n)).
template <int L>
__device__ __forceinline__ void fwht4(float (&x)[4], int lane, float norm) {
    float a0 = x[0] + x[1], a1 = x[0] - x[1], a2 = x[2] + x[3], a3 = x[2] - x[3];
    x[0] = a0 + a2; x[2] = a0 - a2; x[1] = a1 + a3; x[3] = a1 - a3;
    fwht4_lanes<L, 1>(x, lane);
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = x[e] * norm;
}

// Per-vector scale s = amax/448 (1 when the vector is zero) and E4M3 codes of
// x/s. Returns the four codes of this lane packed little-endian.
template <int L>
__device__ __forceinline__ uint32_t quant4(const float (&x)[4], float* scale_out) {
    float amax = fmaxf(fmaxf(fabsf(x[0]), fabsf(x[1])), fmaxf(fabsf(x[2]), fabsf(x[3])));
    amax = group_max<L>(amax);
    float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    *scale_out = s;
    return cvt_e4m3x4(x[0] / s, x[1] / s, x[2] / s, x[3] / s);
}

// ------------------------------------------------------------ keys ----------
// Channels 4j .. 4j+3 of the pooled key (before rotation) of the kpool tokens
// whose k_idx and gate rows are tok_row(0) .. tok_row(kpool-1): per channel, a
// softmax over the pool's tokens of gate + ape, then the weighted sum of k_idx.
template <int L, int KP, typename TokRow>
__device__ __forceinline__ void pool_vector(float (&x)[4], const uint16_t* __restrict__ k_idx,
                                            const uint16_t* __restrict__ gate, const float* __restrict__ ape,
                                            int kpool, int j, TokRow tok_row) {
    constexpr int N = 4 * L;
    if (KP > 0) {
        // max-subtracted softmax over a fixed pool size, values held in registers
        float a[KP > 0 ? KP : 1][4], kv[KP > 0 ? KP : 1][4];
        float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
        for (int i = 0; i < KP; ++i) {
            const size_t r = tok_row(i);
            uint2 g = reinterpret_cast<const uint2*>(gate + r * N)[j];
            uint2 k = reinterpret_cast<const uint2*>(k_idx + r * N)[j];
            float4 e = reinterpret_cast<const float4*>(ape + (size_t)i * N)[j];
            a[i][0] = bf16_lo(g.x) + e.x; a[i][1] = bf16_hi(g.x) + e.y;
            a[i][2] = bf16_lo(g.y) + e.z; a[i][3] = bf16_hi(g.y) + e.w;
            kv[i][0] = bf16_lo(k.x); kv[i][1] = bf16_hi(k.x);
            kv[i][2] = bf16_lo(k.y); kv[i][3] = bf16_hi(k.y);
#pragma unroll
            for (int c = 0; c < 4; ++c) m[c] = fmaxf(m[c], a[i][c]);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float den = 0.0f, num = 0.0f;
#pragma unroll
            for (int i = 0; i < KP; ++i) {
                float e = expf(a[i][c] - m[c]);
                den += e;
                num += e * kv[i][c];
            }
            x[c] = num / den;
        }
    } else {
        // any pool size: running max with rescaled partial sums
        float m[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        float den[4] = {0.f, 0.f, 0.f, 0.f}, num[4] = {0.f, 0.f, 0.f, 0.f};
        for (int i = 0; i < kpool; ++i) {
            const size_t r = tok_row(i);
            uint2 g = reinterpret_cast<const uint2*>(gate + r * N)[j];
            uint2 k = reinterpret_cast<const uint2*>(k_idx + r * N)[j];
            float4 e = reinterpret_cast<const float4*>(ape + (size_t)i * N)[j];
            float av[4] = {bf16_lo(g.x) + e.x, bf16_hi(g.x) + e.y, bf16_lo(g.y) + e.z, bf16_hi(g.y) + e.w};
            float kk[4] = {bf16_lo(k.x), bf16_hi(k.x), bf16_lo(k.y), bf16_hi(k.y)};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float mn = fmaxf(m[c], av[c]);
                float r2 = expf(m[c] - mn);   // 0 on the first token
                float w = expf(av[c] - mn);
                den[c] = den[c] * r2 + w;
                num[c] = num[c] * r2 + w * kk[c];
                m[c] = mn;
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) x[c] = num[c] / den[c];
    }
}

// One pool per L lanes. Capacity rows (num_tokens / kpool) past the last pool
// get pool_start -1, zero codes and a zero scale.
// LAYOUT says where the pool layout comes from:
//   POOL_LAYOUT_READ: cu_pools in memory, written by layout_scan_kernel before;
//   POOL_LAYOUT_ONE:  one document (cu = {0, num_tokens}): pool p starts at
//                     token kpool*p, and no layout is read before the key rows;
//   POOL_LAYOUT_LDS:  at most POOL_LDS_DOCS documents: every workgroup reads cu
//                     and scans the pool counts in LDS.
// With ONE and LDS, workgroup 0 also writes cu_pools (the launch is the whole
// of the layout and pooling).
enum { POOL_LAYOUT_READ = 0, POOL_LAYOUT_ONE = 1, POOL_LAYOUT_LDS = 2 };
constexpr int POOL_LDS_DOCS = 1024;
template <int L, int KP, int LAYOUT>
__global__ __launch_bounds__(256) void pool_keys_kernel(
    const int32_t* __restrict__ cu, int num_docs, int num_tokens, int32_t* __restrict__ cu_pools,
    const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ gate,
    const float* __restrict__ ape, int kpool, int pool_cap, float norm,
    int32_t* __restrict__ pool_start, uint8_t* __restrict__ k8, float* __restrict__ ks,
    float* __restrict__ kf32, int p_base, int token_lo) {
    constexpr int N = 4 * L;
    const int lane = threadIdx.x & 63;
    const int j = lane % L;
    const int p = p_base + (int)((blockIdx.x * blockDim.x + threadIdx.x) / L);
    int total, d = 0, s;
    if constexpr (LAYOUT == POOL_LAYOUT_ONE) {
        total = num_tokens / kpool;
        if (blockIdx.x == 0 && threadIdx.x == 0) { cu_pools[0] = 0; cu_pools[1] = total; }
        if (p >= pool_cap) return;
        s = kpool * p;
    } else if constexpr (LAYOUT == POOL_LAYOUT_LDS) {
        // cu into LDS, then an exclusive scan of floor(length / kpool): thread t
        // owns documents 4t .. 4t+3
        __shared__ int scu[POOL_LDS_DOCS + 1], scp[POOL_LDS_DOCS + 1];
        __shared__ int wtot[4];
        const int tid = threadIdx.x;
        for (int e = tid; e <= num_docs; e += 256) scu[e] = cu[e];
        __syncthreads();
        int cnt[4], sum = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int dd = 4 * tid + k;
            cnt[k] = dd < num_docs ? (scu[dd + 1] - scu[dd]) / kpool : 0;
            sum += cnt[k];
        }
        const int incl = wave_incl_scan(sum);
        if (lane == 63) wtot[tid >> 6] = incl;
        __syncthreads();
        int run = incl - sum;
        for (int w = 0; w < (tid >> 6); ++w) run += wtot[w];
        if (tid == 0) scp[0] = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            run += cnt[k];
            if (4 * tid + k < num_docs) scp[4 * tid + k + 1] = run;
        }
        __syncthreads();
        if (blockIdx.x == 0)
            for (int e = tid; e <= num_docs; e += 256) cu_pools[e] = scp[e];
        if (p >= pool_cap) return;
        total = scp[num_docs];
        if (p < total) {
            // document of pool p: the d with cu_pools[d] <= p < cu_pools[d+1]
            d = find_doc(scp, num_docs, p);
            s = scu[d] + kpool * (p - scp[d]);
        }
    } else {
        if (p >= pool_cap) return;
        total = cu_pools[num_docs];
        if (p < total) {
            d = find_doc(cu_pools, num_docs, p);
            s = cu[d] + kpool * (p - cu_pools[d]);
        }
    }
    if (p >= total) {
        if (j == 0) { pool_start[p] = -1; ks[p] = 0.0f; }
        reinterpret_cast<uint32_t*>(k8 + (size_t)p * N)[j] = 0u;
        if (kf32) reinterpret_cast<float4*>(kf32 + (size_t)p * N)[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        return;
    }
    if (s + kpool - 1 < token_lo) return;   // a pool of the caller's cache

    float x[4];
    pool_vector<L, KP>(x, k_idx, gate, ape, kpool, j, [&](int i) { return (size_t)(s + i); });
    if (kf32) reinterpret_cast<float4*>(kf32 + (size_t)p * N)[j] = make_float4(x[0], x[1], x[2], x[3]);
    fwht4<L>(x, lane, norm);
    float sc;
    uint32_t codes = quant4<L>(x, &sc);
    reinterpret_cast<uint32_t*>(k8 + (size_t)p * N)[j] = codes;
    if (j == 0) { ks[p] = sc; pool_start[p] = s; }
}

// Paged cache: document d's tokens live in pages of 32*kpool token slots and
// its pools in pages of 32 pool rows, page q of d at table[d*max_pages + q]
// (token l of d in slot table[..][l / (32 kpool)] * 32 kpool + l % (32 kpool),
// pool j in row table[..][j / 32] * 32 + j % 32). Grid: per_doc pool slots per
// document, one pool per L lanes; slot u of d is pool j_first(d) + u, the pools
// whose last token is among d's last `last_tokens` tokens. A page number
// outside [0, num_pages), or a pool past the document's max_pages pages, is
// left unwritten.
template <int L, int KP>
__global__ __launch_bounds__(256) void pool_keys_paged_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ table, int max_pages,
    int num_pages, const uint16_t* __restrict__ k_idx, const uint16_t* __restrict__ gate,
    const float* __restrict__ ape, int kpool, float norm, uint8_t* __restrict__ k8, float* __restrict__ ks,
    int last_tokens, int per_doc) {
    constexpr int N = 4 * L;
    const int lane = threadIdx.x & 63;
    const int j = lane % L;
    const long long u = ((long long)blockIdx.x * blockDim.x + threadIdx.x) / L;
    if (u >= (long long)num_docs * per_doc) return;
    const int d = (int)(u / per_doc);
    const int len = cu[d + 1] - cu[d];
    const int first_tok = len - last_tokens;                  // pools ending at or after it
    const int lo = first_tok <= kpool - 1 ? 0 : (first_tok - (kpool - 1) + kpool - 1) / kpool;
    const int pj = lo + (int)(u % per_doc);
    if (pj >= len / kpool) return;
    const int page_tok = 32 * kpool;
    const int* trow = table + (size_t)d * max_pages;
    const int s = kpool * pj;                                  // the pool's first token (of d)
    if (s / page_tok >= max_pages || (pj >> 5) >= max_pages) return;   // past the document's table row
    const int tpage = trow[s / page_tok];                      // (the pool's tokens share a page)
    const int ppage = trow[pj >> 5];
    if (tpage < 0 || tpage >= num_pages || ppage < 0 || ppage >= num_pages) return;
    const size_t tok0 = (size_t)tpage * page_tok + s % page_tok;

    float x[4];
    pool_vector<L, KP>(x, k_idx, gate, ape, kpool, j, [&](int i) { return tok0 + i; });
    fwht4<L>(x, lane, norm);
    float sc;
    uint32_t codes = quant4<L>(x, &sc);
    const size_t prow = (size_t)ppage * 32 + (pj & 31);
    reinterpret_cast<uint32_t*>(k8 + prow * N)[j] = codes;
    if (j == 0) ks[prow] = sc;
}

// ---------------------------------------------------------- queries ---------
// One (query, head) vector per L lanes: bf16 -> fp32 (exact), rotate, quantise.
// A block covers R groups of 256/L consecutive vectors and each lane loads its
// R pieces before any shuffle, so R loads per lane are in flight at once (one
// per lane leaves too few bytes in flight to cover HBM latency). Vectors past
// `rows` are computed on zeros and not stored; every lane stays active for the
// shuffles.
template <int L, int R>
__global__ __launch_bounds__(256) void rotate_quant_kernel(const uint16_t* __restrict__ q_idx,
                                                           long long rows, float norm,
                                                           uint8_t* __restrict__ codes,
                                                           float* __restrict__ scales) {
    constexpr int N = 4 * L;
    constexpr int GROUP = 256 / L;   // vectors per block per step
    const int lane = threadIdx.x & 63;
    const int j = lane % L;
    const long long r0 = (long long)blockIdx.x * (GROUP * R) + threadIdx.x / L;
    uint2 q[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const long long r = r0 + (long long)k * GROUP;
        q[k] = r < rows ? reinterpret_cast<const uint2*>(q_idx + (size_t)r * N)[j] : make_uint2(0u, 0u);
    }
#pragma unroll
    for (int k = 0; k < R; ++k) {
        const long long r = r0 + (long long)k * GROUP;
        float x[4] = {bf16_lo(q[k].x), bf16_hi(q[k].x), bf16_lo(q[k].y), bf16_hi(q[k].y)};
        fwht4<L>(x, lane, norm);
        float sc;
        uint32_t c = quant4<L>(x, &sc);
        if (r < rows) {
            reinterpret_cast<uint32_t*>(codes + (size_t)r * N)[j] = c;
            if (j == 0) scales[r] = sc;
        }
    }
}

// ------------------------------------------------------------ launchers -----
template <int KP, int LAYOUT>
static void launch_pool_keys(int blocks, hipStream_t stream, int d_idx, const int32_t* cu, int num_docs,
                             int num_tokens, int32_t* cu_pools, const uint16_t* k_idx, const uint16_t* gate,
                             const float* ape, int kpool, int pool_cap, float norm, int32_t* pool_start,
                             uint8_t* k8, float* ks, float* kf32, int p_base, int token_lo) {
#define KP_POOL_ARGS cu, num_docs, num_tokens, cu_pools, k_idx, gate, ape, kpool, pool_cap, norm, pool_start, k8, ks, \
                     kf32, p_base, token_lo
    switch (d_idx) {
        case 32: pool_keys_kernel<8, KP, LAYOUT><<<blocks, 256, 0, stream>>>(KP_POOL_ARGS); break;
        case 64: pool_keys_kernel<16, KP, LAYOUT><<<blocks, 256, 0, stream>>>(KP_POOL_ARGS); break;
        default: pool_keys_kernel<32, KP, LAYOUT><<<blocks, 256, 0, stream>>>(KP_POOL_ARGS); break;
    }
#undef KP_POOL_ARGS
}

template <int LAYOUT>
static void launch_pool_keys_kp(int blocks, hipStream_t stream, int d_idx, const int32_t* cu, int num_docs,
                                int num_tokens, int32_t* cu_pools, const uint16_t* k_idx, const uint16_t* gate,
                                const float* ape, int kpool, int pool_cap, float norm, int32_t* pool_start,
                                uint8_t* k8, float* ks, float* kf32, int p_base, int token_lo) {
    if (kpool == 4)
        launch_pool_keys<4, LAYOUT>(blocks, stream, d_idx, cu, num_docs, num_tokens, cu_pools, k_idx, gate, ape,
                                    kpool, pool_cap, norm, pool_start, k8, ks, kf32, p_base, token_lo);
    else
        launch_pool_keys<0, LAYOUT>(blocks, stream, d_idx, cu, num_docs, num_tokens, cu_pools, k_idx, gate, ape,
                                    kpool, pool_cap, norm, pool_start, k8, ks, kf32, p_base, token_lo);
}

hipError_t launch_layout_pool(const int32_t* cu, int num_docs, int num_tokens, const uint16_t* k_idx,
                              const uint16_t* gate, const float* ape, int d_idx, int kpool,
                              float norm, int32_t* cu_pools, int32_t* pool_start, uint8_t* k8,
                              float* ks, float* kf32, int token_lo, hipStream_t stream) {
    const int pool_cap = num_tokens / kpool;
    // (one launch does the layout and the pooling when the documents fit the
    // in-workgroup scan; a row of more documents scans them first, in its own launch)
    const int layout = num_docs == 1 ? POOL_LAYOUT_ONE : num_docs <= POOL_LDS_DOCS ? POOL_LAYOUT_LDS
                                                                                  : POOL_LAYOUT_READ;
    if (layout == POOL_LAYOUT_READ || pool_cap == 0) {
        layout_scan_kernel<<<1, 1024, 0, stream>>>(cu, num_docs, kpool, cu_pools);
        if (pool_cap == 0) return hipGetLastError();
    }
    // With token_lo > 0 only pools ending at or after token_lo (and the rows past
    // the last pool) are written. Every such pool has a global number of at least
    // (token_lo - (kpool-1) - num_docs*(kpool-1)) / kpool, since each document
    // leaves fewer than kpool of its tokens out of its pools; the launch starts
    // there, and the pools between that bound and token_lo return at once.
    int p_base = 0;
    if (token_lo > 0) {
        const long long lb = ((long long)token_lo - (kpool - 1) - (long long)num_docs * (kpool - 1)) / kpool;
        p_base = (int)(lb > 0 ? (lb < pool_cap ? lb : pool_cap) : 0);
    }
    if (p_base >= pool_cap) return hipGetLastError();
    const int L = d_idx / 4;
    const long long threads = (long long)(pool_cap - p_base) * L;
    const int blocks = (int)((threads + 255) / 256);
#define KP_POOL_LAUNCH(LAYOUT_)                                                                      \
    launch_pool_keys_kp<LAYOUT_>(blocks, stream, d_idx, cu, num_docs, num_tokens, cu_pools, k_idx, gate, ape, \
                                 kpool, pool_cap, norm, pool_start, k8, ks, kf32, p_base, token_lo)
    if (layout == POOL_LAYOUT_ONE) KP_POOL_LAUNCH(POOL_LAYOUT_ONE);
    else if (layout == POOL_LAYOUT_LDS) KP_POOL_LAUNCH(POOL_LAYOUT_LDS);
    else KP_POOL_LAUNCH(POOL_LAYOUT_READ);
#undef KP_POOL_LAUNCH
    return hipGetLastError();
}

hipError_t launch_pool_paged(const int32_t* cu, int num_docs, const int32_t* table, int max_pages, int num_pages,
                             const uint16_t* k_idx, const uint16_t* gate, const float* ape, int d_idx, int kpool,
                             float norm, uint8_t* k8, float* ks, int last_tokens, hipStream_t stream) {
    if (num_docs == 0 || last_tokens == 0) return hipSuccess;
    // a document's last `last_tokens` tokens close at most last_tokens / kpool + 1 pools
    const int per_doc = last_tokens / kpool + 1;
    const int L = d_idx / 4;
    const long long threads = (long long)num_docs * per_doc * L;
    const long long blocks = (threads + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
#define KP_PAGED_ARGS cu, num_docs, table, max_pages, num_pages, k_idx, gate, ape, kpool, norm, k8, ks, last_tokens, per_doc
    const unsigned b = (unsigned)blocks;
    if (kpool == 4) {
        switch (d_idx) {
            case 32: pool_keys_paged_kernel<8, 4><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
            case 64: pool_keys_paged_kernel<16, 4><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
            default: pool_keys_paged_kernel<32, 4><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
        }
    } else {
        switch (d_idx) {
            case 32: pool_keys_paged_kernel<8, 0><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
            case 64: pool_keys_paged_kernel<16, 0><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
            default: pool_keys_paged_kernel<32, 0><<<b, 256, 0, stream>>>(KP_PAGED_ARGS); break;
        }
    }
#undef KP_PAGED_ARGS
    return hipGetLastError();
}

hipError_t launch_layout(const int32_t* cu, int num_docs, int kpool, int32_t* cu_pools, hipStream_t stream) {
    layout_scan_kernel<<<1, 1024, 0, stream>>>(cu, num_docs, kpool, cu_pools);
    return hipGetLastError();
}

hipError_t launch_rotate_quant(const uint16_t* q_idx, long long rows, int d_idx, float norm,
                               uint8_t* codes, float* scales, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    constexpr int R = 4;
    const int L = d_idx / 4;
    const long long per_block = (256 / L) * R;
    const unsigned blocks = (unsigned)((rows + per_block - 1) / per_block);
    switch (d_idx) {
        case 32: rotate_quant_kernel<8, R><<<blocks, 256, 0, stream>>>(q_idx, rows, norm, codes, scales); break;
        case 64: rotate_quant_kernel<16, R><<<blocks, 256, 0, stream>>>(q_idx, rows, norm, codes, scales); break;
        default: rotate_quant_kernel<32, R><<<blocks, 256, 0, stream>>>(q_idx, rows, norm, codes, scales); break;
    }
    return hipGetLastError();
}

}  // namespace kp
