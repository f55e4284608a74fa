// Fused FP8 indexer scoring and top-k for rows of many pools (decode over a
// long context): the [queries x pools] score tensor is never written.
//
// The selection is the one of topk.hip (prime-rl PR "GLM-5.3-Flash text
// model", Summary, third bullet: the top-k visible pools by indexer score,
// equal scores keeping the lower pool, listed ascending, then the query's own
// incomplete pool); only the route to it differs. Order pools by (score key
// descending, pool ascending): a total order in which the kept pools are
// exactly the first k. Any threshold (key, pool) whose count of pools at or
// above it lies in [k, cap] therefore holds every kept pool among those
// candidates, and an exact selection over the candidates gives the answer.
// Three launches:
//
//   1. fused_thresh_kernel, one workgroup per query: rows of at most `cap`
//      visible pools take every pool as a candidate; longer rows score every
//      s-th pool and take as threshold the sample of rank r = T*m/n in that
//      order (m samples, n pools, T the target count max(4k, cap/4), at most
//      3/4 cap; s ~ T/16, so r ~ 16 and at most 16384 samples): about T pools
//      clear it when the samples are representative, with a spread of about a
//      quarter of T (1/sqrt(r)); falling below k or above cap needs a count
//      some seven spreads away. Only its count decides correctness.
//   2. score_kernel in its emitting form (score.hip) scores every visible
//      pair and appends the pairs at or above the threshold, as (score bits,
//      pool), to the query's candidate list, counting all of them.
//   3. fused_select_kernel, one workgroup per query: when the count lies in
//      [k, cap], a radix select over the candidates in LDS (ties on the key
//      resolved by a second select over the pools), then the k kept pools in
//      ascending order through a bitmap of the row (a bitonic sort for rows
//      too long for it); otherwise (adversarial rows only) the workgroup
//      rescores every visible pool itself for each digit of an exact radix
//      select and writes the kept pools in one ordered pass.
//
// Scores here are computed as score_kernel computes them, bit for bit: the
// same MFMA dots (16 heads x 16 pools per v_mfma_f32_16x16x128_f8f6f4, the
// heads on the M dimension because one query is scored), then, per pool,
// acc = fma(w*sq of head h, ReLU(dot_h), acc) over h in order from acc = 0,
// and acc * sk; the running sum hops across the four 16-lane groups that hold
// the heads in turn.
//
// Pooled keys are addressed by global pool number, or through a page table of
// 32-pool pages; index rows then hold the page slots of the kept tokens.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_select.h"

namespace kp {

constexpr int FT_TH_THREADS = 512;
constexpr int FT_SEL_THREADS = 1024;
constexpr int FT_SEL_WAVES = FT_SEL_THREADS / 64;

// Pooled-key rows, by global pool number or through 32-pool pages.
struct KeyRows {
    const uint8_t* k8;
    const float* sk;
    const int32_t* table;   // nullptr: row = pool number
    int max_pages;
    int num_pages;          // page numbers outside [0, num_pages): no page
};

// Row of pool p of the document whose first pool is plo and whose page-table
// row starts at tab (-1: its page is missing or past the table row).
template <bool PAGED>
__device__ __forceinline__ long long key_row(const KeyRows& kr, int p, int plo, long long tab) {
    if (!PAGED) return p;
    const int l = p - plo;
    if ((l >> 5) >= kr.max_pages) return -1;
    const int pn = kr.table[tab + (l >> 5)];
    return (unsigned)pn < (unsigned)kr.num_pages ? (long long)pn * 32 + (l & 31) : -1;
}

// One query's operands with its heads as the MFMA's rows: a[hg] holds, in
// lane (n, g), bytes 32g .. 32g+31 of the codes of head 16*hg + n (zero past
// d_idx and past h_idx); wv[hg][e] = w*sq of head 16*hg + 4g + e.
struct HmQuery {
    i32x8 a[4];
    float wv[4][4];
};

// (every load is unconditional, its address clamped into the query's rows and
// the value zeroed after when it lies outside: a load under a condition costs
// a wait for all loads in flight)
__device__ __forceinline__ void hm_load_query(HmQuery& hq, const uint8_t* __restrict__ q8,
                                              const float* __restrict__ sq, const float* __restrict__ w, int i,
                                              int h_idx, int d_idx) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int dchunks = d_idx >> 4;
    uint4 lo4[4], hi4[4];
    float wv[4][4], sv[4][4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
        const int head = min(16 * hg + n, h_idx - 1);
        const uint8_t* src = q8 + ((size_t)i * h_idx + head) * d_idx;
        lo4[hg] = *reinterpret_cast<const uint4*>(src + 16 * min(2 * g, dchunks - 1));
        hi4[hg] = *reinterpret_cast<const uint4*>(src + 16 * min(2 * g + 1, dchunks - 1));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const size_t o = (size_t)i * h_idx + min(16 * hg + 4 * g + e, h_idx - 1);
            wv[hg][e] = w[o];
            sv[hg][e] = sq[o];
        }
    }
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
        const bool hv = 16 * hg + n < h_idx;
        const uint32_t ml = hv && 2 * g < dchunks ? 0xFFFFFFFFu : 0u;
        const uint32_t mh = hv && 2 * g + 1 < dchunks ? 0xFFFFFFFFu : 0u;
        const uint4 l = lo4[hg], u = hi4[hg];
        hq.a[hg] = i32x8{(int)(l.x & ml), (int)(l.y & ml), (int)(l.z & ml), (int)(l.w & ml),
                         (int)(u.x & mh), (int)(u.y & mh), (int)(u.z & mh), (int)(u.w & mh)};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t mw = 16 * hg + 4 * g + e < h_idx ? 0xFFFFFFFFu : 0u;
            hq.wv[hg][e] = __uint_as_float(__float_as_uint(wv[hg][e] * sv[hg][e]) & mw);
        }
    }
}

// Key of pool n of a 16-pool tile for the query of hq: lane (n, g) names the
// pool's key row (row < 0: no pool, key 0) and every lane of column n gets the
// key. Called by whole waves.
// B operand (32 code bytes of column n per lane) and key scale of the pool in
// key row `row`; row < 0: zero (the loads read row 0 and are dropped).
__device__ __forceinline__ void hm_load_pool(i32x8& b, float& s, const KeyRows& kr, int d_idx, long long row) {
    const int g = (threadIdx.x & 63) >> 4;
    const int dchunks = d_idx >> 4;
    const size_t r = row >= 0 ? (size_t)row : 0;
    const uint8_t* src = kr.k8 + r * d_idx;
    const uint4 lo4 = *reinterpret_cast<const uint4*>(src + 16 * min(2 * g, dchunks - 1));
    const uint4 hi4 = *reinterpret_cast<const uint4*>(src + 16 * min(2 * g + 1, dchunks - 1));
    const uint32_t sc = __float_as_uint(kr.sk[r]);
    // (zeroed by masks, not by selects: the compiler turns a select of a
    // loaded value into a branch that waits for the load right there)
    const uint32_t ml = row >= 0 && 2 * g < dchunks ? 0xFFFFFFFFu : 0u;
    const uint32_t mh = row >= 0 && 2 * g + 1 < dchunks ? 0xFFFFFFFFu : 0u;
    const uint32_t ms = row >= 0 ? 0xFFFFFFFFu : 0u;
    b = i32x8{(int)(lo4.x & ml), (int)(lo4.y & ml), (int)(lo4.z & ml), (int)(lo4.w & ml),
              (int)(hi4.x & mh), (int)(hi4.y & mh), (int)(hi4.z & mh), (int)(hi4.w & mh)};
    s = __uint_as_float(sc & ms);
}

__device__ __forceinline__ uint32_t hm_tile_key(const HmQuery& hq, int h_idx, int d_idx, const KeyRows& kr,
                                                long long row) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    i32x8 b;
    float s;
    hm_load_pool(b, s, kr, d_idx, row);
    f32x4 d[4];
#pragma unroll
    for (int hg = 0; hg < 4; ++hg)
        d[hg] = 16 * hg < h_idx ? mfma_fp8_16x16x128(hq.a[hg], b, f32x4{0.f, 0.f, 0.f, 0.f}) : f32x4{0.f, 0.f, 0.f, 0.f};
    // heads 16hg + 4gp .. +3 sit in lane group gp: each group folds its four
    // into the running sum, and the sum of group gp goes on to every lane
    float acc = 0.0f;
#pragma unroll
    for (int hg = 0; hg < 4; ++hg) {
#pragma unroll
        for (int gp = 0; gp < 4; ++gp) {
            if (16 * hg + 4 * gp < h_idx) {
                float t = acc;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (16 * hg + 4 * g + e < h_idx) t = __builtin_fmaf(hq.wv[hg][e], relu_f32(d[hg][e]), t);
                acc = __shfl(t, n + 16 * gp, 64);
            }
        }
    }
    return row >= 0 ? score_key(acc * s) : 0u;
}

// Key of the pool of lane (16g + n) among 64 consecutive entries (4 tiles);
// row_of(j) gives lane (n, *)'s key row for tile j.
template <typename RowOf>
__device__ __forceinline__ uint32_t hm_block_key(const HmQuery& hq, int h_idx, int d_idx, const KeyRows& kr,
                                                 RowOf row_of) {
    const int g = (threadIdx.x & 63) >> 4;
    uint32_t mine = 0u;
#pragma unroll 1
    for (int j = 0; j < 4; ++j) {
        const uint32_t k = hm_tile_key(hq, h_idx, d_idx, kr, row_of(j));
        if (g == j) mine = k;
    }
    return mine;
}

// Sampled keys: the threshold needs only a good estimate, so the head sum is
// a tree (each lane sums its own heads, then two cross-group adds) rather
// than score_kernel's sequential order. B operands of a wave's 4 tiles are
// loaded together, one block ahead of their use.
struct HmTiles {
    i32x8 b[4];
    float s[4];
};

__device__ __forceinline__ void hm_load_tiles(HmTiles& t, const KeyRows& kr, int d_idx, const long long (&row)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) hm_load_pool(t.b[j], t.s[j], kr, d_idx, row[j]);
}

// Key of the pool of lane (16g + n) among the 64 of a loaded block; NHG head
// groups of 16 (a compile-time count: a branch per group would keep the
// compiler from interleaving the tiles' MFMAs).
template <int NHG>
__device__ __forceinline__ uint32_t hm_sample_key(const HmQuery& hq, const HmTiles& t) {
    const int g = (threadIdx.x & 63) >> 4;
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg) {
            const f32x4 d = mfma_fp8_16x16x128(hq.a[hg], t.b[j], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = __builtin_fmaf(hq.wv[hg][e], relu_f32(d[e]), acc);
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        const uint32_t key = score_key(acc * t.s[j]);
        if (g == j) mine = key;
    }
    return mine;
}

// ------------------------------------------------------------ threshold -----
// One workgroup per query: each wave scores blocks wave, wave + NW, ... of 64
// samples, all the loads of its blocks issued before the first MFMA (one
// memory latency), then the workgroup selects the threshold from the samples
// in LDS.
constexpr int FT_TH_BATCH = 2;   // sample blocks per wave per round
template <bool PAGED, int NHG>
__global__ __launch_bounds__(FT_TH_THREADS) void fused_thresh_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const uint8_t* __restrict__ q8, const float* __restrict__ sq,
    const float* __restrict__ w, int h_idx, int d_idx, KeyRows kr, int topk, int cap,
    uint32_t* __restrict__ tau, int32_t* __restrict__ count) {
    constexpr int NTH = FT_TH_THREADS, NW = NTH / 64;
    __shared__ __align__(16) uint32_t keys[FT_SAMPLE_MAX];
    __shared__ int hist[2][RS_BINS];
    __shared__ int wave_buf[NW];
    __shared__ int sel[3];
    __shared__ int found;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15;
    const int i = blockIdx.x;
    // the query's operands depend on i alone: their loads go out before the
    // document lookup's
    HmQuery hq;
    hm_load_query(hq, q8, sq, w, i, h_idx, d_idx);
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = qp.n_vis;
    const int k = n < topk ? n : topk;
    if (k == 0 || n <= cap) {
        // nothing to keep: a threshold above every (key, pool); short row: every pool
        if (tid == 0) {
            tau[2 * i] = k == 0 ? 0xFFFFFFFFu : 0u;
            tau[2 * i + 1] = k == 0 ? 0xFFFFFFFFu : 0x7FFFFFFFu;
            count[i] = 0;
        }
        return;
    }
    // target count T = max(4k, cap/4) (at most 3/4 cap), stride about T/16, so
    // that the threshold is the sample of rank r ~ 16 (T = r n / m)
    const int target = min(cap / 4 * 3, max(4 * k, cap / 4));
    const int ss = max((n + FT_SAMPLE_MAX - 1) / FT_SAMPLE_MAX, max(1, target / 16));
    const int m = (n + ss - 1) / ss;   // samples: pools pool_lo + ss*j, j < m
    const long long tab = PAGED ? (long long)qp.doc * kr.max_pages : 0;
    for (int b0 = wave * 64; b0 < m; b0 += FT_TH_BATCH * NW * 64) {
        HmTiles tb[FT_TH_BATCH];
#pragma unroll
        for (int u = 0; u < FT_TH_BATCH; ++u) {
            long long row[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int sidx = b0 + u * NW * 64 + 16 * j + n16;
                row[j] = sidx < m ? key_row<PAGED>(kr, qp.pool_lo + ss * sidx, qp.pool_lo, tab) : -1;
            }
            hm_load_tiles(tb[u], kr, d_idx, row);
        }
#pragma unroll
        for (int u = 0; u < FT_TH_BATCH; ++u) {
            const int bu = b0 + u * NW * 64;
            const uint32_t key = hm_sample_key<NHG>(hq, tb[u]);
            if (bu + lane < m) keys[bu + lane] = key;
        }
    }
    __syncthreads();

    const int r = (int)max(1LL, min((long long)m, (long long)target * m / n));
    uint32_t th;
    int teq;
    radix_select<NTH>([&](auto f) {
        for (int j = tid; j < m; j += NTH) f(keys[j]);
    }, r, hist, sel, &th, &teq);
    uint32_t tp = 0x7FFFFFFFu;
    if (teq != RS_ALL_EQ) {
        // the teq-th sample with key th, in pool order (samples are in pool order)
        const int chunk = (m + NTH - 1) / NTH;
        const int j0 = min(m, tid * chunk), j1 = min(m, j0 + chunk);
        int c = 0;
        for (int j = j0; j < j1; ++j) c += keys[j] == th;
        int tot;
        const int before = block_excl_scan<NTH>(c, wave_buf, &tot);
        if (before < teq && before + c >= teq) {
            int need = teq - before;
            for (int j = j0; j < j1; ++j)
                if (keys[j] == th && --need == 0) found = j;
        }
        __syncthreads();
        tp = (uint32_t)(qp.pool_lo + ss * found);
    }
    if (tid == 0) {
        tau[2 * i] = th;
        tau[2 * i + 1] = tp;
        count[i] = 0;
    }
}

// -------------------------------------------------------------- select ------
template <bool PAGED>
__global__ __launch_bounds__(FT_SEL_THREADS) void fused_select_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const uint8_t* __restrict__ q8, const float* __restrict__ sq,
    const float* __restrict__ w, int h_idx, int d_idx, KeyRows kr, int topk, int cap,
    const int32_t* __restrict__ count, const uint2* __restrict__ cand, int row_width,
    int32_t* __restrict__ indices, int32_t* __restrict__ num_valid, int32_t* __restrict__ row_path) {
    constexpr int NTH = FT_SEL_THREADS, NW = FT_SEL_WAVES;
    constexpr int PER = FT_CAP / NTH;   // candidates per thread, at most
    __shared__ __align__(16) uint32_t ckey[FT_CAP];   // candidate keys, then the kept pools
    __shared__ __align__(16) int cpool[FT_CAP];
    __shared__ int hist[2][RS_BINS];
    __shared__ int wave_buf[NW];
    __shared__ int sel[3];
    __shared__ uint32_t red[2 * NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, n16 = lane & 15;
    const int i = blockIdx.x;
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = qp.n_vis, lo = qp.pool_lo, hi = qp.pool_lo + qp.n_vis;
    const int k = n < topk ? n : topk;
    const int doc_start = cu[qp.doc];
    const int page_tok = 32 * kpool;
    const long long tab = PAGED ? (long long)qp.doc * kr.max_pages : 0;
    int32_t* row = indices + (size_t)i * row_width;

    // slot of the document's token l (l counted from its first token; -1 when
    // its page is missing)
    auto slot = [&](int l) -> int {
        if (!PAGED) return doc_start + l;
        if (l / page_tok >= kr.max_pages) return -1;
        const int pn = kr.table[tab + l / page_tok];
        return (unsigned)pn < (unsigned)kr.num_pages ? pn * page_tok + l % page_tok : -1;
    };
    // the kpool tokens of pool p at rank pos of the row (a pool's tokens share a page)
    auto put_pool = [&](int pos, int p) {
        const int s0 = slot(kpool * (p - lo));
        const int st = s0 < 0 ? 0 : 1;
        if (kpool == 4) {
            *reinterpret_cast<int4*>(row + 4 * pos) = make_int4(s0, s0 + st, s0 + 2 * st, s0 + 3 * st);
        } else {
            for (int r = 0; r < kpool; ++r) row[pos * kpool + r] = s0 + r * st;
        }
    };

    const int cnt = count[i];
    const bool fits = k > 0 && cnt >= k && cnt <= cap;
    if (fits) {
        // the candidates into LDS, eight loads in flight per thread; keys are
        // kept relative to the smallest (all candidates cleared one threshold,
        // so they crowd the top few bins of a plain 32-bit digit)
        const uint2* src = cand + (size_t)i * cap;
        uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
        for (int j0 = 0; j0 < cnt; j0 += NTH * 8) {
            uint2 c[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)   // (unconditional loads: entries past cnt re-read the last)
                c[u] = src[min(j0 + tid + NTH * u, cnt - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + tid + NTH * u;
                if (j < cnt) {
                    const uint32_t key = score_key(__uint_as_float(c[u].x));   // (stored as score bits)
                    ckey[j] = key;
                    cpool[j] = (int)c[u].y;
                    kmin = min(kmin, key);
                    kmax = max(kmax, key);
                }
            }
        }
        block_min_max<NTH>(kmin, kmax, red, &kmin, &kmax);   // (its barriers publish ckey, cpool)
        uint32_t th = 0u, th2 = 0u;
        int teq = RS_ALL_EQ;
        if (k < cnt) {
            const int bits = kmax == kmin ? 0 : 32 - __builtin_clz(kmax - kmin);
            radix_select<NTH>([&](auto f) {
                for (int j = tid; j < cnt; j += NTH) f(ckey[j] - kmin);
            }, k, hist, sel, &th, &teq, bits);
            th += kmin;
            if (teq != RS_ALL_EQ) {
                // keys equal to th: keep the teq lowest pools (hi-1-pool largest);
                // pools are distinct, so this select is exact
                int teq2;
                const int pbits = n <= 1 ? 0 : 32 - __builtin_clz((uint32_t)(n - 1));
                radix_select<NTH>([&](auto f) {
                    for (int j = tid; j < cnt; j += NTH)
                        if (ckey[j] == th) f((uint32_t)(hi - 1 - cpool[j]));
                }, teq, hist, sel, &th2, &teq2, pbits);
            }
        }
        // kept flags of this thread's candidates j = tid + NTH*s, then their ranks
        uint32_t keep = 0u;
        int nk = 0;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int j = tid + NTH * s;
            if (j < cnt) {
                const uint32_t v = ckey[j];
                const bool kp = teq == RS_ALL_EQ ? v >= th
                                                 : (v > th || (v == th && (uint32_t)(hi - 1 - cpool[j]) >= th2));
                keep |= (uint32_t)kp << s;
                nk += kp;
            }
        }
        int tot;
        int pos = block_excl_scan<NTH>(nk, wave_buf, &tot);   // (its barriers end every read of ckey)
        int* list = reinterpret_cast<int*>(ckey);
        constexpr int MAP_WORDS = FT_CAP;   // the bitmap of a row of up to 32 * FT_CAP pools
        if (n <= 32 * MAP_WORDS) {
            // ascending pools through a bitmap of the row's pools: set the kept
            // ones, then each thread counts a run of words and writes its pools
            // at their ranks
            uint32_t* map = ckey;
            const int words = (n + 31) >> 5;
            for (int u = tid; u < words; u += NTH) map[u] = 0u;
            __syncthreads();
#pragma unroll
            for (int s = 0; s < PER; ++s)
                if (keep >> s & 1u) {
                    const int l = cpool[tid + NTH * s] - lo;
                    atomicOr(&map[l >> 5], 1u << (l & 31));
                }
            __syncthreads();
            const int run = (words + NTH - 1) / NTH;
            const int w0 = min(words, tid * run), w1 = min(words, w0 + run);
            int c = 0;
            for (int u = w0; u < w1; ++u) c += __popc(map[u]);
            int tot2;
            int r = block_excl_scan<NTH>(c, wave_buf, &tot2);
            for (int u = w0; u < w1; ++u)
                for (uint32_t b = map[u]; b; b &= b - 1)
                    if (r < k) put_pool(r++, lo + 32 * u + __builtin_ctz(b));   // (tot2 == k)
        } else {
#pragma unroll
        for (int s = 0; s < PER; ++s)
            if (keep >> s & 1u) list[pos++] = cpool[tid + NTH * s];
        __syncthreads();
        {
            // bitonic sort of the kept pools, padded to a power of two
            int P = 1;
            while (P < tot) P <<= 1;
            for (int p = tot + tid; p < P; p += NTH) list[p] = 0x7FFFFFFF;
            __syncthreads();
            for (int size = 2; size <= P; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int p = tid; p < P / 2; p += NTH) {
                        const int a_i = 2 * stride * (p / stride) + (p % stride), b_i = a_i + stride;
                        const bool up = (a_i & size) == 0;
                        const int a = list[a_i], b = list[b_i];
                        if ((a > b) == up) {
                            list[a_i] = b;
                            list[b_i] = a;
                        }
                    }
                    __syncthreads();
                }
            }
            for (int p = tid; p < min(tot, k); p += NTH) put_pool(p, list[p]);   // (tot == k)
        }
        }
    } else if (k > 0) {
        // exact selection by rescoring every visible pool for each digit
        HmQuery hq;
        hm_load_query(hq, q8, sq, w, i, h_idx, d_idx);
        auto block_key = [&](int base) -> uint32_t {   // key of pool base + lane (0 past hi)
            return hm_block_key(hq, h_idx, d_idx, kr, [&](int j) -> long long {
                const int p = base + 16 * j + n16;
                return p < hi ? key_row<PAGED>(kr, p, lo, tab) : -1;
            });
        };
        uint32_t th;
        int teq;
        radix_select<NTH>([&](auto f) {
            for (int base = lo + wave * 64; base < hi; base += NW * 64) {
                const uint32_t key = block_key(base);
                if (base + lane < hi) f(key);
            }
        }, k, hist, sel, &th, &teq);
        // one ordered pass: every pool above th, and the first teq equal to th
        int eq_run = 0, pos_run = 0;
        for (int base = lo; base < hi; base += NW * 64) {
            const int p = base + wave * 64 + lane;
            const uint32_t key = block_key(base + wave * 64);
            const bool valid = p < hi;
            const bool eq = valid && teq != RS_ALL_EQ && key == th;
            const bool gt = valid && (teq == RS_ALL_EQ ? key >= th : key > th);
            int tot_eq, tot_keep;
            const int eqb = eq_run + block_excl_scan<NTH>(eq, wave_buf, &tot_eq);
            const bool kp = gt || (eq && eqb < teq);
            const int pos = pos_run + block_excl_scan<NTH>(kp, wave_buf, &tot_keep);
            if (kp && pos < k) put_pool(pos, p);   // (exactly k are kept)
            eq_run += tot_eq;
            pos_run += tot_keep;
        }
    }
    // own incomplete pool, then padding
    const int base = k * kpool;
    const int n_tail = t - qp.tail_start + 1;
    for (int r = tid; r < row_width - base; r += NTH)
        row[base + r] = r < n_tail ? slot(kpool * n + r) : -1;
    if (tid == 0) {
        if (num_valid) num_valid[i] = base + n_tail;
        if (row_path) row_path[i] = fits || k == 0 ? 0 : 1;
    }
}

hipError_t launch_fused_topk(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                             const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq, const float* w,
                             int h_idx, int d_idx, const uint8_t* k8, const float* sk, int max_pools,
                             const int32_t* page_table, int max_pages, int num_pages, int topk, int row_width,
                             int32_t* indices, int32_t* num_valid, int32_t* row_path, const FusedState& st,
                             hipStream_t stream) {
    if (num_q == 0) return hipSuccess;
    const KeyRows kr{k8, sk, page_table, max_pages, num_pages};
#define KP_TH(PG, NH)                                                                                     \
    fused_thresh_kernel<PG, NH><<<num_q, FT_TH_THREADS, 0, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, q8, sq, \
                                                                     w, h_idx, d_idx, kr, topk, FT_CAP, st.tau,    \
                                                                     st.count)
    const int nhg = (h_idx + 15) / 16;
    if (page_table) {
        if (nhg == 1) KP_TH(true, 1); else if (nhg == 2) KP_TH(true, 2); else if (nhg == 3) KP_TH(true, 3);
        else KP_TH(true, 4);
    } else {
        if (nhg == 1) KP_TH(false, 1); else if (nhg == 2) KP_TH(false, 2); else if (nhg == 3) KP_TH(false, 3);
        else KP_TH(false, 4);
    }
#undef KP_TH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_score_emit(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w, h_idx, d_idx, k8, sk, max_pools,
                          page_table, max_pages, num_pages, st.tau, st.count, st.cand, FT_CAP, stream);
    if (e != hipSuccess) return e;
    if (page_table)
        fused_select_kernel<true><<<num_q, FT_SEL_THREADS, 0, stream>>>(
            cu, num_docs, cu_pools, kpool, q_pos, q8, sq, w, h_idx, d_idx, kr, topk, FT_CAP, st.count, st.cand,
            row_width, indices, num_valid, row_path);
    else
        fused_select_kernel<false><<<num_q, FT_SEL_THREADS, 0, stream>>>(
            cu, num_docs, cu_pools, kpool, q_pos, q8, sq, w, h_idx, d_idx, kr, topk, FT_CAP, st.count, st.cand,
            row_width, indices, num_valid, row_path);
    return hipGetLastError();
}

size_t fused_state_bytes(int num_q) {
    auto a = [](size_t x) { return (x + 255) & ~(size_t)255; };
    return a((size_t)num_q * 2 * sizeof(uint32_t)) + a((size_t)num_q * sizeof(int32_t)) +
           a((size_t)num_q * FT_CAP * sizeof(uint2));
}

FusedState fused_state_at(void* ws, int num_q) {
    auto a = [](size_t x) { return (x + 255) & ~(size_t)255; };
    uint8_t* p = static_cast<uint8_t*>(ws);
    FusedState st;
    st.tau = reinterpret_cast<uint32_t*>(p);
    p += a((size_t)num_q * 2 * sizeof(uint32_t));
    st.count = reinterpret_cast<int32_t*>(p);
    p += a((size_t)num_q * sizeof(int32_t));
    st.cand = reinterpret_cast<uint2*>(p);
    return st;
}

}  // namespace kp
