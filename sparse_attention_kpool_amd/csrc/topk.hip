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
// stops early when the bin holding the k-th key is kept whole (then no
// ordering among equal keys is needed). A final pass
// over contiguous per-thread chunks, in pool order, keeps every pool above K
// and the first pools equal to K, and writes each kept pool's tokens at its
// rank: the kept pools come out ascending with no sort. The keys of a row
// short enough stay in LDS between passes; longer rows are re-read.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_select.h"

namespace kp {

constexpr int TK_THREADS = 512;
constexpr int TK_LDS_KEYS = 8192;    // keys cached in LDS (32 KB)
constexpr int TK_BINS = 2048;        // histogram bins of the widest digit

// Keys j .. j+3 of the row (j a multiple of 4); entries at or past n read as 0.
// Cached rows read one 16-byte LDS vector; others read the scores.
template <bool CACHED>
__device__ __forceinline__ void fetch4(uint32_t (&kk)[4], const uint32_t* keys_lds, const float* srow,
                                       int j, int n) {
    if (CACHED) {
        const uint4 v = *reinterpret_cast<const uint4*>(keys_lds + j);
        kk[0] = v.x; kk[1] = v.y; kk[2] = v.z; kk[3] = v.w;
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[e] = j + e < n ? score_key(srow[j + e]) : 0u;
    }
}

template <bool CACHED>
__device__ __forceinline__ void topk_row(const uint32_t* keys_lds, int (*hist)[TK_BINS], int* wave_buf,
                                         int* sel, const float* srow, int n, int k, int kpool,
                                         int doc_start, int32_t* row) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool all = k >= n;        // every visible pool is kept (no scores needed)
    uint32_t thresh = 0xFFFFFFFFu;  // key of the k-th largest score (k == 0: above every key)
    int take_eq = 0;                // how many pools equal to thresh are kept (lowest first)
    constexpr int ALL_EQ = 0x7FFFFFFF;
    if (!all && k > 0) {
        for (int b = tid; b < TK_BINS; b += TK_THREADS) hist[0][b] = 0;
        __syncthreads();            // cached keys and the first histogram are ready
        int remaining = k;          // still to choose among keys matching the prefix
        uint32_t prefix = 0u, pmask = 0u;
        take_eq = -1;
        // Two barriers per digit: the histogram is complete, then the bin is
        // known. The histograms alternate between two buffers, so the one for
        // the next digit is cleared while this one is counted.
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int width = pass < 2 ? 11 : 10;
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nb = 1 << width;
            int* h = hist[pass & 1];
#pragma unroll 2
            for (int j = 4 * tid; j < n; j += 4 * TK_THREADS) {
                uint32_t kk[4];
                fetch4<CACHED>(kk, keys_lds, srow, j, n);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < n && (kk[e] & pmask) == prefix)
                        atomicAdd(&h[(kk[e] >> shift) & (uint32_t)(nb - 1)], 1);
            }
            for (int b = tid; b < TK_BINS; b += TK_THREADS) hist[(pass + 1) & 1][b] = 0;
            __syncthreads();
            if (wave == 0) {
                // lane l owns bins [nb - per*(l+1), nb - per*l): a scan over lanes
                // counts the keys in the bins above each lane's
                const int per = nb >> 6;    // 32 or 16
                const int base = nb - per * (lane + 1);
                int4 r[8];
                int own = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    r[q] = make_int4(0, 0, 0, 0);
                    if (4 * q < per) r[q] = *reinterpret_cast<const int4*>(h + base + 4 * q);
                    own += r[q].x + r[q].y + r[q].z + r[q].w;
                }
                const int incl = wave_incl_scan(own);
                const int before = incl - own;
                if (before < remaining && incl >= remaining) {
                    int acc = before;
#pragma unroll
                    for (int m = 31; m >= 0; --m) {
                        if (m < per) {
                            const int4 v = r[m >> 2];
                            const int c = (m & 3) == 0 ? v.x : (m & 3) == 1 ? v.y : (m & 3) == 2 ? v.z : v.w;
                            if (acc < remaining && acc + c >= remaining) {
                                sel[0] = base + m;
                                sel[1] = acc;
                                sel[2] = c;
                            }
                            acc += c;
                        }
                    }
                }
            }
            __syncthreads();
            const int sel_digit = sel[0], sel_above = sel[1], sel_cnt = sel[2];
            remaining -= sel_above;
            prefix |= (uint32_t)sel_digit << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            if (sel_cnt == remaining) {
                // the whole bin is kept: every key >= prefix (low bits zero) is selected
                take_eq = ALL_EQ;
                break;
            }
        }
        thresh = prefix;
        if (take_eq < 0) take_eq = remaining;
    }

    // final pass: contiguous chunks (multiples of 4) per thread, in pool order
    const int chunk = ((n + TK_THREADS - 1) / TK_THREADS + 3) & ~3;
    const int j0 = min(n, tid * chunk), j1 = min(n, j0 + chunk);
    int tot;
    // rank among the keys equal to thresh, needed only when ties are split
    int eq_before = 0;
    if (!all && take_eq != ALL_EQ) {
        int n_eq = 0;
        for (int j = j0; j < j1; j += 4) {
            uint32_t kk[4];
            fetch4<CACHED>(kk, keys_lds, srow, j, n);
#pragma unroll
            for (int e = 0; e < 4; ++e) n_eq += (j + e < j1 && kk[e] == thresh);
        }
        eq_before = block_excl_scan<TK_THREADS>(n_eq, wave_buf, &tot);
    }
    int n_sel = 0;
    if (!all) {
        int e_rank = eq_before;
        for (int j = j0; j < j1; j += 4) {
            uint32_t kk[4];
            fetch4<CACHED>(kk, keys_lds, srow, j, n);
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (j + e < j1) n_sel += kk[e] > thresh || (kk[e] == thresh && e_rank++ < take_eq);
        }
    } else {
        n_sel = j1 - j0;
    }
    const int sel_before = block_excl_scan<TK_THREADS>(n_sel, wave_buf, &tot);
    int e_rank = eq_before, pos = sel_before;
    for (int j = j0; j < j1; j += 4) {
        uint32_t kk[4] = {0u, 0u, 0u, 0u};
        if (!all) fetch4<CACHED>(kk, keys_lds, srow, j, n);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (j + e >= j1) break;
            const bool keep = all || kk[e] > thresh || (kk[e] == thresh && e_rank++ < take_eq);
            if (keep) {
                const int tok = doc_start + kpool * (j + e);
                if (kpool == 4) {   // the four tokens of the pool as one 16-byte store
                    *reinterpret_cast<int4*>(row + 4 * pos) = make_int4(tok, tok + 1, tok + 2, tok + 3);
                } else {
                    for (int r = 0; r < kpool; ++r) row[pos * kpool + r] = tok + r;
                }
                ++pos;
            }
        }
    }
}

__device__ void mw_init(int32_t* row, int row_width, int n, int k);

__global__ __launch_bounds__(TK_THREADS) void topk_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices, int32_t* __restrict__ num_valid, int skip_long) {
    __shared__ __align__(16) uint32_t keys_lds[TK_LDS_KEYS];
    __shared__ __align__(16) int hist[2][TK_BINS];
    __shared__ int wave_buf[TK_THREADS / 64];
    __shared__ int sel[3];   // selected digit, keys in bins above it, keys in it

    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = qp.n_vis;
    const int k = n < topk ? n : topk;
    const int doc_start = cu[qp.doc];
    int32_t* row = indices + (size_t)i * row_width;
    const float* srow = scores + (size_t)i * max_pools + qp.pool_lo;
    if (skip_long && n > TK_LDS_KEYS) {   // a row for the long-row kernels
        if (skip_long == 2) mw_init(row, row_width, n, k);
        return;
    }

    if (n <= TK_LDS_KEYS) {
        if (k < n && k > 0) {
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
        topk_row<true>(keys_lds, hist, wave_buf, sel, srow, n, k, kpool, doc_start, row);
    } else {
        topk_row<false>(keys_lds, hist, wave_buf, sel, srow, n, k, kpool, doc_start, row);
    }
    // own incomplete pool, then padding
    const int base = k * kpool;
    const int n_tail = t - qp.tail_start + 1;
    for (int r = tid; r < row_width - base; r += TK_THREADS)
        row[base + r] = r < n_tail ? qp.tail_start + r : -1;
    if (tid == 0 && num_valid) num_valid[i] = base + n_tail;
}

// ------------------------------------------------------- one wave per row ----
// When no row has more than TW_KEYS visible pools, each row gets one wave that
// holds the row's keys in registers. The same radix select then runs with no
// barrier: the histogram is the wave's own LDS array (lane l owns the bins
// below nb - per*l, which it reads to pick the digit and clears for the next
// one), counting is branchless, and the ordered final pass ranks the kept pools
// with ballots or a scan over lanes. Registers are visited in chunks of TW_C,
// one scalar test per chunk.
//
// Slots: the row is read from `base`, its first score or (with 16-byte loads)
// the 16-byte boundary at or below it, a = 0..3 slots earlier; slot s holds pool
// s - a. With 16-byte loads (vec4: the score rows' stride is a multiple of four
// and the buffer is 16-byte aligned, so a row's 16-byte chunks lie in its own
// row) register 4g + c of lane l holds slot 256g + 4l + c; otherwise register r
// holds slot 64r + l.
constexpr int TW_KEYS = 8192, TW_R = TW_KEYS / 64, TW_WAVES = 4, TW_C = 16;

// BODY runs for r = 0 .. TW_C*nch - 1 (r a compile-time constant in it). nch
// passes through an empty asm first, so the compiler recomputes the scalar
// chunk tests in each loop instead of keeping them live across the kernel.
#define TW_FOR_REGS(nch, BODY)                                                   \
    {                                                                            \
        int nc_ = (nch);                                                         \
        __asm__ volatile("" : "+s"(nc_));                                        \
        _Pragma("unroll") for (int c_ = 0; c_ < R / TW_C; ++c_) {                \
            if (c_ < nc_) {                                                      \
                _Pragma("unroll") for (int u_ = 0; u_ < TW_C; ++u_) {            \
                    const int r = TW_C * c_ + u_;                                \
                    BODY                                                         \
                }                                                                \
            }                                                                    \
        }                                                                        \
    }
// the same over groups g of four registers (4g .. 4g+3)
#define TW_FOR_GROUPS(nch, BODY)                                                 \
    {                                                                            \
        int nc_ = (nch);                                                         \
        __asm__ volatile("" : "+s"(nc_));                                        \
        _Pragma("unroll") for (int c_ = 0; c_ < R / TW_C; ++c_) {                \
            if (c_ < nc_) {                                                      \
                _Pragma("unroll") for (int u_ = 0; u_ < TW_C / 4; ++u_) {        \
                    const int g = TW_C / 4 * c_ + u_;                            \
                    BODY                                                         \
                }                                                                \
            }                                                                    \
        }                                                                        \
    }

// add + the lanes below this one set in each of the four masks
__device__ __forceinline__ int tw_mbcnt4(uint64_t b0, uint64_t b1, uint64_t b2, uint64_t b3, int add) {
    uint32_t x = __builtin_amdgcn_mbcnt_lo((uint32_t)b0, (uint32_t)add);
    x = __builtin_amdgcn_mbcnt_hi((uint32_t)(b0 >> 32), x);
    x = __builtin_amdgcn_mbcnt_lo((uint32_t)b1, x);
    x = __builtin_amdgcn_mbcnt_hi((uint32_t)(b1 >> 32), x);
    x = __builtin_amdgcn_mbcnt_lo((uint32_t)b2, x);
    x = __builtin_amdgcn_mbcnt_hi((uint32_t)(b2 >> 32), x);
    x = __builtin_amdgcn_mbcnt_lo((uint32_t)b3, x);
    return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b3 >> 32), x);
}

// One compare-exchange step of a bitonic sort of one value per lane: the partner
// is lane ^ J; in blocks of KK lanes with (lane & KK) == 0 the lower lane keeps
// the larger value (descending), in the others the smaller.
#define TW_BITONIC_STEP(KK, J)                                                                   \
    {                                                                                            \
        const uint32_t p_ = __float_as_uint(lane_xor<J>(__uint_as_float(v)));                   \
        const bool desc_ = (lane & (KK)) == 0 || (KK) == 64, low_ = (lane & (J)) == 0;           \
        v = desc_ == low_ ? max(v, p_) : min(v, p_);                                             \
    }

// R key registers per lane: this instance takes the rows of 64*RLO < S <= 64*R
// slots, so that shorter rows run with fewer registers and more waves per SIMD.
template <bool KP4, int R, int RLO>
__global__ __launch_bounds__(64 * TW_WAVES, R > 64 ? 2 : 5) void topk_wave_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices, int32_t* __restrict__ num_valid, int num_q, int vec4) {
    static_assert(R % TW_C == 0 && R <= TW_R, "register count");
    // digits of at most MAXW bits: 2048 bins for the long rows, 1024 for the short
    // ones (a smaller LDS share per wave, so that more waves fit per SIMD)
    constexpr int NB = R > 64 ? 2048 : 1024, MAXW = R > 64 ? 11 : 10;
    // per wave: NB bins, then one spare word per lane that takes the counts and
    // writes of lanes with nothing to count or keep (no branch around them)
    __shared__ __align__(16) int hist_all[TW_WAVES][NB + 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // rows are taken last first: under the causal mask the later queries of a
    // document see more pools, so the longest rows start first and the launch
    // ends on short ones
    const int j = __builtin_amdgcn_readfirstlane(blockIdx.x * TW_WAVES + wave);
    if (j >= num_q) return;
    const int i = num_q - 1 - j;
    if (KP4) kpool = 4;
    int* hist = hist_all[wave];
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = __builtin_amdgcn_readfirstlane(qp.n_vis);
    const float* srow = scores + (size_t)i * max_pools + qp.pool_lo;
    const int a = vec4 ? (int)(((uintptr_t)srow >> 2) & 3) : 0;   // slots before the row's first pool
    const int S = n + a;                                            // slots up to the row's last pool
    if (S > 64 * R || (RLO > 0 && S <= 64 * RLO)) return;          // another instance's row
    const int k = n < topk ? n : topk;
    const int doc_start = cu[qp.doc];
    int32_t* row = indices + (size_t)i * row_width;
    const uint64_t below = (1ull << lane) - 1ull;
    auto put = [&](int pos, int j) __attribute__((always_inline)) {
        const int tok = doc_start + kpool * j;
        if (KP4) {   // the four tokens of the pool as one 16-byte store
            *reinterpret_cast<int4*>(row + 4 * pos) = make_int4(tok, tok + 1, tok + 2, tok + 3);
        } else {
            for (int q = 0; q < kpool; ++q) row[pos * kpool + q] = tok + q;
        }
    };
    // the slot of register r in this lane
    auto slot_of = [&](int r) __attribute__((always_inline)) {
        return vec4 ? 256 * (r >> 2) + 4 * lane + (r & 3) : 64 * r + lane;
    };

    if (k >= n) {
        // every visible pool is kept, in order
        for (int j = lane; j < n; j += 64) put(j, j);
    } else if (k > 0) {
        const int nch = (S + 64 * TW_C - 1) / (64 * TW_C);   // chunks of registers in use
        const int n_pad = 64 * TW_C * nch - n;               // their slots outside the row
        uint32_t key[R];
        // the sample (below) is loaded first, then the row: a buffer that ends with
        // the row (with 16-byte loads: with the 16-byte chunk holding its last pool),
        // so slots past its end read 0
        const float sample = srow[(lane * n) >> 6];
        const __amdgpu_buffer_rsrc_t srsc = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(srow - a), 0, vec4 ? 4 * ((S + 3) & ~3) : 4 * n, 0x00020000);
        if (vec4) {
            typedef int v4i __attribute__((ext_vector_type(4)));
            TW_FOR_GROUPS(nch, {
                const v4i v = __builtin_amdgcn_raw_buffer_load_b128(srsc, 16 * lane + 1024 * g, 0, 0);
                key[4 * g] = v.x; key[4 * g + 1] = v.y; key[4 * g + 2] = v.z; key[4 * g + 3] = v.w;
            })
            // slots of the first and last 16-byte chunks outside the row: 0
            if (lane == 0) {
#pragma unroll
                for (int c = 0; c < 3; ++c)
                    if (c < a) key[c] = 0u;
            }
            const int gl = (S - 1) >> 8, ll = ((S - 1) >> 2) & 63, cl = (S - 1) & 3;
            TW_FOR_GROUPS(nch, {
                if (g == gl && lane == ll) {
                    if (cl < 1) key[4 * g + 1] = 0u;
                    if (cl < 2) key[4 * g + 2] = 0u;
                    if (cl < 3) key[4 * g + 3] = 0u;
                }
            })
        } else {
            TW_FOR_REGS(nch, key[r] = __builtin_amdgcn_raw_buffer_load_b32(srsc, 4 * lane + 256 * r, 0, 0);)
        }
        // A lower bound lo (in key space) from 64 pools sampled along the row: the
        // sample of rank t from the top (t samples at least as large before it), t
        // about twice the expected 64 k / n plus 4, so that the k-th largest key lies
        // above lo but for rare rows. Only keys at or above lo enter the histograms;
        // a row where fewer than k do is selected again over every key (lo = 0: the
        // plain radix select).
        uint32_t lo = 0u, smax = 0u;   // smax: the largest sample
        if (n >= 2048) {
            // the samples' keys sorted across the wave, largest in lane 0 (bitonic:
            // blocks of kk lanes, even blocks descending, merged at distance j)
            uint32_t v = score_key(sample);
            TW_BITONIC_STEP(2, 1)
            TW_BITONIC_STEP(4, 2) TW_BITONIC_STEP(4, 1)
            TW_BITONIC_STEP(8, 4) TW_BITONIC_STEP(8, 2) TW_BITONIC_STEP(8, 1)
            TW_BITONIC_STEP(16, 8) TW_BITONIC_STEP(16, 4) TW_BITONIC_STEP(16, 2) TW_BITONIC_STEP(16, 1)
            TW_BITONIC_STEP(32, 16) TW_BITONIC_STEP(32, 8) TW_BITONIC_STEP(32, 4) TW_BITONIC_STEP(32, 2)
            TW_BITONIC_STEP(32, 1)
            TW_BITONIC_STEP(64, 32) TW_BITONIC_STEP(64, 16) TW_BITONIC_STEP(64, 8) TW_BITONIC_STEP(64, 4)
            TW_BITONIC_STEP(64, 2) TW_BITONIC_STEP(64, 1)
            const int tr = min(63, (128 * k + n - 1) / n + 4);
            lo = (uint32_t)__builtin_amdgcn_readlane((int)v, tr);
            smax = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
        }
#pragma unroll
        for (int q = 0; q < NB / 256; ++q)
            *reinterpret_cast<int4*>(hist + (NB / 64) * lane + 4 * q) = make_int4(0, 0, 0, 0);

        int remaining = k;
        uint32_t prefix = 0u, pmask = 0u;
        bool pad_bin0 = false;   // the slots outside the row (key 0) are counted in bin 0
        // the digit of bits [shift, shift + width) of the counted offsets from the
        // counts in hist: the bin holding the remaining-th largest key. Returns 1 when
        // that whole bin is kept, 0 when not, -1 when fewer than `remaining` keys were
        // counted (then nothing has changed but the histogram, which is cleared).
        auto pick = [&](int shift, int width) __attribute__((always_inline)) -> int {
            const int nb = 1 << width;
            // a wave's LDS operations complete in order
            if (lane == 0 && pad_bin0 && prefix == 0u && n_pad > 0) hist[0] -= n_pad;
            // lane l owns bins [nb - per*(l+1), nb - per*l) (with fewer than 64 bins,
            // lanes l < nb own one each): a scan over lanes counts the keys in the bins
            // above each lane's
            const int per = nb >= 64 ? nb >> 6 : 1;   // 1 .. NB / 64
            const int base = nb - per * (lane + 1);
            int own = 0;
            if (per >= 4) {
#pragma unroll
                for (int q = 0; q < NB / 256; ++q)
                    if (4 * q < per) {
                        const int4 v = *reinterpret_cast<const int4*>(hist + base + 4 * q);
                        own += (v.x + v.y) + (v.z + v.w);
                    }
            } else if (base >= 0) {
                own = hist[base] + (per == 2 ? hist[base + 1] : 0);
            }
            const int incl = wave_incl_scan(own);
            const bool enough = __builtin_amdgcn_readlane(incl, 63) >= remaining;
            int res = -1;
            if (enough) {
                // the lane whose bins hold the remaining-th largest key; then one of its
                // bins per lane (lane m: the m-th from the top) and a scan over them
                const int before = incl - own;
                const int src = __builtin_ctzll(__ballot(before < remaining && incl >= remaining));
                const int acc0 = __builtin_amdgcn_readlane(before, src);
                const int top_bin = nb - 1 - per * src;
                const int c = lane < per ? hist[top_bin - lane] : 0;
                const int ci = wave_incl_scan(c);
                const int m = __builtin_ctzll(__ballot(lane < per && acc0 + ci - c < remaining && acc0 + ci >= remaining));
                const int sel_digit = top_bin - m;
                const int sel_above = acc0 + __builtin_amdgcn_readlane(ci - c, m);
                const int sel_cnt = __builtin_amdgcn_readlane(c, m);
                remaining -= sel_above;
                prefix |= (uint32_t)sel_digit << shift;
                pmask |= (uint32_t)(nb - 1) << shift;
                res = sel_cnt == remaining ? 1 : 0;
            }
            // clear the bins for the next digit (after the reads above)
            if (per >= 4) {
#pragma unroll
                for (int q = 0; q < NB / 256; ++q)
                    if (4 * q < per) *reinterpret_cast<int4*>(hist + base + 4 * q) = make_int4(0, 0, 0, 0);
            } else if (base >= 0) {
                hist[base] = 0;
                if (per == 2) hist[base + 1] = 0;
            }
            return res;
        };
        // count one for lane's value in bin b when `in` (else in the lane's spare word)
        int* const spare = hist + NB + lane;
        auto count = [&](bool in, uint32_t b) __attribute__((always_inline)) {
            atomicAdd(in ? hist + b : spare, 1);
        };
        bool whole = false;
        uint32_t thr, top;   // the threshold and the largest counted value, in the keys' units

        // Positive bound: every kept pool has a positive score, and the raw bits of
        // positive floats order as the scores do, so the keys stay raw (slots outside
        // the row hold +0, never counted). A raw value v is counted when lo_raw <= v
        // <= +inf (0x7F800000), one unsigned test that also drops negative scores
        // (sign bit set) and NaN; the digits are cut from the span [lo_raw, largest
        // counted value] as in the general path below.
        bool fast = lo > 0x80000000u;
        if (fast) {
            const uint32_t lo_raw = lo & 0x7FFFFFFFu, lim0 = 0x7F800000u - lo_raw;
            // the first digit's span from the largest sample (values above it are
            // counted in the top bin); should the k-th largest value fall in that top
            // bin, the row is counted again with the span from its largest value
            int B = 32 - __builtin_clz(((smax & 0x7FFFFFFFu) - lo_raw) | 1u);
            bool est = smax > lo;
#pragma unroll 1
            for (int tries = 0; tries < 2; ++tries) {
                // (the bound passes through an empty asm, so that no per-register test is
                // hoisted out of this loop)
                uint32_t lr = lo_raw;
                __asm__ volatile("" : "+s"(lr));
                if (!est) {
                    uint32_t omax = 0u;   // largest counted offset v - lo_raw
                    TW_FOR_REGS(nch, {
                        const uint32_t o = key[r] - lr;
                        omax = max(omax, o <= lim0 ? o : 0u);
                    })
#pragma unroll
                    for (int m = 1; m < 64; m <<= 1) omax = max(omax, (uint32_t)__shfl_xor((int)omax, m, 64));
                    omax = __builtin_amdgcn_readfirstlane(omax);
                    B = omax == 0u ? 0 : 32 - __builtin_clz(omax);
                }
                // B == 0: every counted value equals lo_raw (handled by the final pass)
                if (B == 0) break;
                const int s0 = max(B - MAXW, 0), w0 = B - s0;
                const uint32_t top0 = (1u << w0) - 1u;
                TW_FOR_REGS(nch, {
                    const uint32_t o = key[r] - lr;
                    count(o <= lim0, min(o >> s0, top0));
                })
                const int res = pick(s0, w0);
                if (res < 0) {
                    fast = false;
                    lo = 0u;
                    break;
                }
                if (est && (prefix >> s0) == top0) {   // the top bin (clamped values): exact span
                    est = false;
                    remaining = k;
                    prefix = pmask = 0u;
                    continue;
                }
                whole = res > 0;
#pragma unroll 1
                for (int low = s0; low > 0 && !whole;) {
                    const int width = min(low, MAXW), shift = low - width;
                    low = shift;
                    const uint32_t kb0 = lo_raw + prefix, lim = 1u << (shift + width);
                    TW_FOR_REGS(nch, {
                        const uint32_t o = key[r] - kb0;
                        count(o < lim, o >> shift);
                    })
                    whole = pick(shift, width) > 0;
                }
                break;
            }
            if (fast && B == 0) {
                // nothing above lo_raw: the count of values equal to lo_raw decides
                int cnt = 0;
                TW_FOR_REGS(nch, cnt += __popcll(__ballot(key[r] == lo_raw));)
                if (cnt < k) {
                    fast = false;
                    lo = 0u;
                }
            }
            if (fast) {
                thr = lo_raw + prefix;
                top = 0x7F800000u;
            }
        }
        if (!fast) {
            // order-preserving keys; slots outside the row get key 0
            TW_FOR_REGS(nch, key[r] = (uint32_t)(slot_of(r) - a) < (uint32_t)n ? score_key(__uint_as_float(key[r]))
                                                                                : 0u;)
            uint32_t kmax = 0u;
            TW_FOR_REGS(nch, kmax = max(kmax, key[r]);)
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) kmax = max(kmax, (uint32_t)__shfl_xor((int)kmax, m, 64));
            kmax = __builtin_amdgcn_readfirstlane(kmax);
#pragma unroll 1
            for (int attempt = 0; attempt < 2; ++attempt) {
                pad_bin0 = lo == 0u;
                // the span's significant bits are cut into digits from the top, MAXW bits
                // each but the last (the first digit as fine as the bins allow)
                const uint32_t span = kmax - lo;
                const int B = span == 0u ? 0 : 32 - __builtin_clz(span);
                if (B == 0) break;   // every key at or above lo is equal: ties in pool order
                // first digit: every key at or above lo
                const int s0 = max(B - MAXW, 0), w0 = B - s0;
                TW_FOR_REGS(nch, count(key[r] >= lo, (key[r] - lo) >> s0);)
                const int res = pick(s0, w0);
                if (res < 0) {   // lo was above the k-th largest key: all keys
                    lo = 0u;
                    continue;
                }
                whole = res > 0;
                // later digits: the keys matching the digits so far, lo + prefix <= key <
                // lo + prefix + 2^(shift + width) (a bound that changes every pass, so no
                // test is hoisted)
#pragma unroll 1
                for (int low = s0; low > 0 && !whole;) {
                    const int width = min(low, MAXW), shift = low - width;
                    low = shift;
                    const uint32_t kb0 = lo + prefix, lim = 1u << (shift + width);
                    TW_FOR_REGS(nch, count(key[r] - kb0 < lim, (key[r] - kb0) >> shift);)
                    whole = pick(shift, width) > 0;
                }
                break;
            }
            thr = lo + prefix;
            top = 0xFFFFFFFFu;
        }

        // Ordered final pass: with a whole bin kept, every value v with thr <= v <=
        // top (thr is above 0: fewer than n pools are kept); otherwise those above thr
        // and the first `remaining` equal to it, in pool order. Slots outside the row
        // (0) are never kept: 0 is below thr, those after the row come after every
        // pool equal to thr, and those before it are left out of the equal ones.
        const uint32_t lge = top - thr;
        const bool has_gt = thr < top;
        const uint32_t agt = thr + 1u, lgt = top - thr - 1u;
        int pos = 0;
        auto mbcnt = [&](uint64_t m, int add) __attribute__((always_inline)) {
            return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, add));
        };
        // pools of 4 tokens and k <= NB: the kept pools' numbers go to the wave's
        // histogram array at their ranks, and the index row is written from there
        // with contiguous 16-byte stores; otherwise each kept pool is stored directly
        const bool via_lds = KP4 && k <= NB;
        // register r: ranks by ballot (slot 64r + lane)
#define TW_FINAL_REGS(EMIT)                                                                               \
    if (whole) {                                                                                          \
        TW_FOR_REGS(nch, {                                                                                \
            const bool keep = key[r] - thr <= lge;                                                        \
            const uint64_t kb = __ballot(keep);                                                           \
            EMIT(keep, mbcnt(kb, pos), 64 * r + lane);                                                    \
            pos += __popcll(kb);                                                                          \
        })                                                                                                \
    } else {                                                                                              \
        int eq_seen = 0;                                                                                  \
        TW_FOR_REGS(nch, {                                                                                \
            const bool eq = key[r] == thr;                                                                \
            const uint64_t eb = __ballot(eq);                                                             \
            const bool keep = (has_gt & (key[r] - agt <= lgt)) | (eq & (mbcnt(eb, eq_seen) < remaining)); \
            eq_seen += __popcll(eb);                                                                      \
            const uint64_t kb = __ballot(keep);                                                           \
            EMIT(keep, mbcnt(kb, pos), 64 * r + lane);                                                    \
            pos += __popcll(kb);                                                                          \
        })                                                                                                \
    }
        // group g (slots 256g + 4*lane + c): a kept slot's rank is the count kept in
        // earlier groups, in the lanes below (all four registers: one ballot each,
        // counted with a chain of mbcnt), and in the lane's own earlier registers
#define TW_MBCNT4(b0, b1, b2, b3, add) tw_mbcnt4(b0, b1, b2, b3, add)
#define TW_FINAL_GROUPS(EMIT)                                                                             \
    {                                                                                                     \
        int eq_seen = 0;                                                                                  \
        TW_FOR_GROUPS(nch, {                                                                              \
            bool kp[4];                                                                                   \
            if (whole) {                                                                                  \
                _Pragma("unroll") for (int c = 0; c < 4; ++c) kp[c] = key[4 * g + c] - thr <= lge;        \
            } else {                                                                                      \
                bool eq[4];                                                                               \
                uint64_t eb[4];                                                                           \
                _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                           \
                    eq[c] = key[4 * g + c] == thr && (g > 0 || lane > 0 || c >= a);                       \
                    eb[c] = __ballot(eq[c]);                                                              \
                }                                                                                         \
                int er = TW_MBCNT4(eb[0], eb[1], eb[2], eb[3], eq_seen);                                  \
                _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                           \
                    kp[c] = (has_gt & (key[4 * g + c] - agt <= lgt)) | (eq[c] & (er < remaining));        \
                    er += eq[c];                                                                          \
                    eq_seen += __popcll(eb[c]);                                                           \
                }                                                                                         \
            }                                                                                             \
            uint64_t kb[4];                                                                               \
            _Pragma("unroll") for (int c = 0; c < 4; ++c) kb[c] = __ballot(kp[c]);                        \
            int p = TW_MBCNT4(kb[0], kb[1], kb[2], kb[3], pos);                                           \
            _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                               \
                EMIT(kp[c], p, 256 * g + 4 * lane + c - a);                                               \
                p += kp[c];                                                                               \
                pos += __popcll(kb[c]);                                                                   \
            }                                                                                             \
        })                                                                                                \
    }
#define TW_EMIT_LDS(keep, p, j) (*((keep) ? hist + (p) : spare) = (j))
#define TW_EMIT_PUT(keep, p, j) \
    if (keep) put((p), (j))
        if (vec4) {
            if (via_lds) {
                TW_FINAL_GROUPS(TW_EMIT_LDS)
            } else {
                TW_FINAL_GROUPS(TW_EMIT_PUT)
            }
        } else {
            if (via_lds) {
                TW_FINAL_REGS(TW_EMIT_LDS)
            } else {
                TW_FINAL_REGS(TW_EMIT_PUT)
            }
        }
#undef TW_FINAL_REGS
#undef TW_FINAL_GROUPS
#undef TW_MBCNT4
#undef TW_EMIT_LDS
#undef TW_EMIT_PUT
        if (via_lds) {
            for (int q = lane; q < k; q += 64) put(q, hist[q]);
        }
    }
    // own incomplete pool, then padding
    const int base = k * kpool;
    const int n_tail = t - qp.tail_start + 1;
    for (int r = lane; r < row_width - base; r += 64) row[base + r] = r < n_tail ? qp.tail_start + r : -1;
    if (lane == 0 && num_valid) num_valid[i] = base + n_tail;
}
#undef TW_FOR_REGS
#undef TW_FOR_GROUPS
#undef TW_BITONIC_STEP

// ------------------------------------------------------------- long rows ----
// Rows with more visible pools than the LDS key cache (decode over a long
// context) go to the many-workgroup kernels below when their index rows have
// room for the scratch; otherwise each gets a workgroup of 1024 threads: the same radix select with the
// scores streamed from memory in 16-byte loads, several in flight per thread;
// when the boundary bin is kept whole (no tie is split) the kept pools are
// collected in LDS in any order, sorted (bitonic) and written out with
// contiguous 16-byte stores. A row whose selection splits ties takes the
// ordered chunk scan of the short-row kernel instead.
constexpr int TL_THREADS = 1024;
constexpr int TL_LIST = 4096;    // kept pools collected in LDS

__device__ __forceinline__ void fetch4_g(uint32_t (&kk)[4], const float* srow, int j, int n, bool aligned) {
    if (aligned && j + 3 < n) {
        const float4 v = *reinterpret_cast<const float4*>(srow + j);
        kk[0] = score_key(v.x); kk[1] = score_key(v.y); kk[2] = score_key(v.z); kk[3] = score_key(v.w);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[e] = j + e < n ? score_key(srow[j + e]) : 0u;
    }
}

__global__ __launch_bounds__(TL_THREADS) void topk_long_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices, int32_t* __restrict__ num_valid) {
    __shared__ __align__(16) int hist[2][TK_BINS];
    __shared__ int wave_buf[TL_THREADS / 64];
    __shared__ int sel[3];
    __shared__ int list[TL_LIST];
    __shared__ int list_n;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int i = blockIdx.x;
    const int t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
    const int n = qp.n_vis;
    if (n <= TK_LDS_KEYS) return;   // a row for topk_kernel
    const int k = n < topk ? n : topk;
    const int doc_start = cu[qp.doc];
    int32_t* row = indices + (size_t)i * row_width;
    const float* srow = scores + (size_t)i * max_pools + qp.pool_lo;
    const bool aligned = (reinterpret_cast<uintptr_t>(srow) & 15) == 0;
    constexpr int ALL_EQ = 0x7FFFFFFF;

    auto put_pool = [&](int pos, int j) {
        const int tok = doc_start + kpool * j;
        if (kpool == 4) {
            *reinterpret_cast<int4*>(row + 4 * pos) = make_int4(tok, tok + 1, tok + 2, tok + 3);
        } else {
            for (int r = 0; r < kpool; ++r) row[pos * kpool + r] = tok + r;
        }
    };

    if (k >= n) {   // every visible pool is kept, in order
        for (int j = tid; j < n; j += TL_THREADS) put_pool(j, j);
    } else if (k > 0) {
        for (int b = tid; b < TK_BINS; b += TL_THREADS) hist[0][b] = 0;
        __syncthreads();
        int remaining = k;
        uint32_t prefix = 0u, pmask = 0u;
        int take_eq = -1;
#pragma unroll 1
        for (int pass = 0; pass < 3; ++pass) {
            const int width = pass < 2 ? 11 : 10;
            const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
            const int nb = 1 << width;
            int* h = hist[pass & 1];
#pragma unroll 4
            for (int j = 4 * tid; j < n; j += 4 * TL_THREADS) {
                uint32_t kk[4];
                fetch4_g(kk, srow, j, n, aligned);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < n && (kk[e] & pmask) == prefix)
                        atomicAdd(&h[(kk[e] >> shift) & (uint32_t)(nb - 1)], 1);
            }
            for (int b = tid; b < TK_BINS; b += TL_THREADS) hist[(pass + 1) & 1][b] = 0;
            __syncthreads();
            if (wave == 0) {
                const int per = nb >> 6;
                const int base = nb - per * (lane + 1);
                int4 r[8];
                int own = 0;
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    r[q] = make_int4(0, 0, 0, 0);
                    if (4 * q < per) r[q] = *reinterpret_cast<const int4*>(h + base + 4 * q);
                    own += r[q].x + r[q].y + r[q].z + r[q].w;
                }
                const int incl = wave_incl_scan(own);
                const int before = incl - own;
                if (before < remaining && incl >= remaining) {
                    int acc = before;
#pragma unroll
                    for (int m = 31; m >= 0; --m) {
                        if (m < per) {
                            const int4 v = r[m >> 2];
                            const int c = (m & 3) == 0 ? v.x : (m & 3) == 1 ? v.y : (m & 3) == 2 ? v.z : v.w;
                            if (acc < remaining && acc + c >= remaining) {
                                sel[0] = base + m;
                                sel[1] = acc;
                                sel[2] = c;
                            }
                            acc += c;
                        }
                    }
                }
            }
            __syncthreads();
            const int sel_digit = sel[0], sel_above = sel[1], sel_cnt = sel[2];
            remaining -= sel_above;
            prefix |= (uint32_t)sel_digit << shift;
            pmask |= (uint32_t)(nb - 1) << shift;
            if (sel_cnt == remaining) {
                take_eq = ALL_EQ;
                break;
            }
        }
        const uint32_t thresh = prefix;
        if (take_eq < 0) take_eq = remaining;

        if (take_eq == ALL_EQ && k <= TL_LIST) {
            // exactly the k keys >= thresh are kept: collect, sort, write
            if (tid == 0) list_n = 0;
            __syncthreads();
#pragma unroll 4
            for (int j = 4 * tid; j < n; j += 4 * TL_THREADS) {
                uint32_t kk[4];
                fetch4_g(kk, srow, j, n, aligned);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < n && kk[e] >= thresh) {
                        const int pos = atomicAdd(&list_n, 1);   // ends at exactly k
                        if (pos < TL_LIST) list[pos] = j + e;
                    }
            }
            __syncthreads();
            int P = 1;
            while (P < k) P <<= 1;
            for (int p = k + tid; p < P; p += TL_THREADS) list[p] = 0x7FFFFFFF;
            __syncthreads();
            for (int size = 2; size <= P; size <<= 1) {
                for (int stride = size >> 1; stride > 0; stride >>= 1) {
                    for (int p = tid; p < P / 2; p += TL_THREADS) {
                        const int lo = 2 * stride * (p / stride) + (p % stride), hi = lo + stride;
                        const bool up = (lo & size) == 0;
                        const int a = list[lo], b = list[hi];
                        if ((a > b) == up) {
                            list[lo] = b;
                            list[hi] = a;
                        }
                    }
                    __syncthreads();
                }
            }
            for (int pos = tid; pos < k; pos += TL_THREADS) put_pool(pos, list[pos]);
        } else {
            // ties split (or too many kept for LDS): ordered contiguous chunks per thread
            const int chunk = ((n + TL_THREADS - 1) / TL_THREADS + 3) & ~3;
            const int j0 = min(n, tid * chunk), j1 = min(n, j0 + chunk);
            int tot, n_eq = 0, n_sel = 0;
            for (int j = j0; j < j1; j += 4) {
                uint32_t kk[4];
                fetch4_g(kk, srow, j, n, aligned);
#pragma unroll
                for (int e = 0; e < 4; ++e) n_eq += (j + e < j1 && kk[e] == thresh);
            }
            const int eq_before = block_excl_scan<TL_THREADS>(n_eq, wave_buf, &tot);
            int e_rank = eq_before;
            for (int j = j0; j < j1; j += 4) {
                uint32_t kk[4];
                fetch4_g(kk, srow, j, n, aligned);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (j + e < j1) n_sel += kk[e] > thresh || (kk[e] == thresh && e_rank++ < take_eq);
            }
            int pos = block_excl_scan<TL_THREADS>(n_sel, wave_buf, &tot);
            e_rank = eq_before;
            for (int j = j0; j < j1; j += 4) {
                uint32_t kk[4];
                fetch4_g(kk, srow, j, n, aligned);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    if (j + e >= j1) break;
                    if (kk[e] > thresh || (kk[e] == thresh && e_rank++ < take_eq)) put_pool(pos++, j + e);
                }
            }
        }
    }
    // own incomplete pool, then padding
    const int base = k * kpool;
    const int n_tail = t - qp.tail_start + 1;
    for (int r = tid; r < row_width - base; r += TL_THREADS)
        row[base + r] = r < n_tail ? qp.tail_start + r : -1;
    if (tid == 0 && num_valid) num_valid[i] = base + n_tail;
}

// ------------------------------------------------ long rows, many workgroups --
// A long row (decode over a long context) is cut into chunks of TM_CHUNK pools,
// one workgroup each, and the radix select runs as a sequence of launches: per
// digit, every chunk adds its histogram to the row's (global atomics), then one
// wave per row picks the digit; then every chunk counts its keys above and equal
// to the threshold, and writes its kept pools at their ranks in pool order. The
// scratch lives in the row's own index slots, which only the last launches write:
//   row[0 .. TK_BINS)                  histogram of the current digit
//   row[W - TM_STATE .. W)             prefix (the threshold when done), digit mask,
//                                      keys still to choose, done, equal keys kept
//   row[W - TM_STATE - 2*C .. )        per chunk: keys above, keys equal
// (C chunks of the widest row). The host takes this path only when the rows have
// room for it; otherwise topk_long_kernel runs.
constexpr int TM_CHUNK = 8192;
constexpr int TM_THREADS = 512;
constexpr int TM_STATE = 8;
constexpr int TM_ALL_EQ = 0x7FFFFFFF;

// digit PASS: width and position of its bits in the key
template <int PASS> struct TmDigit {
    static constexpr int width = PASS < 2 ? 11 : 10;
    static constexpr int shift = PASS == 0 ? 21 : (PASS == 1 ? 10 : 0);
    static constexpr int nb = 1 << width;
};

struct TmRow {
    int n, k, t, tail_start, doc_start;
    const float* srow;
    int32_t* row;
    int32_t* st;   // state
    int32_t* cc;   // chunk counts
};

__device__ __forceinline__ TmRow tm_row(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                                       const int32_t* q_pos, const float* scores, int max_pools, int topk,
                                       int row_width, int32_t* indices, int i) {
    TmRow r;
    r.t = q_pos ? q_pos[i] : i;
    const QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, r.t);
    r.n = qp.n_vis;
    r.k = r.n < topk ? r.n : topk;
    r.tail_start = qp.tail_start;
    r.doc_start = cu[qp.doc];
    r.srow = scores + (size_t)i * max_pools + qp.pool_lo;
    r.row = indices + (size_t)i * row_width;
    r.st = r.row + row_width - TM_STATE;
    r.cc = r.st - 2 * ((max_pools + TM_CHUNK - 1) / TM_CHUNK);
    return r;
}

// by topk_kernel, for a long row: zero histogram, initial state
__device__ void mw_init(int32_t* row, int row_width, int n, int k) {
    for (int b = threadIdx.x; b < TK_BINS; b += blockDim.x) row[b] = 0;
    if (threadIdx.x == 0) {
        int32_t* st = row + row_width - TM_STATE;
        const bool done = k == 0 || k >= n;   // nothing to choose: keep none, or every pool
        st[0] = k == 0 ? (int32_t)0xFFFFFFFFu : 0;   // prefix; once done, the threshold key
        st[1] = 0;                                 // bits of the key fixed by the prefix
        st[2] = k;                                 // keys still to choose among the prefix's
        st[3] = done;
        st[4] = k == 0 ? 0 : TM_ALL_EQ;            // keys equal to the threshold kept
    }
}

template <int PASS>
__global__ __launch_bounds__(TM_THREADS) void topk_mw_hist_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices) {
    using Dg = TmDigit<PASS>;
    __shared__ int h[Dg::nb];
    const TmRow r = tm_row(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices,
                           blockIdx.x);
    const int c0 = blockIdx.y * TM_CHUNK;
    if (r.n <= TK_LDS_KEYS || c0 >= r.n || r.st[3]) return;
    const int c1 = min(r.n, c0 + TM_CHUNK);
    const uint32_t prefix = (uint32_t)r.st[0], pmask = (uint32_t)r.st[1];
    const bool aligned = (reinterpret_cast<uintptr_t>(r.srow) & 15) == 0;
    for (int b = threadIdx.x; b < Dg::nb; b += TM_THREADS) h[b] = 0;
    __syncthreads();
#pragma unroll 4
    for (int j = c0 + 4 * threadIdx.x; j < c1; j += 4 * TM_THREADS) {
        uint32_t kk[4];
        fetch4_g(kk, r.srow, j, c1, aligned);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < c1 && (kk[e] & pmask) == prefix) atomicAdd(&h[(kk[e] >> Dg::shift) & (Dg::nb - 1)], 1);
    }
    __syncthreads();
    for (int b = threadIdx.x; b < Dg::nb; b += TM_THREADS)
        if (h[b]) atomicAdd(&r.row[b], h[b]);
}

// one wave per row: the digit holding the remaining-th largest key
template <int PASS>
__global__ __launch_bounds__(64) void topk_mw_select_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices) {
    using Dg = TmDigit<PASS>;
    const TmRow r = tm_row(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices,
                           blockIdx.x);
    if (r.n <= TK_LDS_KEYS || r.st[3]) return;
    const int lane = threadIdx.x;
    const int remaining = r.st[2];
    // lane l owns bins [nb - per*(l+1), nb - per*l); a scan over lanes counts the
    // keys in the bins above each lane's
    constexpr int per = Dg::nb >> 6;   // 32 or 16
    const int base = Dg::nb - per * (lane + 1);
    int cnt[per];
    int own = 0;
#pragma unroll
    for (int m = 0; m < per; ++m) {
        cnt[m] = r.row[base + m];
        own += cnt[m];
    }
    const int incl = wave_incl_scan(own);
    const int before = incl - own;
    int sdig = 0, sabove = 0, scnt = 0;
    if (before < remaining && incl >= remaining) {
        int acc = before;
#pragma unroll
        for (int m = per - 1; m >= 0; --m) {
            if (acc < remaining && acc + cnt[m] >= remaining) {
                sdig = base + m;
                sabove = acc;
                scnt = cnt[m];
            }
            acc += cnt[m];
        }
    }
    const unsigned long long who = __ballot(before < remaining && incl >= remaining);
    const int src = who ? __builtin_ctzll(who) : 0;   // (one lane holds the boundary)
    sdig = __shfl(sdig, src, 64);
    sabove = __shfl(sabove, src, 64);
    scnt = __shfl(scnt, src, 64);
    for (int b = lane; b < TK_BINS; b += 64) r.row[b] = 0;   // the next digit's histogram
    if (lane == 0) {
        const int rem = remaining - sabove;
        const bool whole = scnt == rem;   // the bin is kept whole: no tie is split
        r.st[0] = (int32_t)((uint32_t)r.st[0] | ((uint32_t)sdig << Dg::shift));
        r.st[1] = (int32_t)((uint32_t)r.st[1] | ((uint32_t)(Dg::nb - 1) << Dg::shift));
        r.st[2] = rem;
        r.st[3] = whole || PASS == 2;
        r.st[4] = whole ? TM_ALL_EQ : rem;
    }
}

// per chunk: keys above and equal to the threshold
__global__ __launch_bounds__(TM_THREADS) void topk_mw_count_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices) {
    __shared__ int wave_buf[TM_THREADS / 64];
    const TmRow r = tm_row(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices,
                           blockIdx.x);
    const int c0 = blockIdx.y * TM_CHUNK;
    if (r.n <= TK_LDS_KEYS || c0 >= r.n) return;
    const int c1 = min(r.n, c0 + TM_CHUNK);
    const uint32_t thresh = (uint32_t)r.st[0];
    const bool aligned = (reinterpret_cast<uintptr_t>(r.srow) & 15) == 0;
    int gt = 0, eq = 0;
#pragma unroll 4
    for (int j = c0 + 4 * threadIdx.x; j < c1; j += 4 * TM_THREADS) {
        uint32_t kk[4];
        fetch4_g(kk, r.srow, j, c1, aligned);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < c1) {
                gt += kk[e] > thresh;
                eq += kk[e] == thresh;
            }
    }
    // (16 bits each: a chunk has at most TM_CHUNK keys)
    int tot;
    block_excl_scan<TM_THREADS>(gt | (eq << 16), wave_buf, &tot);
    if (threadIdx.x == 0) {
        r.cc[2 * blockIdx.y] = tot & 0xFFFF;
        r.cc[2 * blockIdx.y + 1] = tot >> 16;
    }
}

// per chunk: its kept pools at their ranks, in pool order
__global__ __launch_bounds__(TM_THREADS) void topk_mw_write_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices) {
    __shared__ int wave_buf[TM_THREADS / 64];
    const TmRow r = tm_row(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices,
                           blockIdx.x);
    const int c = blockIdx.y, c0 = c * TM_CHUNK;
    if (r.n <= TK_LDS_KEYS || c0 >= r.n) return;
    const int c1 = min(r.n, c0 + TM_CHUNK);
    const uint32_t thresh = (uint32_t)r.st[0];
    const int take_eq = r.st[4];
    // kept pools and keys equal to the threshold in the chunks before this one
    int pos0 = 0, eqb = 0;
    for (int q = 0; q < c; ++q) {
        const int gq = r.cc[2 * q], eqq = r.cc[2 * q + 1];
        const int keq = take_eq == TM_ALL_EQ ? eqq : max(0, min(eqq, take_eq - eqb));
        pos0 += gq + keq;
        eqb += eqq;
    }
    // contiguous runs of TM_RUN keys per thread, in pool order, read once
    constexpr int TM_RUN = TM_CHUNK / TM_THREADS;
    static_assert(TM_RUN % 4 == 0, "runs of whole 16-byte groups");
    const int j0 = c0 + (int)threadIdx.x * TM_RUN;
    const bool aligned = (reinterpret_cast<uintptr_t>(r.srow) & 15) == 0;
    uint32_t kk[TM_RUN];
#pragma unroll
    for (int q = 0; q < TM_RUN; q += 4) {
        uint32_t k4[4];
        fetch4_g(k4, r.srow, j0 + q, c1, aligned);   // (keys at or past c1 read as 0 and are skipped)
#pragma unroll
        for (int e = 0; e < 4; ++e) kk[q + e] = k4[e];
    }
    int tot, n_eq = 0;
#pragma unroll
    for (int q = 0; q < TM_RUN; ++q) n_eq += (j0 + q < c1 && kk[q] == thresh);
    const int eq_before = eqb + block_excl_scan<TM_THREADS>(n_eq, wave_buf, &tot);
    int e_rank = eq_before, n_sel = 0;
#pragma unroll
    for (int q = 0; q < TM_RUN; ++q)
        if (j0 + q < c1) n_sel += kk[q] > thresh || (kk[q] == thresh && e_rank++ < take_eq);
    int pos = pos0 + block_excl_scan<TM_THREADS>(n_sel, wave_buf, &tot);
    e_rank = eq_before;
#pragma unroll
    for (int q = 0; q < TM_RUN; ++q) {
        if (j0 + q < c1 && (kk[q] > thresh || (kk[q] == thresh && e_rank++ < take_eq))) {
            const int tok = r.doc_start + kpool * (j0 + q);
            if (kpool == 4) {
                *reinterpret_cast<int4*>(r.row + 4 * pos) = make_int4(tok, tok + 1, tok + 2, tok + 3);
            } else {
                for (int u = 0; u < kpool; ++u) r.row[pos * kpool + u] = tok + u;
            }
            ++pos;
        }
    }
}

// the row's own incomplete pool and padding (over the scratch), and its slot count
__global__ __launch_bounds__(256) void topk_mw_tail_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, const float* __restrict__ scores, int max_pools, int topk,
    int row_width, int32_t* __restrict__ indices, int32_t* __restrict__ num_valid) {
    const TmRow r = tm_row(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices,
                           blockIdx.x);
    if (r.n <= TK_LDS_KEYS) return;
    const int base = r.k * kpool;
    const int n_tail = r.t - r.tail_start + 1;
    for (int q = threadIdx.x; q < row_width - base; q += 256)
        r.row[base + q] = q < n_tail ? r.tail_start + q : -1;
    if (threadIdx.x == 0 && num_valid) num_valid[blockIdx.x] = base + n_tail;
}

hipError_t launch_topk(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                       const int32_t* q_pos, int num_q, const float* scores, int max_pools,
                       int topk, int row_width, int32_t* indices, int32_t* num_valid,
                       hipStream_t stream) {
    if (num_q == 0) return hipSuccess;
    // rows with more visible pools than the key cache holds go to the long-row
    // kernels: many workgroups per row when the rows have room for the scratch
    // (a histogram in the token slots, the state and chunk counts in the padding),
    // otherwise one workgroup per row
    const int has_long = max_pools > TK_LDS_KEYS;
    const int chunks = (max_pools + TM_CHUNK - 1) / TM_CHUNK;
    const bool many = has_long && (long long)kpool * topk >= TK_BINS &&
                      (long long)row_width >= (long long)kpool * topk + kpool + TM_STATE + 2 * chunks;
    if (!has_long) {
        // rows of up to 4096 slots with 64 key registers per lane, longer ones with 128
        // (a launch per instance: each wave first looks up its row's length, so a
        // third instance costs more than its extra waves per SIMD gain);
        // 16-byte loads when every row's 16-byte chunks lie in the score tensor's row
        // (a row's slots then end at most at its stride, a multiple of four)
        const int g = (num_q + TW_WAVES - 1) / TW_WAVES;
        const int vec4 = max_pools % 4 == 0 && ((uintptr_t)scores & 15) == 0;
#define KP_TW(KP4, R, RLO)                                                                                     \
    topk_wave_kernel<KP4, R, RLO><<<g, 64 * TW_WAVES, 0, stream>>>(cu, num_docs, cu_pools, kpool, q_pos,       \
                                                                   scores, max_pools, topk, row_width, indices, \
                                                                   num_valid, num_q, vec4)
        if (kpool == 4) {
            KP_TW(true, 64, 0);
            if (max_pools > 4096) KP_TW(true, 128, 64);
        } else {
            KP_TW(false, 64, 0);
            if (max_pools > 4096) KP_TW(false, 128, 64);
        }
#undef KP_TW
        return hipGetLastError();
    }
    topk_kernel<<<num_q, TK_THREADS, 0, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools,
                                                  topk, row_width, indices, num_valid,
                                                  !has_long ? 0 : (many ? 2 : 1));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !has_long) return e;
    if (!many) {
        topk_long_kernel<<<num_q, TL_THREADS, 0, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, scores,
                                                           max_pools, topk, row_width, indices, num_valid);
        return hipGetLastError();
    }
    const dim3 cg(num_q, chunks);   // rows on x (up to 2^31 - 1), chunks on y
#define KP_MW_ARGS cu, num_docs, cu_pools, kpool, q_pos, scores, max_pools, topk, row_width, indices
    topk_mw_hist_kernel<0><<<cg, TM_THREADS, 0, stream>>>(KP_MW_ARGS);
    topk_mw_select_kernel<0><<<num_q, 64, 0, stream>>>(KP_MW_ARGS);
    topk_mw_hist_kernel<1><<<cg, TM_THREADS, 0, stream>>>(KP_MW_ARGS);
    topk_mw_select_kernel<1><<<num_q, 64, 0, stream>>>(KP_MW_ARGS);
    topk_mw_hist_kernel<2><<<cg, TM_THREADS, 0, stream>>>(KP_MW_ARGS);
    topk_mw_select_kernel<2><<<num_q, 64, 0, stream>>>(KP_MW_ARGS);
    topk_mw_count_kernel<<<cg, TM_THREADS, 0, stream>>>(KP_MW_ARGS);
    topk_mw_write_kernel<<<cg, TM_THREADS, 0, stream>>>(KP_MW_ARGS);
    topk_mw_tail_kernel<<<num_q, 256, 0, stream>>>(KP_MW_ARGS, num_valid);
#undef KP_MW_ARGS
    return hipGetLastError();
}

}  // namespace kp
