// FP8 lightning-indexer scoring over pools on gfx950 matrix cores.
//
// prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet: a query
// scores, in FP8, the complete pools ending at or before it (pools of its own
// document), after Hadamard rotation of both sides. Score of query i and
// pool p:
//   I[i,p] = sk[p] * sum_h (w[i,h] * sq[i,h]) * ReLU(<q8[i,h], k8[p]>)
// which equals sum_h w * ReLU(sq * sk * <q8, k8>) because both scales are
// positive.
//
// Work decomposition: a workgroup takes 16 queries, stages their codes in LDS
// once, and walks the pools its queries see in chunks of 512 (all of them, or
// every n-th when there are too few query tiles to fill the GPU); for each chunk,
// each of its 8 waves holds the E4M3 codes of 64 pools (4 tiles of 16) in
// registers as the B operand (the kernel is held to 128 registers, four waves
// per SIMD, so one wave's ReLU/weighting overlaps another's MFMAs). The query
// tile sits in LDS head-major; for each indexer head h, one
// v_mfma_f32_16x16x128_f8f6f4 per pool tile computes the full 128-wide dots of
// 16 queries x 16 pools, and each lane folds its 4 (query, pool) results into
// running sums with w*sq of that query and head after the ReLU; the MFMAs of
// the next head are issued before that fold. The head sum thus stays inside
// the lane: no cross-lane reduction. Chunks and waves outside every query's
// visible range are skipped; query tiles are dispatched last-first so the
// longest causal rows start early.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_select.h"

namespace kp {

constexpr int SC_QT = 16;     // queries per workgroup
constexpr int SC_NJ = 4;      // 16-pool tiles per wave
constexpr int SC_PW = 16 * SC_NJ;  // pools per wave
constexpr int SC_WAVES = 8;
constexpr int SC_THREADS = 64 * SC_WAVES;
constexpr int SC_PC = SC_PW * SC_WAVES;  // pools per workgroup

__global__ void fill_f32_kernel(float* __restrict__ dst, size_t n, float v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = v;
}

hipError_t launch_fill_f32(float* dst, size_t n, float value, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_f32_kernel<<<(unsigned)blocks, 256, 0, stream>>>(dst, n, value);
    return hipGetLastError();
}

// LDS layout of the query tile: [head][query][128 bytes]; the 16-byte chunk c
// of query row q is stored at chunk c ^ ((q >> 1) & 7), so the 16 rows one
// A-operand read touches fall in distinct banks.

// All heads of one 64-pool block of a wave: acc[j][e] += w*sq(query 4g+e, h) *
// ReLU(<q8[query, h], k8[pool 16j+n]>) summed over h. The heads run as a
// two-stage pipeline over two register slots: the MFMAs of head h+1 are issued
// before the results of head h are folded in (so the matrix core works while
// the VALU does the ReLU and weighting, and no fold waits on a fresh MFMA), and
// the A operands of head h+2 are read from LDS meanwhile. The loop body covers
// two heads, so every slot index is a constant (no register copies).
__device__ __forceinline__ void score_heads(const uint8_t* __restrict__ q_lds, const float* __restrict__ wq_lds,
                                            int h_idx, const i32x8 (&b)[SC_NJ], f32x4 (&acc)[SC_NJ]) {
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int sw = (n >> 1) & 7;
    const uint8_t* rowp = q_lds + n * 128;
    const int off0 = ((2 * g) ^ sw) << 4, off1 = ((2 * g + 1) ^ sw) << 4;
    i32x8 a[2];
    f32x4 c[2][SC_NJ];
    auto load = [&](int slot, int h) __attribute__((always_inline)) {
        const uint8_t* r = rowp + h * (16 * 128);
        const uint4 lo = *reinterpret_cast<const uint4*>(r + off0);
        const uint4 hi = *reinterpret_cast<const uint4*>(r + off1);
        a[slot] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };
    auto issue = [&](int slot) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SC_NJ; ++j) c[slot][j] = mfma_fp8_16x16x128(a[slot], b[j], f32x4{0.f, 0.f, 0.f, 0.f});
    };
    auto fold = [&](int slot, const f32x4& wv) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < SC_NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[j][e] = __builtin_fmaf(wv[e], relu_f32(c[slot][j][e]), acc[j][e]);
    };
    // the loop covers pairs of heads with a head pair after them, with no
    // condition inside (so the waits on its LDS reads are exact and the reads
    // may be hoisted); the last one or two heads follow it
    load(0, 0);
    issue(0);
    if (h_idx > 1) load(1, 1);
    int h = 0;
#pragma unroll 1
    for (; h + 2 < h_idx; h += 2) {
        // head h: MFMAs in flight in slot 0; head h+1: operands in slot 1. The
        // weights of both heads are read here, so their LDS latency hides behind
        // the MFMAs of head h+1 (no weight is carried from one iteration to the next)
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wq_lds + h * 16 + 4 * g);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wq_lds + (h + 1) * 16 + 4 * g);
        issue(1);
        fold(0, w0);
        load(0, h + 2);
        issue(0);
        fold(1, w1);
        load(1, min(h + 3, h_idx - 1));
    }
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(wq_lds + h * 16 + 4 * g);
    if (h + 1 < h_idx) {
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wq_lds + (h + 1) * 16 + 4 * g);
        issue(1);
        fold(0, w0);
        fold(1, w1);
    } else {
        fold(0, w0);
    }
}

// Pooled keys in pages of 32 pools (a page holds the pools of kpool*32
// tokens): pool p of document d (global number p, d's pools starting at
// cu_pools[d]) is row table[d*max_pages + (p - cu_pools[d]) / 32] * 32 +
// (p - cu_pools[d]) % 32 of k8 and sk (a page number outside [0, num_pages),
// or a pool past d's max_pages pages: no row, its key reads as zero).
// table == nullptr: row p.
struct PageArgs {
    const int32_t* table;
    int max_pages;
    int num_pages;
};

// Candidate emission of the fused scoring + top-k: query i keeps every
// visible pool whose (key, pool) is at least (tau[2i], tau[2i+1]) in the
// order "larger key first, then lower pool first"; count[i] counts them all
// and the first `cap` go to cand[i*cap ...] as (score bits, pool) in any order.
struct EmitArgs {
    const uint32_t* tau;
    int32_t* count;
    uint2* cand;
    int cap;
};

// (at least four waves per SIMD: 128 registers)
template <bool EMIT, bool PAGED>
__global__ __launch_bounds__(SC_THREADS, 4) void score_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, int num_q, const uint8_t* __restrict__ q8,
    const float* __restrict__ sq, const float* __restrict__ w, int h_idx, int d_idx,
    const uint8_t* __restrict__ k8, const float* __restrict__ sk, int max_pools,
    float* __restrict__ scores, int nsplit, EmitArgs em, PageArgs pg) {
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* q_lds = smem;                                                 // [h_idx][QT][128]
    float* wq_lds = reinterpret_cast<float*>(smem + (size_t)h_idx * SC_QT * 128);  // [h_idx][QT]
    __shared__ int lo_s[SC_QT], hi_s[SC_QT];
    __shared__ int plo_s, phi_s, maxlo_s, minhi_s;
    // emission: thresholds (as the score whose key they are, and "every pool"),
    // per-chunk candidate counts and write cursors
    __shared__ float tf_s[SC_QT];
    __shared__ int tp_s[SC_QT], tall_s[SC_QT], lcnt_s[SC_QT], lcur_s[SC_QT];
    // paged keys: the distinct documents of the tile (pool range, table row)
    __shared__ int ndoc_s, dlo_s[SC_QT], dhi_s[SC_QT], dtab_s[SC_QT];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int nqt = (num_q + SC_QT - 1) / SC_QT;
    // query tile, and which of the tile's 512-pool chunks this workgroup takes
    // (every nsplit-th: few query tiles, as in decode, still fill the GPU)
    const int qtile = nqt - 1 - (int)(blockIdx.x / nsplit);
    const int split = (int)(blockIdx.x % nsplit);
    const int q0 = qtile * SC_QT;

    if (tid < SC_QT) {
        int lo = 0, hi = 0, doc = -1;
        int i = q0 + tid;
        if (EMIT) {   // (a slot past the last query: no pool clears its threshold)
            tf_s[tid] = __uint_as_float(0x7FFFFFFFu);
            tall_s[tid] = 0;
            tp_s[tid] = -1;
        }
        if (i < num_q) {
            int t = q_pos ? q_pos[i] : i;
            QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
            lo = qp.pool_lo;
            hi = qp.pool_lo + qp.n_vis;
            doc = qp.doc;
            if (EMIT) {
                // key K = tau[2i] as a score: a score s of key k has k >= K exactly when
                // s >= that score (keys order scores; -0 and +0 share a key and compare
                // equal). K = 0 (every pool, NaN included) is the flag tall.
                const uint32_t tk = em.tau[2 * i];
                tf_s[tid] = __uint_as_float((tk & 0x80000000u) ? (tk & 0x7FFFFFFFu) : ~tk);
                tall_s[tid] = tk == 0u;
                tp_s[tid] = (int)em.tau[2 * i + 1];
            }
        }
        lo_s[tid] = lo;
        hi_s[tid] = hi;
        if (EMIT) lcnt_s[tid] = 0;
        if (PAGED) dtab_s[tid] = doc;   // (documents, deduplicated below)
    }
    __syncthreads();
    if (tid == 0) {
        // the pools any query of the tile sees lie in [plo, phi); every query of
        // the tile sees all of [maxlo, minhi)
        int plo = 0x7FFFFFFF, phi = 0, maxlo = 0, minhi = 0x7FFFFFFF;
        for (int q = 0; q < SC_QT; ++q) {
            if (lo_s[q] < hi_s[q]) {
                plo = min(plo, lo_s[q]);
                phi = max(phi, hi_s[q]);
            }
            if (q0 + q < num_q) {
                maxlo = max(maxlo, lo_s[q]);
                minhi = min(minhi, hi_s[q]);
            }
        }
        plo_s = plo;
        phi_s = phi;
        maxlo_s = maxlo;
        minhi_s = minhi;
        if (PAGED) {
            // per distinct document: its first pool, the end of what the tile's
            // queries see of it, and its row of the page table
            int nd = 0;
            for (int q = 0; q < SC_QT; ++q) {
                if (lo_s[q] >= hi_s[q]) continue;
                int f = -1;
                for (int e = 0; e < nd; ++e)
                    if (dlo_s[e] == lo_s[q]) f = e;
                if (f < 0) {
                    f = nd++;
                    dlo_s[f] = lo_s[q];
                    dhi_s[f] = hi_s[q];
                    dtab_s[f] = dtab_s[q] * pg.max_pages;
                } else {
                    dhi_s[f] = max(dhi_s[f], hi_s[q]);
                }
            }
            ndoc_s = nd;
        }
    }
    __syncthreads();
    const int plo = plo_s, phi = phi_s, maxlo = maxlo_s, minhi = minhi_s;
    const int P_first = (plo / SC_PC + split) * SC_PC;
    if (plo >= phi || P_first >= phi) return;

    // stage the query tile, head-major: codes (zero-padded to 128 bytes) and w*sq
    const int dchunks = d_idx >> 4;
    {
        // 16-byte chunk c = tid + SC_THREADS * k: head c >> 7, query (c >> 3) & 15,
        // chunk c & 7; eight loads are put in flight before their LDS stores
        constexpr int SB = 8;
        const int nch = h_idx * SC_QT * 8;
        const int ch = tid & 7, q = (tid >> 3) & (SC_QT - 1);
        const bool qok = q0 + q < num_q && ch < dchunks;
        const uint8_t* src = q8 + (size_t)(qok ? q0 + q : 0) * h_idx * d_idx + ch * 16;
        uint8_t* dst = q_lds + (size_t)q * 128 + ((ch ^ ((q >> 1) & 7)) << 4);
        for (int c0 = 0; c0 < nch; c0 += SC_THREADS * SB) {
            uint4 v[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int h = (c0 + tid + SC_THREADS * k) >> 7;
                v[k] = make_uint4(0u, 0u, 0u, 0u);
                if (qok && c0 + SC_THREADS * k + tid < nch) v[k] = *reinterpret_cast<const uint4*>(src + (size_t)h * d_idx);
            }
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const int h = (c0 + tid + SC_THREADS * k) >> 7;
                if (c0 + SC_THREADS * k + tid < nch) *reinterpret_cast<uint4*>(dst + (size_t)h * SC_QT * 128) = v[k];
            }
        }
    }
    for (int c = tid; c < h_idx * SC_QT; c += SC_THREADS) {
        const int q = c & (SC_QT - 1), h = c >> 4;
        float v = 0.0f;
        if (q0 + q < num_q) {
            const size_t o = (size_t)(q0 + q) * h_idx + h;
            v = w[o] * sq[o];
        }
        wq_lds[c] = v;
    }

    __syncthreads();

    // (the chunk loop is uniform over the workgroup: emission synchronises it)
    for (int P0 = P_first; P0 < phi; P0 += SC_PC * nsplit) {
        const int Pw = P0 + wave * SC_PW;
        // skip the block if it lies outside what the tile's queries see (their
        // union's hull: a block in a gap is computed and then dropped); a block
        // every query sees whole needs no per-pool visibility test
        const bool seen = Pw < phi && Pw + SC_PW > plo;
        const bool full = Pw >= maxlo && Pw + SC_PW <= minhi;
        if (!EMIT && !seen) continue;

        f32x4 acc[SC_NJ];
        float skj[SC_NJ];
        if (seen) {
            // this wave's pools: B operands (32 code bytes of column n per lane) and key scales
            i32x8 b[SC_NJ];
#pragma unroll
            for (int j = 0; j < SC_NJ; ++j) {
                int p = Pw + 16 * j + n;
                uint4 lo4 = make_uint4(0u, 0u, 0u, 0u), hi4 = lo4;
                float s = 0.0f;
                long long row = -1;
                if (PAGED) {
                    // a pool some query of the tile sees; others stay zero
                    for (int e = 0; e < ndoc_s; ++e)
                        if (p >= dlo_s[e] && p < dhi_s[e]) {
                            const int l = p - dlo_s[e];
                            const int pn = (l >> 5) < pg.max_pages ? pg.table[dtab_s[e] + (l >> 5)] : -1;
                            if ((unsigned)pn < (unsigned)pg.num_pages) row = (long long)pn * 32 + (l & 31);
                            break;
                        }
                } else if (p < max_pools) {
                    row = p;
                }
                if (row >= 0) {
                    const uint8_t* src = k8 + (size_t)row * d_idx;
                    if (2 * g < dchunks) lo4 = *reinterpret_cast<const uint4*>(src + 32 * g);
                    if (2 * g + 1 < dchunks) hi4 = *reinterpret_cast<const uint4*>(src + 32 * g + 16);
                    s = sk[row];
                }
                b[j] = i32x8{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                             (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
                skj[j] = s;
            }

            // (a block with only some tiles visible computes all four: the others'
            // results are dropped at the store)
#pragma unroll
            for (int j = 0; j < SC_NJ; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            score_heads(q_lds, wq_lds, h_idx, b, acc);
        }

        if (!EMIT) {
            // lane holds queries 4g + e of the tile for pool Pw + 16j + n
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = 4 * g + e;
                if (q0 + q >= num_q) continue;
                float* orow = scores + (size_t)(q0 + q) * max_pools;
                if (full) {
#pragma unroll
                    for (int j = 0; j < SC_NJ; ++j) orow[Pw + 16 * j + n] = acc[j][e] * skj[j];
                } else {
                    const int lo = lo_s[q], hi = hi_s[q];
#pragma unroll
                    for (int j = 0; j < SC_NJ; ++j) {
                        const int p = Pw + 16 * j + n;
                        if (p >= lo && p < hi) orow[p] = acc[j][e] * skj[j];
                    }
                }
            }
        } else {
            // candidates of this block: bit 4j+e for query 4g+e and pool Pw+16j+n
            // (the threshold test on the score itself; keys are formed in the
            // select, from the stored score bits)
            uint32_t cm = 0u;
            float sc[SC_NJ][4];
            if (seen) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int q = 4 * g + e;
                    const float tf = tf_s[q];
                    const int tp = tp_s[q];
                    const bool tall = tall_s[q] != 0;
                    // (slots past the last query have lo = hi = 0: never "seen in full")
                    const bool fq = full && q0 + q < num_q;
                    const int lo = fq ? 0 : lo_s[q], hi = fq ? 0x7FFFFFFF : hi_s[q];
#pragma unroll
                    for (int j = 0; j < SC_NJ; ++j) {
                        const int p = Pw + 16 * j + n;
                        sc[j][e] = acc[j][e] * skj[j];
                        const bool c = p >= lo && p < hi && (tall || sc[j][e] > tf || (sc[j][e] == tf && p <= tp));
                        cm |= (uint32_t)c << (4 * j + e);
                    }
                }
            }
            // count per query, reserve one range of each query's list, then write
#pragma unroll
            for (int b = 0; b < 4 * SC_NJ; ++b)
                if (cm >> b & 1u) atomicAdd(&lcnt_s[4 * g + (b & 3)], 1);
            __syncthreads();
            if (tid < SC_QT) {
                const int c = lcnt_s[tid];
                lcur_s[tid] = c ? atomicAdd(&em.count[q0 + tid], c) : 0;
                lcnt_s[tid] = 0;
            }
            __syncthreads();
#pragma unroll
            for (int b = 0; b < 4 * SC_NJ; ++b) {
                const int j = b >> 2, e = b & 3, q = 4 * g + e;
                if (cm >> b & 1u) {
                    const int pos = atomicAdd(&lcur_s[q], 1);
                    if (pos < em.cap)
                        em.cand[(size_t)(q0 + q) * em.cap + pos] = make_uint2(__float_as_uint(sc[j][e]), Pw + 16 * j + n);
                }
            }
        }
    }
}

static int score_split(int num_q, int max_pools) {
    // split the pools of a query tile over several workgroups when the tiles
    // alone give fewer than 512 workgroups: two per compute unit (four waves per
    // SIMD) on the 256 CUs, so one round of workgroups fills the GPU and each
    // walks several chunks, which repays staging its 16 queries' codes (more,
    // shorter splits were slower at decode: 2048 of them took 37 us more)
    const int nqt = (num_q + SC_QT - 1) / SC_QT;
    const int nchunks = (max_pools + SC_PC - 1) / SC_PC;
    int nsplit = (512 + nqt - 1) / nqt;
    if (nsplit > nchunks) nsplit = nchunks;
    if (nsplit < 1) nsplit = 1;
    return nsplit;
}

template <bool EMIT, bool PAGED>
static hipError_t launch_score_t(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                                 const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                                 const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                                 int max_pools, float* scores, EmitArgs em, PageArgs pg, hipStream_t stream) {
    if (num_q == 0 || max_pools == 0) return hipSuccess;
    const int nqt = (num_q + SC_QT - 1) / SC_QT;
    const int nsplit = score_split(num_q, max_pools);
    const long long nblk = (long long)nqt * nsplit;
    if (nblk > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk);
    const size_t lds = (size_t)h_idx * SC_QT * (128 + 4);
    hipError_t e = hipFuncSetAttribute((const void*)score_kernel<EMIT, PAGED>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    score_kernel<EMIT, PAGED><<<grid, SC_THREADS, lds, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8,
                                                                  sq, w, h_idx, d_idx, k8, sk, max_pools, scores,
                                                                  nsplit, em, pg);
    return hipGetLastError();
}

hipError_t launch_score(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                        const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                        const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                        int max_pools, float* scores, hipStream_t stream) {
    return launch_score_t<false, false>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w, h_idx, d_idx, k8,
                                        sk, max_pools, scores, EmitArgs{}, PageArgs{nullptr, 0, 0}, stream);
}

hipError_t launch_score_emit(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                             const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                             const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                             int max_pools, const int32_t* page_table, int max_pages, int num_pages,
                             const uint32_t* tau, int32_t* count, uint2* cand, int cap, hipStream_t stream) {
    const EmitArgs em{tau, count, cand, cap};
    const PageArgs pg{page_table, max_pages, num_pages};
    if (page_table)
        return launch_score_t<true, true>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w, h_idx, d_idx,
                                          k8, sk, max_pools, nullptr, em, pg, stream);
    return launch_score_t<true, false>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w, h_idx, d_idx, k8,
                                       sk, max_pools, nullptr, em, pg, stream);
}

}  // namespace kp
