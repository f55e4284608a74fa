// Absorbed, NoPE sparse latent attention (MLA) forward on gfx950.
//
// NeMo AutoModel PR "add GLM-5.3-Flash training support", Changelog: the K
// projection is absorbed into the query, which attends over a shared
// 512-wide latent K/V; prime-rl PR "GLM-5.3-Flash text model", Summary, second
// bullet: the latent serves as both key and value, no RoPE part. Each query
// attends to the rows its index row names (up to 2051 of them, "cuDNN sparse
// MLA parity and performance").
//
// One workgroup of 8 waves (two per SIMD) per query token (64 heads). The
// index row is compacted in LDS (masked entries dropped, order kept); its
// latent rows are gathered 32 at a time: each wave loads 4 whole rows (16-byte
// loads, 1 KB per wave-wide load) into registers and writes them into a 3-tile
// LDS ring one tile later (plain vector loads keep the gather near the memory
// system's random-row bandwidth at this occupancy; the direct-to-LDS loads of
// gfx950 reach well under half of it). The work on a tile t:
//   QK: wave w computes a partial S^T = K[rows_h, cols_c] . Q[:, cols_c]^T for
//       the row half h = w/4 and column quarter c = w%4, all 64 heads (bf16
//       MFMA 16x16x32; Q's columns stay in registers; every K fragment read
//       from LDS feeds four MFMAs, and K is read once per CU);
//   SM: the four column partials meet in LDS; wave w adds them for heads
//       w, w+8, .., w+56 and runs their online softmax, writing P (bf16);
//   PV: wave w accumulates O[:, cols] += P . V[:, cols] over its eighth of the
//       latent columns for all 64 heads: one V fragment, read with the
//       transposing ds_read_b64_tr_b16 (V is read exactly once per CU), feeds
//       four MFMAs.
// The loop is software-pipelined with two barriers per tile: phase 1 runs
// QK(t+1) together with a quarter of PV(t); phase 2 runs SM(t+1) and the
// staging of tile t+2 together with the rest of PV(t), so the MFMA pipe has
// work while the softmax and the staging wait on LDS.
// The softmax reference max of a head is re-based (and O rescaled) only when a
// tile's max exceeds it by more than 8 (log2 units), so weights stay below 2^8
// and O is untouched outside the MFMAs on most tiles. LDS rows keep their
// 16-byte chunks permuted by a per-row xor so the row-wise K reads and the
// column-wise V reads are both free of bank conflicts. A latent narrower than
// 128 is zero-padded to 128 in LDS.
#include "kp_device.h"
#include "kp_launch.h"

namespace kp {

constexpr int MLA_TK = 32;    // latent rows per tile
constexpr int MLA_NW = 8;     // waves per workgroup (two per SIMD)
constexpr int MLA_NBUF = 3;   // LDS tiles in the gather ring
constexpr int MLA_MAX_ROW = 4096;  // index-row entries the LDS list holds

// Chunk permutation of LDS row r: 16-byte chunk c is stored at c ^ row_swz(r)
// (within aligned groups of 16 chunks, one pass over the 64 banks).
// gfx950 services a 16-byte LDS read in four passes of 16 lanes (lanes
// {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31} and the same in the upper half),
// 8-byte and transposing reads in two passes of 32 consecutive lanes, and
// 16-byte writes in passes of 8 consecutive lanes. This linear map of the row
// bits (row bits 0, 1, 2, 3 -> chunk masks 2, 4, 8, 9) is conflict-free, under
// those passes, for the row-wise K reads (16 rows, one chunk column per lane
// group), the column-wise transposing V reads (8 rows per pass) and the
// row-contiguous staging writes.
__device__ __forceinline__ int row_swz(int r) { return ((r & 7) << 1) ^ (((r >> 3) & 1) * 9); }

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((KP_LDS bf16x4*)(p));
}

// compiler-only barrier: keeps LDS accesses on their side of the explicit waits
__device__ __forceinline__ void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

constexpr int P_STRIDE = 96;   // bytes per head row of the P tile (32 bf16 + 32 pad: conflict-free 16-byte reads)
constexpr int SP_STRIDE = 36;  // floats per head row of a partial-S block (32 + 4 pad)

__device__ __forceinline__ void wait_lgkm0() {
    // s_waitcnt lgkmcnt(0) only (vmcnt 63, expcnt 7: no wait)
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Barrier that orders LDS traffic between waves but does not wait for the
// gathers in flight (a __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier() {
    compiler_fence();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

// Workgroups are handed to the eight XCDs round-robin by their index, and each
// XCD has its own L2. Queries of one document that are close in position pick
// mostly the same pools, so the workgroup -> query map gives each XCD runs of
// MLA_XCD_RUN consecutive queries: the latent rows they gather are then shared
// through one L2. Runs go to the XCDs in turn, which keeps the long and the
// short rows of a causal batch spread over all of them. A bijection on
// [0, n): the last n % (8 * MLA_XCD_RUN) workgroups keep their own index.
#define MLA_XCD_RUN 32
__device__ __forceinline__ int xcd_query(int b, int n) {
    constexpr int R = MLA_XCD_RUN;
    const int full = n / (8 * R) * (8 * R);
    if (b >= full) return b;
    const int slot = b >> 3, xcd = b & 7;   // slot-th workgroup that lands on this XCD
    return (slot / R) * (8 * R) + xcd * R + slot % R;
}

template <int D>
__global__ __launch_bounds__(64 * MLA_NW, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ indices,
    int num_kv, int heads, int row_width, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int NW = MLA_NW;
    constexpr int NT = 64 * NW;             // threads
    constexpr int DP = D < 128 ? 128 : D;   // latent width in LDS (zero-padded)
    constexpr int RB = DP * 2;              // LDS bytes per latent row
    constexpr int CH = D / 8;               // 16-byte chunks a gathered row brings
    constexpr int KSW = DP / 128;           // QK k-steps (32 columns) per wave: a quarter of the columns
    constexpr int DTW = DP / 128;           // 16-wide O column tiles per wave: an eighth of the columns
    constexpr int DTA = (DTW + 3) / 4;      // of which PV runs in phase 1 (the rest in phase 2)
    constexpr int TILE_B = MLA_TK * RB;     // bytes per LDS tile
    constexpr int IPW = MLA_TK / NW;        // gathered rows per wave per tile
    constexpr int RPL = (64 / CH) < IPW ? (64 / CH) : IPW;  // rows one wave-wide load covers
    constexpr int NL = IPW / RPL;           // such loads per wave per tile
    static_assert(NW == 8 && CH >= 8 && CH <= 64 && 64 % CH == 0 && IPW % RPL == 0, "tile staging split");
    static_assert((D * 2 + 16) * 64 <= MLA_NBUF * TILE_B, "output staging fits the ring");

    __shared__ __align__(16) uint8_t ring[MLA_NBUF * TILE_B];
    __shared__ int32_t list[MLA_MAX_ROW];
    __shared__ __align__(16) float spart[4 * 64 * SP_STRIDE];   // partial S, [column quarter][head][row]
    __shared__ __align__(16) uint8_t ptile[64 * P_STRIDE];      // P, bf16 [head][row]
    __shared__ __align__(16) float alpha_s[64];                 // per-head rescale of the last softmax tile
    __shared__ int rebase_tile;                                 // last tile (+1) that moved a reference max
    __shared__ float lsum[64 * 2];                              // per-head (rounded, exact) sums
    __shared__ float mref_s[64];                                // per-head final reference max
    __shared__ int wave_buf[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int i = xcd_query(blockIdx.x, gridDim.x);
    const int cq = wave & 3;    // QK: column quarter
    const int rh = wave >> 2;   // QK: row half of the tile

    // ---- compact the index row (valid entries, original order) ----------------
    const int32_t* irow = indices + (size_t)i * row_width;
    const int per = (row_width + NT - 1) / NT;
    const int j0 = min(row_width, tid * per), j1 = min(row_width, j0 + per);
    int cnt = 0;
    for (int j = j0; j < j1; ++j) {
        int v = irow[j];
        cnt += (v >= 0 && v < num_kv);
    }
    int x = cnt;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    if (lane == 63) wave_buf[wave] = x;
    if (DP != D) {   // zero the padding columns of the ring once; the staging never writes them
        for (int e = tid; e < MLA_NBUF * TILE_B / 16; e += NT)
            reinterpret_cast<uint4*>(ring)[e] = make_uint4(0u, 0u, 0u, 0u);
    }
    __syncthreads();
    int before = x - cnt, n_valid = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        if (w < wave) before += wave_buf[w];
        n_valid += wave_buf[w];
    }
    for (int j = j0; j < j1; ++j) {
        int v = irow[j];
        if (v >= 0 && v < num_kv) list[before++] = v;
    }
    __syncthreads();
    // pad the list to whole tiles with a valid row (its scores are masked), so
    // the gather needs no bounds test
    {
        const int pad_end = (n_valid + MLA_TK - 1) / MLA_TK * MLA_TK;
        if (n_valid > 0 && tid < pad_end - n_valid) list[n_valid + tid] = list[0];
    }
    __syncthreads();

    uint16_t* orow = out + (size_t)i * heads * D;
    if (n_valid == 0) {
        for (int e = tid; e < heads * D; e += NT) orow[e] = 0;
        if (lse && tid < heads) lse[(size_t)i * heads + tid] = -INFINITY;
        return;
    }
    const int ntiles = (n_valid + MLA_TK - 1) / MLA_TK;
    if (tid == 0) rebase_tile = 0;   // visible after the first barrier below

    // ---- gather: wave w stages tile rows IPW*w .. IPW*w + IPW-1 --------------------
    // Load j of a tile: lane l (< RPL*CH) covers tile row r = IPW*w + j*RPL + l/CH
    // and its 16-byte chunk l%CH, which lands in LDS at chunk (l%CH) ^ row_swz(r).
    const int lrow = lane / CH, lchunk = lane % CH;
    const bool lact = lane < RPL * CH;
    const int srow0 = wave * IPW + lrow;     // tile row of this lane's first load
    int sto[NL];                             // LDS offsets of this lane's staged chunks
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int r = srow0 + j * RPL;
        sto[j] = r * RB + ((lchunk ^ row_swz(r)) << 4);
    }
    u32x4 stg[NL];                           // a tile in flight
    int rows_next[NL];                       // latent rows of the next tile to load
#define KP_ROWS_OF(kt_)                                                              \
    _Pragma("unroll") for (int j = 0; j < NL; ++j) {                                 \
        rows_next[j] = list[(kt_) * MLA_TK + srow0 + j * RPL];                       \
    }
#define KP_LOAD_TILE()                                                               \
    if (lact) {                                                                      \
        _Pragma("unroll") for (int j = 0; j < NL; ++j)                               \
            stg[j] = *reinterpret_cast<const u32x4*>(                                \
                reinterpret_cast<const uint8_t*>(kv) +                               \
                ((uint32_t)rows_next[j] * (uint32_t)(D * 2) + 16u * (uint32_t)lchunk)); \
    }
#define KP_STORE_TILE(buf_)                                                          \
    if (lact) {                                                                      \
        _Pragma("unroll") for (int j = 0; j < NL; ++j)                               \
            *reinterpret_cast<u32x4*>(ring + (buf_) * TILE_B + sto[j]) = stg[j];     \
    }

    // ---- Q of this wave's column quarter for all 64 heads, B-operand layout ---------
    bf16x8 qf[4][KSW];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int head = 16 * ht + n;
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const int col = cq * (DP / 4) + 32 * s + 8 * g;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (head < heads && col < D) v = *reinterpret_cast<const uint4*>(q + ((size_t)i * heads + head) * D + col);
            qf[ht][s] = __builtin_bit_cast(bf16x8, v);
        }
    }

    // PV state: O for heads 16*ht + 4*g + e, columns 16*(wave*DTW + dtl) + n
    f32x4 o[4][DTW];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int dtl = 0; dtl < DTW; ++dtl) o[ht][dtl] = f32x4{0.f, 0.f, 0.f, 0.f};
    // softmax state: wave w owns heads w, w+8, .., w+56 (lanes 8j..8j+7 hold head
    // w+8j, rows 4*(lane&7) .. +3; a row-group reduction stays inside 8 lanes)
    const int hown = wave + 8 * (lane >> 3);
    const int srow = 4 * (lane & 7);
    float m_ref = -INFINITY, l_run = 0.f, l_lse = 0.f;

    // fixed per-lane LDS offsets
    const int rq = 16 * rh + n;                      // K row this lane feeds
    int kb[KSW];                                     // K chunk of each k-step
#pragma unroll
    for (int s = 0; s < KSW; ++s)
        kb[s] = rq * RB + (((cq * (DP / 32) + 4 * s + g) ^ row_swz(rq)) << 4);
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int vr0 = 8 * g + e4, vr1 = 8 * g + 4 + e4;  // V rows of the two transposing reads
    int vb0[DTW], vb1[DTW];                          // V chunk of each column tile
#pragma unroll
    for (int dtl = 0; dtl < DTW; ++dtl) {
        const int c = 2 * (wave * DTW + dtl) + (q4 >> 1);
        vb0[dtl] = vr0 * RB + ((c ^ row_swz(vr0)) << 4) + 8 * (q4 & 1);
        vb1[dtl] = vr1 * RB + ((c ^ row_swz(vr1)) << 4) + 8 * (q4 & 1);
    }
    float* my_sp = spart + cq * 64 * SP_STRIDE;

    // QK of tile kt_ into partial S (LDS)
#define KP_QK(buf_)                                                                               \
    {                                                                                             \
        const uint8_t* tb_ = ring + (buf_) * TILE_B;                                              \
        u32x4 ka_[KSW];                                                                           \
        _Pragma("unroll") for (int s = 0; s < KSW; ++s) ka_[s] = *reinterpret_cast<const u32x4*>(tb_ + kb[s]); \
        _Pragma("unroll") for (int ht = 0; ht < 4; ++ht) sp[ht] = f32x4{0.f, 0.f, 0.f, 0.f};     \
        _Pragma("unroll") for (int s = 0; s < KSW; ++s) {                                         \
            const bf16x8 af_ = __builtin_bit_cast(bf16x8, ka_[s]);                                \
            _Pragma("unroll") for (int ht = 0; ht < 4; ++ht) sp[ht] = mfma_bf16_16x16x32(af_, qf[ht][s], sp[ht]); \
        }                                                                                         \
    }
    /* lane holds S^T[rows 16*rh + 4*g + e][head 16*ht + n]; stored as [head][row] */
#define KP_QK_STORE()                                                                             \
    _Pragma("unroll") for (int ht = 0; ht < 4; ++ht)                                              \
        *reinterpret_cast<f32x4*>(my_sp + (16 * ht + n) * SP_STRIDE + 16 * rh + 4 * g) = sp[ht];
    // full S of the owned heads (4 rows per lane) for tile kt_: read and sum the partials
#define KP_SM_READ()                                                                              \
    sv = *reinterpret_cast<const f32x4*>(spart + (0 * 64 + hown) * SP_STRIDE + srow);             \
    _Pragma("unroll") for (int w = 1; w < 4; ++w)                                                 \
        sv += *reinterpret_cast<const f32x4*>(spart + (w * 64 + hown) * SP_STRIDE + srow);
    // online softmax of tile kt_; P (bf16) and the per-head rescale to LDS
#define KP_SM_FINISH(kt_)                                                                         \
    {                                                                                             \
        if (((kt_) + 1) * MLA_TK > n_valid) {   /* ragged last tile: mask the rows past the end */ \
            _Pragma("unroll") for (int e = 0; e < 4; ++e)                                         \
                if ((kt_) * MLA_TK + srow + e >= n_valid) sv[e] = -INFINITY;                      \
        }                                                                                         \
        /* the scale is positive: the max of the raw scores, scaled, is the tile max */           \
        const float mt_ = max4_in_8(sv[0], sv[1], sv[2], sv[3]) * scale_log2;                     \
        float alpha_ = 1.0f;                                                                      \
        if (mt_ > m_ref + 8.0f) {                                                                 \
            alpha_ = __builtin_amdgcn_exp2f(m_ref - mt_);                                         \
            m_ref = mt_;                                                                          \
            rebase_tile = (kt_) + 1;   /* any writer stores the same value */                     \
        }                                                                                         \
        float w_[4];                                                                              \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                                             \
            w_[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[e], scale_log2, -m_ref));            \
        bf16x4 pw_;                                                                               \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) pw_[e] = (__bf16)w_[e];                     \
        /* the sum of the rounded weights, from the packed bf16 words */                          \
        const u32x2 pk_ = __builtin_bit_cast(u32x2, pw_);                                         \
        const float ps_ = (bf16_lo(pk_[0]) + bf16_hi(pk_[0])) + (bf16_lo(pk_[1]) + bf16_hi(pk_[1])); \
        const float pe_ = (w_[0] + w_[1]) + (w_[2] + w_[3]);                                      \
        l_run = l_run * alpha_ + ps_;                                                             \
        l_lse = l_lse * alpha_ + pe_;                                                             \
        *reinterpret_cast<bf16x4*>(ptile + hown * P_STRIDE + 2 * srow) = pw_;                     \
        if ((lane & 7) == 0) alpha_s[hown] = alpha_;                                              \
    }
    // O[:, cols] += P . V[:, cols] over the column tiles [d0_, d1_) of tile kt_
#define KP_PV(buf_, d0_, d1_)                                                                     \
    {                                                                                             \
        const uint8_t* tbv_ = ring + (buf_) * TILE_B;                                             \
        _Pragma("unroll") for (int dtl = (d0_); dtl < (d1_); ++dtl) {                             \
            const bf16x4 v0_ = lds_read_tr16(tbv_ + vb0[dtl]);                                    \
            const bf16x4 v1_ = lds_read_tr16(tbv_ + vb1[dtl]);                                    \
            const bf16x8 vb_ = __builtin_shufflevector(v0_, v1_, 0, 1, 2, 3, 4, 5, 6, 7);         \
            _Pragma("unroll") for (int ht = 0; ht < 4; ++ht)                                      \
                o[ht][dtl] = mfma_bf16_16x16x32(pa[ht], vb_, o[ht][dtl]);                         \
        }                                                                                         \
    }
#define KP_READ_P()                                                                               \
    _Pragma("unroll") for (int ht = 0; ht < 4; ++ht)                                              \
        pa[ht] = *reinterpret_cast<const bf16x8*>(ptile + (16 * ht + n) * P_STRIDE + 16 * g);
    // One pipelined step, for a tile kt with a successor (kt + 1 < ntiles); the
    // ring buffers of tiles kt, kt+1 and kt+2 are BV, BK and BS (compile-time,
    // so LDS addresses are immediates):
    //   phase 1: QK(kt+1) and PV(kt) on the first DTA column tiles (the partial
    //            S of QK is stored after PV is issued, so PV hides the QK
    //            latency);
    //   phase 2: SM(kt+1), PV(kt) on the remaining column tiles, tile kt+2
    //            from registers into the ring (its buffer last held tile kt-1,
    //            which every wave finished before the previous barrier) and
    //            the loads of tile kt+3; the MFMAs of PV run under the LDS
    //            traffic and the softmax arithmetic.
    // O is rescaled first when the softmax of tile kt moved a reference max.
#define KP_STEP(BV, BK, BS)                                                                       \
    {                                                                                             \
        const int rb_ = rebase_tile;                                                              \
        if (kt + 3 < ntiles) {                                                                    \
            KP_ROWS_OF(kt + 3)                                                                    \
        }                                                                                         \
        KP_QK(BK)                                                                                 \
        KP_READ_P()                                                                               \
        if (__builtin_amdgcn_readfirstlane(rb_) == kt + 1) {                                      \
            f32x4 al_[4];                                                                         \
            _Pragma("unroll") for (int ht = 0; ht < 4; ++ht)                                      \
                al_[ht] = *reinterpret_cast<const f32x4*>(alpha_s + 16 * ht + 4 * g);             \
            _Pragma("unroll") for (int ht = 0; ht < 4; ++ht)                                      \
                _Pragma("unroll") for (int dtl = 0; dtl < DTW; ++dtl) o[ht][dtl] *= al_[ht];      \
        }                                                                                         \
        KP_PV(BV, 0, DTA)                                                                         \
        KP_QK_STORE()                                                                             \
        lds_barrier();                                                                            \
        KP_SM_READ()                                                                              \
        KP_PV(BV, DTA, DTW)                                                                       \
        if (kt + 2 < ntiles) {                                                                    \
            KP_STORE_TILE(BS)                                                                     \
            if (kt + 3 < ntiles) {                                                                \
                KP_LOAD_TILE()                                                                    \
            }                                                                                     \
        }                                                                                         \
        KP_SM_FINISH(kt + 1)                                                                      \
        lds_barrier();                                                                            \
        ++kt;                                                                                     \
    }

    f32x4 sp[4];
    f32x4 sv;
    bf16x8 pa[4];

    // ---- prologue: tiles 0 and 1 into the ring, tile 2 into registers; SM(0) -------
    KP_ROWS_OF(0)
    KP_LOAD_TILE()
    KP_STORE_TILE(0)
    if (ntiles > 1) {
        KP_ROWS_OF(1)
        KP_LOAD_TILE()
        KP_STORE_TILE(1)
        if (ntiles > 2) {
            KP_ROWS_OF(2)
            KP_LOAD_TILE()
        }
    }
    lds_barrier();
    KP_QK(0)
    KP_QK_STORE()
    lds_barrier();
    KP_SM_READ()
    KP_SM_FINISH(0)
    lds_barrier();

    // the loop runs three steps per pass so that every ring buffer index is a
    // compile-time constant
    int kt = 0;
    for (;;) {
        if (kt + 1 >= ntiles) break;
        KP_STEP(0, 1, 2)
        if (kt + 1 >= ntiles) break;
        KP_STEP(1, 2, 0)
        if (kt + 1 >= ntiles) break;
        KP_STEP(2, 0, 1)
    }
    // last tile: PV only
    if (__builtin_amdgcn_readfirstlane(rebase_tile) == kt + 1) {
        f32x4 al[4];
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) al[ht] = *reinterpret_cast<const f32x4*>(alpha_s + 16 * ht + 4 * g);
#pragma unroll
        for (int ht = 0; ht < 4; ++ht)
#pragma unroll
            for (int dtl = 0; dtl < DTW; ++dtl) o[ht][dtl] *= al[ht];
    }
    KP_READ_P()
    KP_PV(kt % MLA_NBUF, 0, DTW)
#undef KP_STEP
#undef KP_READ_P
#undef KP_PV
#undef KP_SM_FINISH
#undef KP_SM_READ
#undef KP_QK_STORE
#undef KP_QK

    // ---- normalise and write ----------------------------------------------------
    {
        const float lr = sum_in_8(l_run);
        const float le = sum_in_8(l_lse);
        if ((lane & 7) == 0) {
            lsum[hown * 2] = lr;
            lsum[hown * 2 + 1] = le;
            mref_s[hown] = m_ref;
        }
    }
    compiler_fence();
    __syncthreads();   // all waves done with the ring; sums visible
    if (lse && tid < heads)
        lse[(size_t)i * heads + tid] = (mref_s[tid] + log2f(lsum[tid * 2 + 1])) * 0.69314718055994530942f;
    // stage O (bf16, [head][D], rows padded by 16 bytes against bank conflicts)
    // in the ring, then copy the real heads out
    uint16_t* stage = reinterpret_cast<uint16_t*>(ring);
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        f32x4 inv;
#pragma unroll
        for (int e = 0; e < 4; ++e) inv[e] = 1.0f / lsum[(16 * ht + 4 * g + e) * 2];
#pragma unroll
        for (int dtl = 0; dtl < DTW; ++dtl) {
            const int col = 16 * (wave * DTW + dtl) + n;
            if (col < D) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    stage[(16 * ht + 4 * g + e) * (D + 8) + col] = f32_to_bf16_rne(o[ht][dtl][e] * inv[e]);
            }
        }
    }
    __syncthreads();
    uint4* dst = reinterpret_cast<uint4*>(orow);
    const int nvec = heads * D / 8;
    for (int e = tid; e < nvec; e += NT) {
        const int h = e / (D / 8), c = e % (D / 8);
        dst[e] = *reinterpret_cast<const uint4*>(ring + h * (D * 2 + 16) + c * 16);
    }
#undef KP_ROWS_OF
#undef KP_LOAD_TILE
#undef KP_STORE_TILE
}

template <int D>
static hipError_t launch_mla_t(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int num_q,
                               int num_kv, int heads, int row_width, float scale_log2, uint16_t* out,
                               float* lse, hipStream_t stream) {
    sparse_mla_kernel<D><<<num_q, 64 * MLA_NW, 0, stream>>>(q, kv, indices, num_kv, heads, row_width, scale_log2,
                                                             out, lse);
    return hipGetLastError();
}

int sparse_mla_max_row_width() { return MLA_MAX_ROW; }

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int num_q,
                             int num_kv, int heads, int d_latent, int row_width, float scale_log2,
                             uint16_t* out, float* lse, hipStream_t stream) {
    if (num_q == 0) return hipSuccess;
    if (d_latent == 512)
        return launch_mla_t<512>(q, kv, indices, num_q, num_kv, heads, row_width, scale_log2, out, lse, stream);
    return launch_mla_t<64>(q, kv, indices, num_q, num_kv, heads, row_width, scale_log2, out, lse, stream);
}

}  // namespace kp
