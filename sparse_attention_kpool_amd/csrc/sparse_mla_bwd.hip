// Backward of the absorbed sparse latent attention (MLA) on gfx950: dQ and
// dKV for a given output gradient dO, over the same index rows as the forward.
//
// NeMo AutoModel "GLM-5.3-Flash" page, Attention Backends: training runs a
// fast sparse forward and a fast sparse backward, validated against a dense
// SDPA reference by cosine and relative RMSE of the output, dQ and dKV (NeMo
// AutoModel PR "add GLM-5.3-Flash training support", "cuDNN sparse MLA parity
// and performance"); prime-rl PR "GLM-5.3-Flash text model", Summary, third
// bullet: the indexer is frozen, so the index rows are constants here. With
// p the softmax weights of a (query, head) over its valid entries j (latent
// row r_j = key k_j = value v_j):
//   dp_j = <dO, v_j>,  delta = sum_j p_j dp_j = <dO, O>,  ds_j = p_j (dp_j - delta)
//   dQ = scale sum_j ds_j k_j,   dKV[r_j] += scale ds_j q + p_j dO.
// p is recomputed from the forward's lse. delta is first taken from the
// forward's output, which is rounded to bf16; where the softmax is peaked the
// ds terms cancel and that rounding would dominate them. So the dQ kernel also
// sums p_j dp_j in fp32 over the row (the exact delta) and removes the
// difference afterwards: dQ gains scale (delta_used - delta) O (as the keys are
// the values, sum_j p_j k_j is the output), and the dKV product takes
// dO + scale (delta_used - delta) q in place of dO (the p-weighted terms carry
// the same difference).
//
// Two kernels, one workgroup (4 waves, one per SIMD) per query each:
//  * mla_bwd_dq_kernel: for S, dP and ds, wave w owns heads 16w .. 16w+15 and
//    every row of a 64-row tile. The rows are gathered into LDS exactly as in
//    the forward. Per tile: S^T = K . Q^T and dP^T = K . dO^T (each K fragment
//    feeds both MFMAs), then p and scale*ds in registers; the ds values go
//    through LDS, and wave w adds dQ^T += K^T . (scale ds)^T for the w-th
//    quarter of the latent columns (padded to at least 128) of all 64 heads
//    (K^T read with the transposing LDS read, each fragment feeding four head
//    tiles). The K rows enter the QK
//    MFMAs in a permuted order so that each lane's ds values are the B operand
//    layout of the dQ MFMA. dQ stays in registers for the whole row (no merge:
//    the waves own disjoint columns). scale*ds and p of every valid slot are
//    written to the workspace, head-major: coef[query][h][slot] (h < 64:
//    scale*ds, 64 + h: p), bf16.
//  * dKV (below): each valid slot's dKV row is coef^T . [Q; dO], a product
//    over its 128 coefficients (mla_bwd_dkv_part_kernel, MFMA); the rows are
//    then summed per latent row in a fixed order (a stable sort of the slots
//    by row, an ordered reduction), so dKV is bit-reproducible.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_mla_common.h"
#include "kp_select.h"

namespace kp {

constexpr int BW_COEF = 128;   // coefficients per slot: scale*ds and p of 64 heads
constexpr int BW_RING = 4;     // LDS operand fragments in flight ahead of the MFMAs that use them

// Slot stride of the coefficient workspace rows: the index row width rounded
// up to whole 64-slot tiles.
__host__ __device__ __forceinline__ int bwd_coef_stride(int row_width) { return (row_width + 63) / 64 * 64; }

// Compacts the valid entries of an index row (0 <= e < num_kv, original order)
// into list[]: the entries themselves, and their positions in the row into
// pos[] when pos is given. Every thread of the 256-thread workgroup calls it;
// returns the count. Ends with the list visible to all.
__device__ __forceinline__ int bwd_compact(const int32_t* __restrict__ irow, int row_width, int num_kv,
                                           int32_t* list, int* rcnt, int32_t* pos = nullptr) {
    constexpr int NT = 64 * MLA_NW, NRND = MLA_MAX_ROW / NT;
    static_assert(NRND * MLA_NW == 64, "one count per lane");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int ent[NRND];
#pragma unroll
    for (int k = 0; k < NRND; ++k) {
        const int j = NT * k + tid;
        ent[k] = j < row_width ? irow[j] : -1;
    }
    unsigned long long bal[NRND];
#pragma unroll
    for (int k = 0; k < NRND; ++k) {
        bal[k] = __ballot(ent[k] >= 0 && ent[k] < num_kv);
        if (lane == 0) rcnt[k * MLA_NW + wave] = __popcll(bal[k]);
    }
    __syncthreads();
    const int c = rcnt[lane];
    int x = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(x, o, 64);
        if (lane >= o) x += u;
    }
    const int n_valid = __builtin_amdgcn_readfirstlane(__shfl(x, 63, 64));
    const int excl = x - c;
#pragma unroll
    for (int k = 0; k < NRND; ++k) {
        const int base = __shfl(excl, k * MLA_NW + wave, 64);
        const uint32_t below = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[k] >> 32),
                                                         __builtin_amdgcn_mbcnt_lo((uint32_t)bal[k], 0u));
        if (ent[k] >= 0 && ent[k] < num_kv) {
            list[base + below] = ent[k];
            if (pos) pos[base + below] = NT * k + tid;
        }
    }
    __syncthreads();
    return n_valid;
}

// ------------------------------------------------------------------ dQ ------
template <int D>
__global__ __launch_bounds__(64 * MLA_NW, 1) void mla_bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ indices,
    const uint16_t* __restrict__ o, const float* __restrict__ lse, const uint16_t* __restrict__ dout,
    int num_kv, int heads, int row_width, float scale, float scale_log2, uint16_t* __restrict__ dq,
    uint16_t* __restrict__ coef, float* __restrict__ dcorr) {
    constexpr int NT = 64 * MLA_NW;
    constexpr int DP = D < 128 ? 128 : D;   // latent width in LDS (zero-padded)
    constexpr int RB = DP * 2;
    constexpr int CH = D / 8;               // 16-byte chunks a gathered row brings
    constexpr int KS = DP / 32;             // QK k-steps
    constexpr int TILE_B = MLA_TK * (RB + 48);
    constexpr int RPW = MLA_TK / MLA_NW;

    constexpr int CQ = DP / 64;             // dQ column tiles per wave
    constexpr int DSP = 144;                // bytes per head in the ds exchange (64 slots + pad)

    __shared__ __align__(16) uint8_t ring[MLA_NBUF * TILE_B];
    __shared__ __align__(16) int32_t list[MLA_MAX_ROW];
    __shared__ int rcnt[64];
    __shared__ __align__(16) uint8_t dsx[64 * DSP];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int head = 16 * wave + n;        // this lane's head in the S, dP and ds steps
    const bool head_ok = head < heads;
    const int i = xcd_query(blockIdx.x, gridDim.x);
    const int wc = bwd_coef_stride(row_width);

    // Q, dO and O of this lane's head (the B operands of S^T = K . Q^T and
    // dP^T = K . dO^T, k-step ks: columns 32*ks + 8*g .. +7; O for delta = <dO, O>)
    // and its LSE, loaded before the index row is compacted so that the two
    // memory round trips overlap
    bf16x8 qf[KS], gf[KS], ofr[KS];
    float lse_h;
    {
        const size_t rowoff = ((size_t)i * heads + (head_ok ? head : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = 32 * ks + 8 * g;
            const bool in = head_ok && (DP == D || col < D);
            const int c = DP == D ? col : min(col, D - 8);
            qf[ks] = in ? *reinterpret_cast<const bf16x8*>(q + rowoff + c) : bf16x8{};
            gf[ks] = in ? *reinterpret_cast<const bf16x8*>(dout + rowoff + c) : bf16x8{};
            ofr[ks] = in ? *reinterpret_cast<const bf16x8*>(o + rowoff + c) : bf16x8{};
        }
        lse_h = head_ok ? lse[(size_t)i * heads + head] : 0.f;
    }

    const int n_valid = bwd_compact(indices + (size_t)i * row_width, row_width, num_kv, list, rcnt);
    if (n_valid == 0) {
        for (int e = tid; e < heads * D; e += NT) dq[(size_t)i * heads * D + e] = 0;
        return;
    }
    const int ntiles = (n_valid + MLA_TK - 1) / MLA_TK;
    // the gather list: byte offsets, padded to whole tiles with a valid row, adjusted
    // for the shared-M0 immediate offsets (as in the forward)
    {
        const int pad_end = ntiles * MLA_TK;
        if (tid < pad_end - n_valid) list[n_valid + tid] = list[0];
        __syncthreads();
        for (int p = tid; p < pad_end; p += NT)
            list[p] = (int32_t)((uint32_t)list[p] * (uint32_t)(D * 2) + 4096u - (uint32_t)row_base<RB>(p & 3));
        __syncthreads();
    }
    if (DP != D) {
        for (int e = tid; e < MLA_NBUF * TILE_B / 16; e += NT)
            reinterpret_cast<uint4*>(ring)[e] = make_uint4(0u, 0u, 0u, 0u);
        __syncthreads();
    }

    float delta = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) delta += (float)gf[ks][e] * (float)ofr[ks][e];
    // the four lanes of a head (g = 0..3) hold a quarter of the columns each
    delta += shfl_xor(delta, 16);
    delta += shfl_xor(delta, 32);
    const float lse2 = lse_h * 1.4426950408889634f;

    // gather: as in the forward (wave w brings rows 16w .. 16w+15 of each tile)
    const uint32_t ring_lds = lds_addr(ring);
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    const uint32_t wave_lds = ring_lds + (uint32_t)row_base<RB>(RPW * wave_s);
    const uint32_t lane16 = 16u * lane;
    const uint64_t kv_base = reinterpret_cast<uint64_t>(kv) - 4096u;
    const u32x4 kv_rsrc = u32x4{(uint32_t)kv_base, (uint32_t)(kv_base >> 32) & 0xFFFFu,
                                (uint32_t)((uint64_t)num_kv * (D * 2) + 4096u), 0x00020000u};
#define BW_ROWS_OF(kt_)                                                                        \
    int rws_[RPW];                                                                             \
    _Pragma("unroll") for (int c4_ = 0; c4_ < RPW / 4; ++c4_) {                                \
        const int4 rw_ = *reinterpret_cast<const int4*>(list + (kt_) * MLA_TK + RPW * wave_s + 4 * c4_); \
        rws_[4 * c4_] = __builtin_amdgcn_readfirstlane(rw_.x);                                 \
        rws_[4 * c4_ + 1] = __builtin_amdgcn_readfirstlane(rw_.y);                             \
        rws_[4 * c4_ + 2] = __builtin_amdgcn_readfirstlane(rw_.z);                             \
        rws_[4 * c4_ + 3] = __builtin_amdgcn_readfirstlane(rw_.w);                             \
    }                                                                                          \
    kp_sgpr_settle(rws_);
#define BW_ISSUE_ROW(j_, buf_)                                                                \
    {                                                                                          \
        if (DP == D || lane < CH) {                                                            \
            const uint32_t m0_ = __builtin_amdgcn_readfirstlane(                                \
                wave_lds + (uint32_t)((buf_) * TILE_B + row_base<RB>((j_) & ~3)));              \
            if (((j_) & 3) == 0) lds_dma16_row_at<0>(kv_rsrc, lane16, (uint32_t)rws_[j_], m0_);  \
            else if (((j_) & 3) == 1) lds_dma16_row_at<row_base<RB>(1)>(kv_rsrc, lane16, (uint32_t)rws_[j_], m0_); \
            else if (((j_) & 3) == 2) lds_dma16_row_at<row_base<RB>(2)>(kv_rsrc, lane16, (uint32_t)rws_[j_], m0_); \
            else lds_dma16_row_at<row_base<RB>(3)>(kv_rsrc, lane16, (uint32_t)rws_[j_], m0_);    \
        }                                                                                      \
    }
    {
        BW_ROWS_OF(0)
#pragma unroll
        for (int j = 0; j < RPW; ++j) BW_ISSUE_ROW(j, 0)
    }
    wait_vm0();
    lds_barrier();

    // QK A-operand row m of row sub-tile s (16 rows each) is tile row
    // 32*(s/2) + 8*(m/4) + 4*(s%2) + m%4: lane (g, n) then holds the S^T and dP^T
    // values of rows 32*(s/2) + 8*g + 4*(s%2) + e (e = 0..3), so that sub-tiles
    // 2kk and 2kk+1 give the eight rows 32*kk + 8*g .. +7 it feeds to dQ k-step kk
    int kb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) kb[s] = row_base<RB>(32 * (s >> 1) + 8 * (n >> 2) + 4 * (s & 1) + (n & 3)) + 16 * g;
    // K^T A operand of the wave's dQ column tile ct (columns DP/4*wave + 16*ct ..
    // +15), k-step kk: two transposing reads of rows 32*kk + 8*g + 4*b + e4, columns
    // DP/4*wave + 16*ct + 4*q4 .. +3: byte offset vb[kk][b] + 32*ct
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    int vb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int b = 0; b < 2; ++b) vb[kk][b] = row_base<RB>(32 * kk + 8 * g + 4 * b + e4) + 8 * q4 + DP / 2 * wave;

    // dQ^T of the wave's DP/4 columns for all 64 heads: acc[ht][ct] holds columns
    // DP/4*wave + 16*ct + 4*g .. +3 of head 16*ht + n
    f32x4 acc[4][CQ];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int ct = 0; ct < CQ; ++ct) acc[ht][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dsum = 0.f;   // sum of p_j dp_j over the lane's rows
    uint16_t* crow_ds = coef + ((size_t)i * BW_COEF + head) * wc;        // this lane's scale*ds row
    uint16_t* crow_p = coef + ((size_t)i * BW_COEF + 64 + head) * wc;    // and its p row

    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        {
            // the next tile's gather (the last tile gathers its own rows again)
            BW_ROWS_OF(kt + 1 < ntiles ? kt + 1 : kt)
#pragma unroll
            for (int j = 0; j < RPW; ++j) BW_ISSUE_ROW(j, buf ^ 1)
        }
        const uint8_t* tb = ring + buf * TILE_B;
        f32x4 sacc[4], pacc[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            sacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
            pacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        // K fragment u (k-step u / 4, sub-tile u % 4) is read BW_RING - 1 fragments
        // ahead of its two MFMAs; scheduling barriers keep that order (left alone, the
        // compiler reads each fragment right before its MFMAs and waits for it there)
        bf16x8 kr[BW_RING];
#pragma unroll
        for (int u = 0; u < BW_RING - 1; ++u) kr[u] = *reinterpret_cast<const bf16x8*>(tb + kb[u & 3] + 64 * (u >> 2));
#pragma unroll
        for (int u = 0; u < 4 * KS; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            if (u + BW_RING - 1 < 4 * KS) {
                const int un = u + BW_RING - 1;
                kr[un % BW_RING] = *reinterpret_cast<const bf16x8*>(tb + kb[un & 3] + 64 * (un >> 2));
            }
            __builtin_amdgcn_sched_barrier(0);
            sacc[u & 3] = mfma_bf16_16x16x32(kr[u % BW_RING], qf[u >> 2], sacc[u & 3]);
            pacc[u & 3] = mfma_bf16_16x16x32(kr[u % BW_RING], gf[u >> 2], pacc[u & 3]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // p and scale*ds of the lane's rows; rows past the list's end (and heads past
        // `heads`) get zero
        bf16x8 dsb[2], pb[2];
        const int row0 = kt * MLA_TK + 8 * g;
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = row0 + 32 * (s >> 1) + 4 * (s & 1) + e;
                float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[s][e], scale_log2, -lse2));
                if (!(slot < n_valid && head_ok)) p = 0.f;
                dsum = __builtin_fmaf(p, pacc[s][e], dsum);
                const float ds = scale * p * (pacc[s][e] - delta);
                dsb[s >> 1][4 * (s & 1) + e] = (__bf16)ds;
                pb[s >> 1][4 * (s & 1) + e] = (__bf16)p;
            }
        // the coefficients of slots kt*64 + 32*kk + 8*g .. +7 (zero for padded heads)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int slot = kt * MLA_TK + 32 * kk + 8 * g;
            *reinterpret_cast<bf16x8*>(crow_ds + slot) = dsb[kk];
            *reinterpret_cast<bf16x8*>(crow_p + slot) = pb[kk];
        }
        // dQ^T[cols, heads] += K^T[cols, rows] . (scale ds)^T[rows, heads], the columns
        // split over the waves: each wave's ds (its 16 heads) goes through LDS, so
        // that a K^T fragment, read once, feeds the four head tiles. The K^T
        // fragment of step u (k-step u / CQ, column tile u % CQ) is read BW_RING - 1
        // steps ahead of its MFMAs.
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            *reinterpret_cast<bf16x8*>(dsx + head * DSP + 2 * (32 * kk + 8 * g)) = dsb[kk];
        lds_barrier();
        bf16x8 dsf[2][4];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                dsf[kk][ht] = *reinterpret_cast<const bf16x8*>(dsx + (16 * ht + n) * DSP + 2 * (32 * kk + 8 * g));
        auto ktr = [&](int u) __attribute__((always_inline)) {
            const int kk = u / CQ, ct = u % CQ;
            const bf16x4 v0 = lds_read_tr16(tb + vb[kk][0] + 32 * ct);
            const bf16x4 v1 = lds_read_tr16(tb + vb[kk][1] + 32 * ct);
            return __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        };
        constexpr int NU = 2 * CQ, RA = NU < BW_RING ? NU : BW_RING;
        bf16x8 vr[RA];
#pragma unroll
        for (int u = 0; u < RA - 1; ++u) vr[u] = ktr(u);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            __builtin_amdgcn_sched_barrier(0);
            if (u + RA - 1 < NU) vr[(u + RA - 1) % RA] = ktr(u + RA - 1);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                acc[ht][u % CQ] = mfma_bf16_16x16x32(vr[u % RA], dsf[u / CQ][ht], acc[ht][u % CQ]);
        }
        __builtin_amdgcn_sched_barrier(0);
        // the next tile's rows have landed: every vector-memory operation but the
        // four coefficient stores issued after them is done (s_waitcnt vmcnt(4); the
        // counter retires in issue order): the stores may stay in flight across
        // the barrier
        __builtin_amdgcn_s_waitcnt(0x0F74);
        lds_barrier();
    }
#undef BW_ROWS_OF
#undef BW_ISSUE_ROW
    // the exact delta of the lane's head (its four lane groups hold a quarter of
    // the rows each) and the correction of dQ: + scale (delta_used - delta) O, each
    // head's correction passed to the waves that hold its columns through LDS
    dsum += shfl_xor(dsum, 16);
    dsum += shfl_xor(dsum, 32);
    const float corr = head_ok ? delta - dsum : 0.f;
    float* corr_s = reinterpret_cast<float*>(dsx);   // the exchange buffer is free now
    if (g == 0) {
        dcorr[(size_t)i * 64 + head] = corr;
        corr_s[head] = corr;
    }
    __syncthreads();
    // dQ: lane (g, n) holds columns DP/4*wave + 16*ct + 4*g .. +3 of head 16*ht + n
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int h = 16 * ht + n;
        if (h < heads) {
            const uint16_t* o_row = o + ((size_t)i * heads + h) * D;
            uint16_t* dq_h = dq + ((size_t)i * heads + h) * D;
            const float sc = scale * corr_s[h];
#pragma unroll
            for (int ct = 0; ct < CQ; ++ct) {
                const int col = DP / 4 * wave + 16 * ct + 4 * g;
                if (DP == D || col < D) {
                    const uint2 ov = *reinterpret_cast<const uint2*>(o_row + col);
                    const float of[4] = {bf16_lo(ov.x), bf16_hi(ov.x), bf16_lo(ov.y), bf16_hi(ov.y)};
                    bf16x4 r;
#pragma unroll
                    for (int e = 0; e < 4; ++e) r[e] = (__bf16)__builtin_fmaf(sc, of[e], acc[ht][ct][e]);
                    *reinterpret_cast<bf16x4*>(dq_h + col) = r;
                }
            }
        }
    }
}

// ----------------------------------------------------------------- dKV ------
// dKV is a sum over every (query, slot) whose index entry names the row. It is
// made deterministic by fixing the order of that sum instead of leaving it to
// the arrival order of atomic adds: the queries are taken in chunks of at most
// BW_QC; for each chunk
//  1. mla_bwd_dkv_part_kernel writes each valid slot's contribution row
//     coef^T . [Q; dO] (D columns, rounded to bf16) to `part`, at the slot's
//     position e = i * row_width + j in the chunk's index rows;
//  2. a stable least-significant-digit radix sort (8-bit digits) orders the
//     positions e by their index entry (invalid entries get the key num_kv and
//     sort last), so each row's contributions form one run, in e order;
//  3. bwd_dkv_reduce_kernel sums runs of the sorted list in order (fp32) and
//     adds each into dKV; a run that crosses a tile boundary leaves per-tile
//     partial sums that bwd_dkv_fixup_kernel adds in tile order.
// The chunks run in order, so dKV is bit-reproducible.
constexpr int BW_QC = 8192;   // queries per chunk

// LDS layout of a coefficient tile (128 rows of 64 slots, 128 bytes each): row
// r at byte r*176 + 16*(r & 1); the transposing reads of the B operand (two
// groups of 16 lanes per pass, 4 rows x 32 bytes each) then hit distinct banks.
__device__ __forceinline__ constexpr int coef_row(int r) { return r * 176 + 16 * (r & 1); }
constexpr int BW_CTILE_B = 128 * 176;   // bytes per coefficient tile

// two floats rounded to bf16 (nearest even), the first in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t{a, b}), bf16x2_t));
}

template <int D>
__global__ __launch_bounds__(64 * MLA_NW, 1) void mla_bwd_dkv_part_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const int32_t* __restrict__ indices,
    const uint16_t* __restrict__ coef, const float* __restrict__ dcorr, int num_kv, int heads, int row_width,
    float scale, uint16_t* __restrict__ part) {
    constexpr int NT = 64 * MLA_NW;
    constexpr int DP = D < 128 ? 128 : D;
    constexpr int RB = DP * 2;
    constexpr int CW = DP / 4;              // columns per wave
    constexpr int CTW = CW / 16;            // 16-wide column tiles per wave
    constexpr int XB = 64 * (RB + 48);      // bytes of one staged operand (64 heads)

    constexpr int CBUF = 3;                 // coefficient tiles in the LDS ring
    __shared__ __align__(16) uint8_t xs[XB > CBUF * BW_CTILE_B ? XB : CBUF * BW_CTILE_B];
    __shared__ __align__(16) int32_t list[MLA_MAX_ROW];
    __shared__ __align__(16) int32_t jpos[MLA_MAX_ROW];
    __shared__ int rcnt[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int i = xcd_query(blockIdx.x, gridDim.x);
    const int wc = bwd_coef_stride(row_width);

    // The coefficient tile 0 and every Q and dO chunk this thread stages are
    // loaded first, all in flight together and before the index row is compacted
    // (the round trips overlap); head h's scale (delta_used - delta) comes with them.
    constexpr int XC = 64 * (DP / 8) / NT;   // 16-byte chunks of Q (and of dO) per thread
    static_assert(XC * NT == 64 * (DP / 8), "whole chunks per thread");
    const uint16_t* crow = coef + (size_t)i * BW_COEF * wc;
    const int cr = tid >> 1, chalf = tid & 1;
    u32x4 cpre[4];
    auto load_tile = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            cpre[u] = *reinterpret_cast<const u32x4*>(crow + (size_t)cr * wc + kt * MLA_TK + 32 * chalf + 8 * u);
    };
    load_tile(0);
    u32x4 qv[XC], gv[XC];
    float sc[XC];
    {
        const uint16_t* qq = q + (size_t)i * heads * D;
        const uint16_t* gg = dout + (size_t)i * heads * D;
#pragma unroll
        for (int u = 0; u < XC; ++u) {
            // 64 rows (heads) x DP columns; heads past `heads` and padded columns are zero
            const int c = tid + NT * u, h = c / (DP / 8), col = 8 * (c % (DP / 8));
            qv[u] = gv[u] = u32x4{0u, 0u, 0u, 0u};
            sc[u] = 0.f;
            if (h < heads && col < D) {
                qv[u] = *reinterpret_cast<const u32x4*>(qq + (size_t)h * D + col);
                gv[u] = *reinterpret_cast<const u32x4*>(gg + (size_t)h * D + col);
                sc[u] = scale * dcorr[(size_t)i * 64 + h];
            }
        }
    }
    const int n_valid = bwd_compact(indices + (size_t)i * row_width, row_width, num_kv, list, rcnt, jpos);
    if (n_valid == 0) return;
    const int ntiles = (n_valid + MLA_TK - 1) / MLA_TK;

    // A operands of dKV^T[cols, slots] = X^T[cols, coefs] . coef[coefs, slots] with X =
    // [Q; dO] (coefficients 0..63: Q of head c, 64..127: dO of head c - 64): lane (g, n)
    // of k-step kk holds coefficients 32*kk + 8*g .. +7 of column
    // 32*(ct/2) + 8*(n/4) + 4*(ct%2) + n%4 of the wave's columns. Over a pair of
    // column tiles, lane (g, n) of the products then holds the 8 consecutive
    // columns 32*(ct/2) + 8*g .. +7 of its slot: one 16-byte store. Q, then dO + scale (delta_used - delta) Q (rounded to bf16),
    // is staged in LDS (head h at row_base(h)) and read with the transposing read.
    bf16x8 xf[4][CTW];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int u = 0; u < XC; ++u) {
            const int c = tid + NT * u, h = c / (DP / 8), col = 8 * (c % (DP / 8));
            u32x4 v = qv[u];
            if (half == 1) {
                const uint32_t qw[4] = {v.x, v.y, v.z, v.w}, gw[4] = {gv[u].x, gv[u].y, gv[u].z, gv[u].w};
                uint32_t ow[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = f32_to_bf16_rne(__builtin_fmaf(sc[u], bf16_lo(qw[e]), bf16_lo(gw[e])));
                    const uint32_t hi = f32_to_bf16_rne(__builtin_fmaf(sc[u], bf16_hi(qw[e]), bf16_hi(gw[e])));
                    ow[e] = lo | (hi << 16);
                }
                v = u32x4{ow[0], ow[1], ow[2], ow[3]};
            }
            *reinterpret_cast<u32x4*>(xs + row_base<RB>(h) + 2 * col) = v;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                const int colb = 2 * CW * wave + 64 * (ct >> 1) + 16 * q4 + 8 * (ct & 1);
                const bf16x4 v0 = lds_read_tr16(xs + row_base<RB>(32 * kq + 8 * g + e4) + colb);
                const bf16x4 v1 = lds_read_tr16(xs + row_base<RB>(32 * kq + 8 * g + 4 + e4) + colb);
                xf[2 * half + kq][ct] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        __syncthreads();
    }

    // coefficient tiles (128 rows x 64 slots of bf16) through a ring of CBUF LDS
    // tiles: thread t copies 64 bytes of row t/2; the next tile's loads are issued
    // before the current tile's MFMAs
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<u32x4*>(xs + buf * BW_CTILE_B + coef_row(cr) + 64 * chalf + 16 * u) = cpre[u];
    };
    const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
        part + (size_t)i * row_width * D, 0, 2 * row_width * D, 0x00020000);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt % CBUF;
        if (kt + 1 < ntiles) load_tile(kt + 1);
        const uint8_t* tb = xs + buf * BW_CTILE_B;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // B operand: lane (g, n) holds coefficients 32*kk + 8*g .. +7 of slot 16*rt + n
            bf16x8 bf[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x4 v0 = lds_read_tr16(tb + coef_row(32 * kk + 8 * g + e4) + 32 * rt + 8 * q4);
                const bf16x4 v1 = lds_read_tr16(tb + coef_row(32 * kk + 8 * g + 4 + e4) + 32 * rt + 8 * q4);
                bf[kk] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            // lane (g, n) gets slot 16*rt + n, columns CW*wave + 32*p + 8*g .. +7 from the
            // column tiles 2p and 2p + 1. Each column tile has its own accumulator, so the
            // products run back to back; the stores are unconditional buffer stores (a
            // fixed count per tile, so the wait for the next coefficient tile does not
            // cover them), and a slot past the valid ones gets an offset beyond the
            // buffer, which drops it.
            const int slot = kt * MLA_TK + 16 * rt + n;
            const uint32_t voff = slot < n_valid ? 2u * (uint32_t)(jpos[slot] * D + CW * wave + 8 * g) : 0x80000000u;
            f32x4 r[CTW];
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                r[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) r[ct] = mfma_bf16_16x16x32(xf[kk][ct], bf[kk], r[ct]);
            }
#pragma unroll
            for (int pt = 0; pt < CTW / 2; ++pt) {
                if (DP == D || CW * wave + 32 * pt < D) {
                    const f32x4 lo = r[2 * pt], hi = r[2 * pt + 1];
                    const u32x4 o = {pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]),
                                     pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3])};
                    __builtin_amdgcn_raw_buffer_store_b128(o, prs, voff, 64 * pt, 0);
                }
            }
        }
        // tile kt + 1 goes to the ring slot last read in tile kt - 2: every wave has
        // passed the barrier that ended tile kt - 1 since, so one barrier per tile
        if (kt + 1 < ntiles) store_tile((kt + 1) % CBUF);
        __syncthreads();
    }
}

// ---------------------------------------------- stable radix sort by row ----
// Entries are the chunk's index positions e = 0 .. E-1 in order; the key of e is
// its index entry when valid, else num_kv. Each pass orders the entries by one
// 8-bit digit of the key, keeping the previous order among equal digits: a tile
// of RX_TILE consecutive entries counts its digits (bwd_rx_hist_kernel), the
// counts are turned into each tile's first output position per digit
// (bwd_rx_scan_kernel), and the tile writes its entries there in order
// (bwd_rx_scatter_kernel). After the passes that cover the key's bits, equal
// keys are contiguous and in increasing e.
constexpr int RX_NT = 256, RX_ROUNDS = 16, RX_TILE = RX_NT * RX_ROUNDS, RX_BINS = 256;

template <bool FIRST>
__device__ __forceinline__ uint32_t rx_key_at(const int32_t* __restrict__ idx, const uint32_t* __restrict__ keys,
                                              int e, int num_kv) {
    if constexpr (FIRST) {
        const int v = idx[e];
        return (v >= 0 && v < num_kv) ? (uint32_t)v : (uint32_t)num_kv;
    } else {
        return keys[e];
    }
}

// hist[d * ntiles + tile] = entries of the tile whose digit is d
template <bool FIRST>
__global__ __launch_bounds__(RX_NT) void bwd_rx_hist_kernel(const int32_t* __restrict__ idx,
                                                            const uint32_t* __restrict__ keys, int E, int num_kv,
                                                            int shift, uint32_t* __restrict__ hist, int ntiles) {
    __shared__ uint32_t h[RX_BINS];
    const int tid = threadIdx.x;
    h[tid] = 0u;
    __syncthreads();
    const int base = blockIdx.x * RX_TILE;
#pragma unroll 4
    for (int r = 0; r < RX_ROUNDS; ++r) {
        const int e = base + r * RX_NT + tid;
        if (e < E) atomicAdd(&h[(rx_key_at<FIRST>(idx, keys, e, num_kv) >> shift) & (RX_BINS - 1)], 1u);
    }
    __syncthreads();
    hist[(size_t)tid * ntiles + blockIdx.x] = h[tid];
}

// One workgroup per digit: the tiles' counts of that digit become exclusive
// offsets within the digit (in place), and totals[d] the digit's count.
__global__ __launch_bounds__(RX_NT) void bwd_rx_scan_kernel(uint32_t* __restrict__ hist, int ntiles,
                                                            uint32_t* __restrict__ totals) {
    __shared__ int wave_buf[RX_NT / 64];
    uint32_t* row = hist + (size_t)blockIdx.x * ntiles;
    int carry = 0;
    for (int t0 = 0; t0 < ntiles; t0 += RX_NT) {
        const int t = t0 + (int)threadIdx.x;
        const int v = t < ntiles ? (int)row[t] : 0;
        int total;
        const int ex = block_excl_scan<RX_NT>(v, wave_buf, &total);
        if (t < ntiles) row[t] = (uint32_t)(carry + ex);
        carry += total;
    }
    if (threadIdx.x == 0) totals[blockIdx.x] = (uint32_t)carry;
}

template <bool FIRST>
__global__ __launch_bounds__(RX_NT) void bwd_rx_scatter_kernel(
    const int32_t* __restrict__ idx, const uint32_t* __restrict__ keys_in, const uint32_t* __restrict__ vals_in,
    int E, int num_kv, int shift, const uint32_t* __restrict__ hist, const uint32_t* __restrict__ totals, int ntiles,
    uint32_t* __restrict__ keys_out, uint32_t* __restrict__ vals_out) {
    __shared__ int dbase[RX_BINS];                 // next output position of each digit
    __shared__ int wcnt[RX_NT / 64][RX_BINS];      // this round's digit counts per wave
    __shared__ int wave_buf[RX_NT / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    {
        int tot;
        const int ex = block_excl_scan<RX_NT>((int)totals[tid], wave_buf, &tot);
        dbase[tid] = ex + (int)hist[(size_t)tid * ntiles + blockIdx.x];
    }
    const uint64_t below = (1ull << lane) - 1ull;
    const int base = blockIdx.x * RX_TILE;
    for (int r = 0; r < RX_ROUNDS; ++r) {
        // entries are taken in order: round r, then wave, then lane
        const int e = base + r * RX_NT + tid;
        const bool ok = e < E;
        uint32_t key = 0u, val = 0u;
        if (ok) {
            key = rx_key_at<FIRST>(idx, keys_in, e, num_kv);
            val = FIRST ? (uint32_t)e : vals_in[e];
        }
        const int dig = (int)((key >> shift) & (RX_BINS - 1));
        // lanes of this wave with the same digit
        uint64_t peers = __ballot(ok);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
            const uint64_t m = __ballot((dig >> b) & 1);
            peers &= ((dig >> b) & 1) ? m : ~m;
        }
        for (int d = lane; d < RX_BINS; d += 64) wcnt[wave][d] = 0;
        // the lowest lane of each digit group writes the group's size (after the
        // zeroing: a wave's LDS operations complete in order)
        if (ok && (peers & below) == 0ull) wcnt[wave][dig] = __popcll(peers);
        __syncthreads();
        if (ok) {
            int pos = dbase[dig] + __popcll(peers & below);
            for (int w = 0; w < wave; ++w) pos += wcnt[w][dig];
            keys_out[pos] = key;
            vals_out[pos] = val;
        }
        __syncthreads();
        dbase[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
        __syncthreads();
    }
}

// --------------------------------------------------- ordered reduction ------
// Wave t sums the sorted entries [RED_TILE*t, RED_TILE*(t+1)): a run of one
// row that starts and ends inside the tile is added to dKV directly (no other
// wave sees that row in this chunk). The first run, when it began in an earlier
// tile, is left in carry[t][0] (flag RED_HEAD, plus RED_CONT when it also goes
// on past the tile); the last run, when it began here and goes on, is left in
// carry[t][1] with its row in ckey[t] (flag RED_TAIL).
constexpr int RED_TILE = 128;
constexpr int RED_HEAD = 1, RED_CONT = 2, RED_TAIL = 4;

template <int D>
__device__ __forceinline__ void red_load(const uint16_t* __restrict__ part, uint32_t e, int lane, float (&x)[D / 64]) {
    constexpr int CPL = D / 64;
    const uint16_t* p = part + (size_t)e * D + CPL * lane;
    if constexpr (CPL == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
        x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
    } else {
        static_assert(CPL == 1, "D is 512 or 64");
        x[0] = __uint_as_float((uint32_t)p[0] << 16);
    }
}

template <int D>
__device__ __forceinline__ void red_flush(float* __restrict__ dst, int lane, const float (&acc)[D / 64], bool add) {
    constexpr int CPL = D / 64;
    float* p = dst + CPL * lane;
    if constexpr (CPL == 8) {
        float4 a = make_float4(acc[0], acc[1], acc[2], acc[3]), b = make_float4(acc[4], acc[5], acc[6], acc[7]);
        if (add) {
            const float4 o0 = *reinterpret_cast<const float4*>(p), o1 = *reinterpret_cast<const float4*>(p + 4);
            a.x = o0.x + a.x; a.y = o0.y + a.y; a.z = o0.z + a.z; a.w = o0.w + a.w;
            b.x = o1.x + b.x; b.y = o1.y + b.y; b.z = o1.z + b.z; b.w = o1.w + b.w;
        }
        *reinterpret_cast<float4*>(p) = a;
        *reinterpret_cast<float4*>(p + 4) = b;
    } else {
        p[0] = add ? p[0] + acc[0] : acc[0];
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_reduce_kernel(const uint32_t* __restrict__ keys,
                                                             const uint32_t* __restrict__ vals, int E, int num_kv,
                                                             const uint16_t* __restrict__ part,
                                                             float* __restrict__ dkv, float* __restrict__ carry,
                                                             int32_t* __restrict__ cflag, int32_t* __restrict__ ckey) {
    constexpr int CPL = D / 64;
    constexpr int U = 8;   // entries whose rows are loaded together
    const int lane = threadIdx.x & 63;
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    const int k0 = t * RED_TILE;
    if (k0 >= E) return;
    const int kend = min(k0 + RED_TILE, E);
    const uint32_t sent = (uint32_t)num_kv;
    const uint32_t ka = k0 + lane < kend ? keys[k0 + lane] : sent;
    const uint32_t kb = k0 + 64 + lane < kend ? keys[k0 + 64 + lane] : sent;
    const uint32_t va = k0 + lane < kend ? vals[k0 + lane] : 0u;
    const uint32_t vb = k0 + 64 + lane < kend ? vals[k0 + 64 + lane] : 0u;
    const uint32_t prev = k0 > 0 ? keys[k0 - 1] : sent;
    const uint32_t next = kend < E ? keys[kend] : sent;
    // the keys are sorted, so the real entries (key < num_kv) are a prefix
    const int nreal = __popcll(__ballot(ka < sent)) + __popcll(__ballot(kb < sent));
    auto key_at = [&](int j) { return j < 64 ? __builtin_amdgcn_readlane(ka, j) : __builtin_amdgcn_readlane(kb, j - 64); };
    auto val_at = [&](int j) { return j < 64 ? __builtin_amdgcn_readlane(va, j) : __builtin_amdgcn_readlane(vb, j - 64); };

    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    uint32_t cur = sent;
    bool head = false;
    int flags = 0;
    for (int j0 = 0; j0 < nreal; j0 += U) {
        float x[U][CPL];
#pragma unroll
        for (int u = 0; u < U; ++u) red_load<D>(part, val_at(min(j0 + u, nreal - 1)), lane, x[u]);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int j = j0 + u;
            if (j < nreal) {
                const uint32_t key = key_at(j);
                if (key != cur) {
                    if (cur != sent) {
                        // a run that ended inside the tile
                        if (head) {
                            red_flush<D>(carry + (size_t)(2 * t) * D, lane, acc, false);
                            flags |= RED_HEAD;
                        } else {
                            red_flush<D>(dkv + (size_t)cur * D, lane, acc, true);
                        }
                    }
                    cur = key;
                    head = j == 0 && key == prev;
#pragma unroll
                    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
                }
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] += x[u][c];
            }
        }
    }
    if (cur != sent) {
        const bool cont = nreal == kend - k0 && cur == next;
        if (head) {
            red_flush<D>(carry + (size_t)(2 * t) * D, lane, acc, false);
            flags |= RED_HEAD | (cont ? RED_CONT : 0);
        } else if (cont) {
            red_flush<D>(carry + (size_t)(2 * t + 1) * D, lane, acc, false);
            flags |= RED_TAIL;
            if (lane == 0) ckey[t] = (int32_t)cur;
        } else {
            red_flush<D>(dkv + (size_t)cur * D, lane, acc, true);
        }
    }
    if (lane == 0) cflag[t] = flags;
}

// Runs that cross tiles: the wave of the tile where a run began adds its tail
// and the heads of the following tiles, in tile order, into dKV.
template <int D>
__global__ __launch_bounds__(256) void bwd_dkv_fixup_kernel(int ntiles, const int32_t* __restrict__ cflag,
                                                            const int32_t* __restrict__ ckey,
                                                            const float* __restrict__ carry,
                                                            float* __restrict__ dkv) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    const int t = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
    if (t >= ntiles || !(cflag[t] & RED_TAIL)) return;
    float acc[CPL];
    const float* c0 = carry + (size_t)(2 * t + 1) * D + CPL * lane;
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = c0[c];
    for (int u = t + 1; u < ntiles; ++u) {
        const float* cu = carry + (size_t)(2 * u) * D + CPL * lane;
#pragma unroll
        for (int c = 0; c < CPL; ++c) acc[c] += cu[c];
        if (!(cflag[u] & RED_CONT)) break;
    }
    red_flush<D>(dkv + (size_t)ckey[t] * D, lane, acc, true);
}

// Workspace of the backward, for chunks of min(num_q, BW_QC) queries.
struct BwdWs {
    uint16_t* coef;      // [qc][BW_COEF][bwd_coef_stride(W)]
    uint16_t* part;      // [qc * W][D]
    uint32_t* key[2];    // [qc * W] each
    uint32_t* val[2];
    uint32_t* hist;      // [RX_BINS][ceil(qc * W / RX_TILE)]
    uint32_t* totals;    // [RX_BINS]
    float* carry;        // [ceil(qc * W / RED_TILE)][2][D]
    int32_t* cflag;      // [ceil(qc * W / RED_TILE)]
    int32_t* ckey;
    float* dcorr;        // [qc][64]: delta_used - delta per (query, head)
};

static size_t a256(size_t b) { return (b + 255) / 256 * 256; }

static size_t bwd_ws_layout(int num_q, int d, int row_width, uint8_t* base, BwdWs* ws) {
    const size_t qc = (size_t)(num_q < BW_QC ? num_q : BW_QC);
    const size_t E = qc * (size_t)row_width;
    const size_t nx = (E + RX_TILE - 1) / RX_TILE, nr = (E + RED_TILE - 1) / RED_TILE;
    const size_t sz[] = {a256(qc * BW_COEF * (size_t)bwd_coef_stride(row_width) * 2), a256(E * (size_t)d * 2),
                         a256(E * 4), a256(E * 4), a256(E * 4), a256(E * 4), a256(RX_BINS * nx * 4),
                         a256(RX_BINS * 4), a256(nr * 2 * (size_t)d * 4), a256(nr * 4), a256(nr * 4),
                         a256(qc * 64 * 4)};
    size_t off[sizeof(sz) / sizeof(sz[0])], total = 0;
    for (size_t k = 0; k < sizeof(sz) / sizeof(sz[0]); ++k) {
        off[k] = total;
        total += sz[k];
    }
    if (ws) {
        ws->coef = reinterpret_cast<uint16_t*>(base + off[0]);
        ws->part = reinterpret_cast<uint16_t*>(base + off[1]);
        ws->key[0] = reinterpret_cast<uint32_t*>(base + off[2]);
        ws->val[0] = reinterpret_cast<uint32_t*>(base + off[3]);
        ws->key[1] = reinterpret_cast<uint32_t*>(base + off[4]);
        ws->val[1] = reinterpret_cast<uint32_t*>(base + off[5]);
        ws->hist = reinterpret_cast<uint32_t*>(base + off[6]);
        ws->totals = reinterpret_cast<uint32_t*>(base + off[7]);
        ws->carry = reinterpret_cast<float*>(base + off[8]);
        ws->cflag = reinterpret_cast<int32_t*>(base + off[9]);
        ws->ckey = reinterpret_cast<int32_t*>(base + off[10]);
        ws->dcorr = reinterpret_cast<float*>(base + off[11]);
    }
    return total;
}

template <int D>
static hipError_t launch_bwd_t(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* o,
                               const float* lse, const uint16_t* dout, int num_q, int num_kv, int heads,
                               int row_width, float scale, uint16_t* dq, float* dkv, void* workspace,
                               hipStream_t stream) {
    hipError_t e = launch_fill_f32(dkv, (size_t)num_kv * D, 0.0f, stream);
    if (e != hipSuccess) return e;
    BwdWs ws;
    bwd_ws_layout(num_q, D, row_width, static_cast<uint8_t*>(workspace), &ws);
    const float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    // digits cover the key's bits, num_kv (the key of invalid entries) included
    const int key_bits = num_kv > 0 ? 32 - __builtin_clz((unsigned)num_kv) : 1;
    const int passes = (key_bits + 7) / 8;
    for (int c0 = 0; c0 < num_q; c0 += BW_QC) {
        const int nq = num_q - c0 < BW_QC ? num_q - c0 : BW_QC;
        const size_t qo = (size_t)c0 * heads * D;
        const int32_t* idx = indices + (size_t)c0 * row_width;
        mla_bwd_dq_kernel<D><<<nq, 64 * MLA_NW, 0, stream>>>(q + qo, kv, idx, o + qo, lse + (size_t)c0 * heads,
                                                             dout + qo, num_kv, heads, row_width, scale, scale_log2,
                                                             dq + qo, ws.coef, ws.dcorr);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if (num_kv == 0) continue;
        mla_bwd_dkv_part_kernel<D><<<nq, 64 * MLA_NW, 0, stream>>>(q + qo, dout + qo, idx, ws.coef, ws.dcorr, num_kv,
                                                                    heads, row_width, scale, ws.part);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        const int E = nq * row_width;
        const int nx = (E + RX_TILE - 1) / RX_TILE;
        for (int p = 0; p < passes; ++p) {
            const int shift = 8 * p;
            const uint32_t *kin = ws.key[(p + 1) & 1], *vin = ws.val[(p + 1) & 1];
            uint32_t *kout = ws.key[p & 1], *vout = ws.val[p & 1];
            if (p == 0)
                bwd_rx_hist_kernel<true><<<nx, RX_NT, 0, stream>>>(idx, nullptr, E, num_kv, shift, ws.hist, nx);
            else
                bwd_rx_hist_kernel<false><<<nx, RX_NT, 0, stream>>>(nullptr, kin, E, num_kv, shift, ws.hist, nx);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            bwd_rx_scan_kernel<<<RX_BINS, RX_NT, 0, stream>>>(ws.hist, nx, ws.totals);
            if ((e = hipGetLastError()) != hipSuccess) return e;
            if (p == 0)
                bwd_rx_scatter_kernel<true><<<nx, RX_NT, 0, stream>>>(idx, nullptr, nullptr, E, num_kv, shift, ws.hist,
                                                                      ws.totals, nx, kout, vout);
            else
                bwd_rx_scatter_kernel<false><<<nx, RX_NT, 0, stream>>>(nullptr, kin, vin, E, num_kv, shift, ws.hist,
                                                                       ws.totals, nx, kout, vout);
            if ((e = hipGetLastError()) != hipSuccess) return e;
        }
        const uint32_t *ks = ws.key[(passes - 1) & 1], *vs = ws.val[(passes - 1) & 1];
        const int nr = (E + RED_TILE - 1) / RED_TILE;
        bwd_dkv_reduce_kernel<D><<<(nr + 3) / 4, 256, 0, stream>>>(ks, vs, E, num_kv, ws.part, dkv, ws.carry,
                                                                   ws.cflag, ws.ckey);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        bwd_dkv_fixup_kernel<D><<<(nr + 3) / 4, 256, 0, stream>>>(nr, ws.cflag, ws.ckey, ws.carry, dkv);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    return hipSuccess;
}

size_t sparse_mla_bwd_ws_bytes(int num_q, int d_latent, int row_width) {
    return bwd_ws_layout(num_q, d_latent, row_width, nullptr, nullptr);
}

hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* out,
                                 const float* lse, const uint16_t* d_out, int num_q, int num_kv, int heads,
                                 int d_latent, int row_width, float scale, uint16_t* d_q, float* d_kv,
                                 void* workspace, hipStream_t stream) {
    if (num_q == 0) return launch_fill_f32(d_kv, (size_t)num_kv * d_latent, 0.0f, stream);
    if (d_latent == 512)
        return launch_bwd_t<512>(q, kv, indices, out, lse, d_out, num_q, num_kv, heads, row_width, scale, d_q, d_kv,
                                 workspace, stream);
    return launch_bwd_t<64>(q, kv, indices, out, lse, d_out, num_q, num_kv, heads, row_width, scale, d_q, d_kv,
                            workspace, stream);
}

}  // namespace kp
