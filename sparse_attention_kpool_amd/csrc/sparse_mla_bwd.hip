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
// p is recomputed from the forward's lse; delta from the forward's output.
//
// Two kernels, one workgroup (4 waves, one per SIMD) per query each:
//  * mla_bwd_dq_kernel: wave w owns heads 16w .. 16w+15 and every row of a
//    64-row tile. The rows are gathered into LDS exactly as in the forward. Per
//    tile: S^T = K . Q^T and dP^T = K . dO^T (each K fragment feeds both MFMAs),
//    then p and scale*ds in registers, then dQ^T += K^T . (scale ds)^T over all
//    columns (K^T read with the transposing LDS read). The K rows enter the QK
//    MFMAs in a permuted order so that each lane's S values are the ones it
//    feeds to the dQ MFMA. dQ stays in registers for the whole row (no merge:
//    a wave owns its heads). scale*ds and p of every valid slot are written to
//    the workspace, head-major: coef[query][h][slot] (h < 64: scale*ds,
//    64 + h: p), bf16.
//  * mla_bwd_dkv_kernel: dKV rows of the query's slots = coef^T . [Q; dO], a
//    product over the 128 coefficients: wave w owns a quarter of the columns.
//    Its [Q; dO] operands (128 coefficients x its columns) are read once per
//    query through LDS into registers; the coefficient tiles stream through an
//    LDS double buffer. Each 16 x 16 result tile is added to dKV with fp32
//    atomics, one per element and slot: dKV is exact to fp32 rounding but its
//    last bits depend on the order in which queries' additions land.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_mla_common.h"

namespace kp {

constexpr int BW_COEF = 128;   // coefficients per slot: scale*ds and p of 64 heads

// Slot stride of the coefficient workspace rows: the index row width rounded
// up to whole 64-slot tiles.
__host__ __device__ __forceinline__ int bwd_coef_stride(int row_width) { return (row_width + 63) / 64 * 64; }

// Compacts the valid entries of an index row (0 <= e < num_kv, original order)
// into list[]: the entries themselves. Every thread of the 256-thread
// workgroup calls it; returns the count. Ends with the list visible to all.
__device__ __forceinline__ int bwd_compact(const int32_t* __restrict__ irow, int row_width, int num_kv,
                                           int32_t* list, int* rcnt) {
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
        if (ent[k] >= 0 && ent[k] < num_kv) list[base + below] = ent[k];
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
    uint16_t* __restrict__ coef) {
    constexpr int NT = 64 * MLA_NW;
    constexpr int DP = D < 128 ? 128 : D;   // latent width in LDS (zero-padded)
    constexpr int RB = DP * 2;
    constexpr int CH = D / 8;               // 16-byte chunks a gathered row brings
    constexpr int KS = DP / 32;             // QK k-steps
    constexpr int CT = DP / 16;             // dQ column tiles
    constexpr int TILE_B = MLA_TK * (RB + 48);
    constexpr int RPW = MLA_TK / MLA_NW;

    __shared__ __align__(16) uint8_t ring[MLA_NBUF * TILE_B];
    __shared__ __align__(16) int32_t list[MLA_MAX_ROW];
    __shared__ int rcnt[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int head = 16 * wave + n;        // this lane's head
    const bool head_ok = head < heads;
    const int i = xcd_query(blockIdx.x, gridDim.x);
    const int wc = bwd_coef_stride(row_width);

    const int n_valid = bwd_compact(indices + (size_t)i * row_width, row_width, num_kv, list, rcnt);
    uint16_t* dq_row = dq + ((size_t)i * heads + (head_ok ? head : 0)) * D;
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

    // Q and dO of this lane's head as the B operands of S^T = K . Q^T and
    // dP^T = K . dO^T (k-step ks: columns 32*ks + 8*g .. +7); delta = <dO, O>
    bf16x8 qf[KS], gf[KS];
    float delta = 0.f, lse2 = 0.f;
    {
        const size_t rowoff = ((size_t)i * heads + (head_ok ? head : 0)) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = 32 * ks + 8 * g;
            const bool in = head_ok && (DP == D || col < D);
            const int c = DP == D ? col : min(col, D - 8);
            qf[ks] = in ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(q + rowoff + c)) : bf16x8{};
            gf[ks] = in ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(dout + rowoff + c)) : bf16x8{};
            const bf16x8 of = in ? __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(o + rowoff + c))
                                 : bf16x8{};
#pragma unroll
            for (int e = 0; e < 8; ++e) delta += (float)gf[ks][e] * (float)of[e];
        }
        // the four lanes of a head (g = 0..3) hold a quarter of the columns each
        delta += shfl_xor(delta, 16);
        delta += shfl_xor(delta, 32);
        lse2 = head_ok ? lse[(size_t)i * heads + head] * 1.4426950408889634f : 0.f;
    }

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
    // K^T A operand of dQ column tile ct, k-step kk: two transposing reads of rows
    // 32*kk + 8*g + 4*b + e4, columns 16*ct + 4*q4 .. +3: byte offset vb[kk][b] + 32*ct
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    int vb[2][2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int b = 0; b < 2; ++b) vb[kk][b] = row_base<RB>(32 * kk + 8 * g + 4 * b + e4) + 8 * q4;

    f32x4 acc[CT];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
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
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8*>(tb + kb[s] + 64 * ks);
                sacc[s] = mfma_bf16_16x16x32(kf, qf[ks], sacc[s]);
                pacc[s] = mfma_bf16_16x16x32(kf, gf[ks], pacc[s]);
            }
        }
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
        // dQ^T[cols, heads] += K^T[cols, rows] . (scale ds)^T[rows, heads]
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                const bf16x4 v0 = lds_read_tr16(tb + vb[kk][0] + 32 * ct);
                const bf16x4 v1 = lds_read_tr16(tb + vb[kk][1] + 32 * ct);
                acc[ct] = mfma_bf16_16x16x32(__builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7), dsb[kk],
                                             acc[ct]);
            }
        // the next tile's rows have landed: every vector-memory operation but the
        // four coefficient stores issued after them is done (s_waitcnt vmcnt(4); the
        // counter retires in issue order): the stores may stay in flight across
        // the barrier
        __builtin_amdgcn_s_waitcnt(0x0F74);
        lds_barrier();
    }
#undef BW_ROWS_OF
#undef BW_ISSUE_ROW
    // dQ: lane (g, n) holds columns 16*ct + 4*g .. +3 of its head
    if (head_ok) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
            const int col = 16 * ct + 4 * g;
            if (DP == D || col < D) {
                bf16x4 r;
#pragma unroll
                for (int e = 0; e < 4; ++e) r[e] = (__bf16)acc[ct][e];
                *reinterpret_cast<bf16x4*>(dq_row + col) = r;
            }
        }
    }
}

// ----------------------------------------------------------------- dKV ------
// LDS layout of a coefficient tile (128 rows of 64 slots, 128 bytes each): row
// r at byte r*176 + 16*(r & 1); the transposing reads of the A operand (two
// groups of 16 lanes per pass, 4 rows x 32 bytes each) then hit distinct banks.
__device__ __forceinline__ constexpr int coef_row(int r) { return r * 176 + 16 * (r & 1); }
constexpr int BW_CTILE_B = 128 * 176;   // bytes per coefficient tile

template <int D>
__global__ __launch_bounds__(64 * MLA_NW, 1) void mla_bwd_dkv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ dout, const int32_t* __restrict__ indices,
    const uint16_t* __restrict__ coef, int num_kv, int heads, int row_width, float* __restrict__ dkv) {
    constexpr int NT = 64 * MLA_NW;
    constexpr int DP = D < 128 ? 128 : D;
    constexpr int RB = DP * 2;
    constexpr int CW = DP / 4;              // columns per wave
    constexpr int CTW = CW / 16;            // 16-wide column tiles per wave
    constexpr int XB = 64 * (RB + 48);      // bytes of one staged operand (64 heads)
    static_assert(XB >= MLA_NBUF * BW_CTILE_B || true, "");

    __shared__ __align__(16) uint8_t xs[XB > MLA_NBUF * BW_CTILE_B ? XB : MLA_NBUF * BW_CTILE_B];
    __shared__ __align__(16) int32_t list[MLA_MAX_ROW];
    __shared__ int rcnt[64];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int i = xcd_query(blockIdx.x, gridDim.x);
    const int wc = bwd_coef_stride(row_width);

    const int n_valid = bwd_compact(indices + (size_t)i * row_width, row_width, num_kv, list, rcnt);
    if (n_valid == 0) return;
    const int ntiles = (n_valid + MLA_TK - 1) / MLA_TK;

    // B operands of dKV[slots, cols] = coef^T[slots, coefs] . X[coefs, cols] with X =
    // [Q; dO] (coefficients 0..63: Q of head c, 64..127: dO of head c - 64): lane (g, n)
    // of k-step kk holds coefficients 32*kk + 8*g .. +7 of column 16*ct + n of the
    // wave's columns. Q, then dO, is staged in LDS (head h at row_base(h)) and read
    // with the transposing read.
    bf16x8 xf[4][CTW];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        const uint16_t* src = (half == 0 ? q : dout) + (size_t)i * heads * D;
        // 64 rows (heads) x DP columns; heads past `heads` and padded columns are zero
        for (int c = tid; c < 64 * (DP / 8); c += NT) {
            const int h = c / (DP / 8), col = 8 * (c % (DP / 8));
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (h < heads && col < D) v = *reinterpret_cast<const uint4*>(src + (size_t)h * D + col);
            *reinterpret_cast<uint4*>(xs + row_base<RB>(h) + 2 * col) = v;
        }
        __syncthreads();
#pragma unroll
        for (int kq = 0; kq < 2; ++kq)
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                const int colb = 2 * (CW * wave + 16 * ct) + 8 * q4;
                const bf16x4 v0 = lds_read_tr16(xs + row_base<RB>(32 * kq + 8 * g + e4) + colb);
                const bf16x4 v1 = lds_read_tr16(xs + row_base<RB>(32 * kq + 8 * g + 4 + e4) + colb);
                xf[2 * half + kq][ct] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
        __syncthreads();
    }

    // coefficient tiles (128 rows x 64 slots of bf16) through an LDS double buffer:
    // thread t copies 64 bytes of row t/2; the next tile's loads are issued before
    // the current tile's MFMAs
    const uint16_t* crow = coef + (size_t)i * BW_COEF * wc;
    const int cr = tid >> 1, chalf = tid & 1;
    uint4 cpre[4];
    auto load_tile = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            cpre[u] = *reinterpret_cast<const uint4*>(crow + (size_t)cr * wc + kt * MLA_TK + 32 * chalf + 8 * u);
    };
    auto store_tile = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
            *reinterpret_cast<uint4*>(xs + buf * BW_CTILE_B + coef_row(cr) + 64 * chalf + 16 * u) = cpre[u];
    };
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < ntiles) load_tile(kt + 1);
        const uint8_t* tb = xs + buf * BW_CTILE_B;
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
            // A operand: lane (g, n) holds coefficients 32*kk + 8*g .. +7 of slot 16*rt + n
            bf16x8 af[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const bf16x4 v0 = lds_read_tr16(tb + coef_row(32 * kk + 8 * g + e4) + 32 * rt + 8 * q4);
                const bf16x4 v1 = lds_read_tr16(tb + coef_row(32 * kk + 8 * g + 4 + e4) + 32 * rt + 8 * q4);
                af[kk] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            }
            f32x4 r[CTW];
#pragma unroll
            for (int ct = 0; ct < CTW; ++ct) {
                r[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) r[ct] = mfma_bf16_16x16x32(af[kk], xf[kk][ct], r[ct]);
            }
            // lane (g, n) holds slots 16*rt + 4*g + e, column CW*wave + 16*ct + n
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int slot = kt * MLA_TK + 16 * rt + 4 * g + e;
                if (slot < n_valid) {
                    float* drow = dkv + (size_t)list[slot] * D;
#pragma unroll
                    for (int ct = 0; ct < CTW; ++ct) {
                        const int col = CW * wave + 16 * ct + n;
                        if (DP == D || col < D) atomicAdd(drow + col, r[ct][e]);
                    }
                }
            }
        }
        __syncthreads();
        if (kt + 1 < ntiles) {
            store_tile(buf ^ 1);
            __syncthreads();
        }
    }
}

template <int D>
static hipError_t launch_bwd_t(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* o,
                               const float* lse, const uint16_t* dout, int num_q, int num_kv, int heads,
                               int row_width, float scale, uint16_t* dq, float* dkv, uint16_t* coef,
                               hipStream_t stream) {
    hipError_t e = launch_fill_f32(dkv, (size_t)num_kv * D, 0.0f, stream);
    if (e != hipSuccess) return e;
    const float scale_log2 = (float)((double)scale * 1.4426950408889634074);
    mla_bwd_dq_kernel<D><<<num_q, 64 * MLA_NW, 0, stream>>>(q, kv, indices, o, lse, dout, num_kv, heads, row_width,
                                                             scale, scale_log2, dq, coef);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    mla_bwd_dkv_kernel<D><<<num_q, 64 * MLA_NW, 0, stream>>>(q, dout, indices, coef, num_kv, heads, row_width,
                                                              dkv);
    return hipGetLastError();
}

size_t sparse_mla_bwd_coef_bytes(int num_q, int row_width) {
    return (size_t)num_q * BW_COEF * (size_t)bwd_coef_stride(row_width) * 2;
}

hipError_t launch_sparse_mla_bwd(const uint16_t* q, const uint16_t* kv, const int32_t* indices, const uint16_t* out,
                                 const float* lse, const uint16_t* d_out, int num_q, int num_kv, int heads,
                                 int d_latent, int row_width, float scale, uint16_t* d_q, float* d_kv,
                                 void* workspace, hipStream_t stream) {
    uint16_t* coef = static_cast<uint16_t*>(workspace);
    if (num_q == 0) return launch_fill_f32(d_kv, (size_t)num_kv * d_latent, 0.0f, stream);
    if (d_latent == 512)
        return launch_bwd_t<512>(q, kv, indices, out, lse, d_out, num_q, num_kv, heads, row_width, scale, d_q, d_kv,
                                 coef, stream);
    return launch_bwd_t<64>(q, kv, indices, out, lse, d_out, num_q, num_kv, heads, row_width, scale, d_q, d_kv, coef,
                            stream);
}

}  // namespace kp
