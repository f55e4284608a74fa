// Absorbed, NoPE sparse latent attention (MLA) forward on gfx950.
//
// NeMo AutoModel PR "add GLM-5.3-Flash training support", Changelog: the K
// projection is absorbed into the query, which attends over a shared
// 512-wide latent K/V; prime-rl PR "GLM-5.3-Flash text model", Summary, second
// bullet: the latent serves as both key and value, no RoPE part. Each query
// attends to the rows its index row names (up to 2051 of them, "cuDNN sparse
// MLA parity and performance").
//
// One workgroup of 4 waves (one per SIMD, so each wave has the whole 512-entry
// register file) per query token (64 heads). The index row is compacted in LDS
// (masked entries dropped, order kept); its latent rows are gathered 64 at a
// time into a 2-tile LDS ring with the direct-to-LDS loads of gfx950 (each
// wave brings 16 whole rows per tile, issued one tile ahead). Wave w owns the
// row half rh = w/2 of every tile and the head half hh = w%2, and runs the
// whole attention of its (rows, heads) block with no exchange between waves:
//   QK: S^T = K[rows] . Q[heads]^T over all 512 columns (bf16 MFMA 16x16x32;
//       Q of its 32 heads stays in registers; every K fragment feeds two MFMAs);
//   SM: online softmax of each head over its 32 rows, in registers: the MFMA
//       row order is permuted so that each lane's eight S values are exactly the
//       eight P values it feeds to PV as the B operand;
//   PV: O^T[cols, heads] += V^T[cols, rows] . P^T[rows, heads] for all 512
//       columns (V read with the transposing ds_read_b64_tr_b16; one V fragment
//       feeds two MFMAs); O stays in the accumulation registers.
// The two row halves of a head keep separate softmax states and partial O and
// are merged once at the end through LDS. The LDS traffic per 32 gathered rows
// is the 32 KB gather plus 128 KB of K and V reads (each row is read by the
// two head halves), with one barrier per 64 rows.
// A head's softmax reference is fixed for a pass, so O is never rescaled: it
// is the max of the head's first tile, lifted by MLA_REF_LIFT, and later
// weights may exceed 1 up to 2^MLA_HEADROOM; a weight beyond that makes the
// workgroup drop the pass, sweep QK for the exact max of every head, and run
// the attention again. O is normalised by the sum of the weights as rounded to
// bf16 (the values the PV product used). LDS rows use a padded pitch (see
// row_base) so the row-wise K reads and the column-wise V reads are both free
// of bank conflicts. A latent narrower than 128 is zero-padded to 128 in LDS.
#include "kp_device.h"
#include "kp_launch.h"
#include "kp_mla_common.h"

namespace kp {

// A pass with a first-tile reference sets the reference MLA_REF_LIFT above the
// max of the head's first tile with a valid row and accepts later tiles up to
// MLA_HEADROOM above the reference: weights stay below 2^64, so the fp32 sums
// (and O, for latent values up to 2^50) are far from overflow, and those of the
// first tile are at least 2^-32, far from underflow.
#define MLA_REF_LIFT 32.0f
#define MLA_HEADROOM 64.0f
#define MLA_WEIGHT_MAX 0x1p64f   // 2^MLA_HEADROOM

// max / sum over the four lanes n, n+16, n+32, n+48 (v_permlane32_swap and
// v_permlane16_swap with both operands the value: the pair holds the value of
// the lane and of its partner 32, then 16, lanes away)
__device__ __forceinline__ float max_over_groups(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_groups(float v) {
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// O^T accumulation of PV, kept in the accumulation registers: c += a . b with
// the accumulator pinned to AGPRs (the whole 256-entry AGPR file holds a
// wave's O). Every accumulator takes one such MFMA per tile, and its readers
// (the rare rescale and the final merge) come a full tile later. The compiler
// does not see an MFMA inside the assembly, so it inserts no wait states before
// it: its A operands come straight from LDS reads, and its B operands (the
// weights) pass through kp_pin_weights, which ends VALU writes to them with
// the wait states an MFMA read needs.
__device__ __forceinline__ void mfma_acc(f32x4& c, bf16x8 a, bf16x8 b) {
    __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
// The same with a zero accumulator (the first tile of a pass): c = a . b, so O
// needs no zeroing and is not live before the pass.
__device__ __forceinline__ void mfma_set(f32x4& c, bf16x8 a, bf16x8 b) {
    __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=a"(c) : "v"(a), "v"(b));
}

// The weights, computed by VALU code, become the B operands of the PV MFMAs:
// the empty-bodied assembly makes them opaque from here on (the compiler can
// neither recompute nor rewrite them later, right before an MFMA) and its
// s_nop 2 gives the 3 wait states between their last VALU write and an MFMA
// read of them (gfx950 asks for 2).
__device__ __forceinline__ void kp_pin_weights(bf16x8& a, bf16x8& b) {
    __asm__ __volatile__("s_nop 2" : "+v"(a), "+v"(b));
}

// Empty-bodied assembly that takes a value as an operand: the instructions that
// compute it stay where they are written (the compiler would otherwise sink them
// to their first use, past the matrix-core work they are meant to overlap).
__device__ __forceinline__ void kp_keep(float& x) { __asm__ __volatile__("" : "+v"(x)); }
__device__ __forceinline__ void kp_keep_lo(bf16x8& x) {
    // the four weights of sub-tile 0 (the low half of the B operand)
    auto u = __builtin_bit_cast(u32x4, x);
    __asm__ __volatile__("" : "+v"(u[0]), "+v"(u[1]));
    x = __builtin_bit_cast(bf16x8, u);
}

// The 64-column RoPE tail of a latent row (keys 576 wide, the GLM-5.2
// contract) sits in its own LDS tile: row r at r*128 bytes, its 16-byte chunk c
// at position c ^ rope_swz(r). Under gfx950's 16-byte read passes (see
// row_base) the K reads of a pass (16 rows, two chunk columns) then hit 16
// distinct bank groups.
__device__ __forceinline__ constexpr int rope_swz(int r) { return ((r >> 1) & 7) ^ (2 * ((r >> 4) & 1)); }

// Direct-to-LDS copy with a per-lane memory offset: lane l copies the 16 bytes
// at rsrc base + voff to LDS byte M0 + 16*l (the RoPE tails of 8 rows, 128
// bytes each, per instruction).
__device__ __forceinline__ void lds_dma16_lane(u32x4 rsrc, uint32_t voff, uint32_t m0) {
    __asm__ __volatile__("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                         :: "v"(voff), "s"(rsrc), "{m0}"(m0) : "memory");
}

// D: width of the values and of the keys' NoPE part; DR: width of the keys'
// RoPE tail (0, or 64 for the 576-wide keys of the GLM-5.2 contract, whose
// values are the first 512 columns). SPLIT: the rows are split over nsplit
// workgroups per query, which write fp32 partials (with SPLIT false, nsplit is 1;
// the two epilogues are separate kernels so that neither takes registers from
// the other).
template <int D, int DR, bool SPLIT, bool W2>
__global__ __launch_bounds__(W2 ? 128 : 64 * MLA_NW, 1) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ indices,
    int num_kv, int heads, int row_width, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse, int nsplit, float* __restrict__ o_part, float* __restrict__ lse_part) {
    constexpr int NW = W2 ? 2 : MLA_NW;     // waves
    constexpr int TK = W2 ? 32 : MLA_TK;    // latent rows per tile
    constexpr int NT = 64 * NW;             // threads
    constexpr int DP = D < 128 ? 128 : D;   // latent width in LDS (zero-padded)
    constexpr int RB = DP * 2;              // LDS bytes per latent row
    constexpr int CH = D / 8;               // 16-byte chunks a gathered row brings
    constexpr int KS = DP / 32;             // QK k-steps (32 columns each)
    constexpr int CT = DP / 16;             // 16-wide O column tiles
    constexpr int TILE_B = TK * (RB + 48);  // bytes per LDS tile (row_base of row TK)
    constexpr int RPW = TK / NW;            // rows each wave gathers per tile
    constexpr int XB = (CT / 2) * 2 * 64 * 16;  // bytes of O one wave hands to its partner
    constexpr int DQK = D + DR;             // key (and q) width in memory
    constexpr int RK = DR / 32;             // QK k-steps over the RoPE tail
    constexpr int ROPE_RB = DR * 2;         // LDS bytes per RoPE tail row
    constexpr int ROPE_TB = TK * ROPE_RB;
    // the index list: 4096 entries, or 2048 with a RoPE tail (its top-k is at most
    // 2048 tokens) so that the tail's LDS tiles fit, or MLA_W2_MAX_ROW for the
    // two-wave form (two of its workgroups share a compute unit's LDS)
    constexpr int MAXR = W2 ? MLA_W2_MAX_ROW : DR > 0 ? 2048 : MLA_MAX_ROW;
    static_assert(RPW == 16 && CH >= 8 && CH <= 64, "tile split");
    static_assert(W2 ? (NW == 2 && TK == 32) : (NW == 4 && TK == 64), "wave and tile shape");
    static_assert(!W2 || (D == 512 && DR == 0 && !SPLIT), "two-wave form: 512-wide latent, whole rows");
    static_assert(W2 || 4 * XB <= MLA_NBUF * TILE_B, "row-half merge fits the ring");
    static_assert(DR == 0 || (D == 512 && DR == 64), "RoPE tail: 512 + 64 only");
    // the interleaved step (sub-tile 0's weights under sub-tile 1's k-steps) needs
    // ten k-steps of room and no RoPE k-steps
    constexpr bool IL = DR == 0 && KS >= 12;
    // Q of the 512-wide latent comes in through LDS (ring tile 1, free until the
    // first step gathers into it): one 1 KB head row per direct-to-LDS load, rows
    // QP bytes apart, a pitch at which the operand reads of 16 heads x one chunk
    // column hit distinct banks in every read pass
    constexpr bool QDMA = IL && D == 512;
    constexpr int QP = 2 * D + 32;
    static_assert(!QDMA || 64 * QP <= (W2 ? 2 : 1) * TILE_B, "Q fits its LDS region");

    __shared__ __align__(16) uint8_t ring[MLA_NBUF * TILE_B];
    __shared__ __align__(16) int32_t list[MAXR];   // byte offsets of the listed latent rows
    __shared__ float mls[W2 ? 1 : 2][64][3];   // per row half and head: reference max, sums
    __shared__ int wsum[NW];          // valid entries per wave of the compaction
    __shared__ int rflag[2];          // a wave saw a score too far above its reference, by step parity
    __shared__ __align__(16) uint8_t rope[DR > 0 ? MLA_NBUF * ROPE_TB : 16];   // RoPE tail tiles

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int rh = W2 ? 0 : wave >> 1;   // row half of every tile (the two-wave form: all rows)
    const int hh = W2 ? wave : wave & 1; // head half
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // the wave index, in a scalar register
    // one workgroup per query, or (nsplit > 1, few queries) per query and split:
    // split sp takes the tiles [ntiles*sp/nsplit, ntiles*(sp+1)/nsplit) of the
    // compacted row and leaves a normalised partial O and its lse for the combine
    const int ns = SPLIT ? nsplit : 1;
    const int i = SPLIT ? (int)(blockIdx.x / ns) : xcd_query<W2 ? MLA_XCD_RUN_W2 : MLA_XCD_RUN>(blockIdx.x, gridDim.x);
    const int sp = SPLIT ? (int)(blockIdx.x % ns) : 0;

    // ---- compact the index row (valid entries, original order) ----------------
    // Thread t owns the NE consecutive entries from NE*t on: it counts its valid
    // ones, one scan over the workgroup's counts gives its first position, and it
    // writes its valid entries from there. Every entry is read before the scan's
    // barrier and positions only move down, so the list is rewritten in place.
    constexpr int NE = MAXR / NT;
    static_assert(NE % 4 == 0, "whole 16-byte groups per thread");
    const int32_t* irow = indices + (size_t)i * row_width;
    int ent[NE];
    if (QDMA) {
        // The index row comes in through LDS (the list array, which the compaction
        // then rewrites): direct-to-LDS loads of 1 KB, chunk c by wave c % NW. Q's
        // row loads follow (wave w brings head rows QR*w .. QR*w+QR-1 of the query
        // into ring tile 1, or into the whole ring in the two-wave form; rows past
        // `heads` lie outside the descriptor's range and land as zeros), and one wait
        // lets them stay in flight: a wave's loads complete in order, so at most QR
        // outstanding means its index chunks have landed.
        const uint64_t ia = reinterpret_cast<uint64_t>(irow);
        const u32x4 i_rsrc = u32x4{(uint32_t)ia, (uint32_t)(ia >> 32) & 0xFFFFu, (uint32_t)(row_width * 4),
                                   0x00020000u};
        const uint32_t list_lds = lds_addr(list);
        for (int c = wave_u; 256 * c < row_width; c += NW)
            lds_dma16_row_at<0>(i_rsrc, 16u * lane, (uint32_t)(1024 * c),
                                __builtin_amdgcn_readfirstlane(list_lds + (uint32_t)(1024 * c)));
        const uint64_t qa = reinterpret_cast<uint64_t>(q) + (uint64_t)i * (uint64_t)(heads * DQK * 2);
        const u32x4 q_rsrc = u32x4{(uint32_t)qa, (uint32_t)(qa >> 32) & 0xFFFFu, (uint32_t)(heads * DQK * 2),
                                   0x00020000u};
        const uint32_t q_lds = lds_addr(ring) + (uint32_t)(W2 ? 0 : TILE_B);
        constexpr int QR = 64 / NW;   // Q rows each wave brings
#pragma unroll
        for (int r = 0; r < QR; ++r) {
            const int head = QR * wave_u + r;
            lds_dma16_row_at<0>(q_rsrc, 16u * lane, (uint32_t)(head * DQK * 2),
                                __builtin_amdgcn_readfirstlane(q_lds + (uint32_t)(head * QP)));
        }
        wait_vm<QR>();
        lds_barrier();
        // (list entries at or past row_width hold zeros or stale values: the
        // validity test below drops them by position)
#pragma unroll
        for (int k = 0; k < NE / 4; ++k) {
            const int4 e4 = *reinterpret_cast<const int4*>(list + NE * tid + 4 * k);
            ent[4 * k] = e4.x;
            ent[4 * k + 1] = e4.y;
            ent[4 * k + 2] = e4.z;
            ent[4 * k + 3] = e4.w;
        }
    } else if ((reinterpret_cast<uintptr_t>(irow) & 15) == 0) {
        // (row_width is a multiple of 128: a group of four is wholly in the row or past it)
#pragma unroll
        for (int k = 0; k < NE / 4; ++k) {
            int4 e4 = make_int4(-1, -1, -1, -1);
            if (NE * tid + 4 * k < row_width) e4 = *reinterpret_cast<const int4*>(irow + NE * tid + 4 * k);
            ent[4 * k] = e4.x;
            ent[4 * k + 1] = e4.y;
            ent[4 * k + 2] = e4.z;
            ent[4 * k + 3] = e4.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const int j = NE * tid + k;
            ent[k] = j < row_width ? irow[j] : -1;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // ---- Q: B operand of S^T = K . Q^T for this wave's 32 heads (through LDS, above,
    // for the 512-wide latent). Otherwise its loads go straight to the registers,
    // issued after the index row's, so the compaction waits for the index row only
    // (the memory counter retires loads in order) and Q lands under the compaction
    // and the first tile's gather.
    // qf[ht][ks]: head 32*hh + 16*ht + n, columns 32*ks + 8*g .. +7
    // (every lane loads from a valid address; heads past `heads` and the columns
    // of a zero-padded narrow latent are zeroed once the loads have landed)
    bf16x8 qf[2][KS];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        if (QDMA) break;
        const int head = 32 * hh + 16 * ht + n;
        const uint16_t* qrow = q + ((size_t)i * heads + min(head, heads - 1)) * DQK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int col = 32 * ks + 8 * g;
            qf[ht][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(
                                                        qrow + (DP == D ? col : min(col, D - 8))));
        }
    }
    // the RoPE tail of Q: qr[ht][c] holds columns D + 32*c + 8*g .. +7
    bf16x8 qr[2][RK > 0 ? RK : 1];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const int head = 32 * hh + 16 * ht + n;
        const uint16_t* qrow = q + ((size_t)i * heads + min(head, heads - 1)) * DQK;
#pragma unroll
        for (int c = 0; c < RK; ++c)
            qr[ht][c] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qrow + D + 32 * c + 8 * g));
    }

    __builtin_amdgcn_sched_barrier(0);
    if (tid < 2) rflag[tid] = 0;
    if (DP != D) {   // zero the padding columns of the ring once; the gather never writes them
        for (int e = tid; e < MLA_NBUF * TILE_B / 16; e += NT)
            reinterpret_cast<uint4*>(ring)[e] = make_uint4(0u, 0u, 0u, 0u);
    }
    // bit k: entry NE*tid + k is a row of the latent
    uint32_t vmask = 0;
#pragma unroll
    for (int k = 0; k < NE; ++k)
        if ((uint32_t)ent[k] < (uint32_t)num_kv && NE * tid + k < row_width) vmask |= 1u << k;
    const int vcnt = __builtin_popcount(vmask);
    const int vscan = wave_incl_scan(vcnt);
    if (lane == 63) wsum[wave] = vscan;
    __syncthreads();
    // The list holds, for local position p, the byte offset of its latent row plus
    // 4096 - row_base(p % 4): entry p is loaded at immediate offset row_base(p % 4)
    // within its group of four rows, through a descriptor based 4 KB below the
    // latent (all offsets stay positive; the latent is below 4 GiB). It is padded to
    // whole tiles with latent row 0 (the scores of those rows are masked), so the
    // gather needs no bounds test.
    int n_valid;
    {
        int n_all = 0, base = vscan - vcnt;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const int c = wsum[w];
            n_all += c;
            if (w < wave_u) base += c;
        }
        // this workgroup's entries: [e0, e1) of the compacted row, stored from 0
        const int nt_all = (n_all + TK - 1) / TK;
        const int e0 = nt_all * sp / ns * TK;
        const int e1 = min(n_all, nt_all * (sp + 1) / ns * TK);
        n_valid = max(0, e1 - e0);
        const int n_pad = (n_valid + TK - 1) / TK * TK - n_valid;
        int p = base - e0;
#pragma unroll
        for (int k = 0; k < NE; ++k) {
            const bool v = (vmask >> k) & 1u;
            if (v && (uint32_t)p < (uint32_t)n_valid)
                list[p] = (int32_t)((uint32_t)ent[k] * (uint32_t)(DQK * 2) + 4096u - (uint32_t)row_base<RB>(p & 3));
            p += v ? 1 : 0;
        }
        if (tid < n_pad) list[n_valid + tid] = (int32_t)(4096u - (uint32_t)row_base<RB>((n_valid + tid) & 3));
    }
    __syncthreads();

    if (n_valid == 0) {
        if (QDMA) wait_vm0();   // (Q's row loads into LDS end before the workgroup does)
        if (!SPLIT) {
            uint16_t* orow = out + (size_t)i * heads * D;
            for (int e = tid; e < heads * D; e += NT) orow[e] = 0;
            if (lse && tid < heads) lse[(size_t)i * heads + tid] = -INFINITY;
        } else {
            float* prow = o_part + (size_t)blockIdx.x * heads * D;
            for (int e = tid; e < heads * D; e += NT) prow[e] = 0.0f;
            if (tid < heads) lse_part[(size_t)blockIdx.x * heads + tid] = -INFINITY;
        }
        return;
    }
    const int ntiles = (n_valid + TK - 1) / TK;

    // ---- gather: wave w brings tile rows 16w .. 16w+15 straight into the ring;
    // lane l copies the row's 16-byte chunk l to LDS chunk l of ring
    // row r (lanes whose chunk lies in the zero padding of a narrow latent idle)
    const uint32_t ring_lds = lds_addr(ring);
    const int wave_s = wave_u;
    const uint32_t wave_lds = ring_lds + (uint32_t)row_base<RB>(RPW * wave_s);   // LDS row 16w of buffer 0
    const uint32_t lane16 = 16u * lane;   // the lane's byte offset in a gathered row
    const uint32_t rope_lds = lds_addr(rope);
    // the latent as a raw buffer: base (48 bits) 4 KiB below the latent, so that the
    // adjusted scalar offsets of the list stay positive; stride 0; num_kv * D * 2
    // + 4 KiB bytes (at most 4 GiB); the default dword format of gfx9 descriptors
    const uint64_t kv_addr = reinterpret_cast<uint64_t>(kv);
    const uint64_t kv_base = kv_addr - 4096u;
    const u32x4 kv_rsrc = u32x4{(uint32_t)kv_base, (uint32_t)(kv_base >> 32) & 0xFFFFu,
                                (uint32_t)((uint64_t)num_kv * (DQK * 2) + 4096u), 0x00020000u};
    // KP_ROWS_OF reads the (adjusted) byte offsets of this wave's 16 rows of tile kt_
    // into rws_[16]; KP_ISSUE_ROW(j_) issues the gather of the wave's row j_ into
    // buffer buf_ (rows 4m .. 4m+3 share M0)
#define KP_ROWS_OF(kt_)                                                                        \
    int rws_[RPW];   /* wave-uniform: scalar registers */                                      \
    _Pragma("unroll") for (int c4_ = 0; c4_ < RPW / 4; ++c4_) {                                \
        const int4 rw_ = *reinterpret_cast<const int4*>(list + (kt_) * TK + RPW * wave_s + 4 * c4_); \
        rws_[4 * c4_] = __builtin_amdgcn_readfirstlane(rw_.x);                                 \
        rws_[4 * c4_ + 1] = __builtin_amdgcn_readfirstlane(rw_.y);                             \
        rws_[4 * c4_ + 2] = __builtin_amdgcn_readfirstlane(rw_.z);                             \
        rws_[4 * c4_ + 3] = __builtin_amdgcn_readfirstlane(rw_.w);                             \
    }                                                                                          \
    /* the row loads read these scalar registers, which v_readfirstlane (VALU) wrote: */      \
    /* five wait states here, and the values are opaque from here on, so no later */          \
    /* VALU write can land closer to a load */                                                 \
    kp_sgpr_settle(rws_);
#define KP_ISSUE_ROW(j_, buf_)                                                                \
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
// KP_ISSUE_ROPE(kt_, m_, buf_): the RoPE tails of the wave's rows 8m_ .. 8m_+7 of
// tile kt_ into RoPE tile buf_: lane l brings chunk position l % 8 of row
// 16w + 8m_ + l / 8 (source chunk (l % 8) ^ rope_swz(row)); its list entry gives
// the row's offset (the list's adjustment undone by row_base(row % 4))
#define KP_ISSUE_ROPE(kt_, m_, buf_)                                                           \
    if (DR > 0) {                                                                              \
        const int jr_ = RPW * wave + 8 * (m_) + (lane >> 3);                                   \
        const uint32_t voff_ = (uint32_t)list[(kt_) * TK + jr_] + (uint32_t)row_base<RB>(jr_ & 3) + \
                               (uint32_t)(2 * D) + 16u * (uint32_t)((lane & 7) ^ rope_swz(jr_)); \
        const uint32_t m0r_ = __builtin_amdgcn_readfirstlane(                                   \
            rope_lds + (uint32_t)((buf_) * ROPE_TB + (RPW * wave_s + 8 * (m_)) * ROPE_RB));     \
        lds_dma16_lane(kv_rsrc, voff_, m0r_);                                                  \
    }
#define KP_ISSUE_TILE(kt_, buf_)                                                               \
    {                                                                                          \
        KP_ROWS_OF(kt_)                                                                        \
        _Pragma("unroll") for (int j = 0; j < RPW; ++j) KP_ISSUE_ROW(j, buf_)                 \
        KP_ISSUE_ROPE(kt_, 0, buf_)                                                            \
        KP_ISSUE_ROPE(kt_, 1, buf_)                                                            \
    }

    // O^T accumulators: o[ct][ht] holds columns 16*ct + 4*g + e of head 32*hh + 16*ht + n
    f32x4 o[CT][2];
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
            if (!IL) o[ct][ht] = f32x4{0.f, 0.f, 0.f, 0.f};   // (with IL the first tile writes O)
    // softmax state of head 32*hh + 16*ht + n over this wave's rows (the four lanes
    // of a head hold the same reference max and their own partial sums). O is
    // never rescaled inside the loop (its accumulators live in AGPRs, and a
    // rescale there costs more registers than a wave has), so the reference is
    // fixed for a pass: it is set from the max of the head's first tile with a
    // valid row, and the weights of later tiles may exceed 1, up to
    // 2^MLA_HEADROOM. A tile
    // whose max goes beyond that flags the workgroup, which then drops the pass,
    // sweeps QK over all tiles for the exact max of every head, and runs the
    // attention again with that max as the reference. The unset reference is
    // finite and far below any score, so a row half with no valid row at all
    // keeps zero weights.
    float m_ref[2] = {-1e30f, -1e30f}, l_lse[2] = {0.f, 0.f};
    // the sum of the rounded (bf16) weights of head 32*hh + 16*ht + n over the
    // wave's rows, accumulated by an MFMA with an all-ones A operand (every entry
    // of lsum[ht] holds the full sum); l_lse keeps the lane's share of the sum of
    // the unrounded weights
    f32x4 lsum[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u});

    // K rows are fed to the MFMA in a permuted order: A row m of sub-tile s is
    // tile row 32*rh + 8*(m/4) + 4*s + m%4, so that S^T lane (g, n) ends up with
    // rows 32*rh + 8*g + 4*s + e (s = 0, 1; e = 0..3): the eight rows of its P^T
    // B operand for PV. K-step ks reads chunk 4*ks + g of that row: byte offset
    // kb[s] + 64*ks.
    int kb[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) kb[s] = row_base<RB>(32 * rh + 8 * (n >> 2) + 4 * s + (n & 3)) + 16 * g;
    // the same rows' RoPE tails, k-step c (columns D + 32*c + 8*g: chunk 4*c + g)
    int rkb[2][RK > 0 ? RK : 1];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < RK; ++c) {
            const int r = 32 * rh + 8 * (n >> 2) + 4 * s + (n & 3);
            rkb[s][c] = r * ROPE_RB + 16 * ((4 * c + g) ^ rope_swz(r));
        }
    // V^T A operand of column tile ct: lane (g, n) needs rows 32*rh + 8*g .. +7 of
    // column 16*ct + n; two transposing reads (b = 0, 1) of rows
    // 32*rh + 8*g + 4*b + e4, 8 bytes at column 16*ct + 8*(q4/2) + 4*(q4%2): byte
    // offset vb[b] + 32*ct.
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    int vb[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) vb[b] = row_base<RB>(32 * rh + 8 * g + 4 * b + e4) + 8 * q4;

    // K fragments of QK chunk c_ (k-step c_, sub-tiles 0, 1) and the V fragments
    // of PV chunk c_ (column tiles 2c_, 2c_+1); a K chunk is read KP_RING_K-1
    // chunks ahead of its MFMAs, a V chunk KP_RING_V-1
#define KP_RING_K 4
#define KP_RING_V 4
#define KP_RING_U 4   // the interleaved step's K fragments (one sub-tile each)
#define KP_K_FRAG(c_, s_)                                                                      \
    kf_[(c_) % KP_RING_K][s_] = *reinterpret_cast<const bf16x8*>(tbk_[s_] + 64 * (c_));
#define KP_K_CHUNK(c_) { KP_K_FRAG(c_, 0) KP_K_FRAG(c_, 1) }
#define KP_V_HALF(c_, u_, b_) lds_read_tr16(tbv_[b_] + 32 * (2 * (c_) + (u_)))
#define KP_V_CHUNK(c_)                                                                         \
    _Pragma("unroll") for (int u_ = 0; u_ < 2; ++u_) {                                         \
        const int ct_ = 2 * (c_) + u_;                                                         \
        const bf16x4 v0_ = lds_read_tr16(tbv_[0] + 32 * ct_);                                  \
        const bf16x4 v1_ = lds_read_tr16(tbv_[1] + 32 * ct_);                                  \
        vf_[(c_) % KP_RING_V][u_] = __builtin_shufflevector(v0_, v1_, 0, 1, 2, 3, 4, 5, 6, 7); \
    }

    // one tile: QK, softmax, PV; the next tile's gather is issued first (its
    // buffer held tile kt-1, which every wave finished before the last barrier)
// the start of a step: the gather of the next tile is issued (its buffer held
// tile kt-1, which every wave finished before the last barrier), then QK of
// tile kt (rows past the end of the list masked)
#define KP_QK()                                                                                \
        const int buf_ = kt & 1;                                                               \
        /* the gather of the next tile; the last tile gathers its own rows again into the */   \
        /* free buffer (no branch per row; those rows were just read, from the L2) */          \
        const int ktn_ = kt + 1 < ntiles ? kt + 1 : kt;                                        \
        KP_ROWS_OF(ktn_)                                                                       \
        const uint8_t* tb_ = ring + buf_ * TILE_B;                                             \
        /* per-lane bases of the K and V reads in this tile (each read adds a constant) */     \
        const uint8_t* tbk_[2] = {tb_ + kb[0], tb_ + kb[1]};                                   \
        const uint8_t* tbv_[2] = {tb_ + vb[0], tb_ + vb[1]};                                   \
        /* QK by k-steps; the K fragments of a step are read three steps ahead of its */       \
        /* MFMAs (scheduling barriers keep the reads from all being hoisted, which would */    \
        /* take more registers than a wave has left) */                                        \
        f32x4 sacc_[2][2];                                                                     \
        _Pragma("unroll") for (int s = 0; s < 2; ++s)                                          \
            _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) sacc_[s][ht] = f32x4{0.f, 0.f, 0.f, 0.f}; \
        bf16x8 kf_[KP_RING_K][2];                                                              \
        _Pragma("unroll") for (int c = 0; c < KP_RING_K - 1; ++c) KP_K_CHUNK(c)                \
        /* each k-step interleaves its four MFMAs with the reads of a later k-step and */      \
        /* the gather of one row of the next tile (spread over the k-steps so that the */      \
        /* address unit takes it in the background), so that those issue while the */         \
        /* matrix core works */                                                                \
        _Pragma("unroll") for (int c = 0; c < KS; ++c) {                                       \
            const bool ld_ = c + KP_RING_K - 1 < KS;                                           \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[0][0] = mfma_bf16_16x16x32(kf_[c % KP_RING_K][0], qf[0][c], sacc_[0][0]);    \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if (ld_) KP_K_FRAG(c + KP_RING_K - 1, 0)                                           \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[0][1] = mfma_bf16_16x16x32(kf_[c % KP_RING_K][0], qf[1][c], sacc_[0][1]);    \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if (ld_) KP_K_FRAG(c + KP_RING_K - 1, 1)                                           \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[1][0] = mfma_bf16_16x16x32(kf_[c % KP_RING_K][1], qf[0][c], sacc_[1][0]);    \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            _Pragma("unroll") for (int j = c * RPW / KS; j < (c + 1) * RPW / KS; ++j)          \
                KP_ISSUE_ROW(j, buf_ ^ 1)                                                     \
            if (c == 1) KP_ISSUE_ROPE(ktn_, 0, buf_ ^ 1)                                       \
            if (c == KS / 2 + 1) KP_ISSUE_ROPE(ktn_, 1, buf_ ^ 1)                              \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[1][1] = mfma_bf16_16x16x32(kf_[c % KP_RING_K][1], qf[1][c], sacc_[1][1]);    \
        }                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        /* the RoPE tail's k-steps: both sub-tiles' K fragments from the RoPE tile */          \
        _Pragma("unroll") for (int c = 0; c < RK; ++c) {                                       \
            const uint8_t* rt_ = rope + buf_ * ROPE_TB;                                        \
            const bf16x8 kr0_ = *reinterpret_cast<const bf16x8*>(rt_ + rkb[0][c]);             \
            const bf16x8 kr1_ = *reinterpret_cast<const bf16x8*>(rt_ + rkb[1][c]);             \
            sacc_[0][0] = mfma_bf16_16x16x32(kr0_, qr[0][c], sacc_[0][0]);                     \
            sacc_[0][1] = mfma_bf16_16x16x32(kr0_, qr[1][c], sacc_[0][1]);                     \
            sacc_[1][0] = mfma_bf16_16x16x32(kr1_, qr[0][c], sacc_[1][0]);                     \
            sacc_[1][1] = mfma_bf16_16x16x32(kr1_, qr[1][c], sacc_[1][1]);                     \
        }                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        if ((kt + 1) * TK > n_valid) {   /* ragged last tile: mask rows past the end */        \
            const int rb0_ = kt * TK + 32 * rh + 8 * g;                                        \
            _Pragma("unroll") for (int s = 0; s < 2; ++s)                                      \
                _Pragma("unroll") for (int e = 0; e < 4; ++e)                                  \
                    if (rb0_ + 4 * s + e >= n_valid) {                                         \
                        sacc_[s][0][e] = -INFINITY;                                            \
                        sacc_[s][1][e] = -INFINITY;                                            \
                    }                                                                          \
        }                                                                                      \

// the max of each head over this wave's rows of the tile, scaled (the scale is
// positive: the max of the raw scores, scaled, is the max of the scaled scores)
#define KP_TILE_MAX()                                                                          \
        float mt_[2];                                                                          \
        _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                     \
            const float mx_ = fmaxf(fmaxf(fmaxf(sacc_[0][ht][0], sacc_[0][ht][1]), fmaxf(sacc_[0][ht][2], sacc_[0][ht][3])), \
                                    fmaxf(fmaxf(sacc_[1][ht][0], sacc_[1][ht][1]), fmaxf(sacc_[1][ht][2], sacc_[1][ht][3]))); \
            mt_[ht] = max_over_groups(mx_) * scale_log2;                                       \
        }
// the end of a step: this wave's rows of tile kt+1 have landed, then the barrier
// that publishes them and frees the buffer of tile kt
#define KP_STEP_END()                                                                          \
        wait_vm0();                                                                            \
        lds_barrier();                                                                         \
        ++kt;

// PV by pairs of column tiles, V read three pairs ahead (each pair interleaves
// its four MFMAs with the four reads of a later pair); the first three pairs'
// V fragments are in vf_ already
#define KP_PV(FRESH)                                                                           \
        _Pragma("unroll") for (int c = 0; c < CT / 2; ++c) {                                   \
            const bool ld_ = c + KP_RING_V - 1 < CT / 2;                                       \
            bf16x4 vh_[2][2];                                                                  \
            _Pragma("unroll") for (int u = 0; u < 2; ++u) {                                    \
                __builtin_amdgcn_sched_barrier(0);                                             \
                if (FRESH) mfma_set(o[2 * c + u][0], vf_[c % KP_RING_V][u], pb_[0]);           \
                else mfma_acc(o[2 * c + u][0], vf_[c % KP_RING_V][u], pb_[0]);                 \
                __builtin_amdgcn_sched_barrier(0);                                             \
                if (ld_) vh_[u][0] = KP_V_HALF(c + KP_RING_V - 1, u, 0);                      \
                __builtin_amdgcn_sched_barrier(0);                                             \
                if (FRESH) mfma_set(o[2 * c + u][1], vf_[c % KP_RING_V][u], pb_[1]);           \
                else mfma_acc(o[2 * c + u][1], vf_[c % KP_RING_V][u], pb_[1]);                 \
                __builtin_amdgcn_sched_barrier(0);                                             \
                if (ld_) {                                                                     \
                    vh_[u][1] = KP_V_HALF(c + KP_RING_V - 1, u, 1);                            \
                    vf_[(c + KP_RING_V - 1) % KP_RING_V][u] =                                  \
                        __builtin_shufflevector(vh_[u][0], vh_[u][1], 0, 1, 2, 3, 4, 5, 6, 7);  \
                }                                                                              \
            }                                                                                  \
        }                                                                                      \

    // one attention step on tile kt; with FIRST, the reference of a head is set by
    // its first tile with a valid row and a weight above 2^MLA_HEADROOM raises the
    // flag. Once set, the reference does not depend on the tile, so the weights
    // are computed straight from the scores: no cross-lane max on the way to PV.
#define KP_STEP(FIRST, FRESH)                                                                  \
    {                                                                                          \
        KP_QK()                                                                                \
        /* the first V chunks do not depend on the softmax: their reads are issued now, */    \
        /* ahead of it (the scheduling barrier keeps the compiler from sinking them below */  \
        /* the exponentials, which would expose their latency at the first PV MFMA) */         \
        bf16x8 vf_[KP_RING_V][2];                                                              \
        _Pragma("unroll") for (int c = 0; c < KP_RING_V - 1; ++c) KP_V_CHUNK(c)                \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        if (FIRST) {                                                                           \
            /* a head without a reference takes it from this tile (its O is still zero) */     \
            if (__ballot(m_ref[0] < -1e29f || m_ref[1] < -1e29f)) {                            \
                KP_TILE_MAX()                                                                  \
                _Pragma("unroll") for (int ht = 0; ht < 2; ++ht)                               \
                    if (m_ref[ht] < -1e29f) m_ref[ht] = mt_[ht] > -1e29f ? mt_[ht] + MLA_REF_LIFT : -1e30f; \
            }                                                                                  \
        }                                                                                      \
        bf16x8 pb_[2];                                                                         \
        float wmax_ = 0.f;                                                                     \
        _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                     \
            float w_[8];                                                                       \
            _Pragma("unroll") for (int s = 0; s < 2; ++s)                                      \
                _Pragma("unroll") for (int e = 0; e < 4; ++e)                                  \
                    w_[4 * s + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc_[s][ht][e], scale_log2, -m_ref[ht])); \
            _Pragma("unroll") for (int e = 0; e < 8; ++e) pb_[ht][e] = (__bf16)w_[e];         \
            lsum[ht] = mfma_bf16_16x16x32(ones, pb_[ht], lsum[ht]);                            \
            const float ws_ = ((w_[0] + w_[1]) + (w_[2] + w_[3])) + ((w_[4] + w_[5]) + (w_[6] + w_[7])); \
            l_lse[ht] += ws_;                                                                  \
            wmax_ = fmaxf(wmax_, ws_);                                                         \
        }                                                                                      \
        /* a weight above 2^MLA_HEADROOM (or infinite) means a score too far above the */     \
        /* reference: flag the workgroup. The lane's sums bound its weights from above */      \
        /* (a sum over the bound with no single weight over it only costs an exact pass) */   \
        if (FIRST && __ballot(wmax_ > MLA_WEIGHT_MAX)) rflag[kt & 1] = 1;                      \
        kp_pin_weights(pb_[0], pb_[1]);                                                        \
        KP_PV(FRESH)                                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        KP_STEP_END()                                                                          \
    }
    // A step after the first tile of a pass: the reference of every head is set
    // (all 64 rows of the first tile are valid whenever a second tile exists), so
    // the weights of sub-tile 0 are computed while the matrix core runs the k-steps
    // of sub-tile 1, and the reads of the first V fragments fill the last k-steps.
    // In a ragged last tile the rows past the end are masked, sub-tile by sub-tile,
    // before their weights. The arithmetic is that of KP_STEP, in the same order:
    // the two give the same bits.
#define KP_MASK_SUB(s_)                                                                        \
    {                                                                                          \
        _Pragma("unroll") for (int e = 0; e < 4; ++e)                                          \
            if (4 * (s_) + e >= lim_) {                                                        \
                sacc_[s_][0][e] = -INFINITY;                                                   \
                sacc_[s_][1][e] = -INFINITY;                                                   \
            }                                                                                  \
    }
#define KP_KU(u_) ku_[(u_) % KP_RING_U] = *reinterpret_cast<const bf16x8*>(tbk_[(u_) / KS] + 64 * ((u_) % KS));
#define KP_STEP_IL(CHECK)                                                                      \
    {                                                                                          \
        const int buf_ = kt & 1;                                                               \
        /* (the last tile gathers its own rows again, as in KP_QK) */                          \
        const int ktn_ = kt + 1 < ntiles ? kt + 1 : kt;                                        \
        KP_ROWS_OF(ktn_)                                                                       \
        const uint8_t* tb_ = ring + buf_ * TILE_B;                                             \
        const uint8_t* tbk_[2] = {tb_ + kb[0], tb_ + kb[1]};                                   \
        const uint8_t* tbv_[2] = {tb_ + vb[0], tb_ + vb[1]};                                   \
        const bool ragged_ = (kt + 1) * TK > n_valid;                                          \
        const int lim_ = n_valid - (kt * TK + 32 * rh + 8 * g);   /* rows 4s+e < lim_ valid */  \
        f32x4 sacc_[2][2];                                                                     \
        _Pragma("unroll") for (int s = 0; s < 2; ++s)                                          \
            _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) sacc_[s][ht] = f32x4{0.f, 0.f, 0.f, 0.f}; \
        /* K fragment u: sub-tile u / KS, k-step u % KS, read KP_RING_U-1 ahead of its MFMAs */ \
        bf16x8 ku_[KP_RING_U];                                                                 \
        _Pragma("unroll") for (int u = 0; u < KP_RING_U - 1; ++u) KP_KU(u)                     \
        bf16x8 vf_[KP_RING_V][2];                                                              \
        float w_[2][8];                                                                        \
        float ws0_[2];                                                                         \
        bf16x8 pb_[2];                                                                         \
        _Pragma("unroll") for (int u = 0; u < 2 * KS; ++u) {                                   \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[u / KS][0] = mfma_bf16_16x16x32(ku_[u % KP_RING_U], qf[0][u % KS], sacc_[u / KS][0]); \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            if (u + KP_RING_U - 1 < 2 * KS) KP_KU(u + KP_RING_U - 1)                           \
            if (u >= 2 * KS - (KP_RING_V - 1)) KP_V_CHUNK(u - (2 * KS - (KP_RING_V - 1)))      \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            sacc_[u / KS][1] = mfma_bf16_16x16x32(ku_[u % KP_RING_U], qf[1][u % KS], sacc_[u / KS][1]); \
            __builtin_amdgcn_sched_barrier(0);                                                 \
            _Pragma("unroll") for (int j = u * RPW / (2 * KS); j < (u + 1) * RPW / (2 * KS); ++j) \
                KP_ISSUE_ROW(j, buf_ ^ 1)                                                      \
            if (u == KS && ragged_) KP_MASK_SUB(0)                                             \
            /* sub-tile 0: one weight per k-step of sub-tile 1, then its sums and bf16 */     \
            if (u >= KS + 1 && u < KS + 9) {                                                   \
                const int h_ = (u - KS - 1) / 4, e_ = (u - KS - 1) % 4;                        \
                w_[h_][e_] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc_[0][h_][e_], scale_log2, -m_ref[h_])); \
                kp_keep(w_[h_][e_]);                                                           \
            }                                                                                  \
            if (u == KS + 9 || u == KS + 10) {                                                 \
                const int h_ = u - KS - 9;                                                     \
                ws0_[h_] = (w_[h_][0] + w_[h_][1]) + (w_[h_][2] + w_[h_][3]);                  \
                kp_keep(ws0_[h_]);                                                             \
                _Pragma("unroll") for (int e = 0; e < 4; ++e) pb_[h_][e] = (__bf16)w_[h_][e];  \
                kp_keep_lo(pb_[h_]);                                                           \
            }                                                                                  \
        }                                                                                      \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        if (ragged_) KP_MASK_SUB(1)                                                            \
        float wmax_ = 0.f;                                                                     \
        _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                     \
            _Pragma("unroll") for (int e = 0; e < 4; ++e)                                      \
                w_[ht][4 + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc_[1][ht][e], scale_log2, -m_ref[ht])); \
            _Pragma("unroll") for (int e = 4; e < 8; ++e) pb_[ht][e] = (__bf16)w_[ht][e];      \
            lsum[ht] = mfma_bf16_16x16x32(ones, pb_[ht], lsum[ht]);                            \
            const float ws_ = ws0_[ht] + ((w_[ht][4] + w_[ht][5]) + (w_[ht][6] + w_[ht][7]));  \
            l_lse[ht] += ws_;                                                                  \
            wmax_ = fmaxf(wmax_, ws_);                                                         \
        }                                                                                      \
        if (CHECK && __ballot(wmax_ > MLA_WEIGHT_MAX)) rflag[kt & 1] = 1;                      \
        kp_pin_weights(pb_[0], pb_[1]);                                                        \
        KP_PV(false)                                                                           \
        __builtin_amdgcn_sched_barrier(0);                                                     \
        KP_STEP_END()                                                                          \
    }
    // one step of the exact-max sweep: QK only
#define KP_MAX_STEP()                                                                          \
    {                                                                                          \
        KP_QK()                                                                                \
        KP_TILE_MAX()                                                                          \
        _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) m_ref[ht] = fmaxf(m_ref[ht], mt_[ht]); \
        KP_STEP_END()                                                                          \
    }
#define KP_FIRST_TILE()                                                                        \
    KP_ISSUE_TILE(0, 0)                                                                        \
    wait_vm0();                                                                                \
    lds_barrier();

    // (the explicit wait after the first tile's gather also covers the Q loads, so
    // the compiler adds no wait of its own at Q's first use inside the loop, where
    // the gathers of later tiles are in flight)
    compiler_fence();
    if (W2) {
        // Q fills the ring: every wave's Q rows land, each wave reads its 32 heads
        // into the operand registers, and the ring is free for the first tile
        wait_vm0();
        lds_barrier();
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ht][ks] = *reinterpret_cast<const bf16x8*>(ring + (32 * hh + 16 * ht + n) * QP + 64 * ks + 16 * g);
        lds_barrier();
        KP_FIRST_TILE()
    } else if (QDMA) {
        // The first tile's rows are issued, then Q moves from LDS into the operand
        // registers while they are in flight: the wave's Q row loads, issued before
        // the row gathers, have landed once at most RPW loads are outstanding (a
        // wave's loads complete in order), and a barrier makes every wave's rows
        // visible. The second barrier publishes the first tile and frees ring tile
        // 1 (every wave has read its Q) for the first step's gathers.
        KP_ISSUE_TILE(0, 0)
        wait_vm<RPW>();
        lds_barrier();
        const uint8_t* qb = ring + TILE_B;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qf[ht][ks] = *reinterpret_cast<const bf16x8*>(qb + (32 * hh + 16 * ht + n) * QP + 64 * ks + 16 * g);
        wait_vm0();
        lds_barrier();
    } else {
        KP_FIRST_TILE()
    }
    __builtin_amdgcn_sched_barrier(0);
    // heads past `heads` and the columns of a zero-padded narrow latent take zero
    // queries (a full 64-head, full-width launch has neither)
    if (DP != D || heads < 64) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int head = 32 * hh + 16 * ht + n;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                if (!(head < heads && (DP == D || 32 * ks + 8 * g < D))) qf[ht][ks] = bf16x8{};
#pragma unroll
            for (int c = 0; c < RK; ++c)
                if (!(head < heads)) qr[ht][c] = bf16x8{};
        }
    }
    // a score rose too far above its first-tile reference: the pass is dropped,
    // a sweep finds the exact max of every head, and the attention runs again with it
#define KP_RESET_PASS()                                                                        \
    _Pragma("unroll") for (int ct = 0; ct < CT; ++ct)                                          \
        _Pragma("unroll") for (int ht = 0; ht < 2; ++ht)                                       \
            if (!IL) o[ct][ht] = f32x4{0.f, 0.f, 0.f, 0.f};                                    \
    _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                         \
        m_ref[ht] = -1e30f;                                                                    \
        lsum[ht] = f32x4{0.f, 0.f, 0.f, 0.f};                                                  \
        l_lse[ht] = 0.f;                                                                       \
    }
    if (IL) {
        // The first tile sets the references, the later ones run the interleaved
        // step. A flag raised by a step is final after that step's barrier and is not
        // written again before the next one: every wave reads the same value and
        // leaves at the same step. The second pass (after the exact-max sweep) runs
        // the same steps: its weights are at most 1, so it raises no flag, and O stays
        // in the same accumulators through both passes.
        for (int pass = 0;; ++pass) {
            int kt = 0;
            KP_STEP(true, true)
            while (kt < ntiles) {
                const int over_prev = __builtin_amdgcn_readfirstlane(rflag[(kt & 1) ^ 1]);
                KP_STEP_IL(true)
                if (over_prev) break;
            }
            // read after the last barrier of the pass: the same value in every wave
            if (pass == 1 || !__builtin_amdgcn_readfirstlane(rflag[0] | rflag[1])) break;
            KP_RESET_PASS()
            KP_FIRST_TILE()
            if (tid < 2) rflag[tid] = 0;   // every wave read the flags before that barrier
            for (kt = 0; kt < ntiles;) KP_MAX_STEP()
            KP_FIRST_TILE()
        }
    } else {
        for (int kt = 0;;) {
            const int over_prev = __builtin_amdgcn_readfirstlane(rflag[(kt & 1) ^ 1]);
            KP_STEP(true, false)
            if (over_prev || kt >= ntiles) break;
        }
        // read after the last barrier of the pass: the same value in every wave
        if (__builtin_amdgcn_readfirstlane(rflag[0] | rflag[1])) {
            KP_RESET_PASS()
            KP_FIRST_TILE()
            for (int kt = 0; kt < ntiles;) KP_MAX_STEP()
            KP_FIRST_TILE()
            for (int kt = 0; kt < ntiles;) KP_STEP(false, false)
        }
    }
#undef KP_RESET_PASS
#undef KP_STEP
#undef KP_STEP_IL
#undef KP_KU
#undef KP_MASK_SUB
#undef KP_PV
#undef KP_MAX_STEP
#undef KP_QK
#undef KP_TILE_MAX
#undef KP_STEP_END
#undef KP_FIRST_TILE
#undef KP_K_CHUNK
#undef KP_K_FRAG
#undef KP_V_HALF
#undef KP_V_CHUNK
#undef KP_RING_K
#undef KP_RING_V
#undef KP_RING_U
#undef KP_ISSUE_TILE
#undef KP_ISSUE_ROPE
#undef KP_ISSUE_ROW
#undef KP_ROWS_OF

    // ---- the two-wave form: each wave finished every row of its 32 heads --------
    // Its O is divided by the head's normaliser, rounded to bf16 and staged in the
    // ring (free after the last step's barrier) at a pitch of SPW bytes, at which
    // the 8-byte writes of a pass of 16 lanes (16 heads) fall in distinct banks;
    // the wave then stores its 32 head rows of the contiguous output, one 1 KB row
    // per instruction. No other wave reads its staged rows, so no barrier.
    // (lane indices derived again, as below, to keep them out of the main loop)
    if constexpr (W2) {
        int lane_x = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
        __asm__ __volatile__("" : "+v"(lane_x));
        const int n = lane_x & 15, g = lane_x >> 4;
        float inv[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            const int head = 32 * wave_s + 16 * ht + n;
            const float le = sum_over_groups(l_lse[ht]);
            if (lse && g == 0 && head < heads)
                lse[(size_t)i * heads + head] = (m_ref[ht] + log2f(le)) * 0.69314718055994530942f;
            inv[ht] = 1.0f / lsum[ht][0];
        }
        int i_late = i;
        __asm__ __volatile__("" : "+s"(i_late));
        constexpr int SPW = 2 * D + 16;
        static_assert(64 * SPW <= MLA_NBUF * TILE_B, "output staging fits the ring");
        uint8_t* const sb = ring + (size_t)wave_s * 32 * SPW;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
                bf16x4 r_;
#pragma unroll
                for (int e = 0; e < 4; ++e) r_[e] = (__bf16)(o[ct][ht][e] * inv[ht]);
                *reinterpret_cast<bf16x4*>(sb + (16 * ht + n) * SPW + 2 * (16 * ct + 4 * g)) = r_;
            }
        uint8_t* const dst = reinterpret_cast<uint8_t*>(out + ((size_t)i_late * heads + 32 * wave_s) * D) + 16 * lane_x;
#pragma unroll
        for (int r = 0; r < 32; ++r)
            if (32 * wave_s + r < heads)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(sb + r * SPW + 16 * lane_x),
                                            reinterpret_cast<u32x4*>(dst + r * (2 * D)));
        return;
    }

    // ---- merge the two row halves and write ---------------------------------------
    // (the lane and wave indices are derived again from the lane count and the
    // scalar wave index: the values the prologue derived from the thread index would
    // otherwise stay live across the main loop, which leaves them no registers)
    if constexpr (!W2) {
    int lane_x = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    __asm__ __volatile__("" : "+v"(lane_x));
    const int lane = lane_x, n = lane_x & 15, g = lane_x >> 4;
    const int wave = wave_s, rh = wave_s >> 1, hh = wave_s & 1;
    // wave (rh, hh) finishes the column half rh of its heads: it hands its O of
    // the other column half, and its softmax state, to the partner (1-rh, hh)
    float lr[2], le[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        lr[ht] = lsum[ht][0];
        le[ht] = sum_over_groups(l_lse[ht]);
    }
    // (the accumulator array is only ever indexed with compile-time constants, so
    // the two row halves take separate code paths)
#define KP_HAND_OVER(RH)                                                                       \
    {                                                                                          \
        uint8_t* xo_ = ring + (2 * hh + (1 - (RH))) * XB;                                      \
        _Pragma("unroll") for (int j = 0; j < CT / 2; ++j)                                     \
            _Pragma("unroll") for (int ht = 0; ht < 2; ++ht)                                   \
                *reinterpret_cast<f32x4*>(xo_ + ((ht * (CT / 2) + j) * 64 + lane) * 16) = o[(CT / 2) * (1 - (RH)) + j][ht]; \
    }
    if (rh == 0) KP_HAND_OVER(0) else KP_HAND_OVER(1)
#undef KP_HAND_OVER
    if (g == 0) {
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            float* m_ = mls[rh][32 * hh + 16 * ht + n];
            m_[0] = m_ref[ht];
            m_[1] = lr[ht];
            m_[2] = le[ht];
        }
    }
    __syncthreads();
    const uint8_t* xi = ring + (2 * hh + rh) * XB;
    float fa[2], fb[2];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        const int head = 32 * hh + 16 * ht + n;
        const float* mp = mls[1 - rh][head];
        const float M = fmaxf(m_ref[ht], mp[0]);
        fa[ht] = __builtin_amdgcn_exp2f(m_ref[ht] - M);
        fb[ht] = __builtin_amdgcn_exp2f(mp[0] - M);
        const float lse_h = (M + log2f(le[ht] * fa[ht] + mp[2] * fb[ht])) * 0.69314718055994530942f;
        if (rh == 0 && g == 0 && head < heads) {
            if (SPLIT) lse_part[(size_t)blockIdx.x * heads + head] = lse_h;
            else if (lse) lse[(size_t)i * heads + head] = lse_h;
        }
        const float inv = 1.0f / (lr[ht] * fa[ht] + mp[1] * fb[ht]);
        fa[ht] *= inv;   // the merge weights with the normaliser folded in
        fb[ht] *= inv;
    }
    // (the output row address is formed here from the scalar query index, so no
    // 64-bit address stays live, or spilled, across the main loop: a reload of a
    // spill would wait for every output store issued before it)
    int i_late = i;
    __asm__ __volatile__("" : "+s"(i_late));
#define KP_FINISH(RH)                                                                          \
    _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                         \
        const int head_ = 32 * hh + 16 * ht + n;                                               \
        uint16_t* dst_ = out + ((size_t)i_late * heads + head_) * D;                           \
        f32x4 op_[CT / 2];                                                                     \
        _Pragma("unroll") for (int j = 0; j < CT / 2; ++j)                                     \
            op_[j] = *reinterpret_cast<const f32x4*>(xi + ((ht * (CT / 2) + j) * 64 + lane) * 16);    \
        if (head_ < heads) {                                                                   \
            _Pragma("unroll") for (int j = 0; j < CT / 2; ++j) {                               \
                const int ct_ = (CT / 2) * (RH) + j;                                           \
                const int col_ = 16 * ct_ + 4 * g;                                             \
                if (DP == D || col_ < D) {                                                     \
                    bf16x4 r_;                                                                 \
                    _Pragma("unroll") for (int e = 0; e < 4; ++e)                              \
                        r_[e] = (__bf16)(__builtin_fmaf(o[ct_][ht][e], fa[ht], op_[j][e] * fb[ht])); \
                    *reinterpret_cast<bf16x4*>(dst_ + col_) = r_;                              \
                }                                                                              \
            }                                                                                  \
        }                                                                                      \
    }
    // (a split's partial O in fp32: the combine rounds once, at the end)
#define KP_FINISH_PART(RH)                                                                     \
    _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                         \
        const int head_ = 32 * hh + 16 * ht + n;                                               \
        float* dst_ = o_part + ((size_t)blockIdx.x * heads + head_) * D;                       \
        f32x4 op_[CT / 2];                                                                     \
        _Pragma("unroll") for (int j = 0; j < CT / 2; ++j)                                     \
            op_[j] = *reinterpret_cast<const f32x4*>(xi + ((ht * (CT / 2) + j) * 64 + lane) * 16);    \
        if (head_ < heads) {                                                                   \
            _Pragma("unroll") for (int j = 0; j < CT / 2; ++j) {                               \
                const int ct_ = (CT / 2) * (RH) + j;                                           \
                const int col_ = 16 * ct_ + 4 * g;                                             \
                if (DP == D || col_ < D) {                                                     \
                    f32x4 r_;                                                                  \
                    _Pragma("unroll") for (int e = 0; e < 4; ++e)                              \
                        r_[e] = __builtin_fmaf(o[ct_][ht][e], fa[ht], op_[j][e] * fb[ht]);     \
                    *reinterpret_cast<f32x4*>(dst_ + col_) = r_;                               \
                }                                                                              \
            }                                                                                  \
        }                                                                                      \
    }
    // (full-width latent: each wave stages its finished values as bf16 in the
    // hand-over region it has just read, 16 head rows of D/2 columns per head tile
    // at a pitch of SPH bytes, so that the 8-byte writes of a pass of 16 lanes (16 heads) fall in
    // distinct banks; after a barrier each wave stores 16 whole head rows of the
    // query's contiguous output, 16 bytes per lane, the two column halves of a row
    // coming from the regions of the two row-half waves: every store instruction
    // writes D*2 contiguous bytes)
    constexpr int SPH = D + 16;
    static_assert(DP != D || 16 * SPH <= XB / 2, "output staging fits a hand-over region");
#define KP_STAGE(RH)                                                                           \
    _Pragma("unroll") for (int ht = 0; ht < 2; ++ht) {                                         \
        /* head tile ht's hand-over sits in half ht of the region: it is read whole, */       \
        /* then overwritten by the staged rows */                                              \
        f32x4 op_[CT / 2];                                                                     \
        _Pragma("unroll") for (int j = 0; j < CT / 2; ++j)                                     \
            op_[j] = *reinterpret_cast<const f32x4*>(xi + ((ht * (CT / 2) + j) * 64 + lane) * 16); \
        uint8_t* srow_ = ring + (2 * hh + (RH)) * XB + ht * (XB / 2) + n * SPH;                \
        _Pragma("unroll") for (int j = 0; j < CT / 2; ++j) {                                   \
            bf16x4 r_;                                                                         \
            _Pragma("unroll") for (int e = 0; e < 4; ++e)                                      \
                r_[e] = (__bf16)(__builtin_fmaf(o[(CT / 2) * (RH) + j][ht][e], fa[ht], op_[j][e] * fb[ht])); \
            *reinterpret_cast<bf16x4*>(srow_ + 2 * (16 * j + 4 * g)) = r_;                     \
        }                                                                                      \
    }
    if (SPLIT) {
        if (rh == 0) {
            KP_FINISH_PART(0)
        } else {
            KP_FINISH_PART(1)
        }
    } else if (DP != D) {
        if (rh == 0) {
            KP_FINISH(0)
        } else {
            KP_FINISH(1)
        }
    } else {
        if (rh == 0) {
            KP_STAGE(0)
        } else {
            KP_STAGE(1)
        }
        __syncthreads();
        // wave w stores heads 16w .. 16w+15, one 1 KB row per instruction: lane l
        // brings 16 bytes of column half l / 32 from the staged rows of head tile
        // w % 2 in the regions of the waves (0, w / 2) and (1, w / 2)
        static_assert(DP != D || D == 512, "one row per store instruction");
        const uint8_t* const src =
            ring + (2 * (wave >> 1) + (lane >> 5)) * XB + (wave & 1) * (XB / 2) + 16 * (lane & 31);
        uint8_t* const dst = reinterpret_cast<uint8_t*>(out + ((size_t)i_late * heads + 16 * wave) * D) + 16 * lane;
#pragma unroll
        for (int r = 0; r < 16; ++r)
            if (16 * wave + r < heads)
                __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(src + r * SPH),
                                            reinterpret_cast<u32x4*>(dst + r * (2 * D)));
    }
    }
#undef KP_STAGE
#undef KP_FINISH
#undef KP_FINISH_PART
}

// Merge of the splits of each (query, head): lse = log sum_s exp(lse_s), and
// out = sum_s exp(lse_s - lse) O_s, rounded once to bf16. One wave per (query,
// head); lane l holds columns l*CPL .. +CPL-1.
template <int D>
__global__ __launch_bounds__(256) void mla_combine_kernel(const float* __restrict__ o_part,
                                                          const float* __restrict__ lse_part, int num_q, int heads,
                                                          int nsplit, uint16_t* __restrict__ out,
                                                          float* __restrict__ lse) {
    constexpr int CPL = D / 64;
    const int lane = threadIdx.x & 63;
    const long long wq = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (wq >= (long long)num_q * heads) return;
    const int i = (int)(wq / heads), h = (int)(wq % heads);
    // the split lse values, one per lane (nsplit <= 64), and their max
    const float myl = lane < nsplit ? lse_part[((size_t)i * nsplit + lane) * heads + h] : -INFINITY;
    float m = myl;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.0f;
    float L = -INFINITY;
    if (m != -INFINITY) {
        float e = lane < nsplit ? __expf(myl - m) : 0.0f;
        float sum = e;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
        L = m + __logf(sum);
        for (int s = 0; s < nsplit; ++s) {
            const float ls = __shfl(myl, s, 64);
            if (ls == -INFINITY) continue;
            const float wgt = __expf(ls - L);
            const float* src = o_part + (((size_t)i * nsplit + s) * heads + h) * D + lane * CPL;
            if constexpr (CPL % 4 == 0) {
#pragma unroll
                for (int c = 0; c < CPL; c += 4) {
                    const float4 v = *reinterpret_cast<const float4*>(src + c);
                    acc[c] = __builtin_fmaf(wgt, v.x, acc[c]);
                    acc[c + 1] = __builtin_fmaf(wgt, v.y, acc[c + 1]);
                    acc[c + 2] = __builtin_fmaf(wgt, v.z, acc[c + 2]);
                    acc[c + 3] = __builtin_fmaf(wgt, v.w, acc[c + 3]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(wgt, src[c], acc[c]);
            }
        }
    }
    uint16_t* dst = out + ((size_t)i * heads + h) * D + lane * CPL;
    if constexpr (CPL % 8 == 0) {
#pragma unroll
        for (int c = 0; c < CPL; c += 8) {
            uint4 pk;
            pk.x = f32_to_bf16_rne(acc[c]) | ((uint32_t)f32_to_bf16_rne(acc[c + 1]) << 16);
            pk.y = f32_to_bf16_rne(acc[c + 2]) | ((uint32_t)f32_to_bf16_rne(acc[c + 3]) << 16);
            pk.z = f32_to_bf16_rne(acc[c + 4]) | ((uint32_t)f32_to_bf16_rne(acc[c + 5]) << 16);
            pk.w = f32_to_bf16_rne(acc[c + 6]) | ((uint32_t)f32_to_bf16_rne(acc[c + 7]) << 16);
            *reinterpret_cast<uint4*>(dst + c) = pk;
        }
    } else {
#pragma unroll
        for (int c = 0; c < CPL; ++c) dst[c] = f32_to_bf16_rne(acc[c]);
    }
    if (lse && lane == 0) lse[(size_t)i * heads + h] = L;
}

// Splits per query row: few queries (decode) leave most compute units idle
// with one workgroup per query, so each row is cut into up to 16 tile ranges
// (at least two tiles each) when there are fewer than 128 queries.
int sparse_mla_splits(int num_q, int row_width) {
    if (num_q <= 0 || num_q >= 128) return 1;
    const int tiles = (row_width + MLA_TK - 1) / MLA_TK;
    int s = 256 / num_q;
    if (s > 16) s = 16;
    if (s > tiles / 2) s = tiles / 2;
    return s < 1 ? 1 : s;
}

size_t sparse_mla_part_bytes(int num_q, int heads, int d_latent, int row_width) {
    const int s = sparse_mla_splits(num_q, row_width);
    if (s == 1) return 0;
    const int dv = d_latent == 576 ? 512 : d_latent;
    const size_t o = (size_t)num_q * s * heads * dv * sizeof(float);
    return ((o + 255) & ~(size_t)255) + (size_t)num_q * s * heads * sizeof(float);
}

template <int D, int DR>
static hipError_t launch_mla_t(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int num_q,
                               int num_kv, int heads, int row_width, float scale_log2, uint16_t* out,
                               float* lse, void* part, hipStream_t stream) {
    const int ns = part ? sparse_mla_splits(num_q, row_width) : 1;
    float* o_part = static_cast<float*>(part);
    float* lse_part = nullptr;
    if (ns > 1) {
        const size_t o = (size_t)num_q * ns * heads * D * sizeof(float);
        lse_part = reinterpret_cast<float*>(static_cast<uint8_t*>(part) + ((o + 255) & ~(size_t)255));
    }
    if (ns > 1)
        sparse_mla_kernel<D, DR, true, false><<<num_q * ns, 64 * MLA_NW, 0, stream>>>(
            q, kv, indices, num_kv, heads, row_width, scale_log2, out, lse, ns, o_part, lse_part);
    else if (D == 512 && DR == 0 && row_width <= MLA_W2_MAX_ROW)
        // whole rows of the 512-wide latent: the two-wave form, two workgroups per CU
        sparse_mla_kernel<512, 0, false, true><<<num_q, 128, 0, stream>>>(
            q, kv, indices, num_kv, heads, row_width, scale_log2, out, lse, 1, nullptr, nullptr);
    else
        sparse_mla_kernel<D, DR, false, false><<<num_q, 64 * MLA_NW, 0, stream>>>(
            q, kv, indices, num_kv, heads, row_width, scale_log2, out, lse, 1, nullptr, nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || ns == 1) return e;
    const long long waves = (long long)num_q * heads;
    mla_combine_kernel<D><<<(unsigned)((waves + 3) / 4), 256, 0, stream>>>(o_part, lse_part, num_q, heads, ns, out,
                                                                             lse);
    return hipGetLastError();
}

int sparse_mla_max_row_width(int d_latent) { return d_latent == 576 ? 2048 : MLA_MAX_ROW; }

hipError_t launch_sparse_mla(const uint16_t* q, const uint16_t* kv, const int32_t* indices, int num_q,
                             int num_kv, int heads, int d_latent, int row_width, float scale_log2,
                             uint16_t* out, float* lse, void* part, hipStream_t stream) {
    if (num_q == 0) return hipSuccess;
    if (d_latent == 576)
        return launch_mla_t<512, 64>(q, kv, indices, num_q, num_kv, heads, row_width, scale_log2, out, lse, part,
                                     stream);
    if (d_latent == 512)
        return launch_mla_t<512, 0>(q, kv, indices, num_q, num_kv, heads, row_width, scale_log2, out, lse, part,
                                    stream);
    return launch_mla_t<64, 0>(q, kv, indices, num_q, num_kv, heads, row_width, scale_log2, out, lse, part, stream);
}

}  // namespace kp
