// Absorbed, NoPE sparse latent attention (MLA) forward on gfx950.
//
// NeMo AutoModel PR "add GLM-5.3-Flash training support", Changelog: the K
// projection is absorbed into the query, which attends over a shared
// 512-wide latent K/V; prime-rl PR "GLM-5.3-Flash text model", Summary, second
// bullet: the latent serves as both key and value, no RoPE part. Each query
// attends to the rows its index row names (up to 2051 of them, "cuDNN sparse
// MLA parity and performance").
//
// One workgroup of 4 waves per query token (64 heads). The index row is
// compacted in LDS (masked entries dropped, order kept); its latent rows are
// gathered 32 at a time into a ring of 3 LDS tiles with the gfx950
// direct-to-LDS load (global_load_lds_dwordx4), two tiles ahead of the one
// being consumed. Per tile, wave w owns latent columns [w*D/4, (w+1)*D/4):
//   1. partial S^T = K[:, cols_w] . Q[:, cols_w]^T for all 32 rows and all 64
//      heads (bf16 MFMA 16x16x32; Q's columns stay in registers; every K
//      fragment read from LDS feeds four MFMAs, and K is read once per CU);
//   2. the four partial sums meet in LDS; wave w adds them for the 16 heads
//      16w.. and runs their online softmax, writing P (bf16) to LDS;
//   3. O[:, cols_w] += P . V[:, cols_w] for all 64 heads: one V fragment, read
//      with the transposing ds_read_b64_tr_b16 (the slow LDS read, so V is
//      read exactly once per CU), feeds four MFMAs.
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
constexpr int MLA_NW = 4;     // waves per workgroup
constexpr int MLA_NBUF = 3;   // LDS tiles in the gather ring
constexpr int MLA_AHEAD = MLA_NBUF - 1;
constexpr int MLA_MAX_ROW = 4096;  // index-row entries the LDS list holds

// chunk permutation of LDS row r (16-byte chunks, within aligned groups of 8)
__device__ __forceinline__ int row_swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((KP_LDS bf16x4*)(p));
}

// Wait until at most n vector-memory operations of this wave are outstanding
// (loads retire in order, so the oldest tiles are complete).
__device__ __forceinline__ void wait_vm(int n) {
    // s_waitcnt immediate: vmcnt in bits [3:0] and [15:14]; expcnt 7 and
    // lgkmcnt 15 mean "do not wait" on those counters
    switch (n) {
        case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
        case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
        case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
        case 8: __builtin_amdgcn_s_waitcnt(0x0F78); break;
        case 16: __builtin_amdgcn_s_waitcnt(0x4F70); break;
        default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
}

// compiler-only barrier: keeps LDS accesses on their side of the explicit waits
__device__ __forceinline__ void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

// Direct-to-LDS load (gfx950 global_load_lds_dwordx4): lane l copies the 16
// bytes at its own global address `src` to LDS byte address lds_base + 16*l;
// lds_base is wave-uniform and travels in M0. Issued as inline assembly so the
// compiler does not treat later LDS reads of other ring tiles as dependent on
// it (it would wait for every outstanding gather); completion is tracked by
// the explicit vmcnt waits of the ring. M0 is not otherwise used by these
// kernels (gfx9 LDS instructions do not read it).
__device__ __forceinline__ void lds_dma16(const void* src, uint32_t lds_base) {
    __asm__ __volatile__("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                         :: "s"(lds_base), "v"(src) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((KP_LDS const uint8_t*)p);
}

constexpr int P_STRIDE = 80;   // bytes per head row of the P tile (32 bf16 + 16 pad: conflict-free reads)
constexpr int SP_STRIDE = 36;  // floats per head row of a partial-S block (32 + 4 pad)

__device__ __forceinline__ void wait_lgkm0() {
    // s_waitcnt lgkmcnt(0) only (vmcnt 63, expcnt 7: no wait)
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Barrier that orders LDS traffic between waves but leaves the gathers of the
// ring in flight (a __syncthreads would also wait for them).
__device__ __forceinline__ void lds_barrier() {
    compiler_fence();
    wait_lgkm0();
    __builtin_amdgcn_s_barrier();
    compiler_fence();
}

template <int D>
__global__ __launch_bounds__(64 * MLA_NW) void sparse_mla_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const int32_t* __restrict__ indices,
    int num_kv, int heads, int row_width, float scale_log2, uint16_t* __restrict__ out,
    float* __restrict__ lse) {
    constexpr int NW = MLA_NW;
    constexpr int NT = 64 * NW;             // threads
    constexpr int DP = D < 128 ? 128 : D;   // latent width in LDS (zero-padded)
    constexpr int RB = DP * 2;              // LDS bytes per latent row
    constexpr int CH = D / 8;               // 16-byte chunks a gathered row brings
    constexpr int KSW = DP / 128;           // QK k-steps (32 columns) per wave
    constexpr int DTW = DP / 64;            // 16-wide O column tiles per wave
    constexpr int TILE_B = MLA_TK * RB;     // bytes per LDS tile
    constexpr int IPW = MLA_TK / NW;        // gathered rows per wave per tile (one load each)
    static_assert(NW == 4 && CH >= 8 && CH <= 64 && IPW == 8, "tile staging split");
    static_assert(DP * 2 * 64 <= MLA_NBUF * TILE_B, "output staging fits the ring");

    __shared__ __align__(16) uint8_t ring[MLA_NBUF * TILE_B];
    __shared__ int32_t list[MLA_MAX_ROW];
    __shared__ __align__(16) float spart[NW * 64 * SP_STRIDE];  // partial S, [wave][head][row]
    __shared__ __align__(16) uint8_t ptile[64 * P_STRIDE];      // P, bf16 [head][row]
    __shared__ __align__(16) float alpha_s[64];                 // per-head rescale of this tile
    __shared__ float lsum[64 * 2];                              // per-head (rounded, exact) sums
    __shared__ float mref_s[64];                                // per-head final reference max
    __shared__ int wave_buf[NW];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int i = blockIdx.x;

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
    if (DP != D) {   // zero the padding columns of the ring once; the gathers never touch them
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

    uint16_t* orow = out + (size_t)i * heads * D;
    if (n_valid == 0) {
        for (int e = tid; e < heads * D; e += NT) orow[e] = 0;
        if (lse && tid < heads) lse[(size_t)i * heads + tid] = -INFINITY;
        return;
    }
    const int ntiles = (n_valid + MLA_TK - 1) / MLA_TK;

    // ---- gather ring: wave w moves tile rows 8w .. 8w+7, one load per row ------
    // Lane l (< CH) writes LDS chunk l of the row and reads the logical chunk
    // that the row's xor permutation places there.
    // Row numbers of a tile: lane c (< IPW) of wave w reads list entry
    // kt*32 + 8w + c; the loads then take them with readlane, so the IPW
    // gathers issue back to back.
    auto tile_rows = [&](int kt) {
        const int li = kt * MLA_TK + wave * IPW + (lane & (IPW - 1));
        return list[li < n_valid ? li : 0];
    };
    auto issue_rows = [&](int kt, int rows_v) {
        const uint32_t tb = lds_addr(ring) + (uint32_t)((kt % MLA_NBUF) * TILE_B);
#pragma unroll
        for (int c = 0; c < IPW; ++c) {
            const int r = wave * IPW + c;
            const int row = __builtin_amdgcn_readlane(rows_v, c);
            if (lane < CH) {
                const uint16_t* src = kv + (size_t)row * D + 8 * (lane ^ row_swz(r));
                lds_dma16(src, __builtin_amdgcn_readfirstlane(tb + (uint32_t)(r * RB)));
            }
        }
    };
    auto issue_tile = [&](int kt) { issue_rows(kt, tile_rows(kt)); };

    // ---- Q columns of this wave for all 64 heads, B-operand layout -------------
    bf16x8 qf[4][KSW];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht) {
        const int head = 16 * ht + n;
#pragma unroll
        for (int s = 0; s < KSW; ++s) {
            const int col = wave * (DP / 4) + 32 * s + 8 * g;
            uint4 v = make_uint4(0u, 0u, 0u, 0u);
            if (head < heads && col < D) v = *reinterpret_cast<const uint4*>(q + ((size_t)i * heads + head) * D + col);
            qf[ht][s] = __builtin_bit_cast(bf16x8, v);
        }
    }
    // Complete the Q loads now: the compiler cannot see the gathers (inline
    // assembly), and if Q were still pending on entry to the tile loop it
    // would wait for every outstanding gather before each tile's first MFMA.
    wait_vm(0);
    compiler_fence();
    for (int kt = 0; kt < MLA_AHEAD && kt < ntiles; ++kt) issue_tile(kt);

    // PV state: O for heads 16*ht + 4*g + e, columns 16*(wave*DTW + dtl) + n
    f32x4 o[4][DTW];
#pragma unroll
    for (int ht = 0; ht < 4; ++ht)
#pragma unroll
        for (int dtl = 0; dtl < DTW; ++dtl) o[ht][dtl] = f32x4{0.f, 0.f, 0.f, 0.f};
    // softmax state of the owned heads 16*wave + n (rows 8g .. 8g+7 of each tile)
    float m_ref = -INFINITY, l_run = 0.f, l_lse = 0.f;

    // fixed per-lane LDS offsets
    int kb[2][2];                                    // K rows 16*rt + n, chunk parity
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
        const int r = 16 * rt + n;
        const int base_c = wave * (DP / 4) / 8;      // first chunk of this wave's columns
        kb[rt][0] = r * RB + (((base_c + g) ^ row_swz(r)) << 4);
        kb[rt][1] = r * RB + (((base_c + 4 + g) ^ row_swz(r)) << 4);
    }
    const int e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int vr0 = 8 * g + e4, vr1 = 8 * g + 4 + e4;  // V rows of the two transposing reads
    int vb0[4], vb1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int c = 2 * j + (q4 >> 1);
        vb0[j] = vr0 * RB + ((c ^ row_swz(vr0)) << 4) + 8 * (q4 & 1);
        vb1[j] = vr1 * RB + ((c ^ row_swz(vr1)) << 4) + 8 * (q4 & 1);
    }
    float* my_sp = spart + wave * 64 * SP_STRIDE;

    for (int kt = 0; kt < ntiles; ++kt) {
        const int next_rows = tile_rows(kt + MLA_AHEAD);   // LDS read overlaps the waits below
        // tile kt complete for this wave, then for all waves
        const int newer = min(MLA_AHEAD - 1, ntiles - 1 - kt);   // tiles issued after kt
        compiler_fence();
        wait_vm(newer * IPW);
        wait_lgkm0();   // this wave's reads of tile kt-1 have landed
        __builtin_amdgcn_s_barrier();
        compiler_fence();
        // every wave is done with tile kt-1, so its buffer can take tile kt+2
        if (kt + MLA_AHEAD < ntiles) issue_rows(kt + MLA_AHEAD, next_rows);
        compiler_fence();
        const uint8_t* tb = ring + (kt % MLA_NBUF) * TILE_B;

        // ---- 1. partial S^T over this wave's columns: 2 row tiles x 4 head tiles ----
        f32x4 sp[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) sp[rt][ht] = f32x4{0.f, 0.f, 0.f, 0.f};
        uint4 ka[2][KSW];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int s = 0; s < KSW; ++s)
                ka[rt][s] = *reinterpret_cast<const uint4*>(tb + kb[rt][s & 1] + 128 * (s >> 1));
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int s = 0; s < KSW; ++s) {
                const bf16x8 af = __builtin_bit_cast(bf16x8, ka[rt][s]);
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) sp[rt][ht] = mfma_bf16_16x16x32(af, qf[ht][s], sp[rt][ht]);
            }
        // lane holds S^T[rows 16*rt + 4*g + e][head 16*ht + n]; store as [head][row]
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
                *reinterpret_cast<f32x4*>(my_sp + (16 * ht + n) * SP_STRIDE + 16 * rt + 4 * g) = sp[rt][ht];
        lds_barrier();

        // ---- 2. full S of the owned heads, rows 8g .. 8g+7; online softmax ----
        const int hown = 16 * wave + n;
        float sv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float* src = spart + (w * 64 + hown) * SP_STRIDE + 8 * g;
            const f32x4 lo = *reinterpret_cast<const f32x4*>(src);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) { sv[e] += lo[e]; sv[4 + e] += hi[e]; }
        }
        float mt = -INFINITY;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int li = kt * MLA_TK + 8 * g + e;
            sv[e] = li < n_valid ? sv[e] * scale_log2 : -INFINITY;
            mt = fmaxf(mt, sv[e]);
        }
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        float alpha = 1.0f;
        if (mt > m_ref + 8.0f) {
            alpha = __builtin_amdgcn_exp2f(m_ref - mt);
            m_ref = mt;
        }
        bf16x8 pw;
        float ps = 0.f, pe = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float w = __builtin_amdgcn_exp2f(sv[e] - m_ref);
            pw[e] = (__bf16)w;
            ps += (float)pw[e];
            pe += w;
        }
        l_run = l_run * alpha + ps;
        l_lse = l_lse * alpha + pe;
        *reinterpret_cast<bf16x8*>(ptile + hown * P_STRIDE + 16 * g) = pw;
        if (g == 0) alpha_s[hown] = alpha;
        lds_barrier();

        // ---- 3. O[:, cols_w] += P . V[:, cols_w] for all heads ----
        bf16x8 pa[4];
        f32x4 al[4];
        bool moved = false;
#pragma unroll
        for (int ht = 0; ht < 4; ++ht) {
            pa[ht] = *reinterpret_cast<const bf16x8*>(ptile + (16 * ht + n) * P_STRIDE + 16 * g);
            al[ht] = *reinterpret_cast<const f32x4*>(alpha_s + 16 * ht + 4 * g);
            moved |= (al[ht][0] != 1.0f) | (al[ht][1] != 1.0f) | (al[ht][2] != 1.0f) | (al[ht][3] != 1.0f);
        }
        if (__builtin_amdgcn_ballot_w64(moved) != 0) {
            // rare: keep it a real branch (not a multiply by 1 on every tile)
            __asm__ __volatile__("");
#pragma unroll
            for (int ht = 0; ht < 4; ++ht)
#pragma unroll
                for (int dtl = 0; dtl < DTW; ++dtl) o[ht][dtl] *= al[ht];
        }
        bf16x4 va[2][2];
        auto vread = [&](int dtl, bf16x4 (&dst)[2]) {
            const int dt = wave * DTW + dtl;
            const int off = 128 * (dt >> 2);
            dst[0] = lds_read_tr16(tb + vb0[dt & 3] + off);
            dst[1] = lds_read_tr16(tb + vb1[dt & 3] + off);
        };
        vread(0, va[0]);
        if (DTW > 1) vread(1, va[1]);
#pragma unroll
        for (int dtl = 0; dtl < DTW; ++dtl) {
            const bf16x8 vb = __builtin_shufflevector(va[dtl & 1][0], va[dtl & 1][1], 0, 1, 2, 3, 4, 5, 6, 7);
            if (dtl + 2 < DTW) vread(dtl + 2, va[dtl & 1]);
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) o[ht][dtl] = mfma_bf16_16x16x32(pa[ht], vb, o[ht][dtl]);
        }
    }

    // ---- normalise and write ----------------------------------------------------
    {
        float lr = l_run + shfl_xor(l_run, 16);
        lr += shfl_xor(lr, 32);
        float le = l_lse + shfl_xor(l_lse, 16);
        le += shfl_xor(le, 32);
        const int hown = 16 * wave + n;
        if (g == 0) {
            lsum[hown * 2] = lr;
            lsum[hown * 2 + 1] = le;
            mref_s[hown] = m_ref;
        }
    }
    compiler_fence();
    __syncthreads();   // all waves done with the ring; sums visible
    if (lse && tid < heads)
        lse[(size_t)i * heads + tid] = (mref_s[tid] + log2f(lsum[tid * 2 + 1])) * 0.69314718055994530942f;
    // stage O (bf16, [head][D]) in the ring, then copy the real heads out
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
                    stage[(16 * ht + 4 * g + e) * D + col] = f32_to_bf16_rne(o[ht][dtl][e] * inv[e]);
            }
        }
    }
    __syncthreads();
    const uint4* src = reinterpret_cast<const uint4*>(stage);
    uint4* dst = reinterpret_cast<uint4*>(orow);
    const int nvec = heads * D / 8;
    for (int e = tid; e < nvec; e += NT) dst[e] = src[e];
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
