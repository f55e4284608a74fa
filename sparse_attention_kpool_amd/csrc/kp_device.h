// Device helpers shared by the gfx950 kernels of libkpool: vector types, MFMA
// wrappers, the FP8 convert, wave shuffles, and the per-query document lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kp {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define KP_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------- MFMA ------
// D(16x16, fp32) += A(16x32, bf16) * B(32x16, bf16).
// Lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16] and
// D[4*(l/16) + i][l%16] for i = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D(16x16, fp32) += A(16x128, e4m3) * B(128x16, e4m3), unit block scales.
// Lane l holds 32 A bytes of row l%16 and 32 B bytes of column l%16 (the same
// k positions for A and B), and D[4*(l/16) + i][l%16].
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
    // operand formats 0/0 = FP8 E4M3; E8M0 scale 127 = 2^0 for both operands
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// max(x, 0) on the bit pattern: a set sign bit reads as a negative integer
// (-0 included), so one integer max clears every negative value; positive
// values pass unchanged. One instruction, and no quieting of the MFMA result.
__device__ __forceinline__ float relu_f32(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ----------------------------------------------------------------- FP8 ------
// Four fp32 values to four OCP E4M3FN codes (round to nearest even), packed
// little-endian: byte 0 holds x0.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float x0, float x1, float x2, float x3) {
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x2, x3, v, true);
    return (uint32_t)v;
}

// --------------------------------------------------------------- bf16 -------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// ------------------------------------------------------------- shuffles -----
__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ float shfl_idx(float v, int src) { return __shfl(v, src, 64); }

// Data-parallel moves inside a row of 16 lanes (no LDS traffic). CTRL is the
// DPP control: 0xB1 = quad_perm(1,0,3,2) (lane ^ 1), 0x4E = quad_perm(2,3,0,1)
// (lane ^ 2), 0x141 = row_half_mirror (lane i of each 8 reads lane 7 - i).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    // every source lane exists for these controls, so bound_ctrl (zero for a
    // missing source) never applies; setting it lets the move fold into the ALU op
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// max / sum over each aligned group of 8 lanes, result in all 8
__device__ __forceinline__ float max_in_8(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    return fmaxf(v, dpp_mov<0x141>(v));
}
__device__ __forceinline__ float sum_in_8(float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    return v + dpp_mov<0x141>(v);
}

// max(a, b, c, d) over each aligned group of 8 lanes, result in all 8. The
// inputs are finite or -inf. Written out so the three cross-lane steps are
// single v_max_f32 DPP instructions (the compiler's IEEE-mode max would quiet
// each DPP result first). A VALU write followed by a DPP read of the same VGPR
// needs two wait states, hence the s_nop 1 before each DPP step.
__device__ __forceinline__ float max4_in_8(float a, float b, float c, float d) {
    float r;
    __asm__("v_max3_f32 %0, %1, %2, %3\n\t"
            "v_max_f32 %0, %0, %4\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
            "s_nop 1\n\t"
            "v_max_f32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf bound_ctrl:1"
            : "=&v"(r)
            : "v"(a), "v"(b), "v"(c), "v"(d));
    return r;
}

// v from lane (lane ^ M). Distances below 16 stay inside a 16-lane DPP row and
// are made of row moves that run on the vector ALU: quad_perm swaps for 1 and 2
// (and 3); the half-row mirror reads lane ^ 7 and the row mirror lane ^ 15, so
// 4 = 3 then 7 and 8 = 7 then 15. Distances 16 and 32 use gfx950's lane swaps:
// v_permlane16_swap with both operands v leaves the odd 16-lane rows' values in
// the first result's odd rows and the even rows' in the second result's even
// rows, so lane l takes its partner l ^ 16 from the first result when l is in an
// odd row and from the second otherwise; v_permlane32_swap does the same for the
// two halves of the wave. The source lane must be active (callers keep whole
// lane groups together).
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    int i = __float_as_int(v);
    if constexpr (M == 32) {
        const auto p = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
        i = (int)((threadIdx.x & 32) ? p[0] : p[1]);
    } else if constexpr (M == 16) {
        const auto p = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
        i = (int)((threadIdx.x & 16) ? p[0] : p[1]);
    } else if constexpr (M == 1) {
        i = __builtin_amdgcn_mov_dpp(i, 0xB1, 0xF, 0xF, false);           // quad_perm [1,0,3,2]
    } else if constexpr (M == 2) {
        i = __builtin_amdgcn_mov_dpp(i, 0x4E, 0xF, 0xF, false);           // quad_perm [2,3,0,1]
    } else if constexpr (M == 4) {
        i = __builtin_amdgcn_mov_dpp(i, 0x1B, 0xF, 0xF, false);           // quad_perm [3,2,1,0]
        i = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, false);          // row_half_mirror
    } else {
        static_assert(M == 8, "lane_xor: power-of-two distance up to 32");
        i = __builtin_amdgcn_mov_dpp(i, 0x141, 0xF, 0xF, false);          // row_half_mirror
        i = __builtin_amdgcn_mov_dpp(i, 0x140, 0xF, 0xF, false);          // row_mirror
    }
    return __int_as_float(i);
}

template <int W, int M = 1>
__device__ __forceinline__ float group_max(float v) {
    if constexpr (M < W) {
        v = fmaxf(v, lane_xor<M>(v));
        return group_max<W, 2 * M>(v);
    } else {
        return v;
    }
}

// --------------------------------------------------------- doc lookup -------
// Document d holding token t: the d with cu[d] <= t < cu[d+1] (empty
// documents are skipped because cu[d] == cu[d+1]).
__device__ __forceinline__ int find_doc(const int32_t* __restrict__ cu, int num_docs, int t) {
    int lo = 0, hi = num_docs + 1;  // first index with cu[i] > t lies in [lo, hi)
    while (lo < hi) {
        int mid = (lo + hi) >> 1;
        if (cu[mid] > t) hi = mid; else lo = mid + 1;
    }
    return lo - 1;
}

struct QueryPools {
    int doc;        // document of the query
    int pool_lo;    // global number of the document's first pool
    int n_vis;      // complete pools of the document ending at or before t
    int tail_start; // first token of the query's incomplete pool
};

__device__ __forceinline__ QueryPools query_pools(const int32_t* __restrict__ cu, int num_docs,
                                                  const int32_t* __restrict__ cu_pools, int kpool,
                                                  int t) {
    QueryPools r;
    r.doc = find_doc(cu, num_docs, t);
    int start = cu[r.doc];
    r.pool_lo = cu_pools[r.doc];
    r.n_vis = (t - start + 1) / kpool;
    r.tail_start = start + kpool * r.n_vis;
    return r;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves (no LDS):
// row_shr 1, 2, 4, 8 scan each row of 16 lanes; row_bcast 15 and 31 carry the
// row totals into the rows above.
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31 into rows 2, 3
    return x;
}

}  // namespace kp
