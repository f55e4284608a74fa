// Pieces shared by the sparse latent attention kernels of libkpool (forward
// and backward): the tile geometry, the LDS row layout, the direct-to-LDS row
// gather of gfx950, wait and barrier helpers, and the workgroup -> query map.
#pragma once

#include "kp_device.h"

namespace kp {

constexpr int MLA_TK = 64;    // latent rows per tile
constexpr int MLA_NW = 4;     // waves per workgroup (one per SIMD)
constexpr int MLA_NBUF = 2;   // LDS tiles in the gather ring
constexpr int MLA_MAX_ROW = 4096;  // index-row entries the LDS list holds
// index-row entries of the two-wave attention form (two of its workgroups share a
// compute unit's 160 KB of LDS: a ring of two 32-row tiles and this list each)
constexpr int MLA_W2_MAX_ROW = 2560;

// LDS layout of a tile row: row r starts at byte r*(RB + 48) + 16*(r & 1) of its
// tile (RB bytes of latent, chunks in order). gfx950 services a 16-byte LDS read
// in four passes of 16 lanes (lanes {0-3, 12-15, 20-27}, {4-11, 16-19, 28-31}
// and the same in the upper half) and 8-byte and transposing reads in two
// passes of 32 consecutive lanes; under those passes this pitch and odd-row
// shift spread the row-wise K reads (16 rows, one chunk column per lane group)
// and the column-wise transposing V reads (8 rows per pass) over all 64 banks
// with no conflict. Every read address is then a per-lane base plus a constant
// (the k-step or column tile), which the read instruction carries as its
// offset: no address arithmetic per read.
template <int RB>
__device__ __forceinline__ constexpr int row_base(int r) { return r * (RB + 48) + 16 * (r & 1); }

__device__ __forceinline__ bf16x4 lds_read_tr16(const uint8_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((KP_LDS bf16x4*)(p));
}

// compiler-only barrier: keeps LDS accesses on their side of the explicit waits
__device__ __forceinline__ void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

__device__ __forceinline__ void wait_lgkm0() {
    // s_waitcnt lgkmcnt(0) only (vmcnt 63, expcnt 7: no wait)
    __builtin_amdgcn_s_waitcnt(0xC07F);
}

// Direct-to-LDS copy of one latent row (gfx950 buffer_load_dwordx4 ... lds): lane
// l copies the 16 bytes at rsrc base + soff + voff + OFF to LDS byte M0 + OFF +
// 16*l. The latent is a raw buffer resource, the row's byte offset the scalar
// offset and the lane's chunk offset the vector offset, so no 64-bit address is
// formed per row. The immediate OFF moves both the memory and the LDS address:
// rows that share M0 (the LDS address of a group's first row, passed as an
// operand so that the compiler writes M0 once per group) land OFF bytes above
// it, and their scalar offsets carry -OFF. Issued as inline assembly so the
// compiler does not make LDS reads of the other ring tile wait for it;
// completion is tracked by the explicit vmcnt wait before each barrier.
template <int OFF>
__device__ __forceinline__ void lds_dma16_row_at(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t m0) {
    __asm__ __volatile__("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                         :: "v"(voff), "s"(rsrc), "s"(soff), "n"(OFF), "{m0}"(m0) : "memory");
}

// Five wait states after VALU writes (v_readfirstlane) of these 16 scalar
// registers, which vector-memory instructions read next (gfx9 needs five).
__device__ __forceinline__ void kp_sgpr_settle(int (&r)[16]) {
    __asm__ __volatile__("s_nop 4"
                         : "+s"(r[0]), "+s"(r[1]), "+s"(r[2]), "+s"(r[3]), "+s"(r[4]), "+s"(r[5]), "+s"(r[6]),
                           "+s"(r[7]), "+s"(r[8]), "+s"(r[9]), "+s"(r[10]), "+s"(r[11]), "+s"(r[12]),
                           "+s"(r[13]), "+s"(r[14]), "+s"(r[15]));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)((KP_LDS const uint8_t*)p);
}

// wait until none of this wave's vector-memory operations is outstanding
// (vmcnt 0; expcnt 7 and lgkmcnt 15 mean "do not wait" on those counters)
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// wait until at most N of this wave's vector-memory operations are outstanding
// (vmcnt N: bits 3:0 and 15:14 of the wait's immediate)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
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
// (the two-wave attention form keeps two workgroups per CU, so an XCD holds 64
// queries at a time: runs of 64 keep them consecutive)
#define MLA_XCD_RUN_W2 64
template <int R = MLA_XCD_RUN>
__device__ __forceinline__ int xcd_query(int b, int n) {
    const int full = n / (8 * R) * (8 * R);
    if (b >= full) return b;
    const int slot = b >> 3, xcd = b & 7;   // slot-th workgroup that lands on this XCD
    return (slot / R) * (8 * R) + xcd * R + slot % R;
}

}  // namespace kp
