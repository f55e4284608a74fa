// Selection helpers shared by the top-k kernels: the order-preserving score
// key, a block scan, and a most-significant-digit-first radix select.
#pragma once

#include "kp_device.h"

namespace kp {

// Order-preserving 32-bit key of a score: a larger score has a larger key;
// -0 is folded onto +0 and NaN sorts below -inf (key 0).
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;                                      // -0 == +0
    // negative: all bits flipped; otherwise the sign bit set
    const uint32_t k = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    return (u & 0x7FFFFFFFu) > 0x7F800000u ? 0u : k;                    // NaN: lowest
}

// Exclusive scan of one int per thread over a block of NTH threads; returns
// the prefix and writes the total to *total.
template <int NTH>
__device__ __forceinline__ int block_excl_scan(int v, int* wave_buf, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wave_buf[wave] = x;
    __syncthreads();
    int add = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
        int t = wave_buf[w];
        if (w < wave) add += t;
        tot += t;
    }
    __syncthreads();
    *total = tot;
    return add + x - v;
}

constexpr int RS_BINS = 2048;             // histogram bins of the widest digit
constexpr int RS_ALL_EQ = 0x7FFFFFFF;     // the boundary bin is kept whole

// k-th largest key by a most-significant-digit-first radix select, keys of
// `bits` significant bits (32 by default, else every key is below 2^bits),
// digits of at most 11 bits from the top (32 bits: 11, 11 and 10), histograms
// in LDS. visit(f) calls f(key) for every key of this thread's share (the
// shares of the NTH threads together are the keys taking part; a pass may
// visit them in any order, the same set each time). Requires 0 < k <= number
// of keys. On return *thresh is the key K of the k-th largest and *take_eq
// the number of keys equal to K that are kept (which ones is the caller's tie
// rule), or, when a digit's boundary bin is kept whole, *thresh is that bin's
// prefix (lower bits zero), *take_eq = RS_ALL_EQ, and exactly k keys are >=
// *thresh. Called by all NTH threads of the block; hist is [2][RS_BINS], sel
// holds 3 ints.
template <int NTH, typename Visit>
__device__ __forceinline__ void radix_select(Visit visit, int k, int (*hist)[RS_BINS], int* sel,
                                             uint32_t* thresh, int* take_eq, int bits = 32) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int b = tid; b < RS_BINS; b += NTH) hist[0][b] = 0;
    __syncthreads();
    int remaining = k;
    uint32_t prefix = 0u, pmask = 0u;
    int teq = -1;
    int low = bits;   // bits below the ones fixed so far
#pragma unroll 1
    for (int pass = 0; low > 0; ++pass) {
        const int width = low < 11 ? low : 11;
        const int shift = low - width;
        const int nb = 1 << width;
        int* h = hist[pass & 1];
        visit([&](uint32_t v) {
            if ((v & pmask) == prefix) atomicAdd(&h[(v >> shift) & (uint32_t)(nb - 1)], 1);
        });
        for (int b = tid; b < RS_BINS; b += NTH) hist[(pass + 1) & 1][b] = 0;
        __syncthreads();
        if (wave == 0) {
            // lane l owns bins [nb - per*(l+1), nb - per*l) (none past the
            // first nb lanes): a scan over lanes counts the keys in the bins
            // above each lane's. A lane's (up to 32) counts are read with
            // 16-byte LDS loads, all in flight together.
            const int per = nb >= 64 ? nb >> 6 : 1;
            const int base = nb - per * (lane + 1);
            int cnt[32];
            int own = 0;
            if (per >= 4) {
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    int4 v = make_int4(0, 0, 0, 0);
                    if (4 * q < per) v = *reinterpret_cast<const int4*>(h + base + 4 * q);
                    cnt[4 * q] = v.x;
                    cnt[4 * q + 1] = v.y;
                    cnt[4 * q + 2] = v.z;
                    cnt[4 * q + 3] = v.w;
                }
            } else {
#pragma unroll
                for (int m = 0; m < 32; ++m) cnt[m] = m < per && base >= 0 ? h[base + m] : 0;
            }
#pragma unroll
            for (int m = 0; m < 32; ++m) own += cnt[m];
            const int incl = wave_incl_scan(own);
            const int before = incl - own;
            if (base >= 0 && before < remaining && incl >= remaining) {
                int acc = before;
#pragma unroll
                for (int m = 31; m >= 0; --m) {
                    if (m < per) {
                        const int c = cnt[m];
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
        // (sel is rewritten only after the next digit's histogram barrier)
        const int sel_digit = sel[0], sel_above = sel[1], sel_cnt = sel[2];
        remaining -= sel_above;
        prefix |= (uint32_t)sel_digit << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        low = shift;
        if (sel_cnt == remaining) {
            teq = RS_ALL_EQ;
            break;
        }
    }
    *thresh = prefix;
    *take_eq = teq < 0 ? remaining : teq;
}

// Minimum and maximum over the block (all NTH threads call it; red holds
// 2 * NTH / 64 ints).
template <int NTH>
__device__ __forceinline__ void block_min_max(uint32_t lo, uint32_t hi, uint32_t* red, uint32_t* out_lo,
                                              uint32_t* out_hi) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        lo = min(lo, (uint32_t)__shfl_xor((int)lo, o, 64));
        hi = max(hi, (uint32_t)__shfl_xor((int)hi, o, 64));
    }
    if (lane == 0) {
        red[wave] = lo;
        red[NTH / 64 + wave] = hi;
    }
    __syncthreads();
    uint32_t a = 0xFFFFFFFFu, b = 0u;
#pragma unroll
    for (int w = 0; w < NTH / 64; ++w) {
        a = min(a, red[w]);
        b = max(b, red[NTH / 64 + w]);
    }
    __syncthreads();
    *out_lo = a;
    *out_hi = b;
}

}  // namespace kp
