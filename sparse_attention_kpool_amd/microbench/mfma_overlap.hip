// What a single wave per SIMD pays for other work between its bf16 MFMAs on
// gfx950, in cycles per v_mfma_f32_16x16x32_bf16 (clock64 of wave 0 of each of
// 256 workgroups of 256 threads: one wave per SIMD on every compute unit):
//   chains:  16 MFMAs per loop iteration over 1, 2, 4, 8 or 16 independent
//            accumulators (VGPR or AGPR), and the older 16x16x16 instruction,
//            which takes as long for half the work;
//   overlap: after each MFMA, one 16-byte LDS read (its result feeding the MFMA
//            four reads later, waited for with lgkmcnt(3)), or two transposing
//            8-byte reads (ds_read_b64_tr_b16, one V operand), and/or
//            independent VALU FMAs.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_overlap.hip -o mfma_overlap
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int NCH, bool AGPR, bool K16>
__global__ __launch_bounds__(256) void chain_kernel(float* out, int iters) {
    f32x4 c[16];
    for (int k = 0; k < 16; ++k) c[k] = f32x4{0, 0, 0, 0};
    bf16x8 a, b;
    bf16x4 a4, b4;
    for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(threadIdx.x * 0.001f + e); b[e] = (__bf16)(e * 0.5f); }
    for (int e = 0; e < 4; ++e) { a4[e] = a[e]; b4[e] = b[e]; }
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            if (K16) {
                if (AGPR) __asm__ __volatile__("v_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+a"(c[k % NCH]) : "v"(a4), "v"(b4));
                else __asm__ __volatile__("v_mfma_f32_16x16x16_bf16 %0, %1, %2, %0" : "+v"(c[k % NCH]) : "v"(a4), "v"(b4));
            } else {
                if (AGPR) __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c[k % NCH]) : "v"(a), "v"(b));
                else __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c[k % NCH]) : "v"(a), "v"(b));
            }
        }
    }
    const long long t1 = clock64();
    __asm__ __volatile__("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = 0;
    for (int k = 0; k < NCH; ++k) r += c[k][0];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x == 0) out[65536 + blockIdx.x] = (float)(t1 - t0) / iters / 16;
}

template <int NR, int NV, bool TR>
__global__ __launch_bounds__(256) void overlap_kernel(float* out, int iters) {
    __shared__ __align__(16) unsigned lds[16384];
    for (int e = threadIdx.x; e < 16384; e += 256) lds[e] = e * 0x00010001u;
    __syncthreads();
    f32x4 c[8];
    for (int i = 0; i < 8; ++i) c[i] = f32x4{0, 0, 0, 0};
    bf16x8 b;
    for (int e = 0; e < 8; ++e) b[e] = (__bf16)(e * 0.5f);
    const unsigned base = (threadIdx.x & 63) * 16 + (threadIdx.x >> 6) * 16384;
    u32x4 r0, r1, r2, r3;
    float v[8];
    for (int e = 0; e < 8; ++e) v[e] = threadIdx.x + e;
    __asm__ __volatile__("ds_read_b128 %0, %4\n ds_read_b128 %1, %4 offset:1024\n ds_read_b128 %2, %4 offset:2048\n ds_read_b128 %3, %4 offset:3072\n s_waitcnt lgkmcnt(0)"
                         : "=v"(r0), "=v"(r1), "=v"(r2), "=v"(r3) : "v"(base));
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#define OV_STEP(R, I, OFF)                                                                              \
        __asm__ __volatile__("s_waitcnt lgkmcnt(3)" ::: "memory");                                     \
        __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"                                  \
                             : "+v"(c[I]) : "v"(__builtin_bit_cast(bf16x8, R)), "v"(b));                \
        if (NR >= 1) {                                                                                  \
            if (TR) {                                                                                   \
                u32x2 lo_, hi_;                                                                         \
                __asm__ __volatile__("ds_read_b64_tr_b16 %0, %2 offset:%3\n ds_read_b64_tr_b16 %1, %2 offset:%4" \
                                     : "=v"(lo_), "=v"(hi_) : "v"(base), "i"(OFF), "i"(OFF + 512));       \
                R = __builtin_shufflevector(lo_, hi_, 0, 1, 2, 3);                                      \
            } else {                                                                                    \
                __asm__ __volatile__("ds_read_b128 %0, %1 offset:%2" : "=v"(R) : "v"(base), "i"(OFF));  \
            }                                                                                           \
        }                                                                                               \
        _Pragma("unroll") for (int q = 0; q < NV; ++q) __asm__ __volatile__("v_fma_f32 %0, %0, %0, 1.0" : "+v"(v[(q + I) & 7]));
        OV_STEP(r0, 0, 0) OV_STEP(r1, 1, 1024) OV_STEP(r2, 2, 2048) OV_STEP(r3, 3, 3072)
        OV_STEP(r0, 4, 4096) OV_STEP(r1, 5, 5120) OV_STEP(r2, 6, 6144) OV_STEP(r3, 7, 7168)
#undef OV_STEP
    }
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
    const long long t1 = clock64();
    float r = 0;
    for (int i = 0; i < 8; ++i) r += c[i][0];
    for (int e = 0; e < 8; ++e) r += v[e];
    r += __builtin_bit_cast(float, r0[0]) + __builtin_bit_cast(float, r1[1]) + __builtin_bit_cast(float, r2[2]) +
         __builtin_bit_cast(float, r3[3]);
    out[blockIdx.x * 256 + threadIdx.x] = r;
    if (threadIdx.x == 0) out[65536 + blockIdx.x] = (float)(t1 - t0) / iters / 8;
}

static double mean_cycles(float* d) {
    float h[256];
    if (hipMemcpy(h, d + 65536, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return -1;
    double s = 0;
    for (int b = 0; b < 256; ++b) s += h[b];
    return s / 256;
}

template <int NCH, bool AGPR, bool K16>
void run_chain(float* d) {
    chain_kernel<NCH, AGPR, K16><<<256, 256>>>(d, 2048);
    if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return; }
    printf("chain  %s %2d accumulators (%s): %.1f cycles per MFMA\n", K16 ? "16x16x16" : "16x16x32", NCH,
           AGPR ? "AGPR" : "VGPR", mean_cycles(d));
}

template <int NR, int NV, bool TR>
void run_overlap(float* d) {
    overlap_kernel<NR, NV, TR><<<256, 256>>>(d, 2048);
    if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return; }
    printf("overlap per MFMA: %d %-22s + %d VALU fma: %.1f cycles per MFMA\n", NR,
           NR == 0 ? "LDS reads" : TR ? "x two ds_read_b64_tr_b16" : "x ds_read_b128", NV, mean_cycles(d));
}

int main() {
    float* d;
    if (hipMalloc(&d, (1 << 20) * 4) != hipSuccess) return 1;
    run_chain<1, false, false>(d); run_chain<4, false, false>(d); run_chain<16, false, false>(d);
    run_chain<1, true, false>(d); run_chain<16, true, false>(d);
    run_chain<1, false, true>(d); run_chain<16, true, true>(d);
    run_overlap<0, 0, false>(d); run_overlap<1, 0, false>(d); run_overlap<1, 1, false>(d); run_overlap<1, 2, false>(d);
    run_overlap<1, 0, true>(d); run_overlap<1, 1, true>(d);
    run_overlap<0, 1, false>(d); run_overlap<0, 2, false>(d); run_overlap<0, 3, false>(d);
    printf("done\n");
    return 0;
}
