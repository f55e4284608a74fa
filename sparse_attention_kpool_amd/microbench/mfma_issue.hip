// Issue-rate microbenchmark for gfx950: how much bf16 MFMA throughput a wave
// keeps when other instructions sit between its MFMAs, with one and with two
// waves per SIMD. Each wave runs four independent v_mfma_f32_16x16x32_bf16
// accumulation chains and, after each MFMA, NV instructions of one kind:
// independent VALU FMAs, dependent SALU adds, 16-byte LDS reads (waited for once
// per iteration) or VALU exponentials. One workgroup per compute unit (256);
// 256 threads = one wave per SIMD, 512 = two. The kernel time (HIP events)
// gives the achieved bf16 TFLOP/s; clock64 gives the cycles per iteration of
// wave 0 of each workgroup.
//
//   hipcc -O3 --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops mfma_issue.hip -o mfma_issue
#include <hip/hip_runtime.h>
#include <cstdio>
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// KIND 0: VALU fma, 1: SALU add, 2: LDS read b128 (no wait until the end), 3: v_exp_f32
template <int KIND, int NV>
__global__ __launch_bounds__(512) void mfma_issue_kernel(float* out, int iters, float s) {
    __shared__ __align__(16) float lds[64 * 64];
    for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) lds[e] = e;
    __syncthreads();
    f32x4 c0 = {0,0,0,0}, c1 = c0, c2 = c0, c3 = c0;
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(threadIdx.x * 0.001f + e); b[e] = (__bf16)(e * 0.5f); }
    float v[8];
    for (int e = 0; e < 8; ++e) v[e] = threadIdx.x + e;
    f32x4 ld[4] = {c0, c0, c0, c0};
    int sv = __builtin_amdgcn_readfirstlane(threadIdx.x);
    const unsigned lane_off = (threadIdx.x & 63) * 16;
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
#define MB_FILL(o_)                                                                              \
        _Pragma("unroll") for (int k = 0; k < NV; ++k) {                                         \
            if (KIND == 0) __asm__ __volatile__("v_fma_f32 %0, %0, %1, %1" : "+v"(v[(k + o_) & 7]) : "v"(s)); \
            if (KIND == 1) __asm__ __volatile__("s_add_u32 %0, %0, 3" : "+s"(sv) :: "scc");     \
            if (KIND == 2) __asm__ __volatile__("ds_read_b128 %0, %1 offset:%2" : "=v"(ld[k & 3]) : "v"(lane_off), "i"(1024 * ((k + o_) & 7))); \
            if (KIND == 3) __asm__ __volatile__("v_exp_f32 %0, %0" : "+v"(v[(k + o_) & 7]));   \
        }
        __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
        MB_FILL(0)
        __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
        MB_FILL(3)
        __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a), "v"(b));
        MB_FILL(5)
        __asm__ __volatile__("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a), "v"(b));
        MB_FILL(1)
        if (KIND == 2) __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    const long long t1 = clock64();
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = c0[0] + c1[1] + c2[2] + c3[3] + (float)sv;
    for (int e = 0; e < 8; ++e) r += v[e];
    for (int e = 0; e < 4; ++e) r += ld[e][0];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x == 0) out[gridDim.x * blockDim.x + blockIdx.x] = (float)(t1 - t0) / iters;
}

// The same with four v_mfma_f32_32x32x16_bf16 chains (32,768 flop each, twice
// the 16x16x32 instruction's work): how much of the per-MFMA issue cost a
// wave saves with the larger tile.
template <int KIND, int NV>
__global__ __launch_bounds__(512) void mfma32_issue_kernel(float* out, int iters, float s) {
    __shared__ __align__(16) float lds[64 * 64];
    for (int e = threadIdx.x; e < 64 * 64; e += blockDim.x) lds[e] = e;
    __syncthreads();
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    bf16x8 a, b;
    for (int e = 0; e < 8; ++e) { a[e] = (__bf16)(threadIdx.x * 0.001f + e); b[e] = (__bf16)(e * 0.5f); }
    float v[8];
    for (int e = 0; e < 8; ++e) v[e] = threadIdx.x + e;
    f32x4 ld[4] = {};
    int sv = __builtin_amdgcn_readfirstlane(threadIdx.x);
    const unsigned lane_off = (threadIdx.x & 63) * 16;
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        __asm__ __volatile__("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
        MB_FILL(0)
        __asm__ __volatile__("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
        MB_FILL(3)
        __asm__ __volatile__("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a), "v"(b));
        MB_FILL(5)
        __asm__ __volatile__("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a), "v"(b));
        MB_FILL(1)
        if (KIND == 2) __asm__ __volatile__("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    const long long t1 = clock64();
    __asm__ __volatile__("s_waitcnt lgkmcnt(0)\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    float r = c0[0] + c1[1] + c2[2] + c3[3] + (float)sv;
    for (int e = 0; e < 8; ++e) r += v[e];
    for (int e = 0; e < 4; ++e) r += ld[e][0];
    out[blockIdx.x * blockDim.x + threadIdx.x] = r;
    if (threadIdx.x == 0) out[gridDim.x * blockDim.x + blockIdx.x] = (float)(t1 - t0) / iters;
}

template <int KIND, int NV, bool BIG = false>
void run(float* d, int threads) {
    const int iters = 8192;
    const char* kn[4] = {"VALU fma", "SALU add", "LDS b128", "VALU exp"};
    auto launch = [&]() {
        if (BIG) mfma32_issue_kernel<KIND, NV><<<256, threads>>>(d, iters, 1.0001f);
        else mfma_issue_kernel<KIND, NV><<<256, threads>>>(d, iters, 1.0001f);
    };
    launch();
    if (hipDeviceSynchronize() != hipSuccess) { printf("launch failed\n"); return; }
    hipEvent_t e0, e1;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return;
    (void)hipEventRecord(e0);
    launch();
    (void)hipEventRecord(e1);
    hipError_t e = hipDeviceSynchronize();
    float ms = 0;
    (void)hipEventElapsedTime(&ms, e0, e1);
    const double mf = 256.0 * (threads / 64) * iters * 4 * (BIG ? 2 : 1);   // in 16x16x32 units
    if (e != hipSuccess) { printf("error %s\n", hipGetErrorString(e)); return; }
    float h[1];
    (void)hipMemcpy(h, d + 256 * threads, 4, hipMemcpyDeviceToHost);
    printf("%s %d waves/SIMD %-9s x%2d per MFMA: %6.1f clock64 per 4 MFMA; kernel %.3f ms = %.0f TFLOP/s bf16 (%.1f%% of 2.5 PF)\n", BIG ? "32x32x16" : "16x16x32", threads / 256, kn[KIND], NV, h[0], ms, mf * 16384 / ms / 1e9, mf * 16384 / ms / 1e9 / 25.0);
}

int main() {
    float* d;
    if (hipMalloc(&d, (1 << 20) * 4) != hipSuccess) return 1;
    for (int t = 256; t <= 512; t += 256) {
        run<0, 0>(d, t); run<0, 2>(d, t); run<0, 4>(d, t); run<0, 8>(d, t);
        run<1, 4>(d, t); run<1, 8>(d, t); run<1, 16>(d, t);
        run<2, 1>(d, t); run<2, 2>(d, t); run<2, 4>(d, t);
        run<3, 1>(d, t); run<3, 2>(d, t); run<3, 4>(d, t);
        run<0, 0, true>(d, t); run<0, 2, true>(d, t); run<0, 4, true>(d, t); run<0, 8, true>(d, t);
        run<2, 1, true>(d, t); run<2, 2, true>(d, t); run<3, 2, true>(d, t); run<3, 4, true>(d, t);
    }
    printf("done\n");
    return 0;
}
