// FP8 lightning-indexer scoring over pools on gfx950 matrix cores.
//
// prime-rl PR "GLM-5.3-Flash text model", Summary, third bullet: a query
// scores, in FP8, the complete pools ending at or before it (pools of its own
// document), after Hadamard rotation of both sides. Score of query i and
// pool p:
//   I[i,p] = sk[p] * sum_h (w[i,h] * sq[i,h]) * ReLU(<q8[i,h], k8[p]>)
// which equals sum_h w * ReLU(sq * sk * <q8, k8>) because both scales are
// positive.
//
// Work decomposition: a workgroup takes 16 queries and a chunk of 512 pools;
// each of its 4 waves holds the E4M3 codes of 128 pools (8 tiles of 16) in
// registers as the B operand and streams the query tile from LDS as the A
// operand: one v_mfma_f32_16x16x128_f8f6f4 covers a full 128-wide dot for 16
// heads x 16 pools. The ReLU and head weighting run on the fp32 accumulator
// lanes; the sum over the 16 heads of a tile is finished with two cross-lane
// adds. Workgroups whose pool chunk lies outside every query's visible range
// exit at once; query tiles are dispatched last-first so the longest causal
// rows start early.
#include "kp_device.h"
#include "kp_launch.h"

namespace kp {

constexpr int SC_QT = 16;     // queries per workgroup
constexpr int SC_PW = 128;    // pools per wave
constexpr int SC_WAVES = 4;
constexpr int SC_PC = SC_PW * SC_WAVES;  // pools per workgroup

__global__ void fill_f32_kernel(float* __restrict__ dst, size_t n, float v) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) dst[i] = v;
}

hipError_t launch_fill_f32(float* dst, size_t n, float value, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    size_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    fill_f32_kernel<<<(unsigned)blocks, 256, 0, stream>>>(dst, n, value);
    return hipGetLastError();
}

// LDS layout of the query tile: row (q, h) of 128 bytes = 8 chunks of 16 B;
// chunk c of row with head h is stored at chunk c ^ (h & 7) so that the 16
// rows an A-operand read touches fall in distinct banks.
template <int NHT>
__global__ __launch_bounds__(256) void score_kernel(
    const int32_t* __restrict__ cu, int num_docs, const int32_t* __restrict__ cu_pools, int kpool,
    const int32_t* __restrict__ q_pos, int num_q, const uint8_t* __restrict__ q8,
    const float* __restrict__ sq, const float* __restrict__ w, int h_idx, int d_idx,
    const uint8_t* __restrict__ k8, const float* __restrict__ sk, int max_pools,
    float* __restrict__ scores) {
    constexpr int NH = NHT * 16;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* q_lds = smem;                                           // [QT][NH][128]
    float* wq_lds = reinterpret_cast<float*>(smem + SC_QT * NH * 128);  // [QT][NH]
    __shared__ int lo_s[SC_QT], hi_s[SC_QT];
    __shared__ int any_s;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int nchunks = (max_pools + SC_PC - 1) / SC_PC;
    const int nqt = (num_q + SC_QT - 1) / SC_QT;
    const int qtile = nqt - 1 - (int)(blockIdx.x / nchunks);
    const int q0 = qtile * SC_QT;
    const int P0 = (int)(blockIdx.x % nchunks) * SC_PC;

    if (tid < SC_QT) {
        int lo = 0, hi = 0;
        int i = q0 + tid;
        if (i < num_q) {
            int t = q_pos ? q_pos[i] : i;
            QueryPools qp = query_pools(cu, num_docs, cu_pools, kpool, t);
            lo = qp.pool_lo;
            hi = qp.pool_lo + qp.n_vis;
        }
        lo_s[tid] = lo;
        hi_s[tid] = hi;
    }
    if (tid == 0) any_s = 0;
    __syncthreads();
    if (tid < SC_QT && lo_s[tid] < hi_s[tid] && hi_s[tid] > P0 && lo_s[tid] < P0 + SC_PC) any_s = 1;
    __syncthreads();
    if (!any_s) return;

    // stage the query tile: codes (zero-padded to NH heads x 128 bytes) and w*sq
    const int dchunks = d_idx >> 4;
    for (int c = tid; c < SC_QT * NH * 8; c += 256) {
        int ch = c & 7, row = c >> 3, h = row % NH, q = row / NH;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (q0 + q < num_q && h < h_idx && ch < dchunks)
            v = *reinterpret_cast<const uint4*>(q8 + (((size_t)(q0 + q) * h_idx + h) * d_idx) + ch * 16);
        *reinterpret_cast<uint4*>(q_lds + (size_t)row * 128 + ((ch ^ (h & 7)) << 4)) = v;
    }
    for (int c = tid; c < SC_QT * NH; c += 256) {
        int h = c % NH, q = c / NH;
        float v = 0.0f;
        if (q0 + q < num_q && h < h_idx) {
            size_t o = (size_t)(q0 + q) * h_idx + h;
            v = w[o] * sq[o];
        }
        wq_lds[c] = v;
    }

    // this wave's pools: B operands (32 code bytes of column n per lane) and key scales
    const int Pw = P0 + wave * SC_PW;
    i32x8 b[8];
    float skj[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        int p = Pw + 16 * j + n;
        uint4 lo4 = make_uint4(0u, 0u, 0u, 0u), hi4 = lo4;
        float s = 0.0f;
        if (p < max_pools) {
            const uint8_t* src = k8 + (size_t)p * d_idx;
            if (2 * g < dchunks) lo4 = *reinterpret_cast<const uint4*>(src + 32 * g);
            if (2 * g + 1 < dchunks) hi4 = *reinterpret_cast<const uint4*>(src + 32 * g + 16);
            s = sk[p];
        }
        b[j] = i32x8{(int)lo4.x, (int)lo4.y, (int)lo4.z, (int)lo4.w,
                     (int)hi4.x, (int)hi4.y, (int)hi4.z, (int)hi4.w};
        skj[j] = s;
    }
    __syncthreads();

    for (int q = 0; q < SC_QT; ++q) {
        const int lo = lo_s[q], hi = hi_s[q];
        if (hi <= Pw || lo >= Pw + SC_PW || lo >= hi) continue;
        float acc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = 0.0f;
#pragma unroll
        for (int ht = 0; ht < NHT; ++ht) {
            const int head = ht * 16 + n;
            const uint8_t* row = q_lds + (size_t)(q * NH + head) * 128;
            uint4 a0 = *reinterpret_cast<const uint4*>(row + (((2 * g) ^ (head & 7)) << 4));
            uint4 a1 = *reinterpret_cast<const uint4*>(row + (((2 * g + 1) ^ (head & 7)) << 4));
            i32x8 a = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
            float4 wv = *reinterpret_cast<const float4*>(wq_lds + q * NH + ht * 16 + 4 * g);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                f32x4 c = mfma_fp8_16x16x128(a, b[j], f32x4{0.f, 0.f, 0.f, 0.f});
                acc[j] += wv.x * fmaxf(c[0], 0.0f) + wv.y * fmaxf(c[1], 0.0f) +
                          wv.z * fmaxf(c[2], 0.0f) + wv.w * fmaxf(c[3], 0.0f);
            }
        }
        const size_t orow = (size_t)(q0 + q) * max_pools;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float v = acc[j];
            v += shfl_xor(v, 16);
            v += shfl_xor(v, 32);
            const int p = Pw + 16 * j + n;
            if ((j & 3) == g && p >= lo && p < hi) scores[orow + p] = v * skj[j];
        }
    }
}

hipError_t launch_score(const int32_t* cu, int num_docs, const int32_t* cu_pools, int kpool,
                        const int32_t* q_pos, int num_q, const uint8_t* q8, const float* sq,
                        const float* w, int h_idx, int d_idx, const uint8_t* k8, const float* sk,
                        int max_pools, float* scores, hipStream_t stream) {
    if (num_q == 0 || max_pools == 0) return hipSuccess;
    const int nht = (h_idx + 15) / 16;
    const long long nblk = (long long)((max_pools + SC_PC - 1) / SC_PC) * ((num_q + SC_QT - 1) / SC_QT);
    if (nblk > 0x7FFFFFFFLL) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)nblk);
    const size_t lds = (size_t)SC_QT * nht * 16 * (128 + 4);
    const void* fns[4] = {(const void*)score_kernel<1>, (const void*)score_kernel<2>, (const void*)score_kernel<3>,
                          (const void*)score_kernel<4>};
    hipError_t e = hipFuncSetAttribute(fns[nht - 1], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    switch (nht) {
        case 1:
            score_kernel<1><<<grid, 256, lds, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w,
                                                        h_idx, d_idx, k8, sk, max_pools, scores);
            break;
        case 2:
            score_kernel<2><<<grid, 256, lds, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w,
                                                        h_idx, d_idx, k8, sk, max_pools, scores);
            break;
        case 3:
            score_kernel<3><<<grid, 256, lds, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w,
                                                        h_idx, d_idx, k8, sk, max_pools, scores);
            break;
        default:
            score_kernel<4><<<grid, 256, lds, stream>>>(cu, num_docs, cu_pools, kpool, q_pos, num_q, q8, sq, w,
                                                        h_idx, d_idx, k8, sk, max_pools, scores);
            break;
    }
    return hipGetLastError();
}

}  // namespace kp
