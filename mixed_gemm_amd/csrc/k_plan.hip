// Offline planning kernels of the W4A4 layer ("W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B"):
//   smooth_kernel     Eq. (2) smoothing scales s and their reciprocals;
//   topk_kernel       Eq. (4) static top-k outlier set O (sparse index list) + pos;
//   fold_pack_kernel  Eq. (1) fold s into W, extract the outlier columns to bf16,
//                     pack the bulk into MXFP4 with 1x32 or 32x32 block scales
//                     (block-packing paragraph after Eq. (5)).
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

// ---------------------------------------------------------------------------- Eq. (2)

__global__ void __launch_bounds__(256) smooth_kernel(const float* __restrict__ a,
                                                     const float* __restrict__ w, int32_t K,
                                                     double alpha, int32_t smooth,
                                                     float* __restrict__ s, float* __restrict__ rcp) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    float sj = 1.0f;
    if (smooth) {
        const double aa = fmax((double)a[j], 1e-5);
        const double ww = fmax((double)w[j], 1e-5);
        sj = (float)(pow(aa, alpha) / pow(ww, 1.0 - alpha));
    }
    s[j] = sj;
    rcp[j] = __fdiv_rn(1.0f, sj);
}

// ---------------------------------------------------------------------------- Eq. (4)

constexpr int kTopkThreads = 1024;

// Block-wide inclusive scan of one value per thread (Hillis-Steele in LDS).
__device__ int block_inclusive_scan(int v, int* buf) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = 1; off < kTopkThreads; off <<= 1) {
        int add = t >= off ? buf[t - off] : 0;
        __syncthreads();
        buf[t] += add;
        __syncthreads();
    }
    int r = buf[t];
    __syncthreads();
    return r;
}

__device__ int block_sum(int v, int* buf) {
    const int t = threadIdx.x;
    buf[t] = v;
    __syncthreads();
    for (int off = kTopkThreads / 2; off > 0; off >>= 1) {
        if (t < off) buf[t] += buf[t + off];
        __syncthreads();
    }
    int r = buf[0];
    __syncthreads();
    return r;
}

// One workgroup.  Scores are non-negative floats, compared through their bit
// patterns (same order).  T = the k-th largest score is found by bisection on
// the bit pattern; channels above T are in O, and of the channels equal to T
// the lowest indices fill the remaining places (tie rule: index ascending).
// Thread t owns the contiguous index range [t*C, (t+1)*C) so block scans give
// ascending order directly.
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ a, int32_t K,
                                                            int32_t k, int32_t* __restrict__ O,
                                                            int32_t* __restrict__ pos) {
    __shared__ int buf[kTopkThreads];
    const uint32_t* ab = reinterpret_cast<const uint32_t*>(a);
    const int t = threadIdx.x;
    const int C = (K + kTopkThreads - 1) / kTopkThreads;
    const int j0 = t * C;
    const int j1 = min(K, j0 + C);

    uint32_t T = 0;
    int need = 0;
    if (k > 0 && k < K) {
        uint32_t lo = 0, hi = 0x7F800000u;       // count(score >= 0) = K >= k
        while (lo < hi) {
            const uint32_t mid = lo + (hi - lo + 1) / 2;
            int c = 0;
            for (int j = j0; j < j1; ++j) c += ab[j] >= mid;
            if (block_sum(c, buf) >= k) lo = mid; else hi = mid - 1;
        }
        T = lo;
        int g = 0;
        for (int j = j0; j < j1; ++j) g += ab[j] > T;
        need = k - block_sum(g, buf);
    }
    // ties before my range
    int ties = 0;
    for (int j = j0; j < j1; ++j) ties += ab[j] == T;
    int tie_off = block_inclusive_scan(ties, buf) - ties;
    // membership and ascending positions
    int mine = 0;
    {
        int to = tie_off;
        for (int j = j0; j < j1; ++j) {
            bool in = k >= K || (k > 0 && (ab[j] > T || (ab[j] == T && to < need)));
            to += ab[j] == T;
            mine += in;
        }
    }
    int off = block_inclusive_scan(mine, buf) - mine;
    {
        int to = tie_off;
        for (int j = j0; j < j1; ++j) {
            bool in = k >= K || (k > 0 && (ab[j] > T || (ab[j] == T && to < need)));
            to += ab[j] == T;
            if (in) {
                O[off] = j;
                pos[j] = off;
                ++off;
            } else {
                pos[j] = -1;
            }
        }
    }
}

// ---------------------------------------------------------------------------- fold + pack

// Workgroup = 32 rows x 8 blocks of 32 K.  Thread (ty, tx) folds, extracts and
// encodes row n = 32*blockIdx.y + ty, block b = 8*blockIdx.x + tx.  For the
// 32x32 layout the 32 rows of a tile share their amax through LDS.
template <bool BF16, bool TILE>
__global__ void __launch_bounds__(256) fold_pack_kernel(const void* __restrict__ W, int32_t N, int32_t K,
                                                        int32_t k, const float* __restrict__ s,
                                                        const int32_t* __restrict__ pos,
                                                        uint8_t* __restrict__ Wq, uint8_t* __restrict__ Ws,
                                                        uint8_t* __restrict__ Wst,
                                                        uint16_t* __restrict__ WO) {
    const int tx = threadIdx.x & 7;
    const int ty = threadIdx.x >> 3;
    const int nb = K / 32;
    const int b = blockIdx.x * 8 + tx;
    const int64_t n = (int64_t)blockIdx.y * 32 + ty;
    const bool valid = b < nb && n < N;
    float v[32];
    uint32_t amax = 0;
    if (valid) {
        const int j0 = b * 32;
        if constexpr (BF16) {
            const uint4* src = reinterpret_cast<const uint4*>(
                reinterpret_cast<const uint16_t*>(W) + n * K + j0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 d = src[q];
                const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    v[8 * q + 2 * i] = bf16_to_f32(wd[i] & 0xFFFFu);
                    v[8 * q + 2 * i + 1] = bf16_to_f32(wd[i] >> 16);
                }
            }
        } else {
            const float4* src = reinterpret_cast<const float4*>(
                reinterpret_cast<const float*>(W) + n * K + j0);
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const float4 d = src[q];
                v[4 * q] = d.x; v[4 * q + 1] = d.y; v[4 * q + 2] = d.z; v[4 * q + 3] = d.w;
            }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            float f = __fmul_rn(s[j0 + i], v[i]);          // RN(s_j * W[n][j])
            const int p = pos[j0 + i];
            if (p >= 0) {
                WO[n * k + p] = (uint16_t)f32_to_bf16_rne(f);
                f = 0.0f;
            }
            v[i] = f;
            amax = max(amax, __float_as_uint(f) & 0x7FFFFFFFu);
        }
    }
    if constexpr (TILE) {
        __shared__ uint32_t tmax[32][8];
        tmax[ty][tx] = amax;
        __syncthreads();
        if (ty == 0) {
            uint32_t m = 0;
            for (int r = 0; r < 32; ++r) m = max(m, tmax[r][tx]);
            tmax[0][tx] = m;
        }
        __syncthreads();
        amax = tmax[0][tx];
    }
    if (!valid) return;
    const uint32_t c = e8m0_from_amax_bits(amax);
    uint32_t packed[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t word = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) word |= e2m1_nibble(v[8 * q + i], c) << (4 * i);
        packed[q] = word;
    }
    *reinterpret_cast<uint4*>(Wq + n * (K / 2) + b * 16) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
    Ws[n * nb + b] = (uint8_t)c;
    if (TILE && ty == 0) Wst[(n / 32) * nb + b] = (uint8_t)c;
}

}  // namespace

hipError_t launch_smooth(const float* a, const float* w, int32_t K, double alpha, int32_t smooth,
                         float* s, float* rcp, hipStream_t st) {
    hipLaunchKernelGGL(smooth_kernel, dim3((K + 255) / 256), dim3(256), 0, st, a, w, K, alpha, smooth,
                       s, rcp);
    return hipGetLastError();
}

hipError_t launch_topk(const float* a, int32_t K, int32_t k, int32_t* O, int32_t* pos,
                       hipStream_t st) {
    hipLaunchKernelGGL(topk_kernel, dim3(1), dim3(kTopkThreads), 0, st, a, K, k, O, pos);
    return hipGetLastError();
}

hipError_t launch_fold_pack(const void* W, int32_t dtype, int32_t N, int32_t K, int32_t k,
                            int32_t layout, const float* s, const int32_t* pos, uint8_t* Wq,
                            uint8_t* Ws, uint8_t* Wst, uint16_t* WO, hipStream_t st) {
    dim3 grid((unsigned)((K / 32 + 7) / 8), (unsigned)((N + 31) / 32));
    const bool bf = dtype == MG_BF16;
    const bool tile = layout == MG_W_32X32;
    if (bf && tile)
        hipLaunchKernelGGL((fold_pack_kernel<true, true>), grid, dim3(256), 0, st, W, N, K, k, s, pos, Wq, Ws, Wst, WO);
    else if (bf)
        hipLaunchKernelGGL((fold_pack_kernel<true, false>), grid, dim3(256), 0, st, W, N, K, k, s, pos, Wq, Ws, Wst, WO);
    else if (tile)
        hipLaunchKernelGGL((fold_pack_kernel<false, true>), grid, dim3(256), 0, st, W, N, K, k, s, pos, Wq, Ws, Wst, WO);
    else
        hipLaunchKernelGGL((fold_pack_kernel<false, false>), grid, dim3(256), 0, st, W, N, K, k, s, pos, Wq, Ws, Wst, WO);
    return hipGetLastError();
}

}  // namespace mg
