// Calibration statistics of the W4A4 layer ("W4A4 Quantization for Inference
// on Wan2.2-I2V-A14B", calibration paragraph before Eq. (4)): per-input-channel
// activation maxima max_t |x_tj| (also Eq. (4)'s outlier score) and weight
// column ranges max_n |W[n][j]|.
//
// HBM-bound column reduction.  Each lane owns 16 bytes of one row (8 bf16 or
// 4 f32 channels) so a wave reads 1 KiB contiguous per row; the 4 waves of a
// workgroup walk interleaved rows (four rows' streaming loads in flight per
// lane), keep running maxima of |x| as integer bit
// patterns in registers, combine through LDS, and fold into the output with
// one integer atomicMax per channel (non-negative floats order like their
// bit patterns, so the result is exact and independent of order).
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

constexpr int kWaves = 4;

__global__ void __launch_bounds__(256) fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = v;
}

// VEC channels per lane: 8 (bf16) or 4 (f32).
template <bool BF16>
__global__ void __launch_bounds__(256) colmax_kernel(const void* __restrict__ X, int64_t R, int32_t K,
                                                     uint32_t* __restrict__ out) {
    constexpr int VEC = BF16 ? 8 : 4;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunk = (int64_t)blockIdx.x * 64 + lane;
    const bool valid = chunk * VEC < K;
    uint32_t m[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) m[v] = 0;
    if (valid) {
        const int64_t rstride = (int64_t)gridDim.y * kWaves;
        typedef uint32_t v4u __attribute__((ext_vector_type(4)));
        auto at = [&](int64_t r) {
            return reinterpret_cast<const v4u*>(reinterpret_cast<const uint8_t*>(X) +
                                                (r * K + chunk * VEC) * (BF16 ? 2 : 4));
        };
        int64_t r = (int64_t)blockIdx.y * kWaves + wave;
        // four rows' streaming loads in flight together, then their maxima
        for (; r + 3 * rstride < R; r += 4 * rstride) {
            v4u d[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) d[u] = __builtin_nontemporal_load(at(r + u * rstride));
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if constexpr (BF16) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        m[2 * i] = max(m[2 * i], (d[u][i] & 0x7FFFu) << 16);
                        m[2 * i + 1] = max(m[2 * i + 1], d[u][i] & 0x7FFF0000u);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < 4; ++i) m[i] = max(m[i], d[u][i] & 0x7FFFFFFFu);
                }
            }
        }
        for (; r < R; r += rstride) {
            const uint4 d = *reinterpret_cast<const uint4*>(
                reinterpret_cast<const uint8_t*>(X) + (r * K + chunk * VEC) * (BF16 ? 2 : 4));
            const uint32_t w[4] = {d.x, d.y, d.z, d.w};
            if constexpr (BF16) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // |bf16| as the bit pattern of the equal f32
                    m[2 * i] = max(m[2 * i], (w[i] & 0x7FFFu) << 16);
                    m[2 * i + 1] = max(m[2 * i + 1], w[i] & 0x7FFF0000u);
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) m[i] = max(m[i], w[i] & 0x7FFFFFFFu);
            }
        }
    }
    __shared__ uint32_t red[kWaves][64 * VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wave][lane * VEC + v] = m[v];
    __syncthreads();
    // 256 threads fold the 4 wave rows for 64*VEC channels.
    for (int c = threadIdx.x; c < 64 * VEC; c += 256) {
        uint32_t x = red[0][c];
#pragma unroll
        for (int wv = 1; wv < kWaves; ++wv) x = max(x, red[wv][c]);
        const int64_t col = (int64_t)blockIdx.x * 64 * VEC + c;
        if (col < K && x != 0) atomicMax(out + col, x);
    }
}

}  // namespace

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, st, p, v, n);
    return hipGetLastError();
}

hipError_t launch_colmax(const void* X, int32_t dtype, int64_t R, int32_t K, float* out,
                         hipStream_t st) {
    if (R <= 0) return hipSuccess;
    const int vec = dtype == MG_BF16 ? 8 : 4;
    const int64_t gx = ((int64_t)K / vec + 63) / 64;
    // Enough workgroups to cover every CU several times, each wave at least ~8 rows.
    int64_t gy = (R + kWaves * 8 - 1) / (kWaves * 8);
    int64_t cap = (int64_t)device_cu_count() * 8 / gx;
    if (cap < 1) cap = 1;
    if (gy > cap) gy = cap;
    if (gy > 65535) gy = 65535;
    dim3 grid((unsigned)gx, (unsigned)gy);
    uint32_t* o = reinterpret_cast<uint32_t*>(out);
    if (dtype == MG_BF16)
        hipLaunchKernelGGL(colmax_kernel<true>, grid, dim3(256), 0, st, X, R, K, o);
    else
        hipLaunchKernelGGL(colmax_kernel<false>, grid, dim3(256), 0, st, X, R, K, o);
    return hipGetLastError();
}

}  // namespace mg
