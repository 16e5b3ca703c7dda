// Per-channel percentile statistic for Eq. (4)'s channel mask: the
// nearest-rank q-quantile of |x_tj| over all calibration rows ("W4A4
// Quantization for Inference on Wan2.2-I2V-A14B" ranks channels by a
// calibration statistic; the tail-aware percentile calibration page builds
// its channel mask from a percentile of the activation tail).
//
// Exact two-pass radix selection on the bf16 bit patterns of |x| (15 bits,
// whose integer order is the numeric order of the magnitudes):
//   pass 0: per channel, a histogram of the high byte (bits 14..7);
//   select 0: T = the channel's count, r = ceil(q T) clamped to [1, T]; the
//            high byte h holding rank r and the rank r' inside it; the
//            channel's bins are cleared for pass 1;
//   pass 1: per channel, a histogram of the low 7 bits of the values whose
//           high byte is h;
//   select 1: the low bits l holding rank r'; the value is (h << 7) | l.
// Counting: a workgroup takes 64 channels (128 B of each row: a lane loads
// two channels, 32 lanes a row piece, 8 rows per step) over a chunk of rows
// and counts into 64 x 256 LDS bins with LDS atomics, then adds its non-zero
// bins into the global [K][256] histogram.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

constexpr int kPctCh = 64;        // channels per workgroup
constexpr int kPctBins = 256;

__global__ void __launch_bounds__(256) pct_count_kernel(const uint16_t* __restrict__ X, int64_t M, int32_t K,
                                                        int64_t rows_per_chunk, int pass,
                                                        const int32_t* __restrict__ sel,
                                                        uint32_t* __restrict__ hist) {
    __shared__ uint32_t bins[kPctCh * kPctBins];
    const int t = threadIdx.x;
    for (int i = t; i < kPctCh * kPctBins; i += 256) bins[i] = 0;
    const int cp = t & 31, ri = t >> 5;
    const int c0 = blockIdx.x * kPctCh + 2 * cp;      // this lane's first channel (K even)
    const bool valid = c0 < K;
    int h0 = -1, h1 = -1;                              // pass 1: the selected high bytes
    if (pass == 1 && valid) {
        h0 = sel[2 * c0];
        h1 = sel[2 * (c0 + 1)];
    }
    __syncthreads();
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r_end = r_begin + rows_per_chunk < M ? r_begin + rows_per_chunk : M;
    uint32_t* b0 = bins + (2 * cp) * kPctBins;
    uint32_t* b1 = b0 + kPctBins;
    if (valid) {
        for (int64_t r = r_begin + ri; r < r_end; r += 8) {
            const uint32_t w = *reinterpret_cast<const uint32_t*>(X + r * K + c0);
            const uint32_t a0 = w & 0x7FFFu, a1 = (w >> 16) & 0x7FFFu;
            if (pass == 0) {
                atomicAdd(b0 + (a0 >> 7), 1u);
                atomicAdd(b1 + (a1 >> 7), 1u);
            } else {
                if ((int)(a0 >> 7) == h0) atomicAdd(b0 + (a0 & 0x7Fu), 1u);
                if ((int)(a1 >> 7) == h1) atomicAdd(b1 + (a1 & 0x7Fu), 1u);
            }
        }
    }
    __syncthreads();
    for (int i = t; i < kPctCh * kPctBins; i += 256) {
        const int c = blockIdx.x * kPctCh + i / kPctBins;
        const uint32_t v = bins[i];
        if (v && c < K) atomicAdd(hist + (int64_t)c * kPctBins + (i % kPctBins), v);
    }
}

__global__ void __launch_bounds__(256) pct_select_kernel(int32_t K, int pass, double q,
                                                         uint32_t* __restrict__ hist,
                                                         int32_t* __restrict__ sel,
                                                         float* __restrict__ score) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    uint32_t* hj = hist + (int64_t)j * kPctBins;
    if (pass == 0) {
        uint64_t T = 0;
        for (int b = 0; b < kPctBins; ++b) T += hj[b];
        int64_t r = (int64_t)ceil(q * (double)T);
        if (r > (int64_t)T) r = (int64_t)T;
        if (r < 1) r = 1;
        int h = 0;
        int64_t before = 0;
        if (T > 0) {
            for (h = 0; h < kPctBins; ++h) {
                if (before + (int64_t)hj[h] >= r) break;
                before += hj[h];
            }
        }
        sel[2 * j] = T > 0 ? h : 0;
        sel[2 * j + 1] = T > 0 ? (int32_t)(r - before) : 0;
        for (int b = 0; b < kPctBins; ++b) hj[b] = 0;
    } else {
        const int h = sel[2 * j];
        const int64_t r = sel[2 * j + 1];
        float v = 0.0f;
        if (r > 0) {
            int64_t before = 0;
            int l = 0;
            for (l = 0; l < 128; ++l) {
                if (before + (int64_t)hj[l] >= r) break;
                before += hj[l];
            }
            // l == 128: the passes saw different rows (undefined input): NaN
            v = l < 128 ? __uint_as_float((uint32_t)((h << 7) | l) << 16) : __uint_as_float(0x7FC00000u);
        }
        score[j] = v;
    }
}

__global__ void pct_zero_kernel(uint32_t* __restrict__ hist, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        hist[i] = 0;
}

}  // namespace

hipError_t launch_pct_reset(uint32_t* hist, int32_t K, hipStream_t st) {
    const int64_t n = (int64_t)K * kPctBins;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(pct_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, hist, n);
    return hipGetLastError();
}

hipError_t launch_pct_count(const uint16_t* X, int64_t M, int32_t K, int pass, const int32_t* sel, uint32_t* hist,
                            hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int gx = (K + kPctCh - 1) / kPctCh;
    // about 4 workgroups per CU (64 KB of LDS each), row chunks of at least 64 rows
    int64_t gy = ((int64_t)device_cu_count() * 4 + gx - 1) / gx;
    int64_t max_gy = (M + 63) / 64;
    if (gy > max_gy) gy = max_gy;
    if (gy < 1) gy = 1;
    if (gy > 65535) gy = 65535;
    const int64_t rows = (M + gy - 1) / gy;
    gy = (M + rows - 1) / rows;
    hipLaunchKernelGGL(pct_count_kernel, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, X, M, K, rows, pass,
                       sel, hist);
    return hipGetLastError();
}

hipError_t launch_pct_select(int32_t K, int pass, double q, uint32_t* hist, int32_t* sel, float* score,
                             hipStream_t st) {
    hipLaunchKernelGGL(pct_select_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, K, pass, q, hist, sel,
                       score);
    return hipGetLastError();
}

}  // namespace mg
