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
// Counting: a workgroup takes 64 channels (128 B of each row, a whole cache
// line: a lane loads 8 channels, 8 lanes a row piece, 32 rows per step, 4
// rows in flight per lane) over a chunk of at most 65535 rows and counts into
// 64 x 256 16-bit LDS counters (two channels per 32-bit word) with LDS
// atomics, then adds its non-zero bins into the global [K][256] histogram.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

constexpr int kPctCh = 64;        // channels per workgroup: 128 bytes of a bf16 row, one cache line
constexpr int kPctBins = 256;
constexpr int kPctStride = 257;   // LDS words per channel pair: equal bins of different pairs in different banks
constexpr int kPctUnroll = 4;     // rows in flight per thread
constexpr int64_t kPctMaxRows = 65535;   // rows per workgroup chunk: a 16-bit counter cannot overflow

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Halfword e (0..7) of a 16-byte word.
__device__ __forceinline__ uint32_t half_of(const u32x4& w, int e) {
    const uint32_t d = (e & 4) ? ((e & 2) ? w[3] : w[2]) : ((e & 2) ? w[1] : w[0]);
    return (e & 1) ? (d >> 16) : (d & 0xFFFFu);
}

__global__ void __launch_bounds__(256) pct_count_kernel(const uint16_t* __restrict__ X, int64_t M, int32_t K,
                                                        int64_t rows_per_chunk, int pass,
                                                        const int32_t* __restrict__ sel,
                                                        uint32_t* __restrict__ hist) {
    // bins of channel c (of the workgroup's 64) are the 16-bit half c / 32 of
    // words (c % 32) * 257 + bin: two channels share a word, which keeps the
    // histograms of 64 channels in 33 KB
    __shared__ uint32_t bins[(kPctCh / 2) * kPctStride];
    const int t = threadIdx.x;
    for (int i = t; i < (kPctCh / 2) * kPctStride; i += 256) bins[i] = 0;
    // a thread owns 8 consecutive channels (16 bytes of a row) and rows
    // rho, rho + 32, ...; it visits its channels starting at rho % 8, so the
    // lanes of a wave that share channels mostly update different channels
    const int g = t & 7, rho = t >> 3;
    const int c0 = blockIdx.x * kPctCh + 8 * g;        // K % 32 == 0: all 8 in range or none
    const bool valid = c0 < K;
    const uint32_t inc = g >= 4 ? 0x10000u : 1u;       // the counter half of this thread's channels
    int hsel[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) hsel[e] = (pass == 1 && valid) ? sel[2 * (c0 + e)] : -1;
    __syncthreads();
    const int64_t r_begin = (int64_t)blockIdx.y * rows_per_chunk;
    const int64_t r_end = r_begin + rows_per_chunk < M ? r_begin + rows_per_chunk : M;
    uint32_t* bg = bins + 8 * (g & 3) * kPctStride;
    if (valid) {
        for (int64_t r0 = r_begin + rho; r0 < r_end; r0 += 32 * kPctUnroll) {
            u32x4 w[kPctUnroll];
#pragma unroll
            for (int u = 0; u < kPctUnroll; ++u) {
                const int64_t r = r0 + 32 * u;
                w[u] = r < r_end ? *reinterpret_cast<const u32x4*>(X + r * K + c0) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kPctUnroll; ++u) {
                if (r0 + 32 * u >= r_end) break;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int e = (i + rho + 4 * (g >> 2)) & 7;   // halves g and g + 4 share words: offset
                    const uint32_t a = half_of(w[u], e) & 0x7FFFu;
                    const uint32_t hi = a >> 7;
                    int h_e = hsel[0];
#pragma unroll
                    for (int f = 1; f < 8; ++f) h_e = e == f ? hsel[f] : h_e;
                    if (pass == 0)
                        atomicAdd(bg + e * kPctStride + hi, inc);
                    else if ((int)hi == h_e)
                        atomicAdd(bg + e * kPctStride + (a & 0x7Fu), inc);
                }
            }
        }
    }
    __syncthreads();
    for (int i = t; i < kPctCh * kPctBins; i += 256) {
        const int ch = i / kPctBins, b = i % kPctBins;
        const int c = blockIdx.x * kPctCh + ch;
        const uint32_t v = (bins[(ch & 31) * kPctStride + b] >> (16 * (ch >> 5))) & 0xFFFFu;
        if (v && c < K) atomicAdd(hist + (int64_t)c * kPctBins + b, v);
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
    // about 8 workgroups per CU (33 KB of LDS each), row chunks of at least 256
    // rows and at most kPctMaxRows (16-bit counters)
    int64_t gy = ((int64_t)device_cu_count() * 8 + gx - 1) / gx;
    int64_t max_gy = (M + 255) / 256;
    if (gy > max_gy) gy = max_gy;
    const int64_t min_gy = (M + kPctMaxRows - 1) / kPctMaxRows;
    if (gy < min_gy) gy = min_gy;
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
