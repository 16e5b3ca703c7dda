// Internal launcher interface between the C ABI (mg_api.hip) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mixed_gemm.h"

namespace mg {

// Largest supported input width (LDS-resident per-channel tables in the plan kernels).
constexpr int32_t kMaxK = 65536;

// Storage order of the E8M0 scale codes of Aq (As) and Wq (Ws): windows of
// 256 rows x 16 blocks (512 channels), 16 bytes per row, so that one window
// is 4 KB of contiguous memory -- the unit the GEMM copies into LDS.  Byte
// (row, block) sits at ((row / 256) * nwin + block / 16) * 4096 +
// (row % 256) * 16 + block % 16 with nwin = ceil(K / 512); the layout depends
// on K only.  Blocks past K / 32 and rows past the last row of the final
// 256-row group hold code 0, the code of an all-zero block.
constexpr int kScRows = 256;      // rows per window
constexpr int kScBlocks = 16;     // 32-blocks per window row
constexpr int kScWinBytes = kScRows * kScBlocks;
__host__ __device__ constexpr int64_t sc_nwin(int32_t K) { return ((int64_t)K + 511) / 512; }
__host__ __device__ constexpr int64_t sc_bytes(int64_t rows, int32_t K) {
    return (rows + kScRows - 1) / kScRows * sc_nwin(K) * kScWinBytes;
}
// Row stride (in bf16 values) of the outlier operands XO [M][kp] and WO
// [N][kp]: k rounded up to a multiple of 8, so every row starts 16-byte
// aligned; the pad columns k .. kp-1 hold +0.
__host__ __device__ constexpr int32_t xo_cols(int32_t k) { return (k + 7) & ~7; }
__host__ __device__ constexpr int64_t sc_offset(int64_t row, int32_t blk, int64_t nwin) {
    return ((row / kScRows) * nwin + blk / kScBlocks) * kScWinBytes + (row % kScRows) * kScBlocks + blk % kScBlocks;
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, int64_t n, hipStream_t st);
hipError_t launch_colmax(const void* X, int32_t dtype, int64_t R, int32_t K, float* out,
                         hipStream_t st);
hipError_t launch_smooth(const float* a, const float* w, int32_t K, double alpha, int32_t smooth,
                         float* s, float* rcp, hipStream_t st);
// s == nullptr: rank a_j; otherwise rank RN(a_j / s_j)
hipError_t launch_topk(const float* a, const float* s, int32_t K, int32_t k, int32_t* O, int32_t* pos,
                       hipStream_t st);
hipError_t launch_fold_pack(const void* W, int32_t dtype, int32_t N, int32_t K, int32_t k,
                            int32_t layout, const float* s, const int32_t* pos, uint8_t* Wq,
                            uint8_t* Ws, uint8_t* Wst, uint16_t* WO, hipStream_t st);
hipError_t launch_quant(const void* X, int32_t dtype, int64_t M, int32_t K, int32_t k,
                        const float* s, const float* rcp, const int32_t* pos, uint8_t* Aq,
                        uint8_t* As, uint16_t* XO, hipStream_t st, bool gelu = false,
                        float* amax = nullptr);
hipError_t launch_dual_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                            const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                            int32_t N, int32_t K, int32_t k, void* Y, int32_t y_dtype,
                            hipStream_t st);
hipError_t launch_gelu(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t st);
hipError_t launch_pct_reset(uint32_t* hist, int32_t K, hipStream_t st);
hipError_t launch_pct_count(const uint16_t* X, int64_t M, int32_t K, int pass, const int32_t* sel, uint32_t* hist,
                            hipStream_t st);
hipError_t launch_pct_select(int32_t K, int pass, double q, uint32_t* hist, int32_t* sel, float* score,
                             hipStream_t st);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Every argument check of mg_forward except the activation workspace (plan,
// dtypes, M, X, Y, operand sizes); MG_OK or the error (message set).
int check_forward(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const void* Y, int32_t y_dtype);

// Sets the calling thread's mg_last_error() message (printf format) and
// returns code.
int fail_msg(int code, const char* fmt, ...);

}  // namespace mg
