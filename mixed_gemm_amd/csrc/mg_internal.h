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
// is 4 KB of contiguous memory -- the unit the GEMM copies into LDS.  Inside
// a row the even blocks come first, then the odd ones (block b of the window
// at byte 8 (b % 2) + b / 2), so a matrix-core lane, which takes either the
// even or the odd 32-block of each 64-wide K step, finds its codes in 8
// consecutive bytes.  Byte (row, block) sits at ((row / 256) * nwin + block /
// 16) * 4096 + (row % 256) * 16 + 8 (block % 2) + (block % 16) / 2 with nwin
// = ceil(K / 512); the layout depends on K only.  Blocks past K / 32 and rows
// past the last row of the final 256-row group hold code 0, the code of an
// all-zero block.
constexpr int kScRows = 256;      // rows per window
constexpr int kScBlocks = 16;     // 32-blocks per window row
constexpr int kScWinBytes = kScRows * kScBlocks;
__host__ __device__ constexpr int64_t sc_nwin(int32_t K) { return ((int64_t)K + 511) / 512; }
__host__ __device__ constexpr int64_t sc_bytes(int64_t rows, int32_t K) {
    return (rows + kScRows - 1) / kScRows * sc_nwin(K) * kScWinBytes;
}
// Fragment order: the storage order of the GEMM operands Aq, Wq (row_bytes =
// K/2) and XO, WO (row_bytes = 2k).  A [rows][row_bytes] byte matrix is cut
// into blocks of 32 rows x 32 bytes (one 32x32x64 FP4 or 32x32x16 bf16
// matrix-core operand); block (row group g = r / 32, slice c = byte / 32)
// is 1024 contiguous bytes at (g * ns + c) * 1024, ns = 2 ceil(row_bytes /
// 64) (an even number of slices: the GEMM moves two per step), and inside it
// byte b of row r's slice sits at 16 * (r % 32 + 32 * (b / 16)) + b % 16 --
// the byte lane l = r % 32 + 32 * (b / 16) of the instruction holds at
// position b % 16.  Rows up to the next multiple of 32 and bytes up to ns *
// 32 are pads holding 0.
constexpr int kFragRows = 32;
constexpr int kFragSliceBytes = 32;
constexpr int kFragBlock = kFragRows * kFragSliceBytes;
__host__ __device__ constexpr int64_t frag_slices(int64_t row_bytes) { return (row_bytes + 63) / 64 * 2; }
__host__ __device__ constexpr int64_t frag_bytes(int64_t rows, int64_t row_bytes) {
    return (rows + 31) / 32 * frag_slices(row_bytes) * kFragBlock;
}
__host__ __device__ constexpr int64_t frag_offset(int64_t r, int64_t b, int64_t ns) {
    return ((r >> 5) * ns + (b >> 5)) * kFragBlock + (((r & 31) + ((b >> 4) & 1) * 32) << 4) + (b & 15);
}
// position of block b (0..15) inside a window row
__host__ __device__ constexpr int32_t sc_pos(int32_t b) { return 8 * (b & 1) + ((b & 15) >> 1); }
__host__ __device__ constexpr int64_t sc_offset(int64_t row, int32_t blk, int64_t nwin) {
    return ((row / kScRows) * nwin + blk / kScBlocks) * kScWinBytes + (row % kScRows) * kScBlocks + sc_pos(blk);
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
// launch_dual_gemm whose epilogue applies GELU to the bf16-rounded output and
// quantizes it as the input of the next layer (plan s2, rcp2, pos2, k2; its
// input width is N) into Aq2, As2, XO2, instead of writing Y.
hipError_t launch_dual_gemm_gelu_quant(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                                       const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                                       int32_t N, int32_t K, int32_t k, const float* s2, const float* rcp2,
                                       const int32_t* pos2, int32_t k2, uint8_t* Aq2, uint8_t* As2,
                                       uint16_t* XO2, hipStream_t st);
hipError_t launch_gelu(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t st);
hipError_t launch_pct_reset(uint32_t* hist, int32_t K, hipStream_t st);
hipError_t launch_pct_count(const uint16_t* X, int64_t M, int32_t K, int pass, const int32_t* sel, uint32_t* hist,
                            hipStream_t st);
hipError_t launch_pct_select(int32_t K, int pass, double q, uint32_t* hist, int32_t* sel, float* score,
                             hipStream_t st);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Workgroups of 256 threads of kernel `kern` that fit on one CU (registers,
// LDS), looked up once per device and kernel.
int blocks_per_cu(const void* kern);

// Every argument check of mg_forward except the activation workspace (plan,
// dtypes, M, X, Y, operand sizes); MG_OK or the error (message set).
int check_forward(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const void* Y, int32_t y_dtype);

// Sets the calling thread's mg_last_error() message (printf format) and
// returns code.
int fail_msg(int code, const char* fmt, ...);

}  // namespace mg
