// Dual-branch GEMM of the W4A4 layer, Eq. (5) of "W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B" (Eq. (3) with a static outlier set):
//   Y[m][n] = bf16_RNE( sum_b 2^(As[m][b]-127) 2^(Ws[n][b]-127) sum_{j in b} e2m1(Aq[m][j]) e2m1(Wq[n][j])
//                       + sum_i XO[m][i] WO[n][i] )
// The bulk runs on the gfx950 block-scaled FP4 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with E2M1 operands and one E8M0 scale per
// 32 K per row/column); the outlier branch runs on the BF16 matrix cores
// (v_mfma_f32_32x32x16_bf16) into the SAME fp32 accumulators; one RNE to bf16
// at the end.
//
// Operand layouts of both instructions (32x32 output, wave64):
//   A (src0): lane l holds row l%32 and the K range [half*KH, half*KH + KH) of
//             the instruction's K, half = l/32 (KH = 32 FP4 values = 16 bytes,
//             or 8 bf16 = 16 bytes);
//   B (src1): lane l holds column l%32 and the same K range;
//   E8M0 scale of lane l: the 32-block of its K range, byte 0 of the operand;
//   D: lane l, register r holds row 8*(r/4) + 4*(l/32) + r%4, column l%32.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

__device__ __forceinline__ v16f mfma_fp4(uint4 a, uint4 b, int sa, int sb, v16f c) {
    v8i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
    v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, 0, sa, 0, sb);
}

__device__ __forceinline__ v16f mfma_bf16(uint4 a, uint4 b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ void store_out(uint16_t* p, float v) { *p = (uint16_t)f32_to_bf16_rne(v); }
__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }

// 8 bf16 of a row starting at column i0 of a [rows][k] array, zero past k.
__device__ __forceinline__ uint4 load_bf16x8(const uint16_t* __restrict__ row, int i0, int k) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = i0 + 2 * e;
        const uint32_t lo = i < k ? row[i] : 0u;
        const uint32_t hi = i + 1 < k ? row[i + 1] : 0u;
        w[e] = lo | (hi << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// Straightforward kernel: one wave per 32x32 output tile, operands straight
// from global memory.  Used for small problems and as the cross-check of the
// tiled kernel.
template <typename OutT>
__global__ void __launch_bounds__(256) dual_gemm_simple(const uint8_t* __restrict__ Aq,
                                                        const uint8_t* __restrict__ As,
                                                        const uint16_t* __restrict__ XO,
                                                        const uint8_t* __restrict__ Wq,
                                                        const uint8_t* __restrict__ Ws,
                                                        const uint16_t* __restrict__ WO, int64_t M,
                                                        int32_t N, int32_t K, int32_t k,
                                                        OutT* __restrict__ Y) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t m0 = (int64_t)blockIdx.y * 64 + (wave >> 1) * 32;
    const int64_t n0 = (int64_t)blockIdx.x * 64 + (wave & 1) * 32;
    if (n0 >= N || m0 >= M) return;
    const int half = lane >> 5;
    const int64_t row = min(m0 + (lane & 31), M - 1);
    const int64_t col = n0 + (lane & 31);
    const int nb = K / 32;
    v16f acc = {};
    for (int kk = 0; kk < K; kk += 64) {
        const int kb = kk / 32 + half;          // this lane's 32-block
        uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
        int sa = 127, sb = 127;
        if (kb < nb) {
            a = *reinterpret_cast<const uint4*>(Aq + row * (K / 2) + kb * 16);
            b = *reinterpret_cast<const uint4*>(Wq + col * (K / 2) + kb * 16);
            sa = As[row * nb + kb];
            sb = Ws[col * nb + kb];
        }
        acc = mfma_fp4(a, b, sa, sb, acc);
    }
    for (int kk = 0; kk < k; kk += 16) {
        const uint4 a = load_bf16x8(XO + row * k, kk + 8 * half, k);
        const uint4 b = load_bf16x8(WO + col * k, kk + 8 * half, k);
        acc = mfma_bf16(a, b, acc);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int64_t m = m0 + 8 * (r / 4) + 4 * half + (r % 4);
        if (m < M) store_out(Y + m * N + col, acc[r]);
    }
}

}  // namespace

hipError_t launch_dual_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                            const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                            int32_t N, int32_t K, int32_t k, void* Y, int32_t y_dtype,
                            hipStream_t st) {
    if (M <= 0) return hipSuccess;
    dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
    if (y_dtype == MG_BF16)
        hipLaunchKernelGGL(dual_gemm_simple<uint16_t>, grid, dim3(256), 0, st, Aq, As, XO, Wq, Ws, WO, M, N, K, k,
                           static_cast<uint16_t*>(Y));
    else
        hipLaunchKernelGGL(dual_gemm_simple<float>, grid, dim3(256), 0, st, Aq, As, XO, Wq, Ws, WO, M, N, K, k,
                           static_cast<float*>(Y));
    return hipGetLastError();
}

}  // namespace mg
