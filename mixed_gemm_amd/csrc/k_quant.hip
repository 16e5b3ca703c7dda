// Runtime activation path of the W4A4 layer ("W4A4 Quantization for Inference
// on Wan2.2-I2V-A14B": the integration paragraph -- activations divided by s,
// quantized to 4 bits and routed to the bulk or the narrow high-precision
// branch -- and Eq. (5)'s split of the input channels into J and O).
//
// One fused HBM-bound pass over X [M][K]:
//   q = RN_f32(x / s_j)                      exact IEEE quotient
//   XO[m][pos_j] = bf16_RNE(q)               for the k outlier channels
//   q := +0 on outlier channels              (masked in place, 32-alignment kept)
//   As[m][b] = E8M0(amax of q over block b)  1x32 blocks along K
//   Aq[m][j/2] nibble = E2M1_RNE(q / 2^(As-127))
//
// Lane layout: a lane owns 8 consecutive channels (16 B of bf16) of a row, 4
// lanes form one 32-block (amax combined with two quad DPP moves), a wave
// covers 512 channels of a row and walks rows with a stride, RPI rows per
// iteration so several 16-byte loads per lane are in flight.  The per-channel
// s, RN(1/s), outlier positions and keep-masks of a lane's 8 channels stay in
// registers for all of its rows.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int RPI = 4;   // rows per loop iteration

__device__ __forceinline__ float quad_max(float v) {
    // max over the 4 lanes of a quad (one 32-block): quad_perm [1,0,3,2] then [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return v;
}

template <bool BF16>
__global__ void __launch_bounds__(256) quant_kernel(const void* __restrict__ X, int64_t M, int32_t K, int32_t k,
                                                    const float* __restrict__ s,
                                                    const float* __restrict__ rcp,
                                                    const int32_t* __restrict__ pos,
                                                    uint8_t* __restrict__ Aq, uint8_t* __restrict__ As,
                                                    uint16_t* __restrict__ XO) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t chunk = (int64_t)blockIdx.x * 64 + lane;
    const int j0 = (int)(chunk * 8);
    // Whole 32-blocks are either in range or not (K % 32 == 0), so the 4 lanes
    // of a quad agree on `valid` and the quad reduction mixes one block only.
    const bool valid = j0 < K;
    float sv[8], rv[8];
    uint32_t keep[8];
    uint32_t omask = 0;
    bool s_ok = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sv[i] = valid ? s[j0 + i] : 1.0f;
        rv[i] = valid ? rcp[j0 + i] : 1.0f;
        const int p = valid ? pos[j0 + i] : -1;
        keep[i] = p >= 0 ? 0u : 0xFFFFFFFFu;
        omask |= (p >= 0 ? 1u : 0u) << i;
        s_ok &= div_fast_ok_s(sv[i]);
    }
    // The first outlier channel of the lane (if any) is written with one store
    // per row; further outlier channels of the same lane (rare) take a loop.
    const int oc0 = omask ? __builtin_ctz(omask) : 8;
    const int64_t op0 = oc0 < 8 ? (int64_t)pos[j0 + oc0] : 0;
    const uint32_t omask_rest = omask & (omask - 1);
    const int64_t rstride = (int64_t)gridDim.y * kWaves;
    const int64_t ld = K;                                     // row stride of X in elements
    for (int64_t r0 = (int64_t)blockIdx.y * kWaves + wave; r0 < M; r0 += rstride * RPI) {
        float xin[RPI][8];
#pragma unroll
        for (int u = 0; u < RPI; ++u) {
            const int64_t r = r0 + u * rstride;
            if (valid && r < M) {
                if constexpr (BF16) {
                    const u32x4 d = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                        reinterpret_cast<const uint16_t*>(X) + r * ld + j0));
                    const uint32_t wd[4] = {d[0], d[1], d[2], d[3]};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        xin[u][2 * i] = __uint_as_float(wd[i] << 16);
                        xin[u][2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
                    }
                } else {
                    const float4* src = reinterpret_cast<const float4*>(
                        reinterpret_cast<const float*>(X) + r * ld + j0);
                    const float4 d0 = src[0], d1 = src[1];
                    xin[u][0] = d0.x; xin[u][1] = d0.y; xin[u][2] = d0.z; xin[u][3] = d0.w;
                    xin[u][4] = d1.x; xin[u][5] = d1.y; xin[u][6] = d1.z; xin[u][7] = d1.w;
                }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) xin[u][i] = 0.0f;
            }
        }
#pragma unroll
        for (int u = 0; u < RPI; ++u) {
            const int64_t r = r0 + u * rstride;
            if (r >= M) break;                              // uniform across the wave
            float q[8];
            bool fast = BF16 && s_ok;
            if (BF16) {
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    q[i] = div_fast(xin[u][i], sv[i], rv[i]);
                    fast &= div_fast_ok_x(xin[u][i]);
                }
            }
            if (!fast) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = __fdiv_rn(xin[u][i], sv[i]);
            }
            if (omask) {
                float qo = q[0];
#pragma unroll
                for (int i = 1; i < 8; ++i) qo = oc0 == i ? q[i] : qo;
                XO[r * k + op0] = (uint16_t)f32_to_bf16_rne(qo);
                for (uint32_t m = omask_rest; m; m &= m - 1) {
                    const int i = __builtin_ctz(m);
                    float qi = q[0];
#pragma unroll
                    for (int t = 1; t < 8; ++t) qi = i == t ? q[t] : qi;
                    XO[r * k + pos[j0 + i]] = (uint16_t)f32_to_bf16_rne(qi);
                }
            }
            float amax = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                q[i] = __uint_as_float(__float_as_uint(q[i]) & keep[i]);   // outliers -> +0
                amax = fmaxf(amax, __builtin_fabsf(q[i]));
            }
            amax = quad_max(amax);
            const uint32_t c = e8m0_from_amax_bits(__float_as_uint(amax));
            const float scale = e8m0_to_f32(c);
            uint32_t word = 0;
            MG_CVT_FP4X2(word, q[0], q[1], scale, 0);
            MG_CVT_FP4X2(word, q[2], q[3], scale, 1);
            MG_CVT_FP4X2(word, q[4], q[5], scale, 2);
            MG_CVT_FP4X2(word, q[6], q[7], scale, 3);
            if (valid) {
                *reinterpret_cast<uint32_t*>(Aq + r * (K / 2) + j0 / 2) = word;
                if ((lane & 3) == 0) As[r * (K / 32) + j0 / 32] = (uint8_t)c;
            }
        }
    }
}

}  // namespace

hipError_t launch_quant(const void* X, int32_t dtype, int64_t M, int32_t K, int32_t k,
                        const float* s, const float* rcp, const int32_t* pos, uint8_t* Aq,
                        uint8_t* As, uint16_t* XO, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    const int64_t gx = ((int64_t)K / 8 + 63) / 64;
    // ~16 waves per CU, each wave at least RPI rows.
    int64_t gy = (M + kWaves * RPI - 1) / (kWaves * RPI);
    int64_t cap = (int64_t)device_cu_count() * 4 / gx;
    if (cap < 1) cap = 1;
    if (gy > cap) gy = cap;
    if (gy > 65535) gy = 65535;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (dtype == MG_BF16)
        hipLaunchKernelGGL(quant_kernel<true>, grid, dim3(256), 0, st, X, M, K, k, s, rcp, pos, Aq, As, XO);
    else
        hipLaunchKernelGGL(quant_kernel<false>, grid, dim3(256), 0, st, X, M, K, k, s, rcp, pos, Aq, As, XO);
    return hipGetLastError();
}

}  // namespace mg
