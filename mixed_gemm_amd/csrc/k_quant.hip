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
// step, the loads of the next step issued before the current one is
// processed.  The per-channel s, RN(1/s) and outlier masks of a lane's 8
// channels stay in registers for all of its rows.
//
// With GELU, X is the previous projection's bf16 output and the quantized
// input is h = gelu_bf16(X) (the FFN block's hidden activation), computed
// in registers with the GELU kernel's own code: one pass instead of a GELU
// pass that writes h and a quantize pass that reads it back.
//
// bf16 input: the quotient comes from Markstein's correction of x * RN(1/s),
// exact when every x of the lane's row lies in {0} or [2^-100, 2^100]; that
// range is checked on the raw bf16 bits, two channels per 16-bit-lane
// integer instruction.  Rows of a lane that fail it, and f32 input, use the
// correctly rounded division.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int RPI = 1;            // rows per step
constexpr int WAVES_PER_CU = 32;  // launch size: about this many waves per CU

// |x| bit patterns of bf16 2^-100 and 2^100 (biased exponents 27 and 227)
constexpr unsigned short kBf16Lo = 0x0D80, kBf16Hi = 0x7180;

__device__ __forceinline__ float quad_max(float v) {
    // max over the 4 lanes of a quad (one 32-block): quad_perm [1,0,3,2] then [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return v;
}

// Every bf16 of the four words is 0 or has 2^-100 <= |x| <= 2^100.
__device__ __forceinline__ bool bf16x8_in_fast_range(const u32x4& w) {
    u16x2 hi = {0, 0}, lo = {0xFFFF, 0xFFFF};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u16x2 a = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
        hi = __builtin_elementwise_max(hi, a);
        lo = __builtin_elementwise_min(lo, a - (u16x2){1, 1});      // 0 wraps to 0xFFFF
    }
    const unsigned short h = hi[0] > hi[1] ? hi[0] : hi[1];
    const unsigned short l = lo[0] < lo[1] ? lo[0] : lo[1];
    return h <= kBf16Hi && l >= (unsigned short)(kBf16Lo - 1);
}

// E8M0 scale + E2M1 codes of the lane's 8 (masked) quotients; stores the
// packed nibbles and, from one lane per quad, the block's scale byte.
__device__ __forceinline__ void encode_store(const float (&q)[8], int lane, bool valid, uint8_t* aq_row,
                                             uint8_t* as_row, int j0) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(q[i]));
    amax = quad_max(amax);
    const uint32_t c = e8m0_from_amax_bits(__float_as_uint(amax));
    const float scale = e8m0_to_f32(c);
    uint32_t word = 0;
    MG_CVT_FP4X2(word, q[0], q[1], scale, 0);
    MG_CVT_FP4X2(word, q[2], q[3], scale, 1);
    MG_CVT_FP4X2(word, q[4], q[5], scale, 2);
    MG_CVT_FP4X2(word, q[6], q[7], scale, 3);
    if (valid) {
        *reinterpret_cast<uint32_t*>(aq_row + j0 / 2) = word;
        if ((lane & 3) == 0) as_row[j0 / 32] = (uint8_t)c;
    }
}

template <bool GELU>
__global__ void __launch_bounds__(256) quant_bf16_kernel(const uint16_t* __restrict__ X, int64_t M, int32_t K,
                                                         int32_t k, const float* __restrict__ s,
                                                         const float* __restrict__ rcp,
                                                         const int32_t* __restrict__ pos,
                                                         uint8_t* __restrict__ Aq, uint8_t* __restrict__ As,
                                                         uint16_t* __restrict__ XO) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int j0 = (blockIdx.x * 64 + lane) * 8;
    // Whole 32-blocks are either in range or not (K % 32 == 0), so the 4 lanes
    // of a quad agree on `valid` and the quad reduction mixes one block only.
    const bool valid = j0 < K;
    // s, RN(1/s) and pos of the block's 512 channels in LDS, for the lanes
    // that hold more than one outlier channel (their further channels are
    // looked up per row; keeping all 8 positions in registers would cost
    // occupancy).
    __shared__ float t_s[512], t_r[512];
    __shared__ int t_p[512];
    for (int t = threadIdx.x; t < 512; t += 256) {
        const int j = blockIdx.x * 512 + t;
        t_s[t] = j < K ? s[j] : 1.0f;
        t_r[t] = j < K ? rcp[j] : 1.0f;
        t_p[t] = j < K ? pos[j] : -1;
    }
    __syncthreads();
    // the lane's 8 channels: three pairs of 16-byte loads (j0 is a multiple of 8)
    float sv[8] = {1, 1, 1, 1, 1, 1, 1, 1}, rv[8] = {1, 1, 1, 1, 1, 1, 1, 1};
    int pv[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
    if (valid) {
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
            const float4 a = *reinterpret_cast<const float4*>(s + j0 + 4 * h4);
            const float4 b = *reinterpret_cast<const float4*>(rcp + j0 + 4 * h4);
            const int4 c = *reinterpret_cast<const int4*>(pos + j0 + 4 * h4);
            sv[4 * h4] = a.x; sv[4 * h4 + 1] = a.y; sv[4 * h4 + 2] = a.z; sv[4 * h4 + 3] = a.w;
            rv[4 * h4] = b.x; rv[4 * h4 + 1] = b.y; rv[4 * h4 + 2] = b.z; rv[4 * h4 + 3] = b.w;
            pv[4 * h4] = c.x; pv[4 * h4 + 1] = c.y; pv[4 * h4 + 2] = c.z; pv[4 * h4 + 3] = c.w;
        }
    }
    uint32_t omask = 0;
    bool s_ok = true;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        omask |= (pv[i] >= 0 ? 1u : 0u) << i;
        s_ok &= div_fast_ok_s(sv[i]);
    }
    // keep masks of the input words (outlier channels -> +0 in the bulk)
    uint32_t keepw[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
        keepw[w] = ((omask >> (2 * w)) & 1u ? 0u : 0x0000FFFFu) | ((omask >> (2 * w + 1)) & 1u ? 0u : 0xFFFF0000u);
    // The first outlier channel of the lane (if any) is written with one store
    // per row; further outlier channels of the same lane take one more store each.
    const int oc0 = omask ? __builtin_ctz(omask) : 0;
    float so = sv[0], ro = rv[0];
    int op0 = pv[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) {
        so = oc0 == i ? sv[i] : so;
        ro = oc0 == i ? rv[i] : ro;
        op0 = oc0 == i ? pv[i] : op0;
    }
    const uint32_t omask_rest = omask & (omask - 1);

    const int64_t rstride = (int64_t)gridDim.y * kWaves;
    const int64_t rstep = rstride * RPI;
    auto load_rows = [&](int64_t rb, u32x4 (&d)[RPI]) {
#pragma unroll
        for (int u = 0; u < RPI; ++u) {
            const int64_t r = rb + u * rstride;
            d[u] = u32x4{0, 0, 0, 0};
            if (valid && r < M)
                d[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(X + r * K + j0));
        }
    };

    int64_t r0 = (int64_t)blockIdx.y * kWaves + wave;
    u32x4 cur[RPI];
    load_rows(r0, cur);
    for (; r0 < M; r0 += rstep) {
        u32x4 nxt[RPI];
        load_rows(r0 + rstep, nxt);                     // next step's rows in flight meanwhile
#pragma unroll
        for (int u = 0; u < RPI; ++u) {
            const int64_t r = r0 + u * rstride;
            if (r >= M) break;                          // uniform across the wave
            u32x4 w = cur[u];
            if constexpr (GELU) {
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = gelu_bf16(w[i] & 0xFFFFu) | (gelu_bf16(w[i] >> 16) << 16);
            }
            const bool fast = s_ok && bf16x8_in_fast_range(w);
            float x[8], q[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint32_t m = w[i] & keepw[i];
                x[2 * i] = __uint_as_float(m << 16);
                x[2 * i + 1] = __uint_as_float(m & 0xFFFF0000u);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) q[i] = div_fast(x[i], sv[i], rv[i]);
            if (!fast) {
#pragma unroll
                for (int i = 0; i < 8; ++i) q[i] = __fdiv_rn(x[i], sv[i]);
            }
            if (omask) {
                // the outlier channel's own (unmasked) value from the raw words
                uint32_t wo = w[0];
#pragma unroll
                for (int i = 1; i < 4; ++i) wo = (oc0 >> 1) == i ? w[i] : wo;
                const float xo = __uint_as_float((oc0 & 1) ? (wo & 0xFFFF0000u) : (wo << 16));
                const float qo = fast ? div_fast(xo, so, ro) : __fdiv_rn(xo, so);
                XO[r * k + op0] = (uint16_t)f32_to_bf16_rne(qo);
                // further outlier channels of the lane (two or more in its 8)
                for (uint32_t mm = omask_rest; mm; mm &= mm - 1) {
                    const int i = __builtin_ctz(mm);
                    const int jl = lane * 8 + i;
                    const uint32_t wi = w[i >> 1];
                    const float xi = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                    const float si = t_s[jl];
                    const float qi = fast ? div_fast(xi, si, t_r[jl]) : __fdiv_rn(xi, si);
                    XO[r * k + t_p[jl]] = (uint16_t)f32_to_bf16_rne(qi);
                }
            }
            encode_store(q, lane, valid, Aq + r * (K / 2), As + r * (K / 32), j0);
        }
#pragma unroll
        for (int u = 0; u < RPI; ++u) cur[u] = nxt[u];
    }
}

// f32 input (the small f32 layer): correctly rounded division throughout.
__global__ void __launch_bounds__(256) quant_f32_kernel(const float* __restrict__ X, int64_t M, int32_t K,
                                                        int32_t k, const float* __restrict__ s,
                                                        const int32_t* __restrict__ pos,
                                                        uint8_t* __restrict__ Aq, uint8_t* __restrict__ As,
                                                        uint16_t* __restrict__ XO) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int j0 = (blockIdx.x * 64 + lane) * 8;
    const bool valid = j0 < K;
    float sv[8];
    int pv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        sv[i] = valid ? s[j0 + i] : 1.0f;
        pv[i] = valid ? pos[j0 + i] : -1;
    }
    const int64_t rstride = (int64_t)gridDim.y * kWaves;
    for (int64_t r = (int64_t)blockIdx.y * kWaves + wave; r < M; r += rstride) {
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = valid ? X[r * K + j0 + i] : 0.0f;
            q[i] = __fdiv_rn(x, sv[i]);
            if (pv[i] >= 0) {
                XO[r * k + pv[i]] = (uint16_t)f32_to_bf16_rne(q[i]);
                q[i] = 0.0f;
            }
        }
        encode_store(q, lane, valid, Aq + r * (K / 2), As + r * (K / 32), j0);
    }
}

}  // namespace

hipError_t launch_quant(const void* X, int32_t dtype, int64_t M, int32_t K, int32_t k,
                        const float* s, const float* rcp, const int32_t* pos, uint8_t* Aq,
                        uint8_t* As, uint16_t* XO, hipStream_t st, bool gelu) {
    if (M <= 0) return hipSuccess;
    const int64_t gx = ((int64_t)K / 8 + 63) / 64;
    // about WAVES_PER_CU waves per CU, each wave at least RPI rows
    int64_t gy = (M + kWaves * RPI - 1) / (kWaves * RPI);
    int64_t cap = (int64_t)device_cu_count() * (WAVES_PER_CU / kWaves) / gx;
    if (cap < 1) cap = 1;
    if (gy > cap) gy = cap;
    if (gy > 65535) gy = 65535;
    dim3 grid((unsigned)gx, (unsigned)gy);
    if (dtype == MG_BF16 && gelu)
        hipLaunchKernelGGL(quant_bf16_kernel<true>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X), M, K, k,
                           s, rcp, pos, Aq, As, XO);
    else if (dtype == MG_BF16)
        hipLaunchKernelGGL(quant_bf16_kernel<false>, grid, dim3(256), 0, st, static_cast<const uint16_t*>(X), M, K,
                           k, s, rcp, pos, Aq, As, XO);
    else
        hipLaunchKernelGGL(quant_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(X), M, K, k, s, pos,
                           Aq, As, XO);
    return hipGetLastError();
}

}  // namespace mg
