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
// covers 512 channels of a row and walks rows with a stride, the next row's
// load issued before the current one is processed.  The per-channel s,
// RN(1/s) and outlier masks of a lane's 8 channels stay in registers for all
// of its rows.  Rows are read and written through buffer resources built per
// row in scalar registers, so channels past K need no per-lane bounds code.
// The codes As[m][b] are stored in scale windows of 256 rows x 16 blocks
// (sc_offset): a workgroup's 512 channels are one window, so a row's 16
// codes are 16 contiguous bytes; the rows run on to the end of the last
// 256-row group, whose pad rows (and the blocks past K) get code 0.
//
// With GELU, X is the previous projection's bf16 output and the quantized
// input is h = gelu_bf16x2 of X (the FFN block's hidden activation), computed
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
constexpr int WAVES_PER_CU = 32;  // launch size: about this many waves per CU

// |x| bit patterns of bf16 2^-100 and 2^100 (biased exponents 27 and 227)
constexpr unsigned short kBf16Lo = 0x0D80, kBf16Hi = 0x7180;

// Max over the 4 lanes of a quad (one 32-block: quad_perm [1,0,3,2] then
// [2,3,0,1]) of the bit patterns of non-negative f32 values, whose unsigned
// integer order is their numeric order.
__device__ __forceinline__ uint32_t quad_max_bits(uint32_t v) {
    v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));
    v = __builtin_elementwise_max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));
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

// E8M0 scale code c of the lane's 32-block and the packed E2M1 nibbles of its
// 8 (masked) quotients (first value in the low nibble).
__device__ __forceinline__ uint32_t encode8(const float (&q)[8], uint32_t& c) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, __builtin_fabsf(q[i]));
    c = e8m0_from_amax_bits(quad_max_bits(__float_as_uint(amax)));
    const float scale = e8m0_to_f32(c);
    uint32_t word = 0;
    MG_CVT_FP4X2(word, q[0], q[1], scale, 0);
    MG_CVT_FP4X2(word, q[2], q[3], scale, 1);
    MG_CVT_FP4X2(word, q[4], q[5], scale, 2);
    MG_CVT_FP4X2(word, q[6], q[7], scale, 3);
    return word;
}

// encode8, then the packed nibbles (lanes inside K, rows inside M) and, from
// one lane per quad, the block's scale byte into the row's 16 bytes of its
// scale window (every lane: past K or M the code of a zero block).
__device__ __forceinline__ void encode_store(const float (&q)[8], int lane, bool store_q, uint8_t* aq_row,
                                             uint8_t* as_win_row, int j0) {
    uint32_t c;
    const uint32_t word = encode8(q, c);
    if (store_q) *reinterpret_cast<uint32_t*>(aq_row + j0 / 2) = word;
    if ((lane & 3) == 0) as_win_row[lane >> 2] = (uint8_t)c;
}

template <bool GELU, bool STATS>
__global__ void __launch_bounds__(256) quant_bf16_kernel(const uint16_t* __restrict__ X, int64_t M, int32_t K,
                                                         int32_t k, const float* __restrict__ s,
                                                         const float* __restrict__ rcp,
                                                         const int32_t* __restrict__ pos,
                                                         uint8_t* __restrict__ Aq, uint8_t* __restrict__ As,
                                                         uint16_t* __restrict__ XO, uint32_t* __restrict__ amax) {
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
    __shared__ uint32_t t_m[512];    // STATS: the workgroup's per-channel max |x| (bf16 bits)
    for (int t = threadIdx.x; t < 512; t += 256) {
        const int j = blockIdx.x * 512 + t;
        t_s[t] = j < K ? s[j] : 1.0f;
        t_r[t] = j < K ? rcp[j] : 1.0f;
        t_p[t] = j < K ? pos[j] : -1;
        t_m[t] = 0;
    }
    __syncthreads();
    u16x2 mx[4] = {{0, 0}, {0, 0}, {0, 0}, {0, 0}};   // STATS: running max of the lane's |x| bit patterns
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

    // Per-lane byte offsets inside a row.  Rows are addressed through a buffer
    // resource per row (scalar registers), so lanes whose channels lie past
    // K read zeros and drop their stores by the hardware range check, and so
    // do the lanes that store no scale byte or no outlier value (offset
    // kNoStore).  The workgroup's 512 channels are one scale window: a row's
    // 16 scale bytes are contiguous, lane 4 i storing byte i (past K: the
    // code 0 of its all-zero block).
    constexpr uint32_t kNoStore = 0x40000000u;
    const uint32_t offX = 2u * (uint32_t)j0, offAq = (uint32_t)j0 / 2u;
    const uint32_t offAs = (lane & 3) == 0 ? (uint32_t)(lane >> 2) : kNoStore;
    const uint32_t offXO = omask ? 2u * (uint32_t)op0 : kNoStore;
    const bool wave_o = __builtin_amdgcn_ballot_w64(omask != 0) != 0;
    const bool wave_rest = __builtin_amdgcn_ballot_w64(omask_rest != 0) != 0;
    // XO rows are kp = xo_cols(k) values apart; the workgroup of channels
    // 0..511 writes the pad columns k .. kp-1 (+0), one per lane
    const int kp = xo_cols(k);
    const uint32_t rowX = 2u * (uint32_t)K, rowAq = (uint32_t)K / 2u, rowXO = 2u * (uint32_t)kp;
    const bool pad_wg = blockIdx.x == 0 && kp > k;
    const uint32_t offPad = lane < kp - k ? 2u * (uint32_t)(k + lane) : kNoStore;

    auto rsrc = [](const void* p, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
    };
    auto load_row = [&](const uint16_t* px, bool in) -> u32x4 {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(px, in ? rowX : 0u), offX, 0,
                                                                                2));   // nt
    };

    // one row: w its 8 bf16 per lane, pq/ps/po its Aq row, its 16 bytes of
    // the As window and its XO row; live: a row of X (else a pad row of the
    // last 256-row scale group, whose Aq and XO stores are dropped)
    auto process_row = [&](u32x4 w, uint8_t* pq, uint8_t* ps, uint16_t* po, bool live) {
        if constexpr (GELU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = gelu_bf16x2(w[i]);
        }
        if constexpr (STATS) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mx[i] = __builtin_elementwise_max(mx[i], __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
        }
        const bool fast = s_ok & bf16x8_in_fast_range(w);
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
        if (wave_o) {
            // the first outlier channel's own (unmasked) value from the raw words
            uint32_t wo = w[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) wo = (oc0 >> 1) == i ? w[i] : wo;
            const float xo = __uint_as_float((oc0 & 1) ? (wo & 0xFFFF0000u) : (wo << 16));
            const float qo = fast ? div_fast(xo, so, ro) : __fdiv_rn(xo, so);
            const __amdgpu_buffer_rsrc_t rxo = rsrc(po, live ? rowXO : 0u);
            if (omask) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qo), rxo, offXO, 0, 0);
            if (wave_rest) {
                // further outlier channels of the lane (two or more in its 8)
                for (uint32_t mm = omask_rest; mm; mm &= mm - 1) {
                    const int i = __builtin_ctz(mm);
                    const int jl = lane * 8 + i;
                    const uint32_t wi = w[i >> 1];
                    const float xi = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                    const float si = t_s[jl];
                    const float qi = fast ? div_fast(xi, si, t_r[jl]) : __fdiv_rn(xi, si);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qi), rxo, 2u * (uint32_t)t_p[jl],
                                                          0, 0);
                }
            }
        }
        uint32_t c;
        const uint32_t word = encode8(q, c);
        __builtin_amdgcn_raw_buffer_store_b32(word, rsrc(pq, live ? rowAq : 0u), offAq, 0, 0);
        if (pad_wg) __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rsrc(po, live ? rowXO : 0u), offPad, 0, 0);
        if ((lane & 3) == 0)
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)c, rsrc(ps, (uint32_t)kScBlocks), offAs, 0, 0);
    };

    // Rows r0, r0 + rstride, ...: the next row's load is in flight while the
    // current one is processed.  Row addresses advance by a fixed stride
    // (scalar adds).  The rows run on to the end of the last 256-row scale
    // group, so its pad rows get their zero codes.
    // The wave's row counts n (with pad rows) and nv (rows of X) are 32-bit
    // scalars (64-bit scalar compares do not exist on this architecture).
    const int64_t rstride = (int64_t)gridDim.y * kWaves;
    const int64_t r0 = (int64_t)blockIdx.y * kWaves + wave;
    const int64_t Mp = (M + kScRows - 1) / kScRows * kScRows;
    const int n = r0 < Mp ? (int)((Mp - 1 - r0) / rstride) + 1 : 0;
    const int nv = r0 < M ? (int)((M - 1 - r0) / rstride) + 1 : 0;
    const int64_t dX = rstride * K, dQ = rstride * (K / 2), dO = rstride * kp;
    const int64_t win_stride = sc_nwin(K) * kScWinBytes;     // bytes between 256-row groups of As
    static_assert(kScRows == 256, "row group = m >> 8");
    const uint16_t* px = X + r0 * K;
    uint8_t* pq = Aq + r0 * (K / 2);
    uint8_t* const asw = As + (int64_t)blockIdx.x * kScWinBytes;
    uint16_t* po = XO + r0 * kp;
    int64_t m = r0;
    u32x4 a = load_row(px, nv > 0);
    px += dX;
    for (int i = 0; i < n; ++i) {
        const u32x4 b = load_row(px, i + 1 < nv);
        px += dX;
        process_row(a, pq, asw + (m >> 8) * win_stride + (m & 255) * kScBlocks, po, i < nv);   // 256-row groups
        pq += dQ; po += dO; m += rstride;
        a = b;
    }
    if constexpr (STATS) {
        // the magnitudes' bit patterns order like the magnitudes: integer max, in LDS across the
        // workgroup's waves, then one global max per channel and workgroup (f32 bits = bf16 << 16)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            atomicMax(&t_m[lane * 8 + 2 * i], (uint32_t)mx[i][0]);
            atomicMax(&t_m[lane * 8 + 2 * i + 1], (uint32_t)mx[i][1]);
        }
        __syncthreads();
        for (int t = threadIdx.x; t < 512; t += 256) {
            const int j = blockIdx.x * 512 + t;
            if (j < K && t_m[t]) atomicMax(amax + j, t_m[t] << 16);
        }
    }
}

// f32 input (the small f32 layer): correctly rounded division throughout.
__global__ void __launch_bounds__(256) quant_f32_kernel(const float* __restrict__ X, int64_t M, int32_t K,
                                                        int32_t k, const float* __restrict__ s,
                                                        const int32_t* __restrict__ pos,
                                                        uint8_t* __restrict__ Aq, uint8_t* __restrict__ As,
                                                        uint16_t* __restrict__ XO, uint32_t* __restrict__ amax) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    float mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};       // amax != nullptr: running max |x| per channel
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
    const int64_t Mp = (M + kScRows - 1) / kScRows * kScRows;   // through the last scale group's pad rows
    const int64_t nwin = sc_nwin(K);
    const int kp = xo_cols(k);                                   // XO row stride; pads written below
    for (int64_t r = (int64_t)blockIdx.y * kWaves + wave; r < Mp; r += rstride) {
        const bool live = r < M;
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = valid && live ? X[r * K + j0 + i] : 0.0f;
            mx[i] = fmaxf(mx[i], __builtin_fabsf(x));
            q[i] = __fdiv_rn(x, sv[i]);
            if (pv[i] >= 0) {
                if (live) XO[r * kp + pv[i]] = (uint16_t)f32_to_bf16_rne(q[i]);
                q[i] = 0.0f;
            }
        }
        if (live && blockIdx.x == 0 && lane < kp - k) XO[r * kp + k + lane] = 0;
        encode_store(q, lane, valid && live, Aq + r * (K / 2),
                     As + sc_offset(r, (int32_t)blockIdx.x * kScBlocks, nwin), j0);
    }
    if (amax != nullptr && valid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) atomicMax(amax + j0 + i, __float_as_uint(mx[i]));
    }
}

}  // namespace

hipError_t launch_quant(const void* X, int32_t dtype, int64_t M, int32_t K, int32_t k,
                        const float* s, const float* rcp, const int32_t* pos, uint8_t* Aq,
                        uint8_t* As, uint16_t* XO, hipStream_t st, bool gelu, float* amax) {
    if (M <= 0) return hipSuccess;
    const int64_t gx = ((int64_t)K / 8 + 63) / 64;
    // about WAVES_PER_CU waves per CU, each wave at least one row
    int64_t gy = (M + kWaves - 1) / kWaves;
    // the statistics variant holds 7 waves per SIMD (more registers), the others 8
    const int waves_per_cu = amax ? 28 : WAVES_PER_CU;
    int64_t cap = (int64_t)device_cu_count() * (waves_per_cu / kWaves) / gx;
    if (cap < 1) cap = 1;
    if (gy > cap) gy = cap;
    if (gy > 65535) gy = 65535;
    dim3 grid((unsigned)gx, (unsigned)gy);
    uint32_t* am = reinterpret_cast<uint32_t*>(amax);   // non-negative f32 maxima: integer max of the bits
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    if (dtype == MG_BF16) {
        if (gelu && am)
            hipLaunchKernelGGL((quant_bf16_kernel<true, true>), grid, dim3(256), 0, st, Xb, M, K, k, s, rcp, pos, Aq, As,
                               XO, am);
        else if (gelu)
            hipLaunchKernelGGL((quant_bf16_kernel<true, false>), grid, dim3(256), 0, st, Xb, M, K, k, s, rcp, pos, Aq,
                               As, XO, am);
        else if (am)
            hipLaunchKernelGGL((quant_bf16_kernel<false, true>), grid, dim3(256), 0, st, Xb, M, K, k, s, rcp, pos, Aq,
                               As, XO, am);
        else
            hipLaunchKernelGGL((quant_bf16_kernel<false, false>), grid, dim3(256), 0, st, Xb, M, K, k, s, rcp, pos, Aq,
                               As, XO, am);
    } else {
        hipLaunchKernelGGL(quant_f32_kernel, grid, dim3(256), 0, st, static_cast<const float*>(X), M, K, k, s, pos,
                           Aq, As, XO, am);
    }
    return hipGetLastError();
}

}  // namespace mg
