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
// Aq and XO are stored in the GEMM's fragment order (frag_offset): a row's
// bytes sit in 16-byte pieces, one per 32x32-byte block, at an offset that
// splits into a per-row part (scalar) and a per-lane part (constant), so the
// per-row resource covers exactly the row's pieces.  Rows up to the next
// multiple of 32 and the pad half of a last 32-byte slice (K % 64 == 32) get
// zero codes.  The codes As[m][b] are stored in scale windows of 256 rows x
// 16 blocks (sc_offset): a workgroup's 512 channels are one window, so a
// row's 16 codes are 16 contiguous bytes; the rows run on to the end of the
// last 256-row group, whose pad rows (and the blocks past K) get code 0.
//
// With GELU, X is the previous projection's bf16 output and the quantized
// input is h = gelu_bf16x2 of X (the FFN block's hidden activation), computed
// in registers with the GELU kernel's own code: one pass instead of a GELU
// pass that writes h and a quantize pass that reads it back.
//
// bf16 input: the quotient comes from Markstein's correction of x * RN(1/s);
// the conditions under which its codes are the exact ones are checked on the
// quotients and block maxima the encoder forms anyway (process_row), and a
// wave whose row fails them redoes the row with the correctly rounded
// division.  f32 input always uses the correctly rounded division.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kStgRow = 272;      // LDS staging row: 256 bytes of codes + 16 pad

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

// encode8, then the packed nibbles (to aq when non-null) and, from one lane
// per quad, the block's scale byte into the row's 16 bytes of its scale
// window (every lane: past K or M the code of a zero block).
__device__ __forceinline__ void encode_store(const float (&q)[8], int lane, uint8_t* aq, uint8_t* as_win_row) {
    uint32_t c;
    const uint32_t word = encode8(q, c);
    if (aq) *reinterpret_cast<uint32_t*>(aq) = word;
    if ((lane & 3) == 0) as_win_row[sc_pos(lane >> 2)] = (uint8_t)c;
}

// Per-lane parts of frag_offset (the row part is (r / 32) * ns * 1024 +
// (r % 32) * 16): byte b of a row sits at (b / 32) * 1024 + ((b / 16) % 2) *
// 512 + b % 16 past it.  Aq: the 4 bytes of channels j0 .. j0 + 7 (b = j0 / 2);
// XO: outlier column i (b = 2 i).
__device__ __forceinline__ uint32_t frag_lane_off(uint32_t b) { return (b >> 5) * 1024u + ((b >> 4) & 1u) * 512u + (b & 15u); }
__device__ __forceinline__ int64_t frag_row_off(int64_t r, int64_t ns) { return (r >> 5) * ns * kFragBlock + ((r & 31) << 4); }

// 5 waves per SIMD (at most 96 VGPRs each); the statistics variants, which
// also carry the lane's running channel maxima, fit 4 without spills.
template <bool GELU, bool STATS>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(STATS ? 4 : 5, 8))) quant_bf16_kernel(const uint16_t* __restrict__ X, int64_t M, int32_t K,
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
    // Aq codes of each wave's 8 rows (rows of 256 bytes, padded to 272 so
    // that the row writes are conflict-free)
    __shared__ __attribute__((aligned(16))) uint8_t stg[kWaves * 8 * kStgRow];
    for (int t = threadIdx.x; t < 512; t += 256) {
        const int j = blockIdx.x * 512 + t;
        t_s[t] = j < K ? s[j] : 1.0f;
        t_r[t] = j < K ? rcp[j] : 1.0f;
        t_p[t] = j < K ? pos[j] : -1;
        t_m[t] = 0;
    }
    __syncthreads();
    uint8_t* const stgw = stg + wave * 8 * kStgRow;   // this wave's staging rows
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
    // The fast quotient multiplies by rz = RN(1/s), or by 0 on outlier channels:
    // their bulk quotient is then +-0 (no effect on the block maximum) and
    // their nibbles are cleared after encoding (nkeep), so that they encode
    // the +0 of Eq. (5)'s bulk.  The exact-division path divides +0 there.
    float rz[8];
    uint32_t nkeep = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        rz[i] = (omask >> i) & 1u ? 0.0f : rv[i];
        nkeep |= ((omask >> i) & 1u ? 0u : 0xFu) << (4 * i);
    }
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
    const uint32_t osh = (oc0 & 1) ? 0u : 16u;     // brings the first outlier's bf16 to the top half

    // Per-lane byte offsets.  Rows of X are read through a buffer resource
    // per row (scalar registers), so lanes whose channels lie past K read
    // zeros.  XO pieces and As codes are written through one resource per
    // 32-row group; a row's part of the offset, 16 bytes per row of the
    // group, is a per-wave constant plus the row's index in the wave times 16.
    // Lanes that store no scale byte or no outlier value get the offset
    // kNoStore, past every resource's range, and the hardware drops those
    // stores.  The workgroup's 512 channels are one scale window: a row's 16
    // scale bytes are contiguous, lane 4 i storing block i's code at byte
    // sc_pos(i) (past K: the code 0 of its all-zero block).
    constexpr uint32_t kNoStore = 0x40000000u;
    const uint32_t offX = 2u * (uint32_t)j0;
    const uint32_t rowpart = 128u * (uint32_t)wave;                       // 16 (8 wave) bytes
    const uint32_t offAs = ((lane & 3) == 0 ? (uint32_t)sc_pos(lane >> 2) : kNoStore) + rowpart;
    const uint32_t offXO = (omask ? frag_lane_off(2u * (uint32_t)op0) : kNoStore) + rowpart;
    // wave-uniform flags as scalars (readfirstlane), so that branches on them
    // stay scalar
    const int wave_o = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(omask != 0) != 0));
    const int wave_rest = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(omask_rest != 0) != 0));
    // |q0| bound of the fast path, 0 on lanes whose s is outside [2^-20, 2^20]
    // (their rows always take the exact division)
    const uint32_t a0_lim = s_ok ? kF32Pow126 : 0u;
    // Aq rows of K/2 bytes in ns4 slices, XO rows of 2k bytes in nso slices;
    // the workgroup of channels 0..511 writes XO's pad columns k .. 16 nso - 1
    // (+0), one per lane
    const int64_t ns4 = frag_slices(K / 2), nso = frag_slices(2 * (int64_t)k);
    const int kp16 = 16 * (int)nso;
    const uint32_t rowX = 2u * (uint32_t)K;
    const bool pad_wg = blockIdx.x == 0 && kp16 > k;

    auto rsrc = [](const void* p, uint32_t bytes) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
    };
    auto load_row = [&](const uint16_t* px, bool in) -> u32x4 {
        return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc(px, in ? rowX : 0u), offX, 0,
                                                                                2));   // nt
    };

    // Row r (0..7) of the wave's 8 rows in a group: w its 8 bf16 per lane;
    // rxo / ras the group's XO and As resources (rxo of range 0 for a group
    // of pad rows that only have scale codes).
    //
    // The quotient q = RN(x / s) comes from Markstein's correction of
    // q0 = RN(x * RN(1/s)) (div_fast), which is the IEEE quotient whenever
    // |x| >= 2^-100, s lies in [2^-20, 2^20] and |q0| < 2^126.  A smaller
    // nonzero |x| gives |q| < 2^-79 on both the fast and the exact path
    // (same sign; a fast +-0 stands for an exact +-0 or +-2^-149): such values
    // encode to a zero code under any block scale of 2^-76 or more, i.e. when
    // the block maximum is at least 2^-74, and then neither the maximum nor
    // any code depends on which path computed them; an all-zero block gets
    // the code 0 either way.  So the fast codes are the exact ones unless
    // some lane has s out of range, |q0| >= 2^126, or a block maximum in
    // (0, 2^-74); the outlier value (stored itself, in bf16) needs |qo| in
    // [2^-78, 2^126) or qo = +-0.  If any of the wave's lanes fails, the
    // wave redoes the row with the correctly rounded division.
    auto process_row = [&](u32x4 w, int r, __amdgpu_buffer_rsrc_t rxo, __amdgpu_buffer_rsrc_t ras) {
        if constexpr (GELU) {
#pragma unroll
            for (int i = 0; i < 4; ++i) w[i] = gelu_bf16x2(w[i]);
        }
        if constexpr (STATS) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                mx[i] = __builtin_elementwise_max(mx[i], __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu));
        }
        float q[8];
        float a0 = 0.0f, aq = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t wi = w[i >> 1];
            const float x = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
            const float q0 = x * rz[i];
            const float t = __builtin_fmaf(q0, sv[i], -x);
            q[i] = __builtin_fmaf(-t, rz[i], q0);
            a0 = fmaxf(a0, __builtin_fabsf(q0));
            aq = fmaxf(aq, __builtin_fabsf(q[i]));
        }
        uint32_t qb = quad_max_bits(__float_as_uint(aq));
        // lanes failing a check, as wave masks (one compare each)
        uint64_t bad = __builtin_amdgcn_uicmp(__float_as_uint(a0), a0_lim, kCmpUGE) |
                       __builtin_amdgcn_uicmp(qb - 1u, kF32PowM74 - 1u, kCmpULT);
        float xo = 0.0f, qo = 0.0f;
        if (wave_o) {
            // the first outlier channel's own (unmasked) value from the raw words
            uint32_t wo = w[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) wo = (oc0 >> 1) == i ? w[i] : wo;
            xo = __uint_as_float((wo << osh) & 0xFFFF0000u);
            qo = div_fast(xo, so, ro);
            const uint32_t ab = __float_as_uint(qo) & 0x7FFFFFFFu;
            // lanes without an outlier hold +-0 or a harmless value here: only those with one count
            bad |= __builtin_amdgcn_uicmp(omask ? ab - kF32PowM78 : 0u, kF32Pow126 - kF32PowM78, kCmpUGE) &
                   __builtin_amdgcn_uicmp(ab, 0u, kCmpNE);
        }
        if (bad) {
            aq = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wi = w[i >> 1];
                const float x = (omask >> i) & 1u ? 0.0f : __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                q[i] = __fdiv_rn(x, sv[i]);
                aq = fmaxf(aq, __builtin_fabsf(q[i]));
            }
            qb = quad_max_bits(__float_as_uint(aq));
            if (wave_o) qo = __fdiv_rn(xo, so);
        }
        const uint32_t rb = 16u * (uint32_t)r;    // the row's 16 bytes in the wave's part of the group
        if (wave_o) {
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qo), rxo, offXO + rb, 0, 0);
            if (wave_rest) {
                // further outlier channels of the lane (two or more in its 8): exact division
                for (uint32_t mm = omask_rest; mm; mm &= mm - 1) {
                    const int i = __builtin_ctz(mm);
                    const int jl = lane * 8 + i;
                    const uint32_t wi = w[i >> 1];
                    const float xi = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                    const float qi = __fdiv_rn(xi, t_s[jl]);
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qi), rxo,
                                                          frag_lane_off(2u * (uint32_t)t_p[jl]) + rowpart + rb, 0,
                                                          0);
                }
            }
        }
        // E8M0 code c = max(e - 2, 0) of the block maximum's biased exponent e,
        // and its scale 2^(c - 127) as the converter takes it (exponent field c)
        const int32_t sb = __builtin_elementwise_max((int32_t)(qb & 0x7F800000u) - (2 << 23), 0x00200000);
        const float scale = __int_as_float(sb);
        uint32_t word = 0;
        MG_CVT_FP4X2(word, q[0], q[1], scale, 0);
        MG_CVT_FP4X2(word, q[2], q[3], scale, 1);
        MG_CVT_FP4X2(word, q[4], q[5], scale, 2);
        MG_CVT_FP4X2(word, q[6], q[7], scale, 3);
        *reinterpret_cast<uint32_t*>(stgw + r * kStgRow + 4 * lane) = word & nkeep;
        if (pad_wg) {
            const uint32_t offPad = lane < kp16 - k ? frag_lane_off(2u * (uint32_t)(k + lane)) : kNoStore;
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)0, rxo, offPad + rowpart + rb, 0, 0);
        }
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(sb >> 23), ras, offAs + rb, 0, 0);
    };

    // 32-row groups G = blockIdx.y, blockIdx.y + gridDim.y, ...; wave w takes
    // rows 32 G + 8 w .. 32 G + 8 w + 7, loaded together (8 KB per wave) while
    // the wave's previous group is processed, row by row.  The groups run on to the end of the
    // last 256-row scale group, so its pad rows get their zero codes.  The
    // wave's 8 rows fill whole 128-byte lines of the fragment blocks (8 rows x
    // 16 bytes of one slice half), so it stages its Aq codes in its own LDS
    // rows and stores them as 16 full lines (two 1 KB store instructions;
    // lane L of store t takes row L % 8 of line 8 t + L / 8 = (slice, half)).
    // No wave reads another's staging, so no barrier is needed.  Groups past
    // the row groups of Aq (pad rows of the scale group only) store nothing
    // but scale codes.
    const int64_t Mp = (M + kScRows - 1) / kScRows * kScRows;
    const int ngr = (int)(Mp / 32);                                       // groups with scale rows
    const int GA = (int)((M + 31) / 32);                                  // groups with Aq / XO pieces
    const int gstride = (int)gridDim.y;
    const int64_t win_stride = sc_nwin(K) * kScWinBytes;     // bytes between 256-row groups of As
    static_assert(kScRows == 256, "8 row groups per scale group");
    uint8_t* const asw = As + (int64_t)blockIdx.x * kScWinBytes;
    uint8_t* const XOb = reinterpret_cast<uint8_t*>(XO);
    const uint32_t xo_group = (uint32_t)nso * 1024u;                      // XO bytes of a 32-row group
    // rows of group g: row r of the wave's 8, as a load through its own resource
    auto load_group_row = [&](int g, int r) -> u32x4 {
        const int64_t m = (int64_t)g * 32 + wave * 8 + r;
        return load_row(X + m * K, g < ngr && m < M);
    };
    u32x4 xa[4], xb[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) xa[r] = load_group_row((int)blockIdx.y, r);
    for (int G = (int)blockIdx.y; G < ngr; G += gstride) {
        const bool live = G < GA;
        const __amdgpu_buffer_rsrc_t rxo = rsrc(XOb + (int64_t)G * xo_group, live ? xo_group : 0u);
        const __amdgpu_buffer_rsrc_t ras = rsrc(asw + (int64_t)(G >> 3) * win_stride + (G & 7) * 512, 512u);
#pragma unroll
        for (int r = 0; r < 4; ++r) xb[r] = load_group_row(G, 4 + r);
#pragma unroll
        for (int r = 0; r < 4; ++r) process_row(xa[r], r, rxo, ras);
#pragma unroll
        for (int r = 0; r < 4; ++r) xa[r] = load_group_row(G + gstride, r);
#pragma unroll
        for (int r = 0; r < 4; ++r) process_row(xb[r], 4 + r, rxo, ras);
        if (live) {
            const __amdgpu_buffer_rsrc_t rg = rsrc(Aq + (int64_t)G * ns4 * 1024, (uint32_t)ns4 * 1024u);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int line = 8 * t + (lane >> 3), sl = line >> 1, hf = line & 1, rr = lane & 7;
                const u32x4 v = *reinterpret_cast<const u32x4*>(stgw + rr * kStgRow + sl * 32 + hf * 16);
                __builtin_amdgcn_raw_buffer_store_b128(
                    v, rg, (uint32_t)((blockIdx.x * 8 + sl) * 1024 + 16 * (wave * 8 + rr + 32 * hf)), 0, 2);
            }
        }
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
    // Aq and XO in fragment order (rows through M rounded up to 32 get zero
    // codes; lanes past K up to the last 32-byte slice of Aq store zero codes)
    const int64_t ns4 = frag_slices(K / 2), nso = frag_slices(2 * (int64_t)k);
    const int64_t M32 = (M + 31) / 32 * 32;
    const int kp16 = 16 * (int)nso;
    uint8_t* const XOb = reinterpret_cast<uint8_t*>(XO);
    for (int64_t r = (int64_t)blockIdx.y * kWaves + wave; r < Mp; r += rstride) {
        const bool live = r < M, piece = r < M32;
        float q[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x = valid && live ? X[r * K + j0 + i] : 0.0f;
            mx[i] = fmaxf(mx[i], __builtin_fabsf(x));
            q[i] = __fdiv_rn(x, sv[i]);
            if (pv[i] >= 0) {
                if (piece)
                    *reinterpret_cast<uint16_t*>(XOb + frag_offset(r, 2 * (int64_t)pv[i], nso)) =
                        (uint16_t)f32_to_bf16_rne(q[i]);
                q[i] = 0.0f;
            }
        }
        if (piece && blockIdx.x == 0 && lane < kp16 - k)
            *reinterpret_cast<uint16_t*>(XOb + frag_offset(r, 2 * (int64_t)(k + lane), nso)) = 0;
        encode_store(q, lane, piece && j0 < 64 * ns4 ? Aq + frag_offset(r, j0 / 2, ns4) : nullptr,
                     As + sc_offset(r, (int32_t)blockIdx.x * kScBlocks, nwin));
    }
    if (amax != nullptr && valid) {
#pragma unroll
        for (int i = 0; i < 8; ++i) atomicMax(amax + j0 + i, __float_as_uint(mx[i]));
    }
}

}  // namespace

template <typename F, typename... A>
static void launch_rows(F* kern, int64_t M, int64_t gx, hipStream_t st, A... args) {
    // one resident round of workgroups; each takes 32-row groups through the
    // last 256-row scale group
    int64_t gy = (M + kScRows - 1) / kScRows * (kScRows / 32);
    int64_t cap = (int64_t)device_cu_count() * blocks_per_cu(reinterpret_cast<const void*>(kern)) / gx;
    if (cap < 1) cap = 1;
    if (gy > cap) gy = cap;
    if (gy > 65535) gy = 65535;
    hipLaunchKernelGGL(kern, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, st, args...);
}

hipError_t launch_quant(const void* X, int32_t dtype, int64_t M, int32_t K, int32_t k,
                        const float* s, const float* rcp, const int32_t* pos, uint8_t* Aq,
                        uint8_t* As, uint16_t* XO, hipStream_t st, bool gelu, float* amax) {
    if (M <= 0) return hipSuccess;
    const int64_t gx = ((int64_t)K / 8 + 63) / 64;
    uint32_t* am = reinterpret_cast<uint32_t*>(amax);   // non-negative f32 maxima: integer max of the bits
    const uint16_t* Xb = static_cast<const uint16_t*>(X);
    if (dtype == MG_BF16) {
        if (gelu && am)
            launch_rows(quant_bf16_kernel<true, true>, M, gx, st, Xb, M, K, k, s, rcp, pos, Aq, As, XO, am);
        else if (gelu)
            launch_rows(quant_bf16_kernel<true, false>, M, gx, st, Xb, M, K, k, s, rcp, pos, Aq, As, XO, am);
        else if (am)
            launch_rows(quant_bf16_kernel<false, true>, M, gx, st, Xb, M, K, k, s, rcp, pos, Aq, As, XO, am);
        else
            launch_rows(quant_bf16_kernel<false, false>, M, gx, st, Xb, M, K, k, s, rcp, pos, Aq, As, XO, am);
    } else {
        launch_rows(quant_f32_kernel, M, gx, st, static_cast<const float*>(X), M, K, k, s, pos, Aq, As, XO, am);
    }
    return hipGetLastError();
}

}  // namespace mg
