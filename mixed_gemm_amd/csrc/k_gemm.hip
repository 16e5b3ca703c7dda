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
#include <stdlib.h>

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

// ---------------------------------------------------------------------------
// Persistent tiled kernel.  One workgroup per CU (4 waves); each walks a list
// of 256x256 output tiles.  Each wave owns a 128x128 quarter = 4x4 MFMA tiles
// of 32x32 (256 fp32 accumulators per lane, held in the accumulation
// registers).
//
// The K dimension is walked in stages that each move 128 bytes per tile row
// into LDS: a bulk stage carries 256 FP4 values (128 B) of Aq / Wq, an outlier
// stage carries 64 bf16 values (128 B) of XO / WO.  Both kinds use the same LDS
// layout and the same fragment addressing -- sub-step ss of a stage reads
// bytes [32 ss + 16 h, 32 ss + 16 h + 16) of a row for lane half h -- which is
// 64 FP4 (one scaled FP4 MFMA) or 16 bf16 (one BF16 MFMA).  Bulk stages come
// first, outlier stages follow, all accumulating into the same registers.
//
// Pipeline.  The stages of all of a workgroup's tiles form one sequence over
// two LDS buffers (2 x 64 KB).  While stage g is multiplied out of one buffer,
// the copies of stage g+1 (which may be the first stage of the next tile) run
// straight from global memory into the other buffer, and two one-lane-per-row
// loads touch the rows of stage g+2 so they are in L2 when their copies are
// issued.  One barrier per stage.  After a tile's last stage its 256x256 bf16
// result is staged through the freed buffer and written as whole 512-byte rows
// while the next tile's first stage already sits in LDS.
//
// LDS rows are 128 B; logical 16-byte chunk c of tile row r is stored at
// physical chunk c ^ ((r >> 1) & 7), which spreads the 16 rows a fragment load
// reads at once over all 64 banks.  Loads use buffer descriptors sized to each
// operand: rows past M (or N) and chunks past K / k read as zeros.  Tiles are
// dealt so that each XCD (workgroups go round-robin to the 8 XCDs) walks a
// contiguous run of the tile order, grouped 8 row-tiles at a time, which keeps
// the operand panels of its concurrently running tiles in its L2.
// ---------------------------------------------------------------------------

constexpr int TBM = 256, TBN = 256;
constexpr int ROWB = 128;                         // bytes per tile row per stage
constexpr int TILE_BYTES = TBM * ROWB;            // 32 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;       // A + B
constexpr int JUNK_OFF = 2 * STAGE_BYTES;         // landing area of the L2 touches
constexpr int GEMM_LDS_BYTES = 2 * STAGE_BYTES + 1024;
constexpr uint32_t OOB = 0xC0000000u;             // offset that reads as zero
constexpr int NXCD = 8;
constexpr int GROUP_M = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint64_t bytes) {
    const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}

template <int OPSEL>
__device__ __forceinline__ v16f mfma_fp4_op(const u32x4& a, const u32x4& b, uint32_t sa, uint32_t sb, v16f c) {
    v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
    v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, c, 4, 4, OPSEL, (int)sa, OPSEL, (int)sb);
}

__device__ __forceinline__ v16f mfma_bf16_v(const u32x4& a, const u32x4& b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a), __builtin_bit_cast(v8bf, b), c,
                                                   0, 0, 0);
}

struct GemmArgs {
    const uint8_t* Aq;
    const uint8_t* As;
    const uint16_t* XO;
    const uint8_t* Wq;
    const uint8_t* Ws;
    const uint16_t* WO;
    void* Y;
    int64_t M;
    int32_t N, K, k;
    int32_t MT, NT;     // tile counts
};

// Origin of an output tile (wave-uniform).
struct TileOrg {
    int64_t m0;
    int n0;
};

// K8: k % 8 == 0 (outlier rows are whole 16-byte chunks); NB8: (K/32) % 8 == 0
// (each stage's 8 scale bytes of a row are one aligned 8-byte word).
template <typename OutT, bool K8, bool NB8>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
dual_gemm_tiled(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int wm = wave >> 1, wn = wave & 1;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int K = g.K, k = g.k, N = g.N;
    const int64_t M = g.M;
    const uint32_t rowA = (uint32_t)(K / 2);       // bytes per Aq / Wq row
    const uint32_t rowX = (uint32_t)(2 * k);       // bytes per XO / WO row
    const int nb = K / 32;
    const int S4 = (K / 2 + ROWB - 1) / ROWB;      // bulk stages
    const int S16 = (2 * k + ROWB - 1) / ROWB;     // outlier stages
    const int S = S4 + S16;

    // ---- this workgroup's tiles: XCD x owns tiles [x per, (x+1) per); its
    // workgroups take every nl-th one.
    const int T = g.MT * g.NT;
    const int per = (T + NXCD - 1) / NXCD;
    const int nl = (int)gridDim.x / NXCD;
    const int xcd = (int)blockIdx.x % NXCD;
    const int t_end = min((xcd + 1) * per, T);
    int t = xcd * per + (int)blockIdx.x / NXCD;
    if (t >= t_end) return;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.Aq, (uint64_t)M * rowA);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.Wq, (uint64_t)N * rowA);
    const __amdgpu_buffer_rsrc_t rAs = make_rsrc(g.As, (uint64_t)M * nb);
    const __amdgpu_buffer_rsrc_t rBs = make_rsrc(g.Ws, (uint64_t)N * nb);
    const __amdgpu_buffer_rsrc_t rXO = make_rsrc(g.XO, (uint64_t)M * rowX);
    const __amdgpu_buffer_rsrc_t rWO = make_rsrc(g.WO, (uint64_t)N * rowX);

    // ---- tile-independent lane constants.  Every per-row offset goes into
    // the range-checked vector offset of the buffer instructions (the scalar
    // offset is not range-checked), so rows past M / N read as zero.
    // Copies: each load instruction of a wave moves 8 tile rows x 128 B = 1 KB
    // into LDS, lane L landing at byte 16 L (row L/8 of the group, physical
    // chunk L%8).  For 8-row group gi that slot holds logical chunk
    // (L%8) ^ ((L/16) + 4 (gi & 1)), which the lane reads from global memory.
    // Wave w copies rows [64 w, 64 w + 64) of the A and of the B tile.
    const int lrow = lane >> 3;
    const uint32_t c16e = (uint32_t)(((lane & 7) ^ (lrow >> 1)) << 4);        // even groups
    const uint32_t c16o = c16e ^ 64u;                                          // odd groups
    const uint32_t lrA0 = (uint32_t)(wave * 64 + lrow) * rowA;                 // copy row (group 0)
    const uint32_t lrX0 = (uint32_t)(wave * 64 + lrow) * rowX;
    const uint32_t ltA = (uint32_t)(wave * 64 + lane) * rowA;                  // L2-touch row
    const uint32_t ltX = (uint32_t)(wave * 64 + lane) * rowX;
    const uint32_t lsA = (uint32_t)(wm * 128 + l32) * (uint32_t)nb;            // scale rows
    const uint32_t lsB = (uint32_t)(wn * 128 + l32) * (uint32_t)nb;
    const uint32_t lds_w = (uint32_t)(wave * 64 * ROWB);
    uint32_t fa[4], fb[4];                        // fragment rows within a stage buffer
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = (uint32_t)((wm * 128 + i * 32 + l32) * ROWB);
        fb[i] = (uint32_t)(TILE_BYTES + (wn * 128 + i * 32 + l32) * ROWB);
    }
    const int sw = (l32 >> 1) & 7;   // (row >> 1) & 7 of every fragment row of this lane

    auto tile_org = [&](int tt) {
        TileOrg o;
        const int grp = tt / (GROUP_M * g.NT);
        const int gsz = min(GROUP_M, g.MT - grp * GROUP_M);
        const int rin = tt - grp * GROUP_M * g.NT;
        o.m0 = (int64_t)__builtin_amdgcn_readfirstlane((grp * GROUP_M + rin % gsz) * TBM);
        o.n0 = __builtin_amdgcn_readfirstlane((rin / gsz) * TBN);
        return o;
    };

    v16f acc[4][4];
    uint32_t scA[4][2], scB[4][2], nA[4][2], nB[4][2];

    auto load_scales = [&](const TileOrg& o, int st) {
        const uint32_t sa0 = __builtin_amdgcn_readfirstlane((uint32_t)o.m0 * (uint32_t)nb);
        const uint32_t sb0 = __builtin_amdgcn_readfirstlane((uint32_t)o.n0 * (uint32_t)nb);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t va = lsA + sa0 + (uint32_t)(32 * i * nb);   // rows past M are out of range
            const uint32_t vb = lsB + sb0 + (uint32_t)(32 * i * nb);
            if constexpr (NB8) {
                const uint32_t sof = __builtin_amdgcn_readfirstlane((uint32_t)st * 8);
                const u32x2 xa = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rAs, va, sof, 0));
                const u32x2 xb = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rBs, vb, sof, 0));
                nA[i][0] = xa[0]; nA[i][1] = xa[1];
                nB[i][0] = xb[0]; nB[i][1] = xb[1];
            } else {
                uint32_t wa[2] = {0, 0}, wb[2] = {0, 0};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = st * 8 + e < nb;
                    const uint32_t ba = ok ? __builtin_amdgcn_raw_buffer_load_b8(rAs, va + (uint32_t)(st * 8 + e), 0, 0) : 0u;
                    const uint32_t bb = ok ? __builtin_amdgcn_raw_buffer_load_b8(rBs, vb + (uint32_t)(st * 8 + e), 0, 0) : 0u;
                    wa[e >> 2] |= (ba & 0xFFu) << (8 * (e & 3));
                    wb[e >> 2] |= (bb & 0xFFu) << (8 * (e & 3));
                }
                nA[i][0] = wa[0]; nA[i][1] = wa[1];
                nB[i][0] = wb[0]; nB[i][1] = wb[1];
            }
        }
    };

    // Copies of stage st of a tile into LDS buffer `buf` (asynchronous).
    auto load_stage = [&](const TileOrg& o, int st, int buf) {
        uint8_t* base = lds + buf * STAGE_BYTES + lds_w;
        // opaque per call: the per-group row offsets below are formed here
        // instead of being hoisted out of the loops and held in registers
        uint32_t lrA = lrA0, lrX = lrX0;
        asm volatile("" : "+v"(lrA), "+v"(lrX));
        if (st < S4) {
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)st * ROWB);   // column offset in the row
            const uint32_t ra = __builtin_amdgcn_readfirstlane((uint32_t)o.m0 * rowA);
            const uint32_t rb = __builtin_amdgcn_readfirstlane((uint32_t)o.n0 * rowA);
            // chunks past K (only when K % 256 != 0) read as zero
            const bool oke = so + c16e < rowA, oko = so + c16o < rowA;
#pragma unroll
            for (int gi = 0; gi < 8; ++gi) {
                const uint32_t c = (gi & 1) ? c16o : c16e;
                const bool ok = (gi & 1) ? oko : oke;
                const uint32_t va = ok ? lrA + c + ra + (uint32_t)gi * 8 * rowA : OOB;
                const uint32_t vb = ok ? lrA + c + rb + (uint32_t)gi * 8 * rowA : OOB;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (lds_ptr_t)(base + gi * 8 * ROWB), 16, va, so, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(base + TILE_BYTES + gi * 8 * ROWB), 16, vb,
                                                         so, 0, 0);
            }
            load_scales(o, st);
        } else {
            const int u = st - S4;
            const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)u * ROWB);
            if constexpr (K8) {
                const uint32_t ra = __builtin_amdgcn_readfirstlane((uint32_t)o.m0 * rowX);
                const uint32_t rb = __builtin_amdgcn_readfirstlane((uint32_t)o.n0 * rowX);
                const bool oke = so + c16e < rowX, oko = so + c16o < rowX;
#pragma unroll
                for (int gi = 0; gi < 8; ++gi) {
                    const uint32_t c = (gi & 1) ? c16o : c16e;
                    const bool ok = (gi & 1) ? oko : oke;
                    const uint32_t va = ok ? lrX + c + ra + (uint32_t)gi * 8 * rowX : OOB;
                    const uint32_t vb = ok ? lrX + c + rb + (uint32_t)gi * 8 * rowX : OOB;
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rXO, (lds_ptr_t)(base + gi * 8 * ROWB), 16, va, so, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rWO, (lds_ptr_t)(base + TILE_BYTES + gi * 8 * ROWB), 16,
                                                             vb, so, 0, 0);
                }
            } else {
                // k % 8 != 0: outlier rows are not 16-byte aligned; gather the
                // bf16 values one by one and store the chunk through registers.
                const int64_t ra0 = o.m0 + wave * 64 + lrow, rb0 = (int64_t)o.n0 + wave * 64 + lrow;
#pragma unroll
                for (int gi = 0; gi < 8; ++gi) {
                    const int cl = (int)(((gi & 1) ? c16o : c16e) >> 4);
                    const int64_t ra = ra0 + 8 * gi, rb = rb0 + 8 * gi;
                    uint32_t wa[4], wb[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        uint32_t xa = 0, xb = 0;
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int col = u * 64 + cl * 8 + 2 * e + q;
                            const uint32_t ea = (col < k && ra < M)
                                ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rXO, (uint32_t)((ra * k + col) * 2), 0, 0) : 0u;
                            const uint32_t eb = (col < k && rb < N)
                                ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rWO, (uint32_t)((rb * k + col) * 2), 0, 0) : 0u;
                            xa |= (ea & 0xFFFFu) << (16 * q);
                            xb |= (eb & 0xFFFFu) << (16 * q);
                        }
                        wa[e] = xa; wb[e] = xb;
                    }
                    *reinterpret_cast<u32x4*>(base + gi * 8 * ROWB + lane * 16) = u32x4{wa[0], wa[1], wa[2], wa[3]};
                    *reinterpret_cast<u32x4*>(base + TILE_BYTES + gi * 8 * ROWB + lane * 16) = u32x4{wb[0], wb[1], wb[2], wb[3]};
                }
            }
        }
    };

    // One-lane-per-row loads that bring both 64-byte halves of the 128-byte
    // rows of a future stage into L2 (4 bytes per lane land in a scratch area
    // of LDS).  Always exactly NTOUCH instructions, so the stage wait can
    // leave them in flight.
    auto touch = [&](const TileOrg* o, int st) {
        uint8_t* junk = lds + JUNK_OFF + wave * 256;
        uint32_t va = OOB, vb = OOB, so = 0;
        __amdgpu_buffer_rsrc_t ra = rA, rb = rB;
        if (o != nullptr && st < S4) {
            va = ltA + (uint32_t)o->m0 * rowA;
            vb = ltA + (uint32_t)o->n0 * rowA;
            so = (uint32_t)st * ROWB;
        } else if (o != nullptr && st < S) {
            va = ltX + (uint32_t)o->m0 * rowX;
            vb = ltX + (uint32_t)o->n0 * rowX;
            so = (uint32_t)(st - S4) * ROWB;
            ra = rXO; rb = rWO;
        }
        so = __builtin_amdgcn_readfirstlane(so);
        const uint32_t so2 = __builtin_amdgcn_readfirstlane(so + 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)junk, 4, va, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)junk, 4, vb, so, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_ptr_t)junk, 4, va, so2, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_ptr_t)junk, 4, vb, so2, 0, 0);
    };

    auto take_scales = [&]() {
        // lane half h uses the odd scale bytes: shift them down so sub-step ss
        // finds its byte at position 2*(ss&1) of word ss>>1.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            scA[i][0] = h ? nA[i][0] >> 8 : nA[i][0];
            scA[i][1] = h ? nA[i][1] >> 8 : nA[i][1];
            scB[i][0] = h ? nB[i][0] >> 8 : nB[i][0];
            scB[i][1] = h ? nB[i][1] >> 8 : nB[i][1];
        }
    };

    auto fetch = [&](const uint8_t* base, int ss, u32x4 (&fA)[4], u32x4 (&fB)[4]) {
        const uint32_t co = (uint32_t)(((2 * ss + h) ^ sw) << 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            fA[i] = *reinterpret_cast<const u32x4*>(base + fa[i] + co);
            fB[i] = *reinterpret_cast<const u32x4*>(base + fb[i] + co);
        }
    };

    // Instruction order of one stage: the 8 fragment reads of sub-step 0, then
    // for each sub-step the reads of the next one threaded between its first 8
    // MFMAs, so LDS latency hides behind matrix-core work.
    auto interleave_schedule = [&]() {
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);          // DS reads
#pragma unroll
        for (int ss = 0; ss < 3; ++ss) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
    };

    // One stage: 4 sub-steps of 16 MFMAs; the fragments of sub-step ss+1 are
    // read from LDS while the MFMAs of sub-step ss run.
    auto bulk_compute = [&](const uint8_t* base) {
        u32x4 fA[2][4], fB[2][4];
        fetch(base, 0, fA[0], fB[0]);
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            if (ss < 3) fetch(base, ss + 1, fA[(ss + 1) & 1], fB[(ss + 1) & 1]);
            const int c = ss & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if ((ss & 1) == 0)
                        acc[i][j] = mfma_fp4_op<0>(fB[c][j], fA[c][i], scB[j][ss >> 1], scA[i][ss >> 1], acc[i][j]);
                    else
                        acc[i][j] = mfma_fp4_op<2>(fB[c][j], fA[c][i], scB[j][ss >> 1], scA[i][ss >> 1], acc[i][j]);
                }
        }
        interleave_schedule();
    };
    auto outlier_compute = [&](const uint8_t* base) {
        u32x4 fA[2][4], fB[2][4];
        fetch(base, 0, fA[0], fB[0]);
#pragma unroll
        for (int ss = 0; ss < 4; ++ss) {
            if (ss < 3) fetch(base, ss + 1, fA[(ss + 1) & 1], fB[(ss + 1) & 1]);
            const int c = ss & 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16_v(fB[c][j], fA[c][i], acc[i][j]);
        }
        interleave_schedule();
    };
    // Wait for this wave's copies of the next stage (everything but the four
    // L2 touches), then for every wave.  The scheduling barrier keeps the
    // MFMAs of the current stage above it, so they run while copies fly.
    // (__syncthreads would add a release fence, i.e. wait for every
    // outstanding memory operation including the L2 touches and the stores of
    // the previous tile; only this wave's copies matter here.)
    auto stage_sync = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    // LDS-only barrier: this wave's LDS writes are done, then every wave arrives.
    auto lds_sync = [&]() {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
    };

    // ---- epilogue of one tile.  The MFMAs take the weight fragment as their
    // first operand, so acc[i][j] holds Y^T for A row-tile i and W row-tile j:
    // lane (l32, h), register 4 q + e holds output row 32 i + l32 and output
    // column 32 j + 8 q + 4 h + e of this wave's quarter -- four consecutive
    // columns per register group.
    auto epilogue = [&](const TileOrg& o, uint8_t* stagebuf) {
        if constexpr (sizeof(OutT) == 2) {
            // bf16: round pairs with the hardware converter (nearest even) and
            // write the tile in 4 passes; pass p stages the rows of accumulator
            // row-block p of every wave -- 64 rows x 512 B -- in one half of
            // the free buffer (alternating halves), then all threads write
            // those rows with 16-byte streaming stores.  In a staged row r'
            // (= 32 wm + l32) the 8-byte unit u lives at unit u ^ (2 (r' % 32)):
            // the 32 rows written by one instruction spread over the banks and
            // the 16-byte chunk c stays contiguous at chunk c ^ (r' % 32).
            uint16_t* Yb = static_cast<uint16_t*>(g.Y);
            const bool full = o.m0 + TBM <= M && o.n0 + TBN <= N;
            // Every lane-dependent value below is derived from an opaque copy of
            // the thread index, so it is formed here, once per tile, instead of
            // being hoisted out of the tile loop and held (or spilled) across it.
            uint32_t et = (uint32_t)tid;
            asm volatile("" : "+v"(et));
            const uint32_t el32 = et & 31u, eh = (et >> 5) & 1u;
            const uint32_t eb = ((uint32_t)wm * 32 + el32) * 512 + eh * 8, em = el32 << 4;
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                uint8_t* sb = stagebuf + (p & 1) * 32768;
                // read row-block p's accumulators here, not earlier
#pragma unroll
                for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[p][j]));
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const f32x2 lo = {acc[p][j][4 * q], acc[p][j][4 * q + 1]};
                        const f32x2 hi = {acc[p][j][4 * q + 2], acc[p][j][4 * q + 3]};
                        const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                         __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
                        const uint32_t cu = (uint32_t)((wn * 32 + 8 * j + 2 * q) << 3);
                        *reinterpret_cast<u32x2*>(sb + eb + (cu ^ em)) = w;
                    }
                lds_sync();
#pragma unroll
                for (int qq = 0; qq < 8; ++qq) {
                    const int c = (int)et + 256 * qq;      // 16-byte chunk of the 64 staged rows
                    const int rr = c >> 5, cc16 = c & 31;
                    const u32x4 v = *reinterpret_cast<const u32x4*>(sb + rr * 512 + ((cc16 ^ (rr & 31)) << 4));
                    const int64_t grow = o.m0 + (rr >> 5) * 128 + 32 * p + (rr & 31);
                    const int gcol = o.n0 + cc16 * 8;
                    // streaming store: Y is written once and must not push the
                    // operand panels out of L2
                    if (full || (grow < M && gcol < N))
                        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(Yb + grow * N + gcol));
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // every wave's staging reads are done (their data fed the stores
            // above) before the next stage's copies reuse the buffer
            __builtin_amdgcn_s_barrier();
        } else {
            // fp32: four consecutive columns per register group -> 16-byte stores
            float* Yf = static_cast<float*>(g.Y);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = o.m0 + wm * 128 + 32 * i + l32;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = o.n0 + wn * 128 + 32 * j + 8 * q + 4 * h;
                        if (row < M && col < N) {
                            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                             acc[i][j][4 * q + 3]};
                            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(Yf + row * N + col));
                        }
                    }
            }
        }
    };

    // ---- prologue: first stage of the first tile
    TileOrg cur = tile_org(t);
    int tn = t + nl;
    load_stage(cur, 0, 0);
    if (S > 1) touch(&cur, 1);
    else if (tn < t_end) { const TileOrg nx = tile_org(tn); touch(&nx, 0); }
    else touch(nullptr, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    take_scales();
    __syncthreads();
    int buf = 0;

    while (true) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
        const bool has_next = tn < t_end;
        // steady state: bulk stages whose next two stages are bulk stages of this tile
        int st = 0;
        for (; st + 2 < S4; ++st) {
            load_stage(cur, st + 1, buf ^ 1);
            touch(&cur, st + 2);
            __builtin_amdgcn_sched_barrier(0);        // all copies issued before the MFMAs
            bulk_compute(lds + buf * STAGE_BYTES);
            stage_sync();
            buf ^= 1;
            take_scales();
        }
        // the remaining stages (the last bulk stages, then the outlier stages)
        // with general bookkeeping for what comes next: a stage of this tile
        // or the first stage of the next tile.  Bulk and outlier stages run in
        // separate loops so each loop body has one kind of MFMA.
        auto prefetch_next = [&](int s0) {
            const TileOrg nx = tile_org(has_next ? tn : t);
            if (s0 + 1 < S) load_stage(cur, s0 + 1, buf ^ 1);
            else if (has_next) load_stage(nx, 0, buf ^ 1);
            if (s0 + 2 < S) touch(&cur, s0 + 2);
            else if (has_next && s0 + 2 - S < S) touch(&nx, s0 + 2 - S);
            else touch(nullptr, 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        for (; st < S4; ++st) {
            prefetch_next(st);
            bulk_compute(lds + buf * STAGE_BYTES);
            stage_sync();
            buf ^= 1;
            if ((st + 1 < S4) || (st + 1 == S && has_next)) take_scales();
        }
        for (; st < S; ++st) {
            prefetch_next(st);
            outlier_compute(lds + buf * STAGE_BYTES);
            stage_sync();
            buf ^= 1;
            if (st + 1 == S && has_next) take_scales();
        }
        // buffer buf^1 held the last stage and is free; buf holds the next
        // tile's first stage (if any)
        epilogue(cur, lds + (buf ^ 1) * STAGE_BYTES);
        if (!has_next) break;
        t = tn;
        tn += nl;
        cur = tile_org(t);
    }
}

template <typename OutT, bool K8, bool NB8>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
    static thread_local int configured_dev = -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorNoDevice;
    if (configured_dev != dev) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dual_gemm_tiled<OutT, K8, NB8>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES);
        if (e != hipSuccess) return e;
        configured_dev = dev;
    }
    const int T = a.MT * a.NT;
    const int per = (T + NXCD - 1) / NXCD;
    const int cus_per_xcd = device_cu_count() / NXCD;
    const int wg_per_xcd = per < cus_per_xcd ? per : (cus_per_xcd > 0 ? cus_per_xcd : 1);
    hipLaunchKernelGGL((dual_gemm_tiled<OutT, K8, NB8>), dim3((unsigned)(wg_per_xcd * NXCD)), dim3(256),
                       GEMM_LDS_BYTES, st, a);
    return hipGetLastError();
}

template <typename OutT>
static hipError_t launch_tiled_t(const GemmArgs& a, hipStream_t st) {
    const bool k8 = a.k % 8 == 0;
    const bool nb8 = (a.K / 32) % 8 == 0;
    if (k8 && nb8) return launch_tiled<OutT, true, true>(a, st);
    if (k8) return launch_tiled<OutT, true, false>(a, st);
    if (nb8) return launch_tiled<OutT, false, true>(a, st);
    return launch_tiled<OutT, false, false>(a, st);
}

}  // namespace

hipError_t launch_dual_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                            const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                            int32_t N, int32_t K, int32_t k, void* Y, int32_t y_dtype,
                            hipStream_t st) {
    if (M <= 0) return hipSuccess;
    static const char* impl = getenv("MG_GEMM_IMPL");
    if (impl && impl[0] == 's') {   // the straightforward kernel (cross-checks)
        dim3 grid((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
        if (y_dtype == MG_BF16)
            hipLaunchKernelGGL(dual_gemm_simple<uint16_t>, grid, dim3(256), 0, st, Aq, As, XO, Wq, Ws, WO, M, N, K,
                               k, static_cast<uint16_t*>(Y));
        else
            hipLaunchKernelGGL(dual_gemm_simple<float>, grid, dim3(256), 0, st, Aq, As, XO, Wq, Ws, WO, M, N, K, k,
                               static_cast<float*>(Y));
        return hipGetLastError();
    }
    GemmArgs a{Aq, As, XO, Wq, Ws, WO, Y, M, N, K, k, (int32_t)((M + TBM - 1) / TBM), (N + TBN - 1) / TBN};
    return y_dtype == MG_BF16 ? launch_tiled_t<uint16_t>(a, st) : launch_tiled_t<float>(a, st);
}

}  // namespace mg
