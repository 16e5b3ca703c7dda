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
// The operands are stored in fragment order (frag_offset): every 32 rows x 32
// bytes of Aq, Wq, XO, WO -- one A or B operand of either instruction -- is one
// contiguous 1 KB block whose 16-byte lane pieces sit in lane order, so a copy
// moves whole cache lines and a lane's fragment is one conflict-free 16-byte
// LDS read.
#include <type_traits>
#include <utility>

#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

// ---------------------------------------------------------------------------
// Persistent tiled kernel.  One workgroup per CU (NW waves); each walks a
// list of 256x256 output tiles.  Each wave owns 128 rows x 512/NW columns =
// 4 x JB MFMA tiles of 32x32 (16 JB fp32 accumulators per lane, held in the
// accumulation registers).
//
// K is walked in half-stages of two 32-byte K-slices per tile row: a bulk
// half-stage carries 128 FP4 values of Aq / Wq, an outlier half-stage 32 bf16
// values of XO / WO.  A half-stage of a tile is 2 x 8 x 2 fragment blocks
// (A and B, 8 row groups, 2 slices) = 32 KB.  Slice sl of a half-stage is one
// MFMA sub-step: FP4 (32x32x64, scaled) or BF16 (32x32x16), both on the same
// accumulators.  Bulk half-stages come first, outlier half-stages follow.
//
// Pipeline.  The half-stages of all of a workgroup's tiles form one sequence
// over a ring of four 32 KB LDS slots.  While half-stage g is multiplied out
// of slot g % 4, the copies of half-stage g + 2 (which may belong to the next
// tile) run straight from global memory into slot (g + 2) % 4; at the end of
// g each wave waits for the copies of g + 1 only (its NCOPY younger ones
// stay in flight) and the workgroup meets at one barrier.  Two half-stages of lead
// keep the copy path streaming (with one 64 KB stage in flight and waited at
// every stage end it was latency-bound).  Inside a half-stage the issue order
// is fixed slot by slot, one MFMA per slot: the previous half-stage's second
// sub-step (its fragments read before the barrier) fills the first MPS slots,
// so the matrix cores stay busy while this half-stage's first fragments are
// read; the wave's NCOPY copies go one per two slots.
//
// E8M0 scales.  A bulk half-stage needs 4 scale bytes per tile row.  The 16
// bytes of four consecutive bulk half-stages ("a window") of all 512 tile
// rows are copied into LDS with the copies of the window's first
// half-stage, and each wave reads its rows' 4 bytes per half-stage from
// there.  The scale arrays are stored window by window (256 rows x 16 bytes
// contiguous, the tile's rows), so a window of the A (B) tile is 4 KB of
// contiguous memory: one 16-byte load per lane and row, 8 cache lines per
// load instruction.  Windows rotate over three LDS slots: a window is issued
// two half-stages before its first use, and the two windows between it and
// the previous occupant of its slot span at least two half-stages, so the
// occupant's last read is at least one barrier older than the overwrite
// (with two slots a tile ending one half-stage into a window -- k = 0 and
// K mod 512 in (0, 128] -- would have its window overwritten while read).
//
// After a tile's last half-stage its 256x256 bf16 result is staged through
// the two ring slots that hold no pending copy and written as whole 512-byte
// rows while the next tile's first half-stage already sits in LDS.
// A third epilogue (QuantOut) joins the FFN block's two projections: the
// staged bf16 tile goes through GELU-tanh and the next projection's
// activation quantizer (its channels are this tile's columns) instead of
// being written, producing the bytes that the bf16 output followed by the
// fused GELU + quantize pass would.
// Operand rows past M (or N) and slices past K / k read as zeros through
// buffer range checks.  Tiles are dealt so that each XCD (workgroups go
// round-robin to the 8 XCDs) walks a contiguous run of the tile order,
// grouped 8 row-tiles at a time, which keeps the operand panels of its
// concurrently running tiles in its L2.
// ---------------------------------------------------------------------------

constexpr int TBM = 256, TBN = 256;
constexpr int NRG = TBM / kFragRows;                  // row groups per tile operand (8)
constexpr int HS_SL = 2;                              // K-slices per half-stage
constexpr int OP_BYTES = NRG * HS_SL * kFragBlock;    // one operand of a half-stage (16 KB)
constexpr int HS_BYTES = 2 * OP_BYTES;                // A + B (32 KB)
constexpr int RING = 4;                               // LDS slots
constexpr int LEAD = 2;                               // half-stages copied ahead
// Waves per workgroup, 2 along M x NW/2 along N.  With 8 (two per SIMD, 128
// accumulators each) the matrix cores are busier than with 4 (one per SIMD,
// 256 accumulators) but every fragment is read by more waves; the kernel is
// written for both and runs 8, which measured 0.4-0.7 % faster.
#ifndef MG_GEMM_WAVES
#define MG_GEMM_WAVES 8
#endif
constexpr int NW = MG_GEMM_WAVES;
constexpr int JB = 16 / NW;                           // 32-column B blocks per wave (4 or 2)
constexpr int RPW = 8 / NW;                           // row groups per operand a wave copies
constexpr int NCOPY = 2 * NRG * HS_SL / NW;           // copies per wave and half-stage (8 or 4)
constexpr int MPS = 4 * JB;                           // MFMAs per wave and K-slice
constexpr int SCW_ROWB = 16;                          // scale bytes per row per window (4 half-stages)
constexpr int SCW_BYTES = (TBM + TBN) * SCW_ROWB;     // one window slot: A rows then B rows (8 KB)
constexpr int SCW_SLOTS = 3;
constexpr int SCW_OFF = RING * HS_BYTES;
constexpr int GEMM_LDS_BYTES = SCW_OFF + SCW_SLOTS * SCW_BYTES;   // 152 KB
constexpr uint32_t OOB = 0xC0000000u;                 // offset that reads as zero
constexpr int NXCD = 8;
constexpr int GROUP_M = 8;
static_assert(TBM == kScRows && TBN == kScRows && SCW_ROWB == kScBlocks, "a tile's scale window is one stored window");
static_assert(kScBlocks == 4 * HS_SL * 2, "a window holds the scale bytes of four half-stages");
static_assert(LEAD == 2 && NCOPY * NW == 32, "the end-of-half-stage wait keeps exactly one half-stage of copies in flight");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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

// f(integral_constant<int, Q>) for Q = 0 .. N-1, expanded at compile time
template <typename F, int... Qs>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Qs...>) {
    (f(std::integral_constant<int, Qs>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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
    // GELU + quantize epilogue (QuantOut): the next layer's plan (input width
    // N) and activation workspace
    const float* s2;
    const float* rcp2;
    const int32_t* pos2;
    uint8_t* Aq2;
    uint8_t* As2;
    uint8_t* XO2;
    int32_t k2;
};

// Output tag of the epilogue that applies GELU to the bf16-rounded tile and
// quantizes it as the next layer's activation, instead of writing Y.
struct QuantOut {};

// Per-tile lane constants of the GELU + quantize epilogue: the lane's 8
// channels' s, fast-path reciprocals (0 on outlier channels) and outlier
// routing, and its byte offsets inside the tile's part of Aq, XO, As.
struct QuantLane {
    float sv[8], rz[8];
    float so, ro;
    uint32_t omask, nkeep, a0_lim;
    uint32_t offAq, offXO, offAs, ns4, nso;
    int oc0, cj0, wave_o, wave_rest;
    bool valid;
};

// The GELU + quantize epilogue's arguments, read from the kernel-argument
// segment once per tile through a pointer the compiler cannot see through
// (kernargs_per_tile), so that neither they nor the sizes derived from them
// are held in scalar registers across the tile loop's K steps (which would
// spill them there).  The kernel's one parameter, a GemmArgs passed by value,
// is the start of that segment.
struct QuantArgs {
    const float* s2;
    const float* rcp2;
    const int32_t* pos2;
    uint8_t* Aq2;
    uint8_t* As2;
    uint8_t* XO2;
    int64_t M;
    int32_t N, k2;
};
typedef const __attribute__((address_space(4))) GemmArgs* KernargPtr;
__device__ __forceinline__ QuantArgs kernargs_per_tile() {
    KernargPtr p = (KernargPtr)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(p));
    return QuantArgs{p->s2, p->rcp2, p->pos2, p->Aq2, p->As2, p->XO2, p->M, p->N, p->k2};
}

// bytes of a buffer of `total` bytes from offset `from` on (0 past its end)
__device__ __forceinline__ uint64_t rest_bytes(int64_t total, int64_t from) {
    return total > from ? (uint64_t)(total - from) : 0u;
}
__device__ __forceinline__ uint64_t min_u64(uint64_t a, uint64_t b) { return a < b ? a : b; }

// Origin of an output tile (wave-uniform).
struct TileOrg {
    int64_t m0;
    int n0;
};

template <typename OutT>
__global__ void __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
dual_gemm_tiled(GemmArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar)
    const int wm = wave / (NW / 2), wn = wave % (NW / 2);
    const int h = lane >> 5;
    const int l32 = lane & 31;

    const int K = g.K, k = g.k, N = g.N;
    const int64_t M = g.M;
    const uint32_t ns4 = (uint32_t)frag_slices(K / 2);          // K-slices of a bulk row
    const uint32_t nso = (uint32_t)frag_slices(2 * (int64_t)k); // K-slices of an outlier row
    const int H4 = (int)(ns4 + 1) / 2;                          // bulk half-stages per tile
    const int H = H4 + (int)(nso + 1) / 2;                      // all half-stages per tile

    // ---- this workgroup's tiles: XCD x owns tiles [x per, (x+1) per); its
    // workgroups take every nl-th one.
    const int T = g.MT * g.NT;
    const int per = (T + NXCD - 1) / NXCD;
    const int nl = (int)gridDim.x / NXCD;
    const int xcd = (int)blockIdx.x % NXCD;
    const int t_end = min((xcd + 1) * per, T);
    int t = xcd * per + (int)blockIdx.x / NXCD;
    if (t >= t_end) return;

    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.Aq, (uint64_t)frag_bytes(M, K / 2));
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.Wq, (uint64_t)frag_bytes(N, K / 2));
    const __amdgpu_buffer_rsrc_t rAs = make_rsrc(g.As, (uint64_t)sc_bytes(M, K));
    const __amdgpu_buffer_rsrc_t rBs = make_rsrc(g.Ws, (uint64_t)sc_bytes(N, K));
    const uint32_t nwin = (uint32_t)sc_nwin(K);
    const __amdgpu_buffer_rsrc_t rXO = make_rsrc(g.XO, (uint64_t)frag_bytes(M, 2 * (int64_t)k));
    const __amdgpu_buffer_rsrc_t rWO = make_rsrc(g.WO, (uint64_t)frag_bytes(N, 2 * (int64_t)k));
    // row groups of the operands; tile row groups past them are clamped to
    // the last one (their rows only feed output rows / columns past M / N,
    // which are never stored)
    const int GA = (int)((M + kFragRows - 1) / kFragRows), GB = N / kFragRows;

    // ---- tile-independent lane constants.  A copy moves one 1 KB fragment
    // block (lane L: bytes 16 L .. 16 L + 15, landing at byte 16 L of the
    // block's LDS place).  Wave w copies row groups RPW w .. RPW w + RPW - 1
    // of the A and of the B tile, slices 0 and 1 of the half-stage: block
    // (operand, row group rg, slice sl) of a slot sits at operand * 16 KB +
    // (2 rg + sl) * 1 KB.  The block's global offset goes into the scalar offset, slice 1
    // into the instruction offset (which moves the global and the LDS
    // address alike), the lane's 16 L into the vector offset.
    const uint32_t l16 = (uint32_t)lane * 16u;
    // scale windows: lane L of wave w copies window row 64 w + L of A and of
    // B (NW = 4), or of A (w < 4) or B (NW = 8); a lane reads the 2 codes of a half-stage (slices 0, 1 of its half of
    // the K steps) of each of its fragment rows at these offsets (+ 512 i,
    // + 2 (half-stage % 4)): row * 16 + 8 h
    const uint32_t lwr = (uint32_t)((NW == 4 ? wave : wave & 3) * 64 + lane) * SCW_ROWB;
    const uint32_t scw_a = (uint32_t)((wm * 128 + l32) * SCW_ROWB + 8 * h);
    const uint32_t scw_b = (uint32_t)(TBM * SCW_ROWB + (wn * 32 * JB + l32) * SCW_ROWB + 8 * h);
    // fragment reads: A row group 4 wm + i, B row group 4 wn + j
    const uint32_t fa0 = (uint32_t)(wm * 4 * HS_SL * kFragBlock) + l16;
    const uint32_t fb0 = (uint32_t)(OP_BYTES + wn * JB * HS_SL * kFragBlock) + l16;

    auto tile_org = [&](int tt) {
        TileOrg o;
        const int grp = tt / (GROUP_M * g.NT);
        const int gsz = min(GROUP_M, g.MT - grp * GROUP_M);
        const int rin = tt - grp * GROUP_M * g.NT;
        o.m0 = (int64_t)__builtin_amdgcn_readfirstlane((grp * GROUP_M + rin % gsz) * TBM);
        o.n0 = __builtin_amdgcn_readfirstlane((rin / gsz) * TBN);
        return o;
    };

    v16f acc[4][JB];
    uint32_t scA[4], scB[JB], pA[4], pB[JB];
    int wiss = 0;      // slot of the next scale window to issue (0, 1, 2, 0, ...)
    int wnext = 0;     // slot of the next scale window to take into use
    int wcur = 0;      // slot of the window of the current bulk half-stage

    // ---- copy cursor: the next half-stage to copy -- tile ct, half-stage
    // cst, origin corg -- and its source: the resources of the A and B
    // operands (bulk or outlier) and the global offsets of its slice-0
    // blocks in this wave's RPW A and RPW B row groups.  `issued`
    // half-stages have been copied, into ring slots issued % 4.  Wave-uniform
    // (scalar registers); inside a tile's bulk or outlier run an advance is
    // four scalar adds.
    int ct = t, cst = 0, issued = 0;
    TileOrg corg = tile_org(t);
    __amdgpu_buffer_rsrc_t csA = rA, csB = rB;
    uint32_t cA0 = 0, cA1 = 0, cB0 = 0, cB1 = 0;
    auto cursor_src = [&]() {        // sources of half-stage cst of tile ct (ct < t_end)
        const bool bulk = cst < H4;
        const uint32_t ns = bulk ? ns4 : nso;
        const uint32_t s0 = (uint32_t)(2 * (bulk ? cst : cst - H4)) * (uint32_t)kFragBlock;
        const int ga = (int)(corg.m0 / kFragRows) + RPW * wave, gb = corg.n0 / kFragRows + RPW * wave;
        csA = bulk ? rA : rXO;
        csB = bulk ? rB : rWO;
        cA0 = (uint32_t)min(ga, GA - 1) * ns * (uint32_t)kFragBlock + s0;
        cA1 = (uint32_t)min(ga + 1, GA - 1) * ns * (uint32_t)kFragBlock + s0;
        cB0 = (uint32_t)min(gb, GB - 1) * ns * (uint32_t)kFragBlock + s0;
        cB1 = (uint32_t)min(gb + 1, GB - 1) * ns * (uint32_t)kFragBlock + s0;
    };
    cursor_src();

    // scale window w (bulk half-stages 4w .. 4w+3) of a tile into the next
    // slot: the stored windows of the tile's 256 A rows and 256 B rows (4 KB each)
    auto load_window = [&](const TileOrg& o, int w) {
        const int slot = wiss;
        wiss = wiss == SCW_SLOTS - 1 ? 0 : wiss + 1;
        uint8_t* dst = lds + SCW_OFF + slot * SCW_BYTES + wave * 64 * SCW_ROWB;
        const uint32_t wa = __builtin_amdgcn_readfirstlane(((uint32_t)(o.m0 / TBM) * nwin + (uint32_t)w) * kScWinBytes);
        const uint32_t wb = __builtin_amdgcn_readfirstlane(((uint32_t)(o.n0 / TBN) * nwin + (uint32_t)w) * kScWinBytes);
        if constexpr (NW == 4) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, (lds_ptr_t)dst, 16, lwr, wa, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, (lds_ptr_t)(dst + TBM * SCW_ROWB), 16, lwr, wb, 0, 0);
        } else {
            // waves 0-3: A rows 64 w .., waves 4-7: B rows 64 (w - 4) .. (dst already at the B half)
            if (wave < 4) __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, (lds_ptr_t)dst, 16, lwr, wa, 0, 0);
            else          __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, (lds_ptr_t)dst, 16, lwr, wb, 0, 0);
        }
    };
    // does the cursor's half-stage open a scale window?
    auto cursor_opens_window = [&]() { return ct < t_end && cst < H4 && (cst & 3) == 0; };
    // copy c = 2 RPW op + 2 r + sl of the cursor's half-stage into its ring
    // slot: row group RPW w + r of operand A (op 0) or B (op 1), slice sl
    // (fast: the cursor is known to be in the bulk part, whose resources are
    // rA and rB)
    auto copy_part = [&](int c, bool fast) {
        const int op = c / (2 * RPW), r = (c >> 1) % RPW, sl = c & 1;
        uint8_t* dst = lds + (issued & (RING - 1)) * HS_BYTES + op * OP_BYTES + (2 * (RPW * wave + r)) * kFragBlock;
        const uint32_t so = op ? (r ? cB1 : cB0) : (r ? cA1 : cA0);
        const __amdgpu_buffer_rsrc_t rs = fast ? (op ? rB : rA) : (op ? csB : csA);
        if (sl)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, l16, so, kFragBlock, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, l16, so, 0, 0);
    };
    // after the wave's copies: the cursor moves to the next half-stage (past the
    // last tile it stays put: its copies then re-read valid memory into a
    // free slot)
    auto advance_fast = [&]() {      // the cursor stays in the same tile's bulk part
        ++issued;
        ++cst;
        cA0 += 2 * kFragBlock; cA1 += 2 * kFragBlock; cB0 += 2 * kFragBlock; cB1 += 2 * kFragBlock;
    };
    auto advance = [&]() {
        ++issued;
        if (ct >= t_end) return;
        ++cst;
        if (cst == H) {
            cst = 0;
            ct += nl;
            if (ct >= t_end) return;
            corg = tile_org(ct);
            cursor_src();
        } else if (cst == H4) {
            cursor_src();
        } else {
            cA0 += 2 * kFragBlock; cA1 += 2 * kFragBlock; cB0 += 2 * kFragBlock; cB1 += 2 * kFragBlock;
        }
    };

    // End of a half-stage: this wave's copies of the next half-stage have
    // landed (the NCOPY younger ones, of the half-stage after it, stay in
    // flight; loads complete in order) and its reads of the current slot are
    // done, then every wave arrives.  The scheduling barriers keep the MFMAs
    // above the wait, so they run while copies fly.
    auto stage_sync = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (NCOPY == 8)
            asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- this lane's scale codes of a bulk half-stage (from its window):
    // byte 0 = slice 0, byte 1 = slice 1 (the MFMA's op_sel = slice)
    auto read_scale = [&](const uint8_t* wsc, int q) {
        if (q < 4) scA[q] = *reinterpret_cast<const uint16_t*>(wsc + scw_a + q * 32 * SCW_ROWB);
        else       scB[q - 4] = *reinterpret_cast<const uint16_t*>(wsc + scw_b + (q - 4) * 32 * SCW_ROWB);
    };

    // ---- one half-stage in a fixed issue order of one slot per MFMA (MPS =
    // 4 JB MFMAs per slice):
    //   0 .. MPS-1        the previous half-stage's slice 1 (kind DK: 0 none,
    //                     1 FP4, 2 BF16); its first 4 + JB slots also read
    //                     slice 0's fragments (A0, B0 .. B(JB-1), A1 A2 A3,
    //                     the order its MFMAs need them) and the half-stage's
    //                     scale codes;
    //   MPS .. 2 MPS-1    slice 0; its first 4 + JB slots read slice 1's
    //                     fragments;
    //   2 MPS .. 3 MPS-1  slice 1 when it is not deferred (the last bulk
    //                     half-stage of a tile, and every outlier half-stage).
    // Slot 1 opens the cursor's scale window (if it starts one), slots 2,
    // 4, .., 2 NCOPY issue its copies: never two memory instructions back to
    // back, so the address unit is shared evenly between the waves.
    u32x4 pf[2][2][4];                 // fragment sets [set = slice][A/B][i]
    auto frag_read = [&](const uint8_t* base, int sl, int q) {
        const bool isA = q == 0 || q > JB;
        const int r = q == 0 ? 0 : (q <= JB ? q - 1 : q - JB);
        const uint32_t off = (uint32_t)(r * HS_SL * kFragBlock + sl * kFragBlock);
        if (isA) pf[sl][0][r] = *reinterpret_cast<const u32x4*>(base + fa0 + off);
        else     pf[sl][1][r] = *reinterpret_cast<const u32x4*>(base + fb0 + off);
    };
    // FAST: the cursor copies a bulk half-stage of the current tile and
    // stays in its bulk part (no transition in the advance).
    auto run_hs = [&](auto CUR_BULK, auto DK, auto DEFER_OUT, auto FAST, int hs, int slot) {
        constexpr bool cb = decltype(CUR_BULK)::value;
        constexpr int dk = decltype(DK)::value;
        constexpr bool dout = decltype(DEFER_OUT)::value;
        constexpr bool fast = decltype(FAST)::value;
        const uint8_t* base = lds + slot * HS_BYTES;
        const uint8_t* wsc = nullptr;
        if constexpr (cb) {
            if ((hs & 3) == 0) {
                wcur = wnext;
                wnext = wnext == SCW_SLOTS - 1 ? 0 : wnext + 1;
            }
            wsc = lds + SCW_OFF + wcur * SCW_BYTES + 2 * (hs & 3);
        }
        const bool opens_window = fast ? (cst & 3) == 0 : cursor_opens_window();
        static_for<3 * MPS>([&](auto QC) {
            constexpr int q = decltype(QC)::value;
            if constexpr (q < 2 * MPS || !dout) {
                if constexpr (q < MPS) {
                    constexpr int i = q / JB, j = q % JB;
                    if constexpr (dk == 1)
                        acc[i][j] = mfma_fp4_op<1>(pf[1][1][j], pf[1][0][i], pB[j], pA[i], acc[i][j]);
                    else if constexpr (dk == 2)
                        acc[i][j] = mfma_bf16_v(pf[1][1][j], pf[1][0][i], acc[i][j]);
                } else {
                    constexpr int sl = (q - MPS) / MPS, r = (q - MPS) % MPS, i = r / JB, j = r % JB;
                    if constexpr (cb)
                        acc[i][j] = mfma_fp4_op<sl>(pf[sl][1][j], pf[sl][0][i], scB[j], scA[i], acc[i][j]);
                    else
                        acc[i][j] = mfma_bf16_v(pf[sl][1][j], pf[sl][0][i], acc[i][j]);
                }
                if constexpr (q < 4 + JB) {
                    if constexpr (cb) read_scale(wsc, q);
                    frag_read(base, 0, q);
                }
                if constexpr (q >= MPS && q < MPS + 4 + JB) frag_read(base, 1, q - MPS);
                if constexpr (q == 1) {
                    if (opens_window) load_window(corg, cst >> 2);
                }
                if constexpr (q >= 2 && q <= 2 * NCOPY && q % 2 == 0) copy_part((q - 2) >> 1, fast);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (fast)
            advance_fast();
        else
            advance();
        if constexpr (cb && dout) {
#pragma unroll
            for (int i = 0; i < 4; ++i) pA[i] = scA[i];
#pragma unroll
            for (int j = 0; j < JB; ++j) pB[j] = scB[j];
        }
        stage_sync();
    };

    // ---- GELU + quantize epilogue (QuantOut).  The staged bf16 tile is the
    // next layer's input h = GELU(bf16(Y)) before the GELU: its columns are
    // that layer's input channels.  A lane takes 8 consecutive channels of a
    // row (one staged 16-byte piece), 4 lanes one 32-block, as in the
    // activation quantizer, and produces the same bits as GELU-then-quantize
    // of the bf16 output: the same GELU function, the quotient RN(h / s)
    // (Markstein's correction under the quantizer's checks, else the
    // correctly rounded division), E8M0 of the block maximum, the hardware
    // E2M1 converter; outlier channels go to XO as bf16 and +0 into the bulk.
    // Rows past M and channels past N are zeros (their accumulators are not
    // the layer's); the codes of pad rows and pad slices land inside the
    // buffers' pads, the rest outside the resources' ranges.
    auto quant_lane = [&](const QuantArgs& qa, int cj0, bool cvalid, uint32_t ln) {
        QuantLane L;
        float rv[8];
        int pv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) { L.sv[i] = 1.0f; rv[i] = 1.0f; pv[i] = -1; }
        if (cvalid) {
#pragma unroll
            for (int h4 = 0; h4 < 2; ++h4) {
                const float4 a = *reinterpret_cast<const float4*>(qa.s2 + cj0 + 4 * h4);
                const float4 b = *reinterpret_cast<const float4*>(qa.rcp2 + cj0 + 4 * h4);
                const int4 c = *reinterpret_cast<const int4*>(qa.pos2 + cj0 + 4 * h4);
                L.sv[4 * h4] = a.x; L.sv[4 * h4 + 1] = a.y; L.sv[4 * h4 + 2] = a.z; L.sv[4 * h4 + 3] = a.w;
                rv[4 * h4] = b.x; rv[4 * h4 + 1] = b.y; rv[4 * h4 + 2] = b.z; rv[4 * h4 + 3] = b.w;
                pv[4 * h4] = c.x; pv[4 * h4 + 1] = c.y; pv[4 * h4 + 2] = c.z; pv[4 * h4 + 3] = c.w;
            }
        }
        uint32_t om = 0;
        bool s_ok = true;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            om |= (pv[i] >= 0 ? 1u : 0u) << i;
            s_ok &= div_fast_ok_s(L.sv[i]);
        }
        L.omask = om;
        L.nkeep = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            L.rz[i] = (om >> i) & 1u ? 0.0f : rv[i];
            L.nkeep |= ((om >> i) & 1u ? 0u : 0xFu) << (4 * i);
        }
        const int oc0 = om ? __builtin_ctz(om) : 0;
        L.oc0 = oc0;
        L.so = L.sv[0]; L.ro = rv[0];
        int op0 = pv[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) {
            L.so = oc0 == i ? L.sv[i] : L.so;
            L.ro = oc0 == i ? rv[i] : L.ro;
            op0 = oc0 == i ? pv[i] : op0;
        }
        L.a0_lim = s_ok ? kF32Pow126 : 0u;
        L.valid = cvalid;
        L.cj0 = cj0;
        L.wave_o = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64(om != 0) != 0));
        L.wave_rest = __builtin_amdgcn_readfirstlane((int)(__builtin_amdgcn_ballot_w64((om & (om - 1)) != 0) != 0));
        // byte offsets inside the tile's part of each buffer, the row's part
        // (16 per row of the 32-row group, 1 KB blocks per group) added per row
        const uint32_t ns4b = (uint32_t)frag_slices(qa.N / 2), nsob = (uint32_t)frag_slices(2 * (int64_t)qa.k2);
        const uint32_t b = (uint32_t)cj0 / 2u;
        L.offAq = (b >> 5) * 1024u + ((b >> 4) & 1u) * 512u + (b & 15u);
        const uint32_t bo = 2u * (uint32_t)op0;
        L.offXO = om ? (bo >> 5) * 1024u + ((bo >> 4) & 1u) * 512u + (bo & 15u) : OOB;
        const int blk = cj0 / 32;
        L.offAs = (ln & 3u) == 0u ? (uint32_t)(blk / kScBlocks) * kScWinBytes + (uint32_t)sc_pos(blk) : OOB;
        L.ns4 = ns4b; L.nso = nsob;
        return L;
    };
    // row piece of tile row mt = mu + rl (0..255): w the staged bf16 words
    // (before GELU).  mu is wave-uniform and a multiple of 64 / CH, and
    // rl < 64 / CH, so the row's 32-row group (mu / 32) is wave-uniform and
    // the buffer resources below are formed in scalar registers.
    auto quant_octet = [&](const QuantArgs& qa, const QuantLane& L, const TileOrg& o, u32x4 w, uint32_t mu,
                           uint32_t rl) {
        const uint32_t mt = mu + rl;
        const int64_t m = o.m0 + mt;
        const bool live = m < qa.M && L.valid;
        // zeros for rows past M and channels past N (GELU(0) = 0), with no branch
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = gelu_bf16x2(live ? w[i] : 0u);
        const int wave_o = L.wave_o;
        float q[8];
        float a0 = 0.0f, aq = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t wi = w[i >> 1];
            const float x = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
            const float q0 = x * L.rz[i];
            const float t = __builtin_fmaf(q0, L.sv[i], -x);
            q[i] = __builtin_fmaf(-t, L.rz[i], q0);
            a0 = fmaxf(a0, __builtin_fabsf(q0));
            aq = fmaxf(aq, __builtin_fabsf(q[i]));
        }
        uint32_t qb = quad_max_bits(__float_as_uint(aq));
        uint64_t bad = __builtin_amdgcn_uicmp(__float_as_uint(a0), L.a0_lim, kCmpUGE) |
                       __builtin_amdgcn_uicmp(qb - 1u, kF32PowM74 - 1u, kCmpULT);
        float xo = 0.0f, qo = 0.0f;
        if (wave_o) {
            uint32_t wo = w[0];
#pragma unroll
            for (int i = 1; i < 4; ++i) wo = (L.oc0 >> 1) == i ? w[i] : wo;
            xo = __uint_as_float((L.oc0 & 1) ? (wo & 0xFFFF0000u) : (wo << 16));
            qo = div_fast(xo, L.so, L.ro);
            const uint32_t ab = __float_as_uint(qo) & 0x7FFFFFFFu;
            bad |= __builtin_amdgcn_uicmp(L.omask ? ab - kF32PowM78 : 0u, kF32Pow126 - kF32PowM78, kCmpUGE) &
                   __builtin_amdgcn_uicmp(ab, 0u, kCmpNE);
        }
        if (bad) {
            aq = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t wi = w[i >> 1];
                const float x = (L.omask >> i) & 1u ? 0.0f : __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                q[i] = __fdiv_rn(x, L.sv[i]);
                aq = fmaxf(aq, __builtin_fabsf(q[i]));
            }
            qb = quad_max_bits(__float_as_uint(aq));
            if (wave_o) qo = __fdiv_rn(xo, L.so);
        }
        // the tile's row group and the row inside it
        const uint32_t rg = mu >> 5, rin = (mt & 31u) << 4;
        if (wave_o) {
            // the row's 32-row group of XO (its nso blocks; none past the last group)
            const int64_t xo0 = (o.m0 / 32 + rg) * (int64_t)L.nso * kFragBlock;
            const __amdgpu_buffer_rsrc_t rxo = make_rsrc(
                qa.XO2 + xo0, min_u64(rest_bytes(frag_bytes(qa.M, 2 * (int64_t)qa.k2), xo0), (uint64_t)L.nso * kFragBlock));
            __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qo), rxo, L.offXO + rin, 0, 0);
            // further outlier channels of the lane (two or more in its 8): exact division
            if (L.wave_rest) {
                for (uint32_t mm = L.omask & (L.omask - 1); mm; mm &= mm - 1) {
                    const int i = __builtin_ctz(mm);
                    const uint32_t wi = w[i >> 1];
                    const float xi = __uint_as_float((i & 1) ? (wi & 0xFFFF0000u) : (wi << 16));
                    const float qi = __fdiv_rn(xi, qa.s2[L.cj0 + i]);
                    const uint32_t bi = 2u * (uint32_t)qa.pos2[L.cj0 + i];
                    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)f32_to_bf16_rne(qi), rxo,
                                                          (bi >> 5) * 1024u + ((bi >> 4) & 1u) * 512u + (bi & 15u) + rin,
                                                          0, 0);
                }
            }
        }
        const int32_t sb = __builtin_elementwise_max((int32_t)(qb & 0x7F800000u) - (2 << 23), 0x00200000);
        const float scale = __int_as_float(sb);
        uint32_t word = 0;
        MG_CVT_FP4X2(word, q[0], q[1], scale, 0);
        MG_CVT_FP4X2(word, q[2], q[3], scale, 1);
        MG_CVT_FP4X2(word, q[4], q[5], scale, 2);
        MG_CVT_FP4X2(word, q[6], q[7], scale, 3);
        const int64_t gb = o.m0 / 32 + rg;           // the row's 32-row group
        // the row's 32-row group of Aq (its ns4 blocks: slices past them, of
        // channels past the padded row, fall outside the range)
        const int64_t aq0 = gb * (int64_t)L.ns4 * kFragBlock;
        const __amdgpu_buffer_rsrc_t raq = make_rsrc(
            qa.Aq2 + aq0, min_u64(rest_bytes(frag_bytes(qa.M, qa.N / 2), aq0), (uint64_t)L.ns4 * kFragBlock));
        __builtin_amdgcn_raw_buffer_store_b32(word & L.nkeep, raq, L.offAq + rin, 0, 0);
        const __amdgpu_buffer_rsrc_t ras =
            make_rsrc(qa.As2 + (o.m0 / kScRows) * sc_nwin(qa.N) * kScWinBytes, (uint64_t)sc_nwin(qa.N) * kScWinBytes);
        __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(sb >> 23), ras, L.offAs + mt * (uint32_t)kScBlocks, 0, 0);
    };

    // ---- epilogue of one tile.  The MFMAs take the weight fragment as their
    // first operand, so acc[i][j] holds Y^T for A row-tile i and W row-tile j:
    // lane (l32, h), register 4 q + e holds output row 32 i + l32 and output
    // column 32 j + 8 q + 4 h + e of this wave's part -- four consecutive
    // columns per register group.
    auto epilogue = [&](const TileOrg& o, uint8_t* wbuf) {
        if constexpr (std::is_same_v<OutT, uint16_t> || std::is_same_v<OutT, QuantOut>) {
            // bf16: round pairs with the hardware converter (nearest even).
            // Each wave stages its own 128 x 32 JB part through its own
            // 64 KB / NW of a free ring slot pair (wbuf), 64 rows x 64 JB
            // bytes per pass, and writes the rows back out with 16-byte
            // streaming stores (whole 64 JB-byte row pieces).  No wave reads
            // another wave's staging, so a pass needs no barrier: one wave's
            // LDS accesses are processed in order.  In a staged row r the
            // 16-byte chunk c (columns 8c .. 8c+7 of the part) sits at chunk
            // c ^ (r % (4 JB)).
            // the tile's rows of Y: rows past M are out of the descriptor's
            // range and columns past N get an out-of-range offset, so the
            // stores need no branches
            const uint32_t rowY = (uint32_t)N * 2u;
            const int64_t rows_left = M - o.m0;
            const uint32_t nrec = (uint32_t)(rows_left < TBM ? rows_left : TBM) * rowY;
            const __amdgpu_buffer_rsrc_t rY =
                make_rsrc(static_cast<uint16_t*>(g.Y) + o.m0 * (int64_t)N, (uint64_t)nrec);
            // Lane-dependent values come from an opaque copy of the thread
            // index, so they are formed here, once per tile, instead of being
            // hoisted out of the tile loop and held (or spilled) across it.
            uint32_t et = (uint32_t)tid;
            asm volatile("" : "+v"(et));
            const uint32_t el32 = et & 31u, eh = (et >> 5) & 1u;
            constexpr uint32_t CH = 4 * JB, RBY = 64 * JB;      // chunks and bytes per staged row
            const uint32_t rl = (et & 63u) / CH, cl = et & (CH - 1);  // read side: row (of 64 / CH), chunk
            const int gcol = o.n0 + wn * 32 * JB + (int)cl * 8;
            const bool col_ok = gcol < N;
            const uint32_t cofs = (uint32_t)gcol * 2u;
            [[maybe_unused]] QuantArgs qa;
            [[maybe_unused]] QuantLane ql;
            if constexpr (std::is_same_v<OutT, QuantOut>) {
                qa = kernargs_per_tile();
                ql = quant_lane(qa, gcol, col_ok, (uint32_t)(et & 63u));
            }
#pragma unroll
            for (int p = 0; p < 2; ++p) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = 2 * p + ii;
                    // read row-block i's accumulators here, not earlier
#pragma unroll
                    for (int j = 0; j < JB; ++j) asm volatile("" : "+a"(acc[i][j]));
                    const uint32_t r = (uint32_t)(32 * ii) + el32;
                    const uint32_t rb = r * RBY + eh * 8, rs = r & (CH - 1);
#pragma unroll
                    for (int j = 0; j < JB; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x2 lo = {acc[i][j][4 * q], acc[i][j][4 * q + 1]};
                            const f32x2 hi = {acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
                            *reinterpret_cast<u32x2*>(wbuf + rb + ((((uint32_t)(4 * j + q)) ^ rs) << 4)) = w;
                        }
                }
                if constexpr (std::is_same_v<OutT, QuantOut>) {
                    // row pieces of the staged bf16 rows (lane: 8 columns of a row), each
                    // through GELU and the next layer's quantizer
                    for (int sI = 0; sI < (int)CH; ++sI) {
                        const uint32_t rr = (uint32_t)(64 / CH * sI) + rl;
                        const u32x4 w = *reinterpret_cast<const u32x4*>(wbuf + rr * RBY + ((cl ^ (rr & (CH - 1))) << 4));
                        quant_octet(qa, ql, o, w, (uint32_t)(wm * 128 + 64 * p + 64 / CH * sI), rl);
                    }
                } else {
                    u32x4 v[CH];
#pragma unroll
                    for (int sI = 0; sI < (int)CH; ++sI) {
                        const uint32_t rr = (uint32_t)(64 / CH * sI) + rl;
                        v[sI] = *reinterpret_cast<const u32x4*>(wbuf + rr * RBY + ((cl ^ (rr & (CH - 1))) << 4));
                    }
#pragma unroll
                    for (int sI = 0; sI < (int)CH; ++sI) {
                        const uint32_t rr = (uint32_t)(64 / CH * sI) + rl;
                        const uint32_t off = col_ok ? ((uint32_t)(wm * 128 + 64 * p) + rr) * rowY + cofs : OOB;
                        // streaming store (nt): Y is written once and must not
                        // push the operand panels out of L2
                        __builtin_amdgcn_raw_buffer_store_b128(v[sI], rY, off, 0, 2);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            // every wave's staging reads are done (their data fed the stores
            // above) before the next copies reuse the slots
            __builtin_amdgcn_s_barrier();
        } else {
            // fp32: four consecutive columns per register group -> 16-byte stores
            float* Yf = static_cast<float*>(g.Y);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t row = o.m0 + wm * 128 + 32 * i + l32;
#pragma unroll
                for (int j = 0; j < JB; ++j)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int col = o.n0 + wn * 32 * JB + 32 * j + 8 * q + 4 * h;
                        if (row < M && col < N) {
                            const f32x4 v = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                                             acc[i][j][4 * q + 3]};
                            __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(Yf + row * N + col));
                        }
                    }
            }
        }
    };


    // ---- prologue: the first two half-stages (and the first scale window)
    for (int p = 0; p < LEAD; ++p) {
        if (cursor_opens_window()) load_window(corg, cst >> 2);
#pragma unroll
        for (int c = 0; c < NCOPY; ++c) copy_part(c, false);
        advance();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NCOPY == 8)
        asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    TileOrg cur = tile_org(t);
    int gs = 0;        // half-stages computed so far (the current one's slot: gs % 4)

    using T_ = std::true_type;
    using F_ = std::false_type;
    using D0 = std::integral_constant<int, 0>;
    using D1 = std::integral_constant<int, 1>;
    while (true) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j) acc[i][j] = v16f{};
        // bulk half-stages, each leaving its slice 1 to the next.  While hs
        // + 3 < H4 the copies (two half-stages ahead) stay in this tile's
        // bulk part: the fast cursor step.
        run_hs(T_{}, D0{}, T_{}, F_{}, 0, gs & (RING - 1));
        ++gs;
        int hs = 1;
        for (; hs + 3 < H4; ++hs) {
            run_hs(T_{}, D1{}, T_{}, T_{}, hs, gs & (RING - 1));
            ++gs;
        }
        for (; hs < H4; ++hs) {
            run_hs(T_{}, D1{}, T_{}, F_{}, hs, gs & (RING - 1));
            ++gs;
        }
        // the last bulk half-stage's slice 1
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < JB; ++j)
                acc[i][j] = mfma_fp4_op<1>(pf[1][1][j], pf[1][0][i], pB[j], pA[i], acc[i][j]);
        // outlier half-stages, each complete in itself
        for (; hs < H; ++hs) {
            run_hs(F_{}, D0{}, F_{}, F_{}, hs, gs & (RING - 1));
            ++gs;
        }
        // the slots of the last two half-stages, (gs - 1) % 4 and (gs - 2) % 4,
        // hold no pending copy: the first half of the waves stage their
        // output through the first, the second half through the second
        {
            const int fs = (wave < NW / 2 ? gs - 1 : gs - 2) & (RING - 1);
            epilogue(cur, lds + fs * HS_BYTES + (wave % (NW / 2)) * (HS_BYTES / (NW / 2)));
        }
        t += nl;
        if (t >= t_end) break;
        cur = tile_org(t);
    }
}

template <typename OutT>
static hipError_t launch_tiled(const GemmArgs& a, hipStream_t st) {
    static thread_local int configured_dev = -1;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipErrorNoDevice;
    if (configured_dev != dev) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&dual_gemm_tiled<OutT>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, GEMM_LDS_BYTES);
        if (e != hipSuccess) return e;
        configured_dev = dev;
    }
    const int T = a.MT * a.NT;
    const int per = (T + NXCD - 1) / NXCD;
    const int cus_per_xcd = device_cu_count() / NXCD;
    const int wg_per_xcd = per < cus_per_xcd ? per : (cus_per_xcd > 0 ? cus_per_xcd : 1);
    hipLaunchKernelGGL((dual_gemm_tiled<OutT>), dim3((unsigned)(wg_per_xcd * NXCD)), dim3(64 * NW),
                       GEMM_LDS_BYTES, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dual_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                            const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                            int32_t N, int32_t K, int32_t k, void* Y, int32_t y_dtype,
                            hipStream_t st) {
    if (M <= 0) return hipSuccess;
    GemmArgs a{Aq, As, XO, Wq, Ws, WO, Y, M, N, K, k, (int32_t)((M + TBM - 1) / TBM), (N + TBN - 1) / TBN,
               nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0};
    return y_dtype == MG_BF16 ? launch_tiled<uint16_t>(a, st) : launch_tiled<float>(a, st);
}

hipError_t launch_dual_gemm_gelu_quant(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                                       const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                                       int32_t N, int32_t K, int32_t k, const float* s2, const float* rcp2,
                                       const int32_t* pos2, int32_t k2, uint8_t* Aq2, uint8_t* As2,
                                       uint16_t* XO2, hipStream_t st) {
    if (M <= 0) return hipSuccess;
    // XO2 (its pad columns, and every outlier value of pad rows) and As2 (a
    // last window half past N, when N % 512 != 0, belongs to no tile) start at 0
    if (k2 > 0) {
        hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(XO2), 0u, frag_bytes(M, 2 * (int64_t)k2) / 4, st);
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(As2), 0u, sc_bytes(M, N) / 4, st);
    if (e != hipSuccess) return e;
    GemmArgs a{Aq, As, XO, Wq, Ws, WO, nullptr, M, N, K, k, (int32_t)((M + TBM - 1) / TBM), (N + TBN - 1) / TBN,
               s2, rcp2, pos2, Aq2, As2, reinterpret_cast<uint8_t*>(XO2), k2};
    return launch_tiled<QuantOut>(a, st);
}

}  // namespace mg
