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
// E8M0 scales.  A bulk stage needs 8 scale bytes per tile row.  They are not
// fetched per lane (one cache line per row, per wave, per stage): the 16 bytes
// of two consecutive bulk stages ("a window") of all 512 tile rows are copied
// into LDS, next to the operand copies, and each wave reads its rows' 8 bytes
// from there.  The scale arrays are stored window by window (256 rows x 16
// bytes contiguous, the tile's rows), so a window of the A (B) tile is 4 KB
// of contiguous memory: one 16-byte load per lane and row, 8 cache lines per
// load instruction.  Windows alternate between two LDS slots.
//
// Pipeline.  The stages of all of a workgroup's tiles form one sequence over
// two LDS buffers (2 x 64 KB).  While stage g is multiplied out of one buffer,
// the copies of stage g+1 (which may be the first stage of the next tile) run
// straight from global memory into the other buffer.  One barrier per stage.
// In the steady state (a bulk stage followed by bulk stages of the same tile)
// the instruction order of a stage is fixed slot by slot: each of its 64 MFMAs
// is followed by at most one fragment read, scale read or copy, so memory
// instructions never hold up a run of MFMAs, and sub-step 3 -- whose
// fragments are read before the barrier -- is multiplied after it, so the
// matrix cores stay busy while the next stage's first fragments are read.
// After a tile's last stage its 256x256 bf16 result is staged through the
// freed buffer and written as whole 512-byte rows while the next tile's first
// stage already sits in LDS.
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
constexpr int SCW_ROWB = 16;                      // scale bytes per row per window (two bulk stages)
constexpr int SCW_BYTES = (TBM + TBN) * SCW_ROWB; // one window slot: A rows then B rows (8 KB)
constexpr int SCW_OFF = 2 * STAGE_BYTES;
constexpr int GEMM_LDS_BYTES = 2 * STAGE_BYTES + 2 * SCW_BYTES;
constexpr uint32_t OOB = 0xC0000000u;             // offset that reads as zero
constexpr int NXCD = 8;
constexpr int GROUP_M = 8;
static_assert(TBM == kScRows && TBN == kScRows && SCW_ROWB == kScBlocks, "a tile's scale window is one stored window");

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
};

// Origin of an output tile (wave-uniform).
struct TileOrg {
    int64_t m0;
    int n0;
};

template <typename OutT>
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
    const uint32_t rowX = (uint32_t)(2 * xo_cols(k));   // bytes per XO / WO row (16-byte multiple)
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
    const __amdgpu_buffer_rsrc_t rAs = make_rsrc(g.As, (uint64_t)sc_bytes(M, K));
    const __amdgpu_buffer_rsrc_t rBs = make_rsrc(g.Ws, (uint64_t)sc_bytes(N, K));
    const uint32_t nwin = (uint32_t)sc_nwin(K);
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
    const uint32_t lds_w = (uint32_t)(wave * 64 * ROWB);
    // scale windows: lane L of wave w copies window row 64 w + L of A and of
    // B; a lane reads its fragment rows' 8 bytes at these offsets (+ 512 i)
    const uint32_t lwr = (uint32_t)(wave * 64 + lane) * SCW_ROWB;
    const uint32_t scw_a = (uint32_t)((wm * 128 + l32) * SCW_ROWB);
    const uint32_t scw_b = (uint32_t)(TBM * SCW_ROWB + (wn * 128 + l32) * SCW_ROWB);
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
    int wiss = 0;      // scale windows issued so far (slot of the next one: wiss & 1)
    int wuse = 0;      // scale windows taken into use so far
    int wcur = 0;      // slot of the window of the current bulk stage

    // ---- scale window w (bulk stages 2w, 2w+1) of a tile into the next slot:
    // the stored windows of the tile's 256 A rows and 256 B rows (4 KB each)
    auto load_window = [&](const TileOrg& o, int w) {
        const int slot = wiss & 1;
        ++wiss;
        uint8_t* dst = lds + SCW_OFF + slot * SCW_BYTES + wave * 64 * SCW_ROWB;
        uint32_t r = lwr;
        asm volatile("" : "+v"(r));
        const uint32_t wa = __builtin_amdgcn_readfirstlane(((uint32_t)(o.m0 / TBM) * nwin + (uint32_t)w) * kScWinBytes);
        const uint32_t wb = __builtin_amdgcn_readfirstlane(((uint32_t)(o.n0 / TBN) * nwin + (uint32_t)w) * kScWinBytes);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rAs, (lds_ptr_t)dst, 16, wa + r, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rBs, (lds_ptr_t)(dst + TBM * SCW_ROWB), 16, wb + r, 0, 0, 0);
    };

    // ---- this lane's scale words of bulk stage st (from its window)
    auto read_scales_i = [&](const uint8_t* wsc, int q) {
        if (q < 4) {
            const u32x2 x = *reinterpret_cast<const u32x2*>(wsc + scw_a + q * 32 * SCW_ROWB);
            nA[q][0] = x[0]; nA[q][1] = x[1];
        } else {
            const u32x2 x = *reinterpret_cast<const u32x2*>(wsc + scw_b + (q - 4) * 32 * SCW_ROWB);
            nB[q - 4][0] = x[0]; nB[q - 4][1] = x[1];
        }
    };
    auto window_of = [&](int st) -> const uint8_t* {
        if ((st & 1) == 0) { wcur = wuse & 1; ++wuse; }
        return lds + SCW_OFF + wcur * SCW_BYTES + (st & 1) * 8;
    };
    // lane half h uses the odd scale bytes: shift them down so sub-step ss
    // finds its byte at position 2*(ss&1) of word ss>>1.
    const uint32_t sc_shift = (uint32_t)h * 8u;
    auto take_scales = [&]() {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            scA[i][0] = nA[i][0] >> sc_shift;
            scA[i][1] = nA[i][1] >> sc_shift;
            scB[i][0] = nB[i][0] >> sc_shift;
            scB[i][1] = nB[i][1] >> sc_shift;
        }
    };

    // ---- the stage whose copies are issued during the current one: stage
    // `st` of tile `o` (bulk stages first, then outlier stages), or nothing
    // (st < 0).  Wave-uniform.
    struct NextCopy {
        TileOrg o;
        int st;
    };

    // Copies of one 8-row group of the A (B) tile of stage nc (asynchronous,
    // straight into LDS buffer b).  With nothing to copy every lane reads out
    // of range, which lands zeros in the free buffer.
    auto copy_part = [&](const NextCopy& nc, int b, int part, bool isB) {
        uint8_t* dst = lds + b * STAGE_BYTES + lds_w + (isB ? TILE_BYTES : 0) + part * 8 * ROWB;
        const bool bulk = nc.st < S4;
        const uint32_t rowb = bulk ? rowA : rowX;
        uint32_t lr = bulk ? lrA0 : lrX0;
        asm volatile("" : "+v"(lr));
        const uint32_t so = __builtin_amdgcn_readfirstlane((uint32_t)(bulk ? nc.st : nc.st - S4) * ROWB);
        const uint32_t r0 = __builtin_amdgcn_readfirstlane((isB ? (uint32_t)nc.o.n0 : (uint32_t)nc.o.m0) * rowb);
        const uint32_t c = (part & 1) ? c16o : c16e;
        const bool ok = nc.st >= 0 && so + c < rowb;      // chunks past K / k read as zero
        const uint32_t v = ok ? lr + c + r0 + (uint32_t)part * 8 * rowb : OOB;
        if (bulk)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rB : rA, (lds_ptr_t)dst, 16, v, so, 0, 0);
        else
            __builtin_amdgcn_raw_ptr_buffer_load_lds(isB ? rWO : rXO, (lds_ptr_t)dst, 16, v, so, 0, 0);
    };

    // All copies of stage nc at once (the very first stage), with the scale
    // window it opens.
    auto load_stage = [&](const NextCopy& nc, int b) {
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
            copy_part(nc, b, gi, false);
            copy_part(nc, b, gi, true);
        }
        if (nc.st >= 0 && nc.st < S4 && (nc.st & 1) == 0) load_window(nc.o, nc.st >> 1);
    };

    // End of a stage: this wave's copies into the other buffer have landed and
    // its reads of the current buffer are done, then every wave arrives.  The
    // scheduling barriers keep the stage's MFMAs above the wait, so they run
    // while copies fly.  (__syncthreads would add a release fence and wait
    // for the previous tile's stores as well.)
    auto stage_sync = [&]() {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- one stage, in a fixed issue order of one slot per MFMA.  A stage
    // is 4 sub-steps of 16 MFMAs (FP4 for a bulk stage, BF16 for an outlier
    // stage); sub-step 3 is normally read before the stage barrier and
    // multiplied after it, at the start of the next stage (DEFER_OUT), so
    // the matrix cores have 16 MFMAs of work while the next stage's first
    // fragments are read.  Slots:
    //   0-15   the previous stage's sub-step 3 (kind DK: 0 none, 1 FP4, 2
    //          BF16); slots 0-7 also read this stage's scale words and
    //          sub-step 0's fragments (A0 B0 B1 B2 B3 A1 A2 A3, the order its
    //          MFMAs need them), slot 12 shuffles the scales;
    //   16-63  sub-steps 0, 1, 2; the next sub-step's fragments are read in
    //          the first 8 slots of each;
    //   64-79  sub-step 3 when it is not deferred (the last stage of a tile).
    // The next stage's 16 copies go one per 2 slots from slot 2 to 32, the
    // scale window it opens (if any) in slot 36: never two memory
    // instructions back to back, so the address unit is shared evenly
    // between the four waves.
    u32x4 pf[2][2][4];                 // fragment sets [set][A/B][i]
    uint32_t pA[4], pB[4];             // sub-step 3 scales of the previous stage
    auto frag_read = [&](const uint8_t* base, int ss, int set, int q) {
        const uint32_t co = (uint32_t)(((2 * ss + h) ^ sw) << 4);
        const bool isA = q == 0 || q >= 5;
        const int r = q == 0 ? 0 : (q < 5 ? q - 1 : q - 4);
        if (isA) pf[set][0][r] = *reinterpret_cast<const u32x4*>(base + fa[r] + co);
        else     pf[set][1][r] = *reinterpret_cast<const u32x4*>(base + fb[r] + co);
    };
    auto run_stage = [&](auto CUR_BULK, auto DK, auto DEFER_OUT, const NextCopy& nc, int st, int b) {
        constexpr bool cb = decltype(CUR_BULK)::value;
        constexpr int dk = decltype(DK)::value;
        constexpr bool dout = decltype(DEFER_OUT)::value;
        const uint8_t* base = lds + b * STAGE_BYTES;
        const uint8_t* wsc = nullptr;
        if constexpr (cb) wsc = window_of(st);
        const bool opens_window = nc.st >= 0 && nc.st < S4 && (nc.st & 1) == 0;
        static_for<80>([&](auto QC) {
            constexpr int q = decltype(QC)::value;
            if constexpr (q < 64 || !dout) {
                if constexpr (q < 16) {
                    constexpr int i = q >> 2, j = q & 3;
                    if constexpr (dk == 1)
                        acc[i][j] = mfma_fp4_op<2>(pf[1][1][j], pf[1][0][i], pB[j], pA[i], acc[i][j]);
                    else if constexpr (dk == 2)
                        acc[i][j] = mfma_bf16_v(pf[1][1][j], pf[1][0][i], acc[i][j]);
                } else {
                    constexpr int ss = (q - 16) >> 4, r = (q - 16) & 15, i = r >> 2, j = r & 3, set = ss & 1;
                    if constexpr (cb)
                        acc[i][j] = mfma_fp4_op<(ss & 1) ? 2 : 0>(pf[set][1][j], pf[set][0][i], scB[j][ss >> 1],
                                                                  scA[i][ss >> 1], acc[i][j]);
                    else
                        acc[i][j] = mfma_bf16_v(pf[set][1][j], pf[set][0][i], acc[i][j]);
                }
                if constexpr (q < 8) {
                    if constexpr (cb) read_scales_i(wsc, q);
                    frag_read(base, 0, 0, q);
                }
                if constexpr (cb && q == 12) take_scales();
                if constexpr (q >= 16 && q < 24) frag_read(base, 1, 1, q - 16);
                if constexpr (q >= 32 && q < 40) frag_read(base, 2, 0, q - 32);
                if constexpr (q >= 48 && q < 56) frag_read(base, 3, 1, q - 48);
                if constexpr (q >= 2 && q <= 32 && q % 2 == 0) copy_part(nc, b ^ 1, (q - 2) >> 2, ((q - 2) & 2) != 0);
                if constexpr (q == 36) {
                    if (opens_window) load_window(nc.o, nc.st >> 1);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        if constexpr (cb && dout) {
#pragma unroll
            for (int i = 0; i < 4; ++i) { pA[i] = scA[i][1]; pB[i] = scB[i][1]; }
        }
        stage_sync();
    };

    // ---- epilogue of one tile.  The MFMAs take the weight fragment as their
    // first operand, so acc[i][j] holds Y^T for A row-tile i and W row-tile j:
    // lane (l32, h), register 4 q + e holds output row 32 i + l32 and output
    // column 32 j + 8 q + 4 h + e of this wave's quarter -- four consecutive
    // columns per register group.
    auto epilogue = [&](const TileOrg& o, uint8_t* stagebuf) {
        if constexpr (sizeof(OutT) == 2) {
            // bf16: round pairs with the hardware converter (nearest even).
            // Each wave stages its own 128x128 quarter through its own 16 KB
            // of the free buffer, 64 rows x 256 B per pass, and writes the
            // rows back out with 16-byte streaming stores (four 256-byte row
            // pieces per instruction).  No wave reads another wave's staging,
            // so a pass needs no barrier: one wave's LDS accesses are
            // processed in order.  In a staged row r the 16-byte chunk c
            // (columns 8c .. 8c+7 of the quarter) sits at chunk c ^ (r & 15).
            // the tile's rows of Y: rows past M are out of the descriptor's
            // range and columns past N get an out-of-range offset, so the
            // stores need no branches
            const uint32_t rowY = (uint32_t)N * 2u;
            const int64_t rows_left = M - o.m0;
            const uint32_t nrec = (uint32_t)(rows_left < TBM ? rows_left : TBM) * rowY;
            const __amdgpu_buffer_rsrc_t rY =
                make_rsrc(static_cast<uint16_t*>(g.Y) + o.m0 * (int64_t)N, (uint64_t)nrec);
            uint8_t* wbuf = stagebuf + wave * 16384;
            // Lane-dependent values come from an opaque copy of the thread
            // index, so they are formed here, once per tile, instead of being
            // hoisted out of the tile loop and held (or spilled) across it.
            uint32_t et = (uint32_t)tid;
            asm volatile("" : "+v"(et));
            const uint32_t el32 = et & 31u, eh = (et >> 5) & 1u;
            const uint32_t rl = (et & 63u) >> 4, cl = et & 15u;       // read side: row (of 4), chunk
            const int gcol = o.n0 + wn * 128 + (int)cl * 8;
            const bool col_ok = gcol < N;
            const uint32_t cofs = (uint32_t)gcol * 2u;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
#pragma unroll
                for (int ii = 0; ii < 2; ++ii) {
                    const int i = 2 * p + ii;
                    // read row-block i's accumulators here, not earlier
#pragma unroll
                    for (int j = 0; j < 4; ++j) asm volatile("" : "+a"(acc[i][j]));
                    const uint32_t r = (uint32_t)(32 * ii) + el32;
                    const uint32_t rb = r * 256 + eh * 8, rs = r & 15u;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const f32x2 lo = {acc[i][j][4 * q], acc[i][j][4 * q + 1]};
                            const f32x2 hi = {acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
                            const u32x2 w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2)),
                                             __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2))};
                            *reinterpret_cast<u32x2*>(wbuf + rb + ((((uint32_t)(4 * j + q)) ^ rs) << 4)) = w;
                        }
                }
                u32x4 v[16];
#pragma unroll
                for (int sI = 0; sI < 16; ++sI) {
                    const uint32_t rr = (uint32_t)(4 * sI) + rl;
                    v[sI] = *reinterpret_cast<const u32x4*>(wbuf + rr * 256 + ((cl ^ (rr & 15u)) << 4));
                }
#pragma unroll
                for (int sI = 0; sI < 16; ++sI) {
                    const uint32_t rr = (uint32_t)(4 * sI) + rl;
                    const uint32_t off = col_ok ? ((uint32_t)(wm * 128 + 64 * p) + rr) * rowY + cofs : OOB;
                    // streaming store (nt): Y is written once and must not
                    // push the operand panels out of L2
                    __builtin_amdgcn_raw_buffer_store_b128(v[sI], rY, off, 0, 2);
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
    load_stage(NextCopy{cur, 0}, 0);
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    int buf = 0;

    using T_ = std::true_type;
    using F_ = std::false_type;
    using D0 = std::integral_constant<int, 0>;
    using D1 = std::integral_constant<int, 1>;
    while (true) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};
        const bool has_next = tn < t_end;
        const TileOrg nxt = tile_org(has_next ? tn : t);
        // the stage after st: the next one of this tile, the first one of the
        // next tile, or none
        auto next_of = [&](int st) {
            NextCopy nc{cur, st + 1};
            if (st + 1 == S) nc = has_next ? NextCopy{nxt, 0} : NextCopy{cur, -1};
            return nc;
        };
        // bulk stages, each leaving its sub-step 3 to the next
        run_stage(T_{}, D0{}, T_{}, next_of(0), 0, buf);
        buf ^= 1;
        int st = 1;
        for (; st < S4; ++st) {
            run_stage(T_{}, D1{}, T_{}, next_of(st), st, buf);
            buf ^= 1;
        }
        // the last bulk stage's sub-step 3
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = mfma_fp4_op<2>(pf[1][1][j], pf[1][0][i], pB[j], pA[i], acc[i][j]);
        // outlier stages, each complete in itself
        for (; st < S; ++st) {
            run_stage(F_{}, D0{}, F_{}, next_of(st), st, buf);
            buf ^= 1;
        }
        // buffer buf^1 held the last stage and is free; buf holds the next
        // tile's first stage (if any)
        epilogue(cur, lds + (buf ^ 1) * STAGE_BYTES);
        if (!has_next) break;
        t = tn;
        tn += nl;
        cur = nxt;
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
    hipLaunchKernelGGL((dual_gemm_tiled<OutT>), dim3((unsigned)(wg_per_xcd * NXCD)), dim3(256),
                       GEMM_LDS_BYTES, st, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dual_gemm(const uint8_t* Aq, const uint8_t* As, const uint16_t* XO,
                            const uint8_t* Wq, const uint8_t* Ws, const uint16_t* WO, int64_t M,
                            int32_t N, int32_t K, int32_t k, void* Y, int32_t y_dtype,
                            hipStream_t st) {
    if (M <= 0) return hipSuccess;
    GemmArgs a{Aq, As, XO, Wq, Ws, WO, Y, M, N, K, k, (int32_t)((M + TBM - 1) / TBM), (N + TBN - 1) / TBN};
    return y_dtype == MG_BF16 ? launch_tiled<uint16_t>(a, st) : launch_tiled<float>(a, st);
}

}  // namespace mg
