/*
 * mixed_gemm.h -- C ABI of the smoothed, outlier-split, dual-branch W4A4
 * linear layer for AMD Instinct MI355X (gfx950).
 *
 * The layer is the one of "W4A4 Quantization for Inference on
 * Wan2.2-I2V-A14B" (arXiv 2606.29337):
 *   Eq. (1)  Y = (X / s)(s * W), s applied along input channels;
 *   Eq. (2)  s_j = act_max_j^alpha / w_max_j^(1 - alpha);
 *   Eq. (4)  O = top-k input channels by max_t |x_tj|;
 *   Eq. (5)  Y = X_J W^(q)_J + X_O W^(hp)_O: MXFP4 W4A4 bulk + BF16 outliers.
 * The life cycle is calibrate -> plan(alpha, k) -> forward.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - X is [M][K] row-major (tokens x input channels); W is [N][K] row-major
 *    (nn.Linear layout, K contiguous); Y is [M][N] row-major bf16.
 *  - bf16 values travel as uint16_t bit patterns.
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library allocates no device memory and keeps no device state between
 *    calls.  Base pointers must be 16-byte aligned.
 *  - Every call validates its arguments on the host, then enqueues its
 *    kernels on `stream` and returns without synchronizing.  A device fault
 *    surfaces at the caller's next synchronization on that stream.
 *  - Return value: MG_OK (0) or a negative mg_status; mg_last_error() gives a
 *    message for the last failing call on the calling thread.
 *  - Inputs must be finite; NaN/Inf inputs give unspecified results.
 *  - MXFP4 = E2M1 elements + one E8M0 scale per 32 consecutive K (OCP MX):
 *    scale code c = floor(log2 amax) - 2 + 127 (clamped at 0), elements
 *    rounded to nearest, ties to the even code, saturating at +-6, sign copied
 *    (so -0 encodes as 0x8).  Two elements per byte, even K in the low nibble.
 */
#ifndef MIXED_GEMM_H
#define MIXED_GEMM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MG_OK = 0,
    MG_ERR_ARG = -1,         /* null pointer, bad alpha, bad enum value          */
    MG_ERR_SHAPE = -2,       /* K or N not a multiple of 32, k > K, negative size */
    MG_ERR_DTYPE = -3,       /* dtype not MG_F32 / MG_BF16                        */
    MG_ERR_ALIGN = -4,       /* a base pointer not 16-byte aligned                */
    MG_ERR_UNSUPPORTED = -5, /* a size beyond the documented limits               */
    MG_ERR_HIP = -6          /* a HIP runtime call failed (launch error)          */
} mg_status;

typedef enum { MG_F32 = 0, MG_BF16 = 1 } mg_dtype;

/* Weight block-scale layout (the block-packing paragraph after Eq. (5) and
 * its Fig. 8):
 * MG_W_1X32   one E8M0 per (output row n, 32 consecutive K);
 * MG_W_32X32  one E8M0 per aligned tile of 32 output rows x 32 K (requires N % 32 == 0);
 * MG_W_128X1  one E8M0 per K-major stripe of 128 consecutive K of one output
 *             row (the last stripe of a row covers the remaining K when
 *             K % 128 != 0). */
typedef enum { MG_W_1X32 = 0, MG_W_32X32 = 1, MG_W_128X1 = 2 } mg_wlayout;

/* Score the outlier set of Eq. (4) ranks:
 * MG_SCORE_MAX       the calibration maximum a_j = max_t |x_tj| (Eq. (4) as written);
 * MG_SCORE_SMOOTHED  the smoothed maximum max_t |x_tj / s_j| = RN(a_j / s_j). */
typedef enum { MG_SCORE_MAX = 0, MG_SCORE_SMOOTHED = 1 } mg_score;

/* Plan descriptor.  K, N: input / output widths (multiples of 32, K <= 65536);
 * k: number of outlier columns, 0 <= k <= K; layout: mg_wlayout;
 * smooth: 1 to apply Eq. (2) with alpha in (0, 1), 0 for s = 1;
 * score: mg_score. */
typedef struct {
    int32_t K, N, k;
    int32_t layout;
    int32_t smooth;
    int32_t score;
    double alpha;
} mg_plan_desc;

/* Plan buffers (caller-allocated, sizes from mg_plan_bytes, in this order):
 *  s   [K]        f32  smoothing scales, Eq. (2), evaluated in f64, rounded once;
 *  rcp [K]        f32  RN(1/s_j), used inside the exact division of the forward;
 *  O   [k]        i32  outlier channels, ascending (null allowed when k == 0);
 *  pos [K]        i32  index of channel j in O, or -1;
 *  Wq  [N][K/2]   u8   MXFP4 payload of the folded bulk weights RN(s_j W[n][j]),
 *                      outlier columns set to +0 before encoding, in fragment
 *                      order (below);
 *  Ws             u8   E8M0 scale of each (row, 32-block), in scale windows
 *                      (below) -- for MG_W_32X32 the tile's code repeated on
 *                      each of its 32 rows, for MG_W_128X1 the stripe's code
 *                      on each of its 32-blocks;
 *  Wst                 compact codes: [N/32][K/32] u8 tile codes (MG_W_32X32),
 *                      [N][ceil(K/128)] u8 stripe codes (MG_W_128X1); null
 *                      allowed for MG_W_1X32;
 *  WO  [N][k]     bf16 folded outlier columns (2k bytes per row) in fragment
 *                      order; null allowed when k == 0.
 *
 * Fragment order (Wq, Aq: rows of K/2 bytes; WO, XO: rows of 2k bytes).  The
 * [rows][row_bytes] byte matrix is cut into blocks of 32 rows x 32 bytes --
 * one operand of a 32x32x64 FP4 or 32x32x16 bf16 matrix-core instruction --
 * each stored as 1024 contiguous bytes: block (g = r / 32, c = byte / 32) at
 * (g * ns + c) * 1024 with ns = 2 * ceil(row_bytes / 64) (an even number of
 * 32-byte slices per row), and inside it byte b of row r's slice at
 *     16 * (r % 32 + 32 * (b / 16)) + b % 16,
 * for ceil(rows / 32) * ns * 1024 bytes in all.  Pads -- rows up to the next
 * multiple of 32 and bytes up to ns * 32 per row -- hold 0 (zero codes, +0).
 * The dual GEMM copies whole 1 KB blocks, and a block's 16-byte pieces are
 * already in the order the instruction's 64 lanes take them.
 *
 * Scale windows (Ws, As).  The E8M0 codes of a [rows][K/32] scale matrix are
 * stored in windows of 256 rows x 16 blocks (512 channels), 16 bytes per row,
 * 4096 contiguous bytes per window, windows of a 256-row group consecutive.
 * Inside a window row the codes of the even blocks come first, then those of
 * the odd blocks: the code of (row r, block b) is at byte
 *     ((r / 256) * nwin + b / 16) * 4096 + (r % 256) * 16 + 8 * (b % 2) + (b % 16) / 2,
 * nwin = ceil(K / 512), for ceil(rows / 256) * nwin * 4096 bytes in all.  The
 * layout depends on K only (a buffer sized for more rows serves fewer).  The
 * writers fill the whole last 256-row group: blocks past K/32 and rows past
 * the matrix hold code 0, the code of an all-zero block.  The dual GEMM copies
 * one window of its 256x256 output tile's rows as 4 KB of contiguous memory. */
typedef struct {
    mg_plan_desc d;
    float* s;
    float* rcp;
    int32_t* O;
    int32_t* pos;
    uint8_t* Wq;
    uint8_t* Ws;
    uint8_t* Wst;
    uint16_t* WO;
} mg_plan;

/* Per-forward activation workspace (sizes from mg_act_bytes):
 *  Aq [M][K/2] u8 MXFP4 payload of the bulk quotients in fragment order, As
 *  the E8M0 code of each (row, 32-block) in scale windows, XO [M][k] bf16
 *  outlier quotients in fragment order (null allowed when k == 0); see mg_plan. */
typedef struct {
    uint8_t* Aq;
    uint8_t* As;
    uint16_t* XO;
} mg_act;

/* Library version (major*10000 + minor*100 + patch). */
int mg_version(void);

/* Message for the last failing call on this thread ("" if none). */
const char* mg_last_error(void);

/* Host-only size queries.  out[8] = bytes of s, rcp, O, pos, Wq, Ws, Wst, WO;
 * out[3] = bytes of Aq, As, XO for M rows.  A zero size means "may be null". */
int mg_plan_bytes(const mg_plan_desc* d, size_t out[8]);
int mg_act_bytes(const mg_plan_desc* d, int64_t M, size_t out[3]);

/* ---- calibration: per-input-channel activation maxima and weight column
 * ranges (the calibration paragraph before Eq. (4); Eq. (4)'s score). ---- */

/* act_max[0..K) := +0.  Start of a calibration run. */
int mg_calib_reset(float* act_max, int32_t K, hipStream_t stream);

/* act_max[j] = max(act_max[j], max_t |X[t][j]|) over the M rows of X
 * (dtype MG_F32 or MG_BF16).  Exact, order-independent: batches may be fed
 * in any order and split anywhere.  M == 0 is a no-op. */
int mg_calib_act(const void* X, int32_t dtype, int64_t M, int32_t K, float* act_max,
                 hipStream_t stream);

/* w_max[j] = max_n |W[n][j]| (overwrites w_max). */
int mg_weight_range(const void* W, int32_t dtype, int32_t N, int32_t K, float* w_max,
                    hipStream_t stream);

/* ---- percentile calibration statistic: an alternative score for Eq. (4)'s
 * top-k (the tail-aware percentile calibration page builds its channel mask
 * from a percentile of the activation tail, to damp rare calibration
 * outliers; it gives no formula or level -- the reading here is the nearest
 * rank). ----
 *
 * score[j] = the value of rank r = ceil(q T) (1-based, clamped to [1, T]) in
 * ascending order of |x_tj| over all T calibration rows of all batches, for
 * 0 < q <= 1 (q = 1 gives act_max; r is computed in double precision).  The
 * result is exact (one of the inputs' magnitudes), by a two-pass radix
 * selection on the bf16 bit patterns of |x|:
 *   mg_pct_reset; mg_pct_count(pass 0) on every batch; mg_pct_select(pass 0);
 *                 mg_pct_count(pass 1) on every batch; mg_pct_select(pass 1).
 * Pass 0 counts, per channel, the high byte of each |x|; its select finds the
 * byte holding rank r and the rank inside it, and clears the counts; pass 1
 * counts the low bits of the values with that high byte; its select writes
 * score.  Both passes must see the same rows (in any order and split);
 * otherwise the result is unspecified (NaN where a rank is not found).  With
 * no rows counted, score is 0.  bf16 X only.  The score may be passed to
 * mg_outlier_set in place of act_max (s still comes from act_max).
 *
 * State, caller-owned device memory: hist [K][256] u32 (1 KiB per channel),
 * sel [K][2] i32 (selected high byte, rank inside it).  One state serves one
 * statistic at a time; calls on one state must be stream-ordered. */
typedef struct {
    uint32_t* hist;      /* [K][256] */
    int32_t* sel;        /* [K][2]   */
    int32_t K;           /* multiple of 32 */
    int32_t reserved;    /* 0 */
} mg_pct;

/* Clears hist: the start of a percentile calibration run. */
int mg_pct_reset(const mg_pct* st, hipStream_t stream);

/* Adds the M rows of X [M][K] (bf16) to pass `pass` (0 or 1).  M == 0 is a
 * no-op; M above 65535^2 (4.29e9) rows in one call is MG_ERR_UNSUPPORTED
 * (split the batch).  Pass 1 reads sel (written by mg_pct_select pass 0). */
int mg_pct_count(const mg_pct* st, int32_t pass, const uint16_t* X, int64_t M, hipStream_t stream);

/* Pass 0: from the counts and q, sel := (high byte, rank inside it) per
 * channel, and hist is cleared (score unused, may be NULL).  Pass 1:
 * score[0..K) := the statistic (q unused).  q must lie in (0, 1]. */
int mg_pct_select(const mg_pct* st, int32_t pass, double q, float* score, hipStream_t stream);

/* ---- planning (offline, once per layer) ---- */

/* Eq. (2): s, rcp from act_max and w_max (floor 1e-5 on both before the
 * powers); s = rcp = 1 when d.smooth == 0. */
int mg_smooth_scales(const mg_plan* p, const float* act_max, const float* w_max,
                     hipStream_t stream);

/* Eq. (4): O = the k channels first in the order (score desc, index asc),
 * stored ascending, and pos.  The score is act_max (MG_SCORE_MAX) or
 * RN(act_max / s) (MG_SCORE_SMOOTHED, which reads p->s: call
 * mg_smooth_scales first). */
int mg_outlier_set(const mg_plan* p, const float* act_max, hipStream_t stream);

/* Eq. (1) fold + extraction + block packing of W [N][K] (dtype MG_F32 or
 * MG_BF16) into Wq, Ws, (Wst), WO, reading p->s and p->pos. */
int mg_fold_pack(const mg_plan* p, const void* W, int32_t dtype, hipStream_t stream);

/* All three planning steps in order. */
int mg_plan_build(const mg_plan* p, const float* act_max, const float* w_max, const void* W,
                  int32_t dtype, hipStream_t stream);

/* ---- forward (per batch) ---- */

/* Runtime activation path (the integration paragraph after Eq. (5): at
 * inference a calibrated layer's input is divided in place by s, quantized to
 * 4 bits, and its outlier columns go to the narrow high-precision branch;
 * Eq. (1)'s X / s and Eq. (5)'s split into J and O):
 * q = RN_f32(X[m][j] / s_j) (exact IEEE division), XO[m][pos_j] = bf16(q),
 * bulk q with outlier columns set to +0 MXFP4-encoded into Aq/As.  M == 0 is
 * a no-op. */
int mg_quantize_act(const mg_plan* p, const void* X, int32_t dtype, int64_t M,
                    const mg_act* a, hipStream_t stream);

/* Eq. (5): Y[m][n] = sum_j Aq*Wq with their E8M0 scales + sum_i XO[m][i] WO[n][i],
 * accumulated in fp32.  y_dtype MG_BF16: Y is the layer output [M][N] bf16,
 * the fp32 sum rounded once to nearest-even.  y_dtype MG_F32: Y [M][N] f32
 * holds the fp32 sums unrounded (for callers that keep fp32 activations and
 * for checking the accumulation itself).  M == 0 is a no-op.  Each operand
 * (Aq, As, Wq, Ws, XO, WO) must stay below 3 GiB (32-bit buffer offsets),
 * else MG_ERR_UNSUPPORTED; Y has no limit (it is addressed per output tile).
 * Any K (a multiple of 32) and any k run on the same fast path. */
int mg_dual_gemm(const mg_plan* p, const mg_act* a, int64_t M, void* Y, int32_t y_dtype,
                 hipStream_t stream);

/* mg_quantize_act and mg_calib_act on the same X in one pass: the quantized
 * operands as mg_quantize_act writes them, and act_max[j] = max(act_max[j],
 * max_t |X[t][j]|) over every channel (outlier channels included) as
 * mg_calib_act computes it.  For routing that detects the outlier channels of
 * one step while it runs on the set chosen from the previous step (outlier
 * channels persist across steps; MixQ's quantization ahead of detection,
 * whose port to diffusion steps the pages name as future work).  Same
 * arguments and errors as mg_quantize_act, plus act_max [K] f32 (running;
 * reset it with mg_calib_reset). */
int mg_quantize_act_stats(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const mg_act* a,
                          float* act_max, hipStream_t stream);

/* mg_quantize_act followed by mg_dual_gemm. */
int mg_forward(const mg_plan* p, const void* X, int32_t dtype, int64_t M, const mg_act* a,
               void* Y, int32_t y_dtype, hipStream_t stream);

/* mg_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * activation workspace (Aq, As, XO) is not passed in: it lives in a fixed
 * 64 MiB array inside the library, one copy per GPU, created when the library
 * is first used on that GPU and held until the process ends.  The call makes
 * no hipMalloc / hipFree and no allocating library call.
 * Limit: the workspace of M rows -- Aq, As, XO as mg_act_bytes gives them,
 * each rounded up to 256 bytes -- must fit in 64 MiB (K = 5120, k = 64: up to
 * about 23,500 rows), else MG_ERR_UNSUPPORTED before anything is launched.
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it has to start at zero: the quantize step writes every
 * byte the GEMM reads).  Calls ordered on one stream are safe; calls that
 * overlap on one GPU (other streams, or threads without ordering) race and
 * give wrong results.  Otherwise the arguments, errors and results are those
 * of mg_forward. */
int mg_forward_noalloc(const mg_plan* p, const void* X, int32_t dtype, int64_t M, void* Y, int32_t y_dtype,
                       hipStream_t stream);

/* Between the two projections of the FFN block (the integration paragraph:
 * the calibrated FFN linear layers take their inputs after the SiLU/GELU
 * gates): out[i] = gelu_tanh(in[i]) for n bf16 values (in == out allowed),
 * gelu_tanh(y) = 0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3))).  Evaluated in f32 as the equal y / (1 + exp(-2u))
 * (u the tanh argument) with the hardware exp2 and reciprocal, then rounded
 * to bf16: a faithful bf16 rounding (one of the two bf16 neighbours) of the
 * exact value for every finite input where that is at least 2^-24 in
 * magnitude; smaller results are at most 2^-24 (very negative y give -0). */
int mg_gelu_tanh_bf16(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t stream);

/* The FFN block's second projection fed straight from the first one's bf16
 * output Y [M][K] (K = p->d.K = the first projection's N): quantizes the
 * hidden activation h = bf16_RNE(gelu_tanh(Y)) -- bit for bit what
 * mg_gelu_tanh_bf16 followed by mg_quantize_act computes -- in one pass,
 * without writing h (GELU-gated FFN inputs: the integration paragraph).
 * Same arguments and errors as mg_quantize_act with dtype MG_BF16. */
int mg_gelu_quantize_act(const mg_plan* p, const uint16_t* Y, int64_t M, const mg_act* a, hipStream_t stream);

/* The FFN block's two projections joined in the first one's GEMM epilogue
 * ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B": the integration
 * paragraph -- FFN inputs after the GELU gate are quantized like every
 * linear input -- and Eq. (5) for the first projection): mg_dual_gemm of
 * plan p0 on the workspace a0 (M rows), whose bf16 output is never written;
 * instead each output tile goes through GELU-tanh and the second
 * projection's quantizer (plan p2, p2->d.K == p0->d.N) into a2.  a2 holds bit
 * for bit what mg_dual_gemm(p0, a0, M, Y, MG_BF16) followed by
 * mg_gelu_quantize_act(p2, Y, M, a2) writes, including every pad byte.
 * Device pointers as in those calls; errors: theirs, and MG_ERR_SHAPE when
 * p2->d.K != p0->d.N.  a2 must not overlap a0 or the plans. */
int mg_dual_gemm_gelu_quant(const mg_plan* p0, const mg_act* a0, int64_t M, const mg_plan* p2, const mg_act* a2,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MIXED_GEMM_H */
