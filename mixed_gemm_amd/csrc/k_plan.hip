// Offline planning kernels of the W4A4 layer ("W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B"):
//   smooth_kernel     Eq. (2) smoothing scales s and their reciprocals;
//   topk_kernel       Eq. (4) static top-k outlier set O (sparse index list) + pos;
//   fold_pack_kernel  Eq. (1) fold s into W, extract the outlier columns to bf16,
//                     pack the bulk into MXFP4 with 1x32 or 32x32 block scales
//                     (block-packing paragraph after Eq. (5)).
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

// ---------------------------------------------------------------------------- Eq. (2)

__global__ void __launch_bounds__(256) smooth_kernel(const float* __restrict__ a,
                                                     const float* __restrict__ w, int32_t K,
                                                     double alpha, int32_t smooth,
                                                     float* __restrict__ s, float* __restrict__ rcp) {
    const int j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= K) return;
    float sj = 1.0f;
    if (smooth) {
        const double aa = fmax((double)a[j], 1e-5);
        const double ww = fmax((double)w[j], 1e-5);
        sj = (float)(pow(aa, alpha) / pow(ww, 1.0 - alpha));
    }
    s[j] = sj;
    rcp[j] = __fdiv_rn(1.0f, sj);
}

// ---------------------------------------------------------------------------- Eq. (4)

constexpr int kTopkThreads = 1024;

// Block-wide inclusive scan of one value per thread: a shuffle scan inside
// each wave, then the wave totals (through LDS) added on.
__device__ int block_inclusive_scan(int v, int* buf) {
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(v, o, 64);
        if (lane >= o) v += u;
    }
    if (lane == 63) buf[w] = v;
    __syncthreads();
    int add = 0;
#pragma unroll
    for (int i = 0; i < kTopkThreads / 64; ++i) add += i < w ? buf[i] : 0;   // independent loads
    __syncthreads();                  // buf is free again for the next scan
    return v + add;
}

// One workgroup.  Scores -- a_j, or RN(a_j / s_j) for the smoothed score --
// are non-negative floats, compared through their bit patterns (same order).
// T = the k-th largest score is found by an MSB-first radix select, 8 bits
// per pass with a 256-bin histogram in LDS; channels above T are in O, and of
// the channels equal to T the lowest indices fill the remaining places (tie
// rule: index ascending).  Thread t owns the contiguous index range
// [t*C, (t+1)*C) so block scans give ascending order directly.  Its C <= CMAX
// scores are loaded once, all loads in flight together, and every pass runs
// on the registers.
template <int CMAX>
__global__ void __launch_bounds__(kTopkThreads) topk_kernel(const float* __restrict__ a,
                                                            const float* __restrict__ s, int32_t K,
                                                            int32_t k, int32_t* __restrict__ O,
                                                            int32_t* __restrict__ pos) {
    __shared__ int buf[kTopkThreads];
    __shared__ int hist[256];
    __shared__ uint32_t sel[2];
    const int t = threadIdx.x;
    const int C = (K + kTopkThreads - 1) / kTopkThreads;     // <= CMAX (checked by the launcher)
    const int j0 = t * C;
    const int n = max(0, min(K, j0 + C) - j0);               // this thread's channels
    uint32_t kv[CMAX];
    if (s) {
#pragma unroll
        for (int i = 0; i < CMAX; ++i) kv[i] = i < n ? __float_as_uint(__fdiv_rn(a[j0 + i], s[j0 + i])) : 0u;
    } else {
#pragma unroll
        for (int i = 0; i < CMAX; ++i) kv[i] = i < n ? __float_as_uint(a[j0 + i]) : 0u;
    }

    uint32_t T = 0;
    int need = 0;
    if (k > 0 && k < K) {
        uint32_t prefix = 0, pmask = 0;
        int remaining = k;                        // still to pick among keys matching the prefix
        for (int shift = 24; shift >= 0; shift -= 8) {
            if (t < 256) hist[t] = 0;
            __syncthreads();
            // Counting.  The high bytes of channel maxima take few values (similar
            // exponents), so in the first pass one bin can receive most of the
            // 1024 threads' adds: there, lanes of a wave with the same bin as a
            // leader lane are counted with one atomic (two such rounds per key)
            // and the rest add one by one; the later passes, whose bins are
            // spread, add one by one.
#pragma unroll
            for (int i = 0; i < CMAX; ++i) {
                if (i < C) {                                              // uniform
                    bool act = i < n && (kv[i] & pmask) == prefix;
                    const uint32_t bin = (kv[i] >> shift) & 255u;
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        if (shift != 24) break;                           // uniform
                        const uint64_t m = __builtin_amdgcn_ballot_w64(act);
                        if (m != 0) {                                     // uniform
                            const int leader = __builtin_ctzll(m);
                            const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
                            const uint64_t same = __builtin_amdgcn_ballot_w64(act && bin == b);
                            if ((t & 63) == leader) atomicAdd(&hist[b], (int)__builtin_popcountll(same));
                            act = act && bin != b;
                        }
                    }
                    if (act) atomicAdd(&hist[bin], 1);
                }
            }
            __syncthreads();
            // the bin holding the remaining-th largest key: counts from the top
            // bin down (thread t < 256 takes bin 255 - t), then the thread whose
            // running count first reaches `remaining` records it
            const int hv = t < 256 ? hist[255 - t] : 0;
            const int incl = block_inclusive_scan(hv, buf);
            if (t < 256 && incl - hv < remaining && incl >= remaining) {
                sel[0] = (uint32_t)(255 - t);
                sel[1] = (uint32_t)(remaining - (incl - hv));
            }
            __syncthreads();
            // sel is written again only after the next pass's scan barriers,
            // and hist was read before this pass's: no barrier needed here
            prefix |= sel[0] << shift;
            pmask |= 255u << shift;
            remaining = (int)sel[1];
        }
        T = prefix;
        need = remaining;                         // keys equal to T that are taken
    }
    // ties before my range
    int ties = 0;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) ties += i < n && kv[i] == T;
    const int tie_off = block_inclusive_scan(ties, buf) - ties;
    // membership (bit i of `in`) and ascending positions
    uint64_t in = 0;
    {
        int to = tie_off;
#pragma unroll
        for (int i = 0; i < CMAX; ++i) {
            if (i < n) {
                const bool m = k >= K || (k > 0 && (kv[i] > T || (kv[i] == T && to < need)));
                to += kv[i] == T;
                in |= (uint64_t)m << i;
            }
        }
    }
    const int mine = __builtin_popcountll(in);
    int off = block_inclusive_scan(mine, buf) - mine;
#pragma unroll
    for (int i = 0; i < CMAX; ++i) {
        if (i < n) {
            if ((in >> i) & 1u) {
                O[off] = j0 + i;
                pos[j0 + i] = off;
                ++off;
            } else {
                pos[j0 + i] = -1;
            }
        }
    }
}

// ---------------------------------------------------------------------------- fold + pack

constexpr int kFoldWaves = 4;
constexpr int kFoldStgRow = 272;      // LDS staging row of Wq codes: 256 bytes + 16 pad (conflict-free writes)
typedef uint32_t u32x4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float quad_max_f(float v) {
    // max over the 4 lanes of a quad (one 32-block): quad_perm [1,0,3,2] then [2,3,0,1]
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false)));
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false)));
    return v;
}

// Lane layout as in the activation quantizer: a lane owns 8 consecutive
// input channels (one 16-byte load of a bf16 row), 4 lanes form a 32-block,
// a wave covers 512 channels of a row and walks rows.  Per row and lane:
// W'[n][j] = RN(s_j * W[n][j]); outlier channels go to WO as bf16 and become
// +0; the block amax gives the E8M0 code (1x32), or, for the 32x32 layout, the
// amax over the 32 rows of the tile does (a first pass over the tile's rows,
// the second pass re-reads them from L2), or, for 128x1 stripes, the amax over
// the 16 lanes (128 channels) of the stripe; the hardware converter encodes.
template <bool BF16, int LAY>
__global__ void __launch_bounds__(256) fold_pack_kernel(const void* __restrict__ W, int32_t N, int32_t K,
                                                        int32_t k, const float* __restrict__ s,
                                                        const int32_t* __restrict__ pos,
                                                        uint8_t* __restrict__ Wq, uint8_t* __restrict__ Ws,
                                                        uint8_t* __restrict__ Wst,
                                                        uint16_t* __restrict__ WO) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int j0 = (blockIdx.x * 64 + lane) * 8;
    const bool valid = j0 < K;                       // whole quads agree (K % 32 == 0)
    const int nb = K / 32;
    const int64_t nwin = sc_nwin(K);
    // Ws covers whole 256-row scale groups: rows past N get the zero code
    const int64_t Np = ((int64_t)N + kScRows - 1) / kScRows * kScRows;
    float sv[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int pv[8] = {-1, -1, -1, -1, -1, -1, -1, -1};
    if (valid) {                                     // j0 is a multiple of 8: 16-byte loads
#pragma unroll
        for (int h4 = 0; h4 < 2; ++h4) {
            const float4 a = *reinterpret_cast<const float4*>(s + j0 + 4 * h4);
            const int4 c = *reinterpret_cast<const int4*>(pos + j0 + 4 * h4);
            sv[4 * h4] = a.x; sv[4 * h4 + 1] = a.y; sv[4 * h4 + 2] = a.z; sv[4 * h4 + 3] = a.w;
            pv[4 * h4] = c.x; pv[4 * h4 + 1] = c.y; pv[4 * h4 + 2] = c.z; pv[4 * h4 + 3] = c.w;
        }
    }
    uint32_t keep[8];
    uint32_t omask = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        keep[i] = pv[i] >= 0 ? 0u : 0xFFFFFFFFu;
        omask |= (pv[i] >= 0 ? 1u : 0u) << i;
    }

    // RN(s * W) of the lane's 8 channels of row n (zeros when out of range)
    auto fold_row = [&](int64_t n, float (&f)[8]) {
        float x[8];
        if (valid && n < N) {
            if constexpr (BF16) {
                const uint4 d = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(W) + n * K + j0);
                const uint32_t wd[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    x[2 * i] = __uint_as_float(wd[i] << 16);
                    x[2 * i + 1] = __uint_as_float(wd[i] & 0xFFFF0000u);
                }
            } else {
                const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(W) + n * K + j0);
                const float4 d0 = src[0], d1 = src[1];
                x[0] = d0.x; x[1] = d0.y; x[2] = d0.z; x[3] = d0.w;
                x[4] = d1.x; x[5] = d1.y; x[6] = d1.z; x[7] = d1.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.0f;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = __fmul_rn(sv[i], x[i]);
    };
    // outlier channels of row n to WO, then masked to +0 in f; returns the
    // lane's amax of the masked values.  Wq and WO are stored in fragment
    // order (frag_offset); N % 32 == 0, so there are no pad rows.  The
    // workgroup of channels 0..511 writes each WO row's pad columns k ..
    // 16 * nso - 1 (+0), one per lane.
    const int64_t ns4 = frag_slices(K / 2), nso = frag_slices(2 * (int64_t)k);
    uint8_t* const WOb = reinterpret_cast<uint8_t*>(WO);
    const bool pad_lane = blockIdx.x == 0 && lane < 16 * nso - k;
    auto wo_store = [&](int64_t n, int i, uint16_t v) {
        *reinterpret_cast<uint16_t*>(WOb + frag_offset(n, 2 * (int64_t)i, nso)) = v;
    };
    auto extract = [&](int64_t n, float (&f)[8]) {
        if (pad_lane && n < N) wo_store(n, k + lane, 0);
        if (omask && n < N) {
            for (uint32_t m = omask; m; m &= m - 1) {
                const int i = __builtin_ctz(m);
                float fi = f[0];
#pragma unroll
                for (int t = 1; t < 8; ++t) fi = i == t ? f[t] : fi;
                int pi = pv[0];
#pragma unroll
                for (int t = 1; t < 8; ++t) pi = i == t ? pv[t] : pi;
                wo_store(n, pi, (uint16_t)f32_to_bf16_rne(fi));
            }
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            f[i] = __uint_as_float(__float_as_uint(f[i]) & keep[i]);
            amax = fmaxf(amax, __builtin_fabsf(f[i]));
        }
        return amax;
    };
    // the nibbles of row n (rows inside N; lanes inside K, and past K up to
    // the last 32-byte slice, whose pad half gets the zero codes) and, from
    // one lane per quad, the block's scale code (every lane of rows < Np: past
    // K or N the code 0 of an all-zero block)
    auto encode_word = [&](const float (&f)[8], uint32_t c) {
        const float scale = e8m0_to_f32(c);
        uint32_t word = 0;
        MG_CVT_FP4X2(word, f[0], f[1], scale, 0);
        MG_CVT_FP4X2(word, f[2], f[3], scale, 1);
        MG_CVT_FP4X2(word, f[4], f[5], scale, 2);
        MG_CVT_FP4X2(word, f[6], f[7], scale, 3);
        return word;
    };
    auto encode_store = [&](int64_t n, const float (&f)[8], uint32_t c) {
        const uint32_t word = encode_word(f, c);
        if (j0 < 64 * ns4 && n < N) *reinterpret_cast<uint32_t*>(Wq + frag_offset(n, j0 / 2, ns4)) = word;
        if ((lane & 3) == 0) Ws[sc_offset(n, j0 / 32, nwin)] = (uint8_t)(valid ? c : 0u);   // a short stripe's pads: 0
    };

    const int64_t wstride = (int64_t)gridDim.y * kFoldWaves;
    if constexpr (LAY == MG_W_1X32 || LAY == MG_W_128X1) {
        // 32-row groups G = blockIdx.y, blockIdx.y + gridDim.y, ... through the
        // last scale group; wave w takes rows 32 G + 8 w .. + 7, all 8 loaded
        // before any is folded.  The wave's 8 rows fill whole 128-byte lines of
        // Wq's fragment blocks (8 rows x 16 bytes of one slice half), so it
        // stages its codes in its own LDS rows and stores them as 16 full lines
        // (two 1 KB stores; lane L of store t takes row L % 8 of line 8 t + L / 8
        // = (slice, half)); no wave reads another's staging, so no barrier.
        __shared__ __attribute__((aligned(16))) uint8_t stg[kFoldWaves * 8 * kFoldStgRow];
        uint8_t* const stgw = stg + wave * 8 * kFoldStgRow;
        const int64_t NG = (int64_t)N / 32, NGp = Np / 32;
        const int ns_str = (K + 127) / 128;
        for (int64_t G = blockIdx.y; G < NGp; G += gridDim.y) {
            const int64_t n0 = G * 32 + wave * 8;
            float f[8][8];
#pragma unroll
            for (int r = 0; r < 8; ++r) fold_row(n0 + r, f[r]);
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int64_t n = n0 + r;
                float amax = quad_max_f(extract(n, f[r]));
                if constexpr (LAY == MG_W_128X1) {
                    amax = fmaxf(amax, __shfl_xor(amax, 4, 64));      // the stripe's 4 quads (16 lanes)
                    amax = fmaxf(amax, __shfl_xor(amax, 8, 64));
                }
                const uint32_t c = e8m0_from_amax_bits(__float_as_uint(amax));
                const uint32_t word = encode_word(f[r], c);
                *reinterpret_cast<uint32_t*>(stgw + r * kFoldStgRow + 4 * lane) = word;
                if ((lane & 3) == 0) Ws[sc_offset(n, j0 / 32, nwin)] = (uint8_t)(valid ? c : 0u);
                if constexpr (LAY == MG_W_128X1) {
                    if (valid && n < N && (lane & 15) == 0) Wst[n * ns_str + j0 / 128] = (uint8_t)c;
                }
            }
            if (G < NG) {
                const __amdgpu_buffer_rsrc_t rg = make_rsrc(Wq + G * ns4 * kFragBlock, (uint64_t)ns4 * kFragBlock);
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const int line = 8 * t + (lane >> 3), sl = line >> 1, hf = line & 1, rr = lane & 7;
                    const uint4 v = *reinterpret_cast<const uint4*>(stgw + rr * kFoldStgRow + sl * 32 + hf * 16);
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4f, v), rg,
                        (uint32_t)((blockIdx.x * 8 + sl) * kFragBlock + 16 * (wave * 8 + rr + 32 * hf)), 0, 2);
                }
            }
        }
    } else {
        // 32-row groups through the last scale group (N % 32 == 0: the groups
        // past N are all pad rows)
        const int64_t NG = (int64_t)N / 32, NGp = Np / 32;
        for (int64_t gi = (int64_t)blockIdx.y * kFoldWaves + wave; gi < NGp; gi += wstride) {
            const int64_t n0 = gi * 32;
            float tmax = 0.0f;
            for (int r = 0; r < 32; ++r) {
                float f[8];
                fold_row(n0 + r, f);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    tmax = fmaxf(tmax, __builtin_fabsf(__uint_as_float(__float_as_uint(f[i]) & keep[i])));
            }
            const uint32_t c = e8m0_from_amax_bits(__float_as_uint(quad_max_f(tmax)));
            for (int r = 0; r < 32; ++r) {
                const int64_t n = n0 + r;
                float f[8];
                fold_row(n, f);
                (void)extract(n, f);
                encode_store(n, f, c);
            }
            if (valid && gi < NG && (lane & 3) == 0) Wst[gi * nb + j0 / 32] = (uint8_t)c;
        }
    }
}

}  // namespace

hipError_t launch_smooth(const float* a, const float* w, int32_t K, double alpha, int32_t smooth,
                         float* s, float* rcp, hipStream_t st) {
    hipLaunchKernelGGL(smooth_kernel, dim3((K + 255) / 256), dim3(256), 0, st, a, w, K, alpha, smooth,
                       s, rcp);
    return hipGetLastError();
}

hipError_t launch_topk(const float* a, const float* s, int32_t K, int32_t k, int32_t* O, int32_t* pos,
                       hipStream_t st) {
    const int C = (K + kTopkThreads - 1) / kTopkThreads;    // scores per thread (K <= kMaxK: C <= 64)
    static_assert(kMaxK <= 64 * kTopkThreads, "top-k holds at most 64 scores per thread");
    if (C <= 8)
        hipLaunchKernelGGL(topk_kernel<8>, dim3(1), dim3(kTopkThreads), 0, st, a, s, K, k, O, pos);
    else if (C <= 16)
        hipLaunchKernelGGL(topk_kernel<16>, dim3(1), dim3(kTopkThreads), 0, st, a, s, K, k, O, pos);
    else if (C <= 32)
        hipLaunchKernelGGL(topk_kernel<32>, dim3(1), dim3(kTopkThreads), 0, st, a, s, K, k, O, pos);
    else
        hipLaunchKernelGGL(topk_kernel<64>, dim3(1), dim3(kTopkThreads), 0, st, a, s, K, k, O, pos);
    return hipGetLastError();
}

hipError_t launch_fold_pack(const void* W, int32_t dtype, int32_t N, int32_t K, int32_t k,
                            int32_t layout, const float* s, const int32_t* pos, uint8_t* Wq,
                            uint8_t* Ws, uint8_t* Wst, uint16_t* WO, hipStream_t st) {
    if (N <= 0) return hipSuccess;
    const bool bf = dtype == MG_BF16;
    const bool tile = layout == MG_W_32X32;
    const bool stripe = layout == MG_W_128X1;
    const int64_t gx = ((int64_t)K / 8 + 63) / 64;
    // 32x32: a wave per 32-row group; otherwise a workgroup per 32-row group
    const int64_t groups = ((int64_t)N + kScRows - 1) / kScRows * (kScRows / 32);
    int64_t gy = tile ? (groups + kFoldWaves - 1) / kFoldWaves : groups;
    // one resident round of workgroups
#define MG_FOLD_LAUNCH(BFV, LAYV)                                                                          \
    do {                                                                                                   \
        const void* kern = reinterpret_cast<const void*>(fold_pack_kernel<BFV, LAYV>);                     \
        int64_t cap = (int64_t)device_cu_count() * blocks_per_cu(kern) / gx;                               \
        cap = cap < 1 ? 1 : cap;                                                                           \
        const int64_t gyl = gy > cap ? cap : (gy > 65535 ? 65535 : gy);                                    \
        hipLaunchKernelGGL((fold_pack_kernel<BFV, LAYV>), dim3((unsigned)gx, (unsigned)gyl), dim3(256), 0, st, \
                           W, N, K, k, s, pos, Wq, Ws, Wst, WO);                                           \
    } while (0)
    if (bf) {
        if (tile) MG_FOLD_LAUNCH(true, MG_W_32X32);
        else if (stripe) MG_FOLD_LAUNCH(true, MG_W_128X1);
        else MG_FOLD_LAUNCH(true, MG_W_1X32);
    } else {
        if (tile) MG_FOLD_LAUNCH(false, MG_W_32X32);
        else if (stripe) MG_FOLD_LAUNCH(false, MG_W_128X1);
        else MG_FOLD_LAUNCH(false, MG_W_1X32);
    }
#undef MG_FOLD_LAUNCH
    return hipGetLastError();
}

}  // namespace mg
