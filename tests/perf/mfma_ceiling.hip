// FP4 matrix-core ceiling of this GPU: how fast the block-scaled FP4 MFMA
// (v_mfma_scale_f32_32x32x64_f8f6f4, E2M1 operands, one E8M0 scale per 32 K)
// runs with no memory traffic at all -- the practical upper bound for the
// dual GEMM's bulk, next to the published dense peak.
//
// One 4-wave workgroup per compute unit (one wave per SIMD, as the GEMM runs);
// each wave keeps 16 independent 32x32 accumulators and issues 16 MFMAs per
// iteration on register operands.  Two operand modes:
//   fixed     the same FP4 bits every iteration;
//   changing  the operand bits are re-mixed every iteration (as data streaming
//             through a real GEMM does), which draws more power.
// Prints one JSON line per mode.  Usage: mfma_ceiling [iterations]
#include <hip/hip_runtime.h>

#include <stdio.h>
#include <stdlib.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

#define CK(x)                                                                              \
    do {                                                                                   \
        hipError_t e_ = (x);                                                               \
        if (e_ != hipSuccess) {                                                            \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                      \
        }                                                                                  \
    } while (0)

__device__ __forceinline__ unsigned mix(unsigned x) {   // xorshift32
    x ^= x << 13;
    x ^= x >> 17;
    x ^= x << 5;
    return x;
}

template <bool CHANGING>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
fp4_mfma_loop(int iters, unsigned seed, float* out) {
    const int lane = threadIdx.x;
    v16f acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = v16f{};
    unsigned x = (unsigned)lane * 2654435761u ^ seed ^ (blockIdx.x * 97u);
    v8i a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            x = mix(x);
            a[i][e] = e < 4 ? (int)x : 0;      // FP4 operands use the first 4 registers
            x = mix(x);
            b[i][e] = e < 4 ? (int)x : 0;
        }
    }
    const int sa = 120 + (lane & 7), sb = 121 + (lane & 3);   // E8M0 scales near 2^-6
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[4 * i + j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[4 * i + j], 4, 4, 0,
                                                                                  sa, 0, sb);
        if constexpr (CHANGING) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i][0] ^= (int)(0x9e3779b9u * (unsigned)(it + 1));
                a[i][1] += 0x7f4a7c15;
                a[i][2] ^= a[i][0];
                a[i][3] += a[i][1];
                b[i][0] ^= (int)0x85ebca6bu;
                b[i][1] += b[i][0];
                b[i][2] ^= (int)0xc2b2ae35u;
                b[i][3] += b[i][2];
            }
        }
    }
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[i][lane & 15];
    out[blockIdx.x * 256 + lane] = s;                        // keeps the work observable
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 20000;
    int dev = 0, cus = 0;
    CK(hipGetDevice(&dev));
    CK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    float* out = nullptr;
    CK(hipMalloc((void**)&out, (size_t)cus * 256 * sizeof(float)));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    const double flop = (double)cus * 4 /*waves*/ * iters * 16 /*MFMAs*/ * 2.0 * 32 * 32 * 64;
    for (int mode = 0; mode < 2; ++mode) {
        auto kern = mode == 0 ? fp4_mfma_loop<false> : fp4_mfma_loop<true>;
        hipLaunchKernelGGL(kern, dim3(cus), dim3(256), 0, 0, iters / 4, 1u, out);   // warm-up
        CK(hipGetLastError());
        CK(hipDeviceSynchronize());
        float best = 1e30f;
        for (int rep = 0; rep < 3; ++rep) {
            CK(hipEventRecord(e0, 0));
            hipLaunchKernelGGL(kern, dim3(cus), dim3(256), 0, 0, iters, 1u, out);
            CK(hipEventRecord(e1, 0));
            CK(hipEventSynchronize(e1));
            float ms = 0.0f;
            CK(hipEventElapsedTime(&ms, e0, e1));
            if (ms < best) best = ms;
        }
        const double tflops = flop / best / 1e9;
        printf("{\"operands\": \"%s\", \"cus\": %d, \"iterations\": %d, \"ms\": %.3f, \"tflops\": %.1f, "
               "\"frac_of_10100\": %.4f}\n",
               mode == 0 ? "fixed" : "changing", cus, iters, best, tflops, tflops / 10100.0);
    }
    CK(hipFree(out));
    return 0;
}
