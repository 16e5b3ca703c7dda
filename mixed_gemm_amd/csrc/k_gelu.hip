// GELU (tanh form) between the two projections of the FFN block: the
// calibrated FFN inputs sit after the SiLU/GELU gates ("W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B", integration paragraph).
// out = gelu_tanh(y) rounded to bf16 (gelu_bf16x2: the sigmoid form with the
// hardware exp2 and reciprocal), 8 bf16 per 16-byte vector; a thread takes
// four vectors per iteration with all four streaming (non-temporal) loads
// issued first, so more bytes are in flight per CU.  HBM-bound: 4 bytes per
// element.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

typedef uint32_t v4u __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(256) gelu_kernel(const uint16_t* __restrict__ in,
                                                   uint16_t* __restrict__ out, int64_t n) {
    constexpr int U = 4;                 // 16-byte vectors per thread and iteration, loads issued first
    const int64_t nvec = n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const uint4* __restrict__ vin = reinterpret_cast<const uint4*>(in);
    uint4* __restrict__ vout = reinterpret_cast<uint4*>(out);
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    for (; i + (U - 1) * stride < nvec; i += U * stride) {
        uint4 d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const v4u x = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(&vin[i + u * stride]));
            d[u] = make_uint4(x[0], x[1], x[2], x[3]);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const v4u o = {gelu_bf16x2(d[u].x), gelu_bf16x2(d[u].y), gelu_bf16x2(d[u].z), gelu_bf16x2(d[u].w)};
            __builtin_nontemporal_store(o, reinterpret_cast<v4u*>(&vout[i + u * stride]));
        }
    }
    for (; i < nvec; i += stride) {
        const uint4 d = vin[i];
        vout[i] = make_uint4(gelu_bf16x2(d.x), gelu_bf16x2(d.y), gelu_bf16x2(d.z), gelu_bf16x2(d.w));
    }
    // tail (n % 8 elements)
    const int64_t t = nvec * 8 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (t < n && (int64_t)blockIdx.x * blockDim.x + threadIdx.x < 8) out[t] = (uint16_t)gelu_bf16x2(in[t]);
}

}  // namespace

hipError_t launch_gelu(const uint16_t* in, uint16_t* out, int64_t n, hipStream_t st) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n / 8 + 255) / 256;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gelu_kernel, dim3((unsigned)blocks), dim3(256), 0, st, in, out, n);
    return hipGetLastError();
}

}  // namespace mg
