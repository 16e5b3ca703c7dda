// GELU (tanh form) between the two projections of the FFN block: the
// calibrated FFN inputs sit after the SiLU/GELU gates ("W4A4 Quantization for
// Inference on Wan2.2-I2V-A14B", integration paragraph).
// out = gelu_tanh(y) rounded to bf16 (gelu_bf16x2: the sigmoid form with the
// hardware exp2 and reciprocal), 8 bf16 per lane (16-byte loads and stores).
// HBM-bound: 4 bytes per element.
#include "mg_device.h"
#include "mg_internal.h"

namespace mg {

namespace {

__global__ void __launch_bounds__(256) gelu_kernel(const uint16_t* in,
                                                   uint16_t* out, int64_t n) {
    const int64_t nvec = n / 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
        const uint4 d = reinterpret_cast<const uint4*>(in)[i];
        const uint32_t w[4] = {d.x, d.y, d.z, d.w};
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k] = gelu_bf16x2(w[k]);
        reinterpret_cast<uint4*>(out)[i] = make_uint4(o[0], o[1], o[2], o[3]);
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
