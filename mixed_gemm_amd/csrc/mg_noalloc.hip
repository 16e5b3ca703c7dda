// mg_forward for callers that cannot allocate device memory: the per-forward
// activation workspace (Aq, As, XO) lives in a fixed array of this library,
// one copy per GPU, instead of caller-provided buffers.
#include <mutex>

#include "mg_internal.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // 64 MiB per GPU
constexpr int kMaxDevices = 64;

// Device-side workspace.  In host code `scratch` names a host-side stand-in,
// not device memory: only the address from hipGetSymbolAddress (per device)
// may be handed to kernels.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device.
hipError_t scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return hipSuccess;
}

size_t up256(size_t n) { return (n + 255) & ~size_t(255); }

}  // namespace

extern "C" {

int mg_forward_noalloc(const mg_plan* p, const void* X, int32_t dtype, int64_t M, void* Y, int32_t y_dtype,
                       hipStream_t stream) {
    // every check first (host only): a bad or oversized call fails before any HIP call
    if (int e = mg::check_forward(p, X, dtype, M, Y, y_dtype)) return e;
    if (M == 0) return MG_OK;
    size_t b[3];
    if (int e = mg_act_bytes(&p->d, M, b)) return e;
    const size_t offAs = up256(b[0]), offXO = up256(offAs + b[1]), total = offXO + b[2];
    if (total > kScratchBytes)
        return mg::fail_msg(MG_ERR_UNSUPPORTED,
                            "mg_forward_noalloc: M=%lld, K=%d, k=%d needs %zu workspace bytes, above the %zu-byte limit",
                            (long long)M, p->d.K, p->d.k, total, kScratchBytes);
    void* base = nullptr;
    const hipError_t h = scratch_ptr(&base);
    if (h != hipSuccess)
        return mg::fail_msg(MG_ERR_HIP, "mg_forward_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(h));
    uint8_t* w = static_cast<uint8_t*>(base);
    mg_act a;
    a.Aq = w;
    a.As = w + offAs;
    a.XO = b[2] ? reinterpret_cast<uint16_t*>(w + offXO) : nullptr;
    return mg_forward(p, X, dtype, M, &a, Y, y_dtype, stream);
}

}  // extern "C"
