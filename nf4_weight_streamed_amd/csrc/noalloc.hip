// nf4_lora_linear_fwd_noalloc: the forward of the LoRA linear with its workspace in a
// library-owned device array instead of a caller allocation, for callers that cannot
// allocate (code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc). The kernels and their launch plans are those of nf4_lora_linear_fwd;
// only where the workspace lives differs.
//
// `scratch` is a file-scope device array: every GPU the library runs on holds its own
// copy, at its own address, until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it is only a stand-in for the
// symbol): the device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device.
#include <mutex>

#include "../../include/nf4lora.h"
#include "common.h"

namespace nf4 {
namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // NF4_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == NF4_NOALLOC_SCRATCH_BYTES, "header and library agree on the scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up on first use).
int scratch_ptr(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(NF4_E_HIP, "nf4_lora_linear_fwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices)
        return fail(NF4_E_ARG, "nf4_lora_linear_fwd_noalloc: device %d beyond the %d the library tracks", dev,
                    kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(NF4_E_HIP, "nf4_lora_linear_fwd_noalloc: hipGetSymbolAddress(scratch) on device %d: %s", dev,
                        hipGetErrorString(e));
        g_ptr[dev] = p;
    }
    *out = g_ptr[dev];
    return NF4_OK;
}

}  // namespace
}  // namespace nf4

extern "C" int nf4_lora_linear_fwd_noalloc(const uint8_t* codes, const float* absmax, int64_t N, int64_t K,
                                           const uint16_t* x, int64_t T, const uint16_t* A, const uint16_t* B, int r,
                                           float alpha, uint16_t* y, float* u_save, nf4_stream stream) {
    using namespace nf4;
    const char* fn = "nf4_lora_linear_fwd_noalloc";
    int st = check_linear_args(fn, codes, absmax, N, K, T, r, alpha);
    if (st != NF4_OK) return st;
    if (T == 0) return NF4_OK;
    const size_t need = plan_fwd(T, N, K, r).ws_bytes;
    if (need > kScratchBytes)
        return fail(NF4_E_SHAPE, "%s: T=%lld N=%lld K=%lld r=%d needs %zu bytes of workspace, beyond the %zu-byte "
                                 "scratch; call nf4_lora_linear_fwd with a workspace instead",
                    fn, (long long)T, (long long)N, (long long)K, r, need, kScratchBytes);
    void* ws = nullptr;
    st = scratch_ptr(&ws);
    if (st != NF4_OK) return st;
    return linear_fwd(fn, codes, absmax, nullptr, N, K, x, T, A, B, r, alpha, y, u_save, ws, kScratchBytes, stream);
}
