// Denominator probe: the bf16 MFMA issue rate of this GPU, measured with the same
// instruction the GEMM kernels use (v_mfma_f32_32x32x16_bf16), so that achieved
// TFLOP/s can be reported against a measured ceiling beside the published peak.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

// Each wave runs `iters` rounds of 8 independent 32x32x16 MFMAs on register operands
// (no memory traffic inside the loop) and writes one float so that nothing is elided.
__global__ __launch_bounds__(256) void k_probe_mfma(float* __restrict__ out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = __bf16(float((lane + e) & 7) * 0.125f);
        b[e] = __bf16(float((lane * 3 + e) & 7) * 0.0625f);
    }
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;
    for (int it = 0; it < iters; ++it)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = mfma32x32x16(a, b, acc[i]);
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[i][e];
    if (lane == 0) out[blockIdx.x * 4 + (threadIdx.x >> 6)] = s;
}

// Read-rate probe: coalesced 16-byte loads of `n16` pieces in a grid-stride loop, U
// pieces in flight per thread (non-temporal loads with NT), folded with XOR into one
// word per thread (written to out[workgroup * 256 + thread]) so that no load is elided.
template <int U, bool NT>
__global__ __launch_bounds__(256) void k_probe_read(const u32x4* __restrict__ src, uint64_t n16,
                                                    uint32_t* __restrict__ out) {
    const uint64_t stride = uint64_t(gridDim.x) * 256;
    uint64_t i = uint64_t(blockIdx.x) * 256 + threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    auto ld = [&](uint64_t j) { return NT ? __builtin_nontemporal_load(src + j) : src[j]; };
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = ld(i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= ld(i);
    out[uint64_t(blockIdx.x) * 256 + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

hipError_t launch_probe_read_depth(const void* src, uint64_t bytes, uint32_t* out, int workgroups, int depth,
                                  bool nontemporal, hipStream_t stream) {
    const auto* s = static_cast<const u32x4*>(src);
    const dim3 grid = dim3(unsigned(workgroups)), block = dim3(256);
    const uint64_t n16 = bytes / 16;
#define NF4_PROBE_CASE(U)                                                                                 \
    case U:                                                                                               \
        if (nontemporal)                                                                                  \
            hipLaunchKernelGGL((k_probe_read<U, true>), grid, block, 0, stream, s, n16, out);             \
        else                                                                                              \
            hipLaunchKernelGGL((k_probe_read<U, false>), grid, block, 0, stream, s, n16, out);            \
        break;
    switch (depth) {
        NF4_PROBE_CASE(4)
        NF4_PROBE_CASE(8)
        NF4_PROBE_CASE(16)
        NF4_PROBE_CASE(32)
        default:
            return hipErrorInvalidValue;
    }
#undef NF4_PROBE_CASE
    return hipGetLastError();
}

hipError_t launch_probe_read(const void* src, uint64_t bytes, uint32_t* out, int workgroups, hipStream_t stream) {
    return launch_probe_read_depth(src, bytes, out, workgroups, 8, false, stream);
}

hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(k_probe_mfma, dim3(unsigned(workgroups)), dim3(256), 0, stream, out, iters);
    return hipGetLastError();
}

}  // namespace nf4
