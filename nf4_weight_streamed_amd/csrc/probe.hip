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

}  // namespace

hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream) {
    hipLaunchKernelGGL(k_probe_mfma, dim3(unsigned(workgroups)), dim3(256), 0, stream, out, iters);
    return hipGetLastError();
}

}  // namespace nf4
