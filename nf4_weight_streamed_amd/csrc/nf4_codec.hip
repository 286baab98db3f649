// NF4 quantise / dequantise kernels for gfx950.
//
// Format (Poros API reference, "PorosTrainer.from_pretrained": quantization
// "nf4" = 4-bit NF4 QLoRA; its size per parameter is what "Poros on consumer
// GPUs", "What you need besides VRAM", quotes for the host-resident base):
// 64-element runs along a row share one float32 absmax; each element stores the
// 4-bit index of the NF4 level nearest to RN32(w / absmax), ties to the lower
// index; element 2i of a row sits in the low nibble of byte i.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;

// 8 lanes per 64-element block, 8 consecutive elements per lane: a wave covers
// 8 whole blocks (contiguous in memory because cols % 64 == 0).
template <typename In>
__device__ __forceinline__ void load8(const In* p, float v[8]);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[8]) {
    u32x4 raw = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(raw[i] << 16);
        v[2 * i + 1] = __uint_as_float(raw[i] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[8]) {
    u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = *reinterpret_cast<const u32x4*>(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[i] = __uint_as_float(a[i]);
        v[4 + i] = __uint_as_float(b[i]);
    }
}

// code = #{j : q >= thresh[j]} for q = RN32(w / absmax) in [-1, 1], through 65 buckets
// of width 1/32: bucket i = floor(32 q) + 32 (exact: 32 q is exact and so is the
// floor) holds the count of thresholds at or below its lower edge and the one
// threshold strictly inside it, if any (the thresholds are more than 1/32 apart), so a
// single compare finishes the count.
constexpr int kBuckets = 65;
struct Bucket {
    uint32_t below;  // thresholds <= the bucket's lower edge
    float inside;    // the threshold inside the bucket, or +inf
};

template <typename In>
__global__ __launch_bounds__(kThreads) void k_nf4_quantize(const In* __restrict__ w, int64_t n_blocks,
                                                           uint32_t* __restrict__ codes32,
                                                           float* __restrict__ absmax, Tables tab) {
    __shared__ Bucket buckets[kBuckets];
    if (threadIdx.x < kBuckets) {
        const float lo = float(int(threadIdx.x) - 32) * (1.0f / 32.0f), hi = lo + 1.0f / 32.0f;
        uint32_t below = 0;
        float inside = __builtin_inff();
        for (int j = 0; j < 15; ++j) {
            below += tab.thresh[j] <= lo ? 1u : 0u;
            if (tab.thresh[j] > lo && tab.thresh[j] < hi) inside = tab.thresh[j];
        }
        buckets[threadIdx.x] = Bucket{below, inside};
    }
    __syncthreads();
    const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    const int64_t blk = gid >> 3;
    const int sub = int(gid & 7);
    const bool active = blk < n_blocks;
    float v[8];
    if (active) {
        load8<In>(w + blk * 64 + sub * 8, v);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    // max over the 8 lanes of the block (exact: a max of float32 values)
    m = fmaxf(m, __shfl_xor(m, 1, 8));
    m = fmaxf(m, __shfl_xor(m, 2, 8));
    m = fmaxf(m, __shfl_xor(m, 4, 8));
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t code = 7;  // all-zero block: every element takes the level 0
        if (m > 0.0f) {
            const float q = __fdiv_rn(v[i], m);  // correctly rounded float32 quotient
            const Bucket b = buckets[int(__builtin_floorf(q * 32.0f)) + 32];
            code = b.below + (q >= b.inside ? 1u : 0u);
        }
        packed |= code << (4 * i);
    }
    if (active) {
        codes32[blk * 8 + sub] = packed;
        if (sub == 0) absmax[blk] = m;
    }
}

// One dword of codes (8 elements of one block) per thread -> 16 bytes of bf16.
__global__ __launch_bounds__(kThreads) void k_nf4_dequantize(const uint32_t* __restrict__ codes32,
                                                             const float* __restrict__ absmax, int64_t n_words,
                                                             u32x4* __restrict__ out, Tables tab) {
    __shared__ float lut[16];
    if (threadIdx.x < 16) lut[threadIdx.x] = tab.level[threadIdx.x];
    __syncthreads();
    const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    if (gid >= n_words) return;
    const uint32_t c = codes32[gid];
    const float s = absmax[gid >> 3];
    u32x4 o;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const uint32_t byte = c >> (8 * b);
        // level * absmax rounded to float32, then to bf16: the two roundings of the format
        const float lo = lut[byte & 15] * s;
        const float hi = lut[(byte >> 4) & 15] * s;
        o[b] = pack_bf16x2(lo, hi);
    }
    out[gid] = o;
}

}  // namespace

hipError_t launch_quantize(const void* w, int in_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                           float* absmax, hipStream_t stream) {
    const int64_t n_blocks = rows * (cols / 64);
    const int64_t threads = n_blocks * 8;
    const dim3 grid(unsigned(cdiv(threads, kThreads)));
    if (in_dtype == 0) {
        hipLaunchKernelGGL(k_nf4_quantize<uint16_t>, grid, dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(w), n_blocks, reinterpret_cast<uint32_t*>(codes), absmax,
                           tables());
    } else {
        hipLaunchKernelGGL(k_nf4_quantize<float>, grid, dim3(kThreads), 0, stream, static_cast<const float*>(w),
                           n_blocks, reinterpret_cast<uint32_t*>(codes), absmax, tables());
    }
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols, uint16_t* w,
                             hipStream_t stream) {
    const int64_t n_words = rows * cols / 8;
    const dim3 grid(unsigned(cdiv(n_words, kThreads)));
    hipLaunchKernelGGL(k_nf4_dequantize, grid, dim3(kThreads), 0, stream, reinterpret_cast<const uint32_t*>(codes),
                       absmax, n_words, reinterpret_cast<u32x4*>(w), tables());
    return hipGetLastError();
}

}  // namespace nf4
