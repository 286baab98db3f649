// Merged dense weight of a LoRA-adapted NF4 linear (Poros API reference,
// "PorosModel.merge_and_unload"; LoRA rank and alpha as in "PorosTrainer.from_pretrained"):
//
//   W_m[n][k] = RNbf( RN32( W[n][k] + RN32(s . l) ) ),  l = sum_j B[n][j] A[j][k]  (fp32, rank order)
//
// with W the dequantised NF4 base, RNbf(RN32(level . absmax)). A one-time export, bound by
// HBM: 0.5 B of codes + 1/16 B of scale read and 2 B written per weight. Workgroup = 64 rows
// x 256 columns: the A columns of the tile (r x 256) and the B rows (64 x r) are staged in
// LDS as fp32 (dynamic size, so a small rank leaves room for several workgroups per CU) and
// reused by every row / column of the tile; thread = 8 consecutive columns (one 4-byte code
// word, one scale, one 16-byte store) of 8 rows, all 8 rows' codes and scales loaded first.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;
constexpr int kCols = 256;  // columns per workgroup (32 threads x 8)
constexpr int kRowsPerThread = 8;
constexpr int kRows = (kThreads / 32) * kRowsPerThread;  // 64 rows per workgroup

// dynamic LDS: A [j][k - k0] (r x 256 fp32), then B [n - n0][j] (64 x r fp32)
size_t merge_lds_bytes(int r) { return size_t(r) * (kCols + kRows) * 4; }

__global__ __launch_bounds__(kThreads) void k_nf4_merge_lora(const uint8_t* __restrict__ codes,
                                                             const float* __restrict__ absmax, int N, int K,
                                                             const uint16_t* __restrict__ A,
                                                             const uint16_t* __restrict__ B, int r, float s,
                                                             uint16_t* __restrict__ w_out, Tables tab) {
    extern __shared__ __align__(16) float dyn[];
    float* sA = dyn;
    float* sB = dyn + r * kCols;
    __shared__ float lut[16];
    const int tid = threadIdx.x;
    const int k0 = int(blockIdx.x) * kCols, n0 = int(blockIdx.y) * kRows;
    const int c8 = 8 * (tid % 32), k = k0 + c8, row0 = tid / 32;
    // this thread's codes and scales first (rows past N and columns past K read zero)
    const auto rc = make_rsrc(codes, uint32_t(N) * uint32_t(K / 2));
    const auto rs = make_rsrc(absmax, uint32_t(N) * uint32_t(K / 64) * 4u);
    uint32_t cw[kRowsPerThread];
    float sc[kRowsPerThread];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const uint32_t n = uint32_t(n0 + row0 + 8 * i);
        const bool ok = k < K;
        cw[i] = buf_load_u32(rc, ok ? n * uint32_t(K / 2) + uint32_t(k / 2) : kOutOfRange);
        sc[i] = buf_load_f32(rs, ok ? (n * uint32_t(K / 64) + uint32_t(k / 64)) * 4u : kOutOfRange);
    }
    if (tid < 16) lut[tid] = tab.level[tid];
    // A tile: r rows of 256 columns in 16-byte pieces (columns past K read zero)
    const auto ra = make_rsrc(A, uint32_t(r) * uint32_t(K) * 2u);
    for (int o = tid; o < r * (kCols / 8); o += kThreads) {
        const int j = o / (kCols / 8), p8 = 8 * (o % (kCols / 8));
        const u32x4 v = buf_load16(ra, k0 + p8 < K ? (uint32_t(j) * uint32_t(K) + uint32_t(k0 + p8)) * 2u : kOutOfRange);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            sA[j * kCols + p8 + 2 * e] = __uint_as_float(v[e] << 16);
            sA[j * kCols + p8 + 2 * e + 1] = __uint_as_float(v[e] & 0xFFFF0000u);
        }
    }
    const auto rb = make_rsrc(B, uint32_t(N) * uint32_t(r) * 2u);
    for (int o = tid; o < kRows * r; o += kThreads)  // rows past N read zero
        sB[o] = bf16_to_f32(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(
            rb, int((uint32_t(n0) * uint32_t(r) + uint32_t(o)) * 2u), 0, 0)));
    __syncthreads();
    if (k >= K) return;  // K % 64 == 0: the 8 columns are all in or all out

    float l[kRowsPerThread][8];
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) l[i][e] = 0.0f;
    for (int j = 0; j < r; ++j) {  // rank order
        const f32x4 a0 = *reinterpret_cast<const f32x4*>(&sA[j * kCols + c8]);
        const f32x4 a1 = *reinterpret_cast<const f32x4*>(&sA[j * kCols + c8 + 4]);
#pragma unroll
        for (int i = 0; i < kRowsPerThread; ++i) {
            const float b = sB[(row0 + 8 * i) * r + j];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l[i][e] = __builtin_fmaf(b, a0[e], l[i][e]);
                l[i][4 + e] = __builtin_fmaf(b, a1[e], l[i][4 + e]);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < kRowsPerThread; ++i) {
        const int n = n0 + row0 + 8 * i;
        if (n >= N) break;
        u32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const uint32_t byte = cw[i] >> (8 * e);
            // the dequantised base RNbf(RN32(level . absmax)) (exact in fp32), then
            // RN32(W + RN32(s . l)) with no contraction, then RNbf
            const float w0 = bf16_to_f32(bf16_bits(lut[byte & 15] * sc[i]));
            const float w1 = bf16_to_f32(bf16_bits(lut[(byte >> 4) & 15] * sc[i]));
            o[e] = pack_bf16x2(__fadd_rn(w0, __fmul_rn(s, l[i][2 * e])), __fadd_rn(w1, __fmul_rn(s, l[i][2 * e + 1])));
        }
        *reinterpret_cast<u32x4*>(&w_out[size_t(n) * K + k]) = o;
    }
}

}  // namespace

hipError_t launch_merge_lora(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* w_out, hipStream_t stream) {
    const dim3 grid(unsigned(cdiv(K, kCols)), unsigned(cdiv(N, kRows)));
    hipLaunchKernelGGL(k_nf4_merge_lora, grid, dim3(kThreads), merge_lds_bytes(r), stream, codes, absmax, int(N), int(K),
                       A, B, r, s, w_out, tables());
    return hipGetLastError();
}

}  // namespace nf4
