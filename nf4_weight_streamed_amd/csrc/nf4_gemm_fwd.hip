// Fused NF4-dequantise + bf16 MFMA GEMM with the LoRA side path in its epilogue (forward).
//
//   y = RNbf( x . W^T + s . u . B^T ),  W = dequantised NF4 base [N, K], u = x . A^T [T, r]
//
// The frozen base is only read (HN comment thread on streaming the frozen base,
// main comment) and is NF4 with rank-r LoRA on top (Poros API reference,
// "PorosTrainer.from_pretrained"). Design for gfx950:
//  - workgroup tile BM tokens x BN out-features, 4 waves in a 2x2 grid, each wave
//    (BM/2) x (BN/2) of v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulators;
//  - each K step covers one 64-element NF4 block, so a row of the W tile has one scale;
//  - x tile: 16-byte coalesced loads -> LDS; codes: 16-byte loads (32 codes of one row
//    per thread) -> dequantised in registers through the 16 levels held in LDS ->
//    bf16 tile in LDS: every weight element is dequantised once per workgroup;
//  - the next step's global loads are issued before the current step's MFMAs;
//  - LoRA: (s.u) is split into bf16 hi + lo and contracted with B on the same
//    accumulators (a K-extension of r per part), so y is rounded once;
//  - split-K (for shapes with too few tiles to fill 256 CUs): fp32 partials in the
//    caller's workspace, summed in a fixed order by k_fwd_split_reduce.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBK = 64;        // K per main-loop step (= one NF4 block)
constexpr int kLds = kBK + 8;  // LDS row pitch in bf16 (144 B: conflict-free 16 B fragment reads)
constexpr int kThreads = 256;

template <int BM, int BN>
__global__ __launch_bounds__(kThreads, 2) void k_nf4_gemm_fwd(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const float* __restrict__ u, const uint16_t* __restrict__ B, int T, int N, int K, int r, float s,
    int steps_per_split, uint16_t* __restrict__ y, float* __restrict__ partial, Tables tab) {
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int A_CHUNKS = BM * (kBK / 8) / kThreads;  // 16-byte chunks of x per thread
    constexpr int W_PARTS = BN * 2 / kThreads;            // 32-code half rows per thread
    static_assert(A_CHUNKS >= 1 && W_PARTS >= 1, "tile too small for 256 threads");

    __shared__ __align__(16) uint16_t sA[BM * kLds];
    __shared__ __align__(16) uint16_t sW[BN * kLds];
    __shared__ float sLut[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int ksteps = K / kBK;
    const int kb_begin = blockIdx.z * steps_per_split;
    const int kb_end = min(kb_begin + steps_per_split, ksteps);
    const size_t code_pitch = size_t(K) / 2;
    const size_t scale_pitch = size_t(K) / 64;

    if (tid < 16) sLut[tid] = tab.level[tid];

    u32x4 ra[A_CHUNKS];
    u32x4 rc[W_PARTS];
    float rs[W_PARTS];

    auto gload = [&](int kb) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3, col8 = c & 7;
            const int g = m0 + row;
            ra[i] = (g < T) ? *reinterpret_cast<const u32x4*>(x + size_t(g) * K + size_t(kb) * kBK + col8 * 8)
                            : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < W_PARTS; ++i) {
            const int p = tid + kThreads * i;
            const int row = p >> 1, half = p & 1;
            const int g = n0 + row;
            if (g < N) {
                rc[i] = *reinterpret_cast<const u32x4*>(codes + size_t(g) * code_pitch + size_t(kb) * 32 + half * 16);
                rs[i] = absmax[size_t(g) * scale_pitch + kb];
            } else {
                rc[i] = u32x4{0x77777777u, 0x77777777u, 0x77777777u, 0x77777777u};
                rs[i] = 0.0f;
            }
        }
    };

    auto sstore = [&]() {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3, col8 = c & 7;
            *reinterpret_cast<u32x4*>(sA + row * kLds + col8 * 8) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < W_PARTS; ++i) {
            const int p = tid + kThreads * i;
            const int row = p >> 1, half = p & 1;
            const float sc = rs[i];
            uint16_t* dst = sW + row * kLds + half * 32;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t wq = rc[i][q];
                u32x4 o;
#pragma unroll
                for (int b = 0; b < 4; ++b) {
                    const uint32_t byte = wq >> (8 * b);
                    // level * absmax in fp32, then RNbf: bit-identical to the stand-alone dequantiser
                    o[b] = pack_bf16x2(sLut[byte & 15] * sc, sLut[(byte >> 4) & 15] * sc);
                }
                *reinterpret_cast<u32x4*>(dst + q * 8) = o;
            }
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    if (kb_begin < kb_end) {
        gload(kb_begin);
        __syncthreads();  // sLut visible
        sstore();
        __syncthreads();
        for (int kb = kb_begin; kb < kb_end; ++kb) {
            const bool more = kb + 1 < kb_end;
            if (more) gload(kb + 1);
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                bf16x8 af[FM], bw[FN];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        sA + (wm * WM + 32 * i + frag_row) * kLds + kk * 16 + frag_k));
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    bw[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        sW + (wn * WN + 32 * j + frag_row) * kLds + kk * 16 + frag_k));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(af[i], bw[j], acc[i][j]);
            }
            __syncthreads();
            if (more) {
                sstore();
                __syncthreads();
            }
        }
    }

    if (partial != nullptr) {
        // split-K: fp32 partial tile, reduced (with the LoRA term) by k_fwd_split_reduce
        float* dst = partial + size_t(blockIdx.z) * T * N;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    const int col = n0 + wn * WN + 32 * j + (lane & 31);
                    if (row < T && col < N) dst[size_t(row) * N + col] = acc[i][j][e];
                }
        return;
    }

    // LoRA as a K-extension: acc += (s.u)_hi . B^T + (s.u)_lo . B^T, r padded to 16.
    for (int c0 = 0; c0 < r; c0 += 16) {
        bf16x8 hi[FM], lo[FM], bb[FN];
        const int j0 = c0 + frag_k;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = m0 + wm * WM + 32 * i + frag_row;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (row < T && j0 + e < r) ? s * u[size_t(row) * r + j0 + e] : 0.0f;
                __bf16 h, l;
                split_bf16(v, h, l);
                hi[i][e] = h;
                lo[i][e] = l;
            }
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + wn * WN + 32 * j + frag_row;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t bv = (col < N && j0 + e < r) ? B[size_t(col) * r + j0 + e] : uint16_t(0);
                bb[j][e] = __builtin_bit_cast(__bf16, bv);
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                acc[i][j] = mfma32x32x16(hi[i], bb[j], acc[i][j]);
                acc[i][j] = mfma32x32x16(lo[i], bb[j], acc[i][j]);
            }
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int col = n0 + wn * WN + 32 * j + (lane & 31);
                if (row < T && col < N) y[size_t(row) * N + col] = bf16_bits(acc[i][j][e]);
            }
}

// y = RNbf( sum_z partial[z] + s . u . B^T ), z in increasing order; four consecutive
// outputs of one row per thread (N % 16 == 0), float4 partial loads.
__global__ __launch_bounds__(256) void k_fwd_split_reduce(const float* __restrict__ partial, int splits, int T,
                                                          int N, const float* __restrict__ u,
                                                          const uint16_t* __restrict__ B, int r, float s,
                                                          uint16_t* __restrict__ y) {
    const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = int64_t(T) * N;
    if (q * 4 >= total) return;
    const int64_t idx = q * 4;
    const int row = int(idx / N), col = int(idx % N);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(partial + size_t(z) * total + idx);
    f32x4 lora = {0.f, 0.f, 0.f, 0.f};
    const float* ur = u + size_t(row) * r;
    const uint16_t* br = B + size_t(col) * r;
#pragma unroll 4
    for (int j = 0; j < r; ++j) {
        const float uj = ur[j];
#pragma unroll
        for (int c = 0; c < 4; ++c) lora[c] += uj * bf16_to_f32(br[size_t(c) * r + j]);
    }
    u32x2 o = {pack_bf16x2(acc[0] + s * lora[0], acc[1] + s * lora[1]),
               pack_bf16x2(acc[2] + s * lora[2], acc[3] + s * lora[3])};
    *reinterpret_cast<u32x2*>(y + idx) = o;
}

}  // namespace

FwdPlan plan_fwd(int64_t T, int64_t N, int64_t K, int r) {
    FwdPlan p{};
    p.bm = 128;
    p.bn = 128;
    const int64_t tiles = cdiv(T, p.bm) * cdiv(N, p.bn);
    const int64_t ksteps = K / kBK;
    const int64_t splits = pick_splits(tiles, ksteps, 4);
    p.steps_per_split = int(cdiv(ksteps, splits));
    p.splits = int(cdiv(ksteps, p.steps_per_split));
    // u = x.A^T: 16-token blocks; split K until there are about 512 workgroups
    const int64_t tb = cdiv(T, 16), ks32 = K / 32;
    int64_t ds = std::min<int64_t>(cdiv(512, tb), std::max<int64_t>(1, ks32 / 8));
    ds = std::max<int64_t>(ds, 1);
    p.down_steps = int(cdiv(ks32, ds));
    p.down_splits = r > 0 ? int(cdiv(ks32, p.down_steps)) : 0;
    p.off_upart = 0;
    const size_t upart = p.down_splits > 1 ? align256(size_t(p.down_splits) * size_t(T) * size_t(r) * 4) : 0;
    p.off_ypart = upart;
    const size_t ypart = p.splits > 1 ? align256(size_t(p.splits) * size_t(T) * size_t(N) * 4) : 0;
    p.ws_bytes = upart + ypart;
    return p;
}

hipError_t launch_gemm_fwd(const FwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* x,
                           const float* u, const uint16_t* B, int64_t T, int64_t N, int64_t K, int r, float s,
                           uint16_t* y, void* ws, hipStream_t stream) {
    const dim3 grid(unsigned(cdiv(N, p.bn)), unsigned(cdiv(T, p.bm)), unsigned(p.splits));
    float* partial = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ypart) : nullptr;
    prof_gemm_begin(stream);
    hipLaunchKernelGGL((k_nf4_gemm_fwd<128, 128>), grid, dim3(kThreads), 0, stream, x, codes, absmax, u, B, int(T),
                       int(N), int(K), r, s, p.steps_per_split, y, partial, tables());
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t total = T * N;
    hipLaunchKernelGGL(k_fwd_split_reduce, dim3(unsigned(cdiv(total / 4, 256))), dim3(256), 0, stream, partial,
                       p.splits, int(T), int(N), u, B, r, s, y);
    return hipGetLastError();
}

}  // namespace nf4
