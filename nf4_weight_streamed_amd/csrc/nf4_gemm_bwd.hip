// Fused NF4-dequantise + bf16 MFMA GEMM for the input gradient of the LoRA linear.
//
//   dX = RNbf( dY . W + s . g . A ),  g = dY . B  (fp32, from the LoRA pre-pass)
//
// The base is frozen: only dX flows through it and no weight gradient is formed
// (Poros API reference, "patch_hf_model" Behavior 3; HN comment thread on
// streaming the frozen base, main comment). The contraction runs over N, the
// rows of W, while the codes are contiguous along K: each thread dequantises a
// 4 (n) x 8 (k) patch and packs bf16 pairs across rows, so the tile lands in LDS
// as [k][n] and the MFMA B operand is again a contiguous 16-byte read. The 16-byte
// chunks of each LDS row are XOR-swizzled by (k / 8) % 8: the 8-byte transposed
// stores of a wave then spread over all banks, and the fragment reads (8
// consecutive rows share one swizzle) stay conflict-free.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBN = 64;        // contraction (N) per main-loop step
constexpr int kLds = kBN + 8;  // LDS pitch in bf16
constexpr int kThreads = 256;

template <int BM, int BK>
__global__ __launch_bounds__(kThreads, 2) void k_nf4_gemm_bwd_dx(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const float* __restrict__ g, const uint16_t* __restrict__ A, int T, int N, int K, int r, float s,
    int steps_per_split, uint16_t* __restrict__ dx, float* __restrict__ partial, Tables tab) {
    constexpr int WM = BM / 2, WK = BK / 2;
    constexpr int FM = WM / 32, FK = WK / 32;
    constexpr int A_CHUNKS = BM * (kBN / 8) / kThreads;
    static_assert(BK == 128, "patch mapping assumes 16 row-groups x 16 col-groups");
    static_assert(A_CHUNKS >= 1, "tile too small");

    __shared__ __align__(16) uint16_t sA[BM * kLds];
    __shared__ __align__(16) uint16_t sWt[BK * kLds];
    __shared__ float sLut[16];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wk = wave & 1;
    const int k0 = blockIdx.x * BK;
    const int m0 = blockIdx.y * BM;
    const int nsteps = (N + kBN - 1) / kBN;
    const int nb_begin = blockIdx.z * steps_per_split;
    const int nb_end = min(nb_begin + steps_per_split, nsteps);
    const size_t code_pitch = size_t(K) / 2;
    const size_t scale_pitch = size_t(K) / 64;

    // patch of this thread: rows 4*pr .. 4*pr+3 of the step, columns 8*pc .. 8*pc+7 of the tile
    const int pr = tid >> 4, pc = tid & 15;

    if (tid < 16) sLut[tid] = tab.level[tid];

    u32x4 ra[A_CHUNKS];
    uint32_t rc[4];
    float rs[4];

    auto gload = [&](int nb) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            const int row = c >> 3, col8 = c & 7;
            const int t = m0 + row;
            const int n = nb * kBN + col8 * 8;
            ra[i] = (t < T && n < N) ? *reinterpret_cast<const u32x4*>(dy + size_t(t) * N + n)
                                     : u32x4{0u, 0u, 0u, 0u};
        }
        const int kc = k0 + 8 * pc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int n = nb * kBN + 4 * pr + i;
            if (n < N && kc < K) {
                rc[i] = *reinterpret_cast<const uint32_t*>(codes + size_t(n) * code_pitch + kc / 2);
                rs[i] = absmax[size_t(n) * scale_pitch + kc / 64];
            } else {
                rc[i] = 0x77777777u;
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
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = sLut[(rc[i] >> (4 * e)) & 15] * rs[i];
        // row k = 8*pc + e holds n = 4*pr .. 4*pr+3: chunk pr/2 (swizzled by pc), half pr&1
        const int col = (((pr >> 1) ^ (pc & 7)) << 3) + 4 * (pr & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u32x2 o = {pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e])};
            *reinterpret_cast<u32x2*>(sWt + (8 * pc + e) * kLds + col) = o;
        }
    };

    f32x16 acc[FM][FK];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;

    if (nb_begin < nb_end) {
        gload(nb_begin);
        __syncthreads();
        sstore();
        __syncthreads();
        for (int nb = nb_begin; nb < nb_end; ++nb) {
            const bool more = nb + 1 < nb_end;
            if (more) gload(nb + 1);
#pragma unroll
            for (int kk = 0; kk < kBN / 16; ++kk) {
                bf16x8 af[FM], bw[FK];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        sA + (wm * WM + 32 * i + frag_row) * kLds + kk * 16 + frag_k));
#pragma unroll
                for (int j = 0; j < FK; ++j) {
                    const int row = wk * WK + 32 * j + frag_row;
                    const int chunk = (2 * kk + (lane >> 5)) ^ ((row >> 3) & 7);
                    bw[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(sWt + row * kLds + chunk * 8));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FK; ++j) acc[i][j] = mfma32x32x16(af[i], bw[j], acc[i][j]);
            }
            __syncthreads();
            if (more) {
                sstore();
                __syncthreads();
            }
        }
    }

    if (partial != nullptr) {
        float* dst = partial + size_t(blockIdx.z) * T * K;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FK; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                    const int col = k0 + wk * WK + 32 * j + (lane & 31);
                    if (row < T && col < K) dst[size_t(row) * K + col] = acc[i][j][e];
                }
        return;
    }

    // LoRA as a K-extension: acc += (s.g)_hi . A + (s.g)_lo . A, r padded to 16.
    for (int c0 = 0; c0 < r; c0 += 16) {
        bf16x8 hi[FM], lo[FM], aa[FK];
        const int j0 = c0 + frag_k;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = m0 + wm * WM + 32 * i + frag_row;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (row < T && j0 + e < r) ? s * g[size_t(row) * r + j0 + e] : 0.0f;
                __bf16 h, l;
                split_bf16(v, h, l);
                hi[i][e] = h;
                lo[i][e] = l;
            }
        }
#pragma unroll
        for (int j = 0; j < FK; ++j) {
            const int col = k0 + wk * WK + 32 * j + frag_row;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint16_t av = (col < K && j0 + e < r) ? A[size_t(j0 + e) * K + col] : uint16_t(0);
                aa[j][e] = __builtin_bit_cast(__bf16, av);
            }
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FK; ++j) {
                acc[i][j] = mfma32x32x16(hi[i], aa[j], acc[i][j]);
                acc[i][j] = mfma32x32x16(lo[i], aa[j], acc[i][j]);
            }
    }

#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int col = k0 + wk * WK + 32 * j + (lane & 31);
                if (row < T && col < K) dx[size_t(row) * K + col] = bf16_bits(acc[i][j][e]);
            }
}

// dX = RNbf( sum_z partial[z] + s . g . A ), z in increasing order; four consecutive
// outputs of one row per thread (K % 64 == 0), float4 partial loads.
__global__ __launch_bounds__(256) void k_bwd_split_reduce(const float* __restrict__ partial, int splits, int T,
                                                          int K, const float* __restrict__ g,
                                                          const uint16_t* __restrict__ A, int r, float s,
                                                          uint16_t* __restrict__ dx) {
    const int64_t q = int64_t(blockIdx.x) * 256 + threadIdx.x;
    const int64_t total = int64_t(T) * K;
    if (q * 4 >= total) return;
    const int64_t idx = q * 4;
    const int row = int(idx / K), col = int(idx % K);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(partial + size_t(z) * total + idx);
    f32x4 lora = {0.f, 0.f, 0.f, 0.f};
    const float* gr = g + size_t(row) * r;
#pragma unroll 4
    for (int j = 0; j < r; ++j) {
        const float gj = gr[j];
        const u32x2 a4 = *reinterpret_cast<const u32x2*>(A + size_t(j) * K + col);
        lora[0] += gj * __uint_as_float(a4[0] << 16);
        lora[1] += gj * __uint_as_float(a4[0] & 0xFFFF0000u);
        lora[2] += gj * __uint_as_float(a4[1] << 16);
        lora[3] += gj * __uint_as_float(a4[1] & 0xFFFF0000u);
    }
    u32x2 o = {pack_bf16x2(acc[0] + s * lora[0], acc[1] + s * lora[1]),
               pack_bf16x2(acc[2] + s * lora[2], acc[3] + s * lora[3])};
    *reinterpret_cast<u32x2*>(dx + idx) = o;
}

}  // namespace

BwdPlan plan_bwd(int64_t T, int64_t N, int64_t K, int r) {
    BwdPlan p{};
    p.bm = 128;
    p.bn = 128;
    const int64_t tiles = cdiv(T, p.bm) * cdiv(K, p.bn);
    const int64_t nsteps = cdiv(N, kBN);
    const int64_t splits = pick_splits(tiles, nsteps, 4);
    p.steps_per_split = int(cdiv(nsteps, splits));
    p.splits = int(cdiv(nsteps, p.steps_per_split));
    p.nslab = int(cdiv(N, 64));
    size_t off = 0;
    p.off_g = off;
    off += align256(size_t(T) * size_t(std::max(r, 1)) * 4);
    p.off_gpart = off;
    off += r > 0 ? align256(size_t(p.nslab) * size_t(T) * size_t(r) * 4) : 0;
    p.off_dx = off;
    off += p.splits > 1 ? align256(size_t(p.splits) * size_t(T) * size_t(K) * 4) : 0;
    p.ws_bytes = off;
    return p;
}

hipError_t launch_gemm_bwd_dx(const BwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* dy,
                              const uint16_t* A, int64_t T, int64_t N, int64_t K, int r, float s, uint16_t* dx,
                              void* ws, hipStream_t stream) {
    const dim3 grid(unsigned(cdiv(K, p.bn)), unsigned(cdiv(T, p.bm)), unsigned(p.splits));
    const float* g = reinterpret_cast<const float*>(static_cast<char*>(ws) + p.off_g);
    float* partial = p.splits > 1 ? reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_dx) : nullptr;
    prof_gemm_begin(stream);
    hipLaunchKernelGGL((k_nf4_gemm_bwd_dx<128, 128>), grid, dim3(kThreads), 0, stream, dy, codes, absmax, g, A,
                       int(T), int(N), int(K), r, s, p.steps_per_split, dx, partial, tables());
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t total = T * K;
    hipLaunchKernelGGL(k_bwd_split_reduce, dim3(unsigned(cdiv(total / 4, 256))), dim3(256), 0, stream, partial,
                       p.splits, int(T), int(K), g, A, r, s, dx);
    return hipGetLastError();
}

}  // namespace nf4
