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
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBN = 64;        // contraction (N) per main-loop step
constexpr int kLds = kBN + 8;  // LDS pitch in bf16
constexpr int kThreads = 256;

// Workgroup tile: 128 tokens x 128 input features, 4 waves in a 2x2 grid (64 x 64
// each, 32x32x16 MFMA), contraction steps of 64 over N. Per step each thread loads
// (raw buffer loads, hardware zero outside the tensors) a 4 (n) x 8 (k) patch of
// codes with the 4 row scales, and 4 16-byte chunks of the dY tile, one step ahead;
// after the current step's MFMAs it dequantises the patch - one 8-byte read of a
// 256-entry (level[lo], level[hi]) pair table per code byte, fp32 multiply by the
// row's absmax, bf16 pack pairing rows - and stores the patch transposed into the
// other LDS buffer. dY and the weight tile are double-buffered: one barrier per step.
__global__ __launch_bounds__(kThreads, 2) void k_nf4_gemm_bwd_dx(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const float* __restrict__ g, const uint16_t* __restrict__ A, int T, int N, int K, int r, float s,
    int steps_per_split, uint16_t* __restrict__ dx, float* __restrict__ partial, Tables tab) {
    constexpr int BM = 128, BK = 128;
    constexpr int WM = BM / 2, WK = BK / 2;
    constexpr int FM = WM / 32, FK = WK / 32;
    constexpr int A_CHUNKS = BM * (kBN / 8) / kThreads;  // 4

    __shared__ __align__(16) uint16_t sA[2][BM * kLds];
    __shared__ __align__(16) uint16_t sWt[2][BK * kLds];
    __shared__ __align__(16) float sLut[512];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wk = wave & 1;
    const int k0 = blockIdx.x * BK;
    const int m0 = blockIdx.y * BM;
    const int nsteps = (N + kBN - 1) / kBN;
    const int nb_begin = blockIdx.z * steps_per_split;
    const int nb_end = min(nb_begin + steps_per_split, nsteps);
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    sLut[2 * tid] = tab.level[tid & 15];  // entry b: the two codes of byte b
    sLut[2 * tid + 1] = tab.level[tid >> 4];

    // this thread's patch: rows 4*pr .. 4*pr+3 of the step, columns 8*pc .. 8*pc+7 of the tile
    const int pr = tid >> 4, pc = tid & 15;
    const uint32_t trows = uint32_t(max(0, min(BM, T - m0)));
    const auto rdy = make_rsrc(dy + size_t(m0) * N, trows * uint32_t(N) * 2u);
    // codes/absmax of the whole matrix (the entry points keep N*K/2 below 2^30 bytes);
    // patches beyond N or K load from kOutOfRange and read as zero
    const auto rcd = make_rsrc(codes, uint32_t(N) * uint32_t(K / 2));
    const auto rsc = make_rsrc(absmax, uint32_t(N) * uint32_t(K / 64) * 4u);
    const uint32_t kc = uint32_t(k0 + 8 * pc);
    uint32_t a_off[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + kThreads * i;
        a_off[i] = (uint32_t(c >> 3) * uint32_t(N) + uint32_t(c & 7) * 8u) * 2u;
    }

    u32x4 ra[A_CHUNKS];
    uint32_t rc[4];
    float rs[4];
    auto gload = [&](int nb) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            // dY columns at or beyond N (ragged last step) read as zero
            const bool ok = nb * kBN + 8 * ((tid + kThreads * i) & 7) < N;
            ra[i] = buf_load16(rdy, ok ? a_off[i] + uint32_t(nb) * (kBN * 2) : kOutOfRange);
        }
        // Rows n >= N lie past the end of both buffers and read as zero (scale 0, so
        // the dequantised row is zero). Columns k >= K of a ragged tile read the next
        // row's data: they only reach dX columns that are never stored.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t n = uint32_t(nb * kBN + 4 * pr + i);
            rc[i] = buf_load_u32(rcd, n * uint32_t(K / 2) + kc / 2);
            rs[i] = buf_load_f32(rsc, n * uint32_t(K / 64) * 4u + (kc / 64) * 4u);
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(&sA[buf][(c >> 3) * kLds + (c & 7) * 8]) = ra[i];
        }
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float2 lv = *reinterpret_cast<const float2*>(lut + (((rc[i] >> (8 * b)) & 0xFFu) << 3));
                // level * absmax in fp32, then RNbf (below): the format's two roundings
                v[i][2 * b] = lv.x * rs[i];
                v[i][2 * b + 1] = lv.y * rs[i];
            }
        // row k = 8*pc + e holds n = 4*pr .. 4*pr+3: chunk pr/2 (swizzled by pc), half pr&1
        const int col = (((pr >> 1) ^ (pc & 7)) << 3) + 4 * (pr & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u32x2 o = {pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e])};
            *reinterpret_cast<u32x2*>(&sWt[buf][(8 * pc + e) * kLds + col]) = o;
        }
    };

    f32x16 acc[FM][FK];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (nb_begin < nb_end) {
        gload(nb_begin);
        __syncthreads();  // sLut visible
        sstore(0);
        __syncthreads();
        auto step = [&](int nb, auto c_) {
            constexpr int C = decltype(c_)::value;
            const bool more = nb + 1 < nb_end;
            if (more) gload(nb + 1);
#pragma unroll
            for (int kk = 0; kk < kBN / 16; ++kk) {
                bf16x8 af[FM], bw[FK];
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        &sA[C][(wm * WM + 32 * i + frag_row) * kLds + kk * 16 + frag_k]));
#pragma unroll
                for (int j = 0; j < FK; ++j) {
                    const int row = wk * WK + 32 * j + frag_row;
                    const int chunk = (2 * kk + (lane >> 5)) ^ ((row >> 3) & 7);
                    bw[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sWt[C][row * kLds + chunk * 8]));
                }
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FK; ++j) acc[i][j] = mfma32x32x16(af[i], bw[j], acc[i][j]);
            }
            if (more) sstore(C ^ 1);  // next step's tiles into the other buffers
            __syncthreads();
        };
        for (int nb = nb_begin; nb < nb_end; nb += 2) {
            step(nb, std::integral_constant<int, 0>{});
            if (nb + 1 < nb_end) step(nb + 1, std::integral_constant<int, 1>{});
        }
    }

    // LoRA as a K-extension (split 0 only when split): acc += (s.g)_hi . A + (s.g)_lo . A
    for (int c0 = 0; c0 < (blockIdx.z == 0 ? r : 0); c0 += 16) {
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

    float* pdst = partial ? partial + size_t(blockIdx.z) * T * K : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = m0 + wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int col = k0 + wk * WK + 32 * j + (lane & 31);
                if (row < T && col < K) {
                    if (pdst)
                        pdst[size_t(row) * K + col] = acc[i][j][e];
                    else
                        dx[size_t(row) * K + col] = bf16_bits(acc[i][j][e]);
                }
            }
}

// dX = RNbf( sum_z partial[z] ), z in increasing order (split 0 already holds the
// LoRA term); four consecutive outputs per thread, float4 loads.
__global__ __launch_bounds__(256) void k_split_sum_bf16_dx(const float* __restrict__ partial, int splits,
                                                           int64_t total, uint16_t* __restrict__ out) {
    const int64_t idx = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (idx >= total) return;
    f32x4 acc = *reinterpret_cast<const f32x4*>(partial + idx);
    for (int z = 1; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(partial + size_t(z) * total + idx);
    u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(out + idx) = o;
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
    pick_token_chunks(p.nslab, T, p.pre_chunks, p.pre_tc);
    pick_token_chunks(cdiv(K, 64), T, p.da_chunks, p.da_tc);
    size_t off = 0;
    p.off_g = off;
    off += align256(size_t(T) * size_t(std::max(r, 1)) * 4);
    p.off_gpart = off;
    off += r > 0 ? align256(size_t(p.nslab) * size_t(T) * size_t(r) * 4) : 0;
    p.off_dbpart = off;
    off += (r > 0 && p.pre_chunks > 1) ? align256(size_t(p.pre_chunks) * size_t(N) * size_t(r) * 4) : 0;
    p.off_dapart = off;
    off += (r > 0 && p.da_chunks > 1) ? align256(size_t(p.da_chunks) * size_t(r) * size_t(K) * 4) : 0;
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
    hipLaunchKernelGGL(k_nf4_gemm_bwd_dx, grid, dim3(kThreads), 0, stream, dy, codes, absmax, g, A, int(T), int(N),
                       int(K), r, s, p.steps_per_split, dx, partial, tables());
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t total = T * K;
    hipLaunchKernelGGL(k_split_sum_bf16_dx, dim3(unsigned(cdiv(total / 4, 256))), dim3(256), 0, stream, partial,
                       p.splits, total, dx);
    return hipGetLastError();
}

}  // namespace nf4
