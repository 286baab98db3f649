// NF4-LoRA linear for few tokens (the plans route T <= 16 here; the kernels accept
// T <= 64): the same operations as the 128-token GEMMs, organised for the HBM-bound
// regime, where every weight byte should be read once and streamed at full rate while
// MFMA work is cheap.
//
//   forward:  y  = RNbf( x . W^T + s . u . B^T ),  u = x . A^T (saved)
//   backward: dX = RNbf( dY . W + s . g . A ),     dA = s . g^T . x
//             (g and dB from k_lora_bwd_pre)
//
// The frozen NF4 base is only read (HN comment thread on streaming the frozen base,
// main comment); LoRA rank r and alpha as in the Poros API reference
// ("PorosTrainer.from_pretrained"). Tokens are padded to TB blocks of 16 for
// v_mfma_f32_16x16x32_bf16; both GEMM kernels split their contraction over the grid's
// y dimension and write fp32 partials, which the finish kernels add in split order,
// together with the LoRA terms, and round once.
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRank = 16 * NF4_MAX_RANK_BLOCKS;
constexpr int kSkinnyMaxT = int(kSkinnyT);
constexpr int kRows = 128;    // forward: weight rows per workgroup (4 waves x 2 blocks of 16)
constexpr int kDK = 256;      // forward: K per main-loop step (four NF4 blocks)
constexpr int kXP = kDK + 8;  // LDS pitch of the x tile (bf16)

// ------------------------------------------------------------------ forward
// Weight workgroups: 128 weight rows (wave w: rows 32w .. 32w+31, two 16-row blocks) x
// one K range of 256-wide steps. Within a step the contraction order is permuted
// identically for both operands: lane quarter q (lane / 16) supplies k = 64q + 8c ..
// 64q + 8c + 7 at MFMA chunk c (0..7), so a lane's 32 bytes of codes per row block are
// one whole NF4 block (one scale). Codes, scales and x are loaded two steps ahead into a
// ring of three register sets (about 32 KB of codes in flight per workgroup: the kernel
// is bound by memory latency x bytes in flight); the x tile of the current step is in
// double-buffered LDS. Output: fp32 partials ypart[split][T][N].
//
// u workgroups (blockIdx.x >= row_blocks, kUParts per split): the rows of A (bf16, wave
// w: ranks 16w .. 16w+15) against the same x for u = x.A^T, each over a quarter of the
// split's steps with plain loads (few registers, so the weight workgroups keep their
// occupancy) -> upart[split * kUParts + part][T][r].
constexpr int kUParts = 4;

template <int TB>
__device__ __forceinline__ void skinny_fwd_weights(const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes,
                                                   const float* __restrict__ absmax, int T, int N, int K,
                                                   int steps_per_split, float* __restrict__ ypart,
                                                   uint16_t* sXflat, const float* sLut) {
    constexpr int TP = 16 * TB;
    constexpr int XCH = TP * (kDK / 8) / kThreads;  // 16-byte x chunks per thread per step (2 TB)
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int nsteps = (K + kDK - 1) / kDK;
    const int kb_begin = int(blockIdx.y) * steps_per_split;
    const int kb_end = min(kb_begin + steps_per_split, nsteps);
    const auto rx = make_rsrc(x, uint32_t(T) * uint32_t(K) * 2u);
    const auto rcd = make_rsrc(codes, uint32_t(N) * uint32_t(K / 2));
    const auto rsc = make_rsrc(absmax, uint32_t(N) * uint32_t(K / 64) * 4u);
    // rows past N lie beyond the buffers (zero codes and scale); columns past K read
    // other rows' data against zero x columns
    const int n0 = int(blockIdx.x) * kRows + 32 * wave;
    uint32_t c_off[2], s_off[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const uint32_t n = uint32_t(n0 + 16 * nb + l16);
        c_off[nb] = n * uint32_t(K / 2) + uint32_t(q) * 32u;
        s_off[nb] = (n * uint32_t(K / 64) + uint32_t(q)) * 4u;
    }
    struct Set {
        u32x4 cw[2][2];  // codes [row block][16-byte piece]
        float sc[2];
        u32x4 xv[XCH];
    };
    Set ring[3];
    auto gload = [&](int kb, Set& st) {
        const uint32_t k0 = uint32_t(kb) * kDK;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int p = 0; p < 2; ++p) st.cw[nb][p] = buf_load16(rcd, c_off[nb] + k0 / 2u + uint32_t(p) * 16u);
            st.sc[nb] = buf_load_f32(rsc, s_off[nb] + (k0 / 64u) * 4u);
        }
        // only the threads of real tokens load (the padded rows stay zero in LDS):
        // vector-memory instructions, not bytes, limit this kernel
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;  // token c / 32, columns 8 (c % 32)
            const int t = c / (kDK / 8), k8 = 8 * (c % (kDK / 8));
            if (t < T) {
                const bool ok = int(k0) + k8 < K;
                st.xv[i] = buf_load16(rx, ok ? (uint32_t(t) * uint32_t(K) + k0 + uint32_t(k8)) * 2u : kOutOfRange);
            }
        }
    };
    typedef uint16_t XTile[TP * kXP];
    XTile* sX = reinterpret_cast<XTile*>(sXflat);
    auto store_x = [&](const Set& st, int buf) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;
            if (c / (kDK / 8) < T)
                *reinterpret_cast<u32x4*>(&sX[buf][(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = st.xv[i];
        }
    };
    // rows of the padded token block past T are zero in both buffers for the whole loop
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = tid + kThreads * i;
        if (c / (kDK / 8) >= T) {
            *reinterpret_cast<u32x4*>(&sX[0][(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&sX[1][(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = u32x4{0u, 0u, 0u, 0u};
        }
    }
    const char* lut = reinterpret_cast<const char*>(sLut);

    f32x4 acc[TB][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kb_begin < kb_end) {
        gload(kb_begin, ring[0]);
        gload(kb_begin + 1, ring[1]);
        store_x(ring[0], 0);
        __syncthreads();  // sLut and x tile 0
        // one step on ring slot C (compile-time: the loop is unrolled by three)
        auto step = [&](int kb, auto c_) {
            constexpr int C = decltype(c_)::value;
            const int buf = (kb - kb_begin) & 1;
            gload(kb + 2, ring[(C + 2) % 3]);  // two steps ahead; past the range: unused or zeros
            __builtin_amdgcn_sched_barrier(0);
            const Set& cur = ring[C];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                bf16x8 bw[2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const uint32_t w = cur.cw[nb][c >> 2][c & 3];
                    u32x4 o;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float2 lv = *reinterpret_cast<const float2*>(lut + (((w >> (8 * b)) & 0xFFu) << 3));
                        // level * absmax in fp32, then RNbf: the format's two roundings
                        o[b] = pack_bf16x2(lv.x * cur.sc[nb], lv.y * cur.sc[nb]);
                    }
                    bw[nb] = as_bf16x8(o);
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const bf16x8 xa = as_bf16x8(
                        *reinterpret_cast<const u32x4*>(&sX[buf][(16 * tb + l16) * kXP + 64 * q + 8 * c]));
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) acc[tb][nb] = mfma16x16x32(xa, bw[nb], acc[tb][nb]);
                }
            }
            store_x(ring[(C + 1) % 3], buf ^ 1);  // the next step's x (loaded a step ago)
            __syncthreads();
        };
        int kb = kb_begin;
        for (; kb + 2 < kb_end; kb += 3) {
            step(kb, std::integral_constant<int, 0>{});
            step(kb + 1, std::integral_constant<int, 1>{});
            step(kb + 2, std::integral_constant<int, 2>{});
        }
        if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
        if (kb + 1 < kb_end) step(kb + 1, std::integral_constant<int, 1>{});
    }

    // lane holds D[t = 16 tb + 4 q + e][row = 16 nb + l16]
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * tb + 4 * q + e;
            if (t >= T) continue;
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                const int n = n0 + 16 * nb + l16;
                if (n < N) ypart[(size_t(blockIdx.y) * T + t) * N + n] = acc[tb][nb][e];
            }
        }
}

template <int TB>
__device__ __forceinline__ void skinny_fwd_u(const uint16_t* __restrict__ x, const uint16_t* __restrict__ A, int T,
                                             int K, int r, int steps_per_split, int part, float* __restrict__ upart,
                                             uint16_t* sX) {
    constexpr int TP = 16 * TB;
    constexpr int XCH = TP * (kDK / 8) / kThreads;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int nsteps = (K + kDK - 1) / kDK;
    const int split_begin = int(blockIdx.y) * steps_per_split;
    const int split_end = min(split_begin + steps_per_split, nsteps);
    const int per = (split_end - split_begin + kUParts - 1) / kUParts;
    const int kb_begin = split_begin + part * per;
    const int kb_end = min(kb_begin + per, split_end);
    const auto rx = make_rsrc(x, uint32_t(T) * uint32_t(K) * 2u);
    const auto ra = make_rsrc(A, uint32_t(r) * uint32_t(K) * 2u);  // ranks past r read zero
    const uint32_t a_off = uint32_t(16 * wave + l16) * uint32_t(K) * 2u + uint32_t(q) * 128u;
    f32x4 acc[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // rows of the padded token block past T stay zero; only real tokens' x is loaded
#pragma unroll
    for (int i = 0; i < XCH; ++i) {
        const int c = tid + kThreads * i;
        if (c / (kDK / 8) >= T)
            *reinterpret_cast<u32x4*>(&sX[(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = u32x4{0u, 0u, 0u, 0u};
    }
    for (int kb = kb_begin; kb < kb_end; ++kb) {
        const uint32_t k0 = uint32_t(kb) * kDK;
        u32x4 av[8], xv[XCH];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const bool ok = int(k0) + 64 * q + 8 * p < K;
            av[p] = buf_load16(ra, ok ? a_off + k0 * 2u + uint32_t(p) * 16u : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;
            const int t = c / (kDK / 8), k8 = 8 * (c % (kDK / 8));
            if (t < T) {
                const bool ok = int(k0) + k8 < K;
                xv[i] = buf_load16(rx, ok ? (uint32_t(t) * uint32_t(K) + k0 + uint32_t(k8)) * 2u : kOutOfRange);
            }
        }
        __syncthreads();  // the previous step's x reads are done
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;
            if (c / (kDK / 8) < T)
                *reinterpret_cast<u32x4*>(&sX[(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = xv[i];
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                const bf16x8 xa =
                    as_bf16x8(*reinterpret_cast<const u32x4*>(&sX[(16 * tb + l16) * kXP + 64 * q + 8 * c]));
                acc[tb] = mfma16x16x32(xa, as_bf16x8(av[c]), acc[tb]);
            }
    }
    const int j = 16 * wave + l16;
    float* dst = upart + size_t(int(blockIdx.y) * kUParts + part) * T * r;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int t = 16 * tb + 4 * q + e;
            if (t < T && j < r) dst[size_t(t) * r + j] = acc[tb][e];
        }
}

template <int TB>
__global__ __launch_bounds__(kThreads, 2) void k_skinny_fwd(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ A, int T, int N, int K, int r, int steps_per_split, int row_blocks,
    float* __restrict__ ypart, float* __restrict__ upart, Tables tab) {
    __shared__ __align__(16) uint16_t sX[2 * 16 * TB * kXP];
    __shared__ __align__(16) float sLut[512];
    if (int(blockIdx.x) >= row_blocks) {
        skinny_fwd_u<TB>(x, A, T, K, r, steps_per_split, int(blockIdx.x) - row_blocks, upart, sX);
        return;
    }
    for (int i = threadIdx.x; i < 256; i += kThreads) {
        sLut[2 * i] = tab.level[i & 15];
        sLut[2 * i + 1] = tab.level[i >> 4];
    }
    skinny_fwd_weights<TB>(x, codes, absmax, T, N, K, steps_per_split, ypart, sX, sLut);
}

constexpr int kFinCols = 512;  // finish kernels: features per workgroup
constexpr int kFinT = 8;       // finish kernels: tokens per workgroup (dX / y)

// Stage rows [t0, t0 + rows) of an fp32 [T][r] tensor given as `parts` partials
// (src[p * T * r + t * r + j]) into dst[t - t0][j] with row pitch `pitch` (>= r):
// the sum over p in increasing order; entries with t >= T or j >= r are 0. Every load
// of a thread's items is issued before the first is added (8 parts at a time).
__device__ __forceinline__ void stage_partial_sums(float* dst, const float* src, int parts, int T, int r, int t0,
                                                   int rows, int pitch) {
    const uint32_t stride = uint32_t(T) * uint32_t(r);
    const auto rs = make_rsrc(src, uint32_t(parts) * stride * 4u);
    const int count = rows * pitch;
    for (int o0 = int(threadIdx.x); o0 < count; o0 += 4 * kThreads) {
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        for (int p0 = 0; p0 < parts; p0 += 8) {
            float pv[4][8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = o0 + i * kThreads, t = t0 + o / pitch, j = o % pitch;
                const bool ok = o < count && t < T && j < r;
#pragma unroll
                for (int pp = 0; pp < 8; ++pp)
                    pv[i][pp] = buf_load_f32(rs, ok && p0 + pp < parts
                                                     ? (uint32_t(p0 + pp) * stride + uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u
                                                     : kOutOfRange);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int pp = 0; pp < 8; ++pp)
                    if (p0 + pp < parts) v[i] += pv[i][pp];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (o0 + i * kThreads < count) dst[o0 + i * kThreads] = v[i];
    }
}

// y[t][n] = RNbf( sum_z ypart[z][t][n] + s . sum_j u[t][j] B[n][j] ), u = the sum of
// its partials in partial order, the split partials added in split order. Grid
// (features / 512, tokens / 8): 2 features per thread, their B rows in registers, u of
// the 8 tokens staged in LDS; the column-0 workgroups store u_save. All split partials
// of a thread's 8 tokens are loaded before the first is added.
template <int RB>
__global__ __launch_bounds__(kThreads) void k_skinny_fwd_finish(const float* __restrict__ ypart,
                                                                 const float* __restrict__ upart, int uparts,
                                                                 int splits, const uint16_t* __restrict__ B, int T,
                                                                 int N, int r, float s, uint16_t* __restrict__ y,
                                                                 float* __restrict__ u_save) {
    __shared__ float su[kFinT * kMaxRank];  // u [t - t0][j]
    const int tid = threadIdx.x;
    const int t0 = int(blockIdx.y) * kFinT, nt = min(kFinT, T - t0);
    stage_partial_sums(su, upart, uparts, T, r, t0, nt, r);
    const int n = int(blockIdx.x) * kFinCols + 2 * tid;
    // B rows n, n + 1 (ranks j >= r and rows past N read zero)
    const auto rb = make_rsrc(B, uint32_t(N) * uint32_t(r) * 2u);
    constexpr int R = 16 * RB;  // ranks held per thread (>= r)
    float b0[R], b1[R];
#pragma unroll
    for (int j = 0; j < R; ++j) {
        const bool ok = j < r;
        b0[j] = bf16_to_f32(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(
            rb, int(ok ? (uint32_t(n) * uint32_t(r) + uint32_t(j)) * 2u : kOutOfRange), 0, 0)));
        b1[j] = bf16_to_f32(uint16_t(__builtin_amdgcn_raw_buffer_load_b16(
            rb, int(ok ? (uint32_t(n + 1) * uint32_t(r) + uint32_t(j)) * 2u : kOutOfRange), 0, 0)));
    }
    __syncthreads();
    if (blockIdx.x == 0)
        for (int o = tid; o < nt * r; o += kThreads) u_save[size_t(t0) * r + o] = su[o];
    if (n >= N) return;  // N % 16 == 0: both features are in or out
    const auto rp = make_rsrc(ypart, uint32_t(splits) * uint32_t(T) * uint32_t(N) * 4u);
    f32x2 acc[kFinT];
#pragma unroll
    for (int i = 0; i < kFinT; ++i) acc[i] = f32x2{0.f, 0.f};
    for (int z0 = 0; z0 < splits; z0 += 4) {
        u32x2 pv[4][kFinT];
#pragma unroll
        for (int zz = 0; zz < 4; ++zz)
#pragma unroll
            for (int i = 0; i < kFinT; ++i) {
                const bool ok = z0 + zz < splits && i < nt;
                pv[zz][i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                    rp, int(ok ? ((uint32_t(z0 + zz) * uint32_t(T) + uint32_t(t0 + i)) * uint32_t(N) + uint32_t(n)) * 4u
                               : kOutOfRange), 0, 0));
            }
#pragma unroll
        for (int zz = 0; zz < 4; ++zz)
            if (z0 + zz < splits)
#pragma unroll
                for (int i = 0; i < kFinT; ++i) acc[i] += __builtin_bit_cast(f32x2, pv[zz][i]);
    }
#pragma unroll
    for (int i = 0; i < kFinT; ++i) {
        if (i >= nt) break;
        float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
        for (int j = 0; j < R; ++j)
            if (j < r) {
                const float uj = su[i * r + j];
                l0 += uj * b0[j];
                l1 += uj * b1[j];
            }
        *reinterpret_cast<uint32_t*>(&y[size_t(t0 + i) * N + n]) = pack_bf16x2(acc[i][0] + s * l0, acc[i][1] + s * l1);
    }
}

// ------------------------------------------------------------------ backward dX
// Workgroup = 128 input features (wave w: columns 32w .. 32w+31, two 16-column blocks)
// x one N range of 64-wide steps. Per step each thread dequantises a 4 (n) x 8 (k)
// patch (pair table, as in the large backward kernel) and stores it transposed into
// LDS as [k][n] (16-byte chunks XOR-swizzled by (k/8)%8); dY of the step is staged as
// [t][n]. Both double-buffered, loads one step ahead, one barrier per step.
// Output: fp32 partials dxpart[split][T][K].
constexpr int kBN = 64;       // N per step
constexpr int kCols = 128;    // K per workgroup
constexpr int kWP = kBN + 8;  // LDS pitch (bf16)

template <int TB>
__global__ __launch_bounds__(kThreads, 2) void k_skinny_bwd(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes, const float* __restrict__ absmax, int T,
    int N, int K, int steps_per_split, float* __restrict__ dxpart, Tables tab) {
    constexpr int TP = 16 * TB;
    constexpr int DCH = TP * (kBN / 8);  // 16-byte dY chunks per step (<= 512)

    __shared__ __align__(16) uint16_t sW[2][kCols * kWP];
    __shared__ __align__(16) uint16_t sD[2][TP * kWP];
    __shared__ __align__(16) float sLut[512];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int k0 = int(blockIdx.x) * kCols;
    const int nsteps = (N + kBN - 1) / kBN;
    const int nb_begin = int(blockIdx.y) * steps_per_split;
    const int nb_end = min(nb_begin + steps_per_split, nsteps);
    sLut[2 * tid] = tab.level[tid & 15];
    sLut[2 * tid + 1] = tab.level[tid >> 4];

    const int pr = tid >> 4, pc = tid & 15;  // patch: rows 4 pr .. 4 pr + 3, columns 8 pc .. 8 pc + 7
    const auto rdy = make_rsrc(dy, uint32_t(T) * uint32_t(N) * 2u);
    const auto rcd = make_rsrc(codes, uint32_t(N) * uint32_t(K / 2));
    const auto rsc = make_rsrc(absmax, uint32_t(N) * uint32_t(K / 64) * 4u);
    const uint32_t kc = uint32_t(k0 + 8 * pc);

    uint32_t rc[4];
    float rs[4];
    u32x4 dv[(DCH + kThreads - 1) / kThreads];
    auto gload = [&](int nb) {
        // rows past N are beyond both buffers (zero); columns past K only reach dX
        // columns that are never stored
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t n = uint32_t(nb * kBN + 4 * pr + i);
            rc[i] = buf_load_u32(rcd, n * uint32_t(K / 2) + kc / 2);
            rs[i] = buf_load_f32(rsc, n * uint32_t(K / 64) * 4u + (kc / 64) * 4u);
        }
#pragma unroll
        for (int i = 0; i < (DCH + kThreads - 1) / kThreads; ++i) {
            const int c = tid + kThreads * i, t = c / (kBN / 8), n8 = 8 * (c % (kBN / 8));
            const bool ok = c < DCH && t < T && nb * kBN + n8 < N;
            dv[i] = buf_load16(rdy, ok ? (uint32_t(t) * uint32_t(N) + uint32_t(nb * kBN + n8)) * 2u : kOutOfRange);
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    auto sstore = [&](int buf) {
#pragma unroll
        for (int i = 0; i < (DCH + kThreads - 1) / kThreads; ++i) {
            const int c = tid + kThreads * i;
            if (c < DCH) *reinterpret_cast<u32x4*>(&sD[buf][(c / (kBN / 8)) * kWP + 8 * (c % (kBN / 8))]) = dv[i];
        }
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float2 lv = *reinterpret_cast<const float2*>(lut + (((rc[i] >> (8 * b)) & 0xFFu) << 3));
                v[i][2 * b] = lv.x * rs[i];  // level * absmax in fp32, RNbf below
                v[i][2 * b + 1] = lv.y * rs[i];
            }
        const int col = (((pr >> 1) ^ (pc & 7)) << 3) + 4 * (pr & 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const u32x2 o = {pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e])};
            *reinterpret_cast<u32x2*>(&sW[buf][(8 * pc + e) * kWP + col]) = o;
        }
    };

    f32x4 acc[TB][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) acc[tb][cb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (nb_begin < nb_end) {
        gload(nb_begin);
        __syncthreads();  // sLut
        sstore(0);
        __syncthreads();
        for (int nb = nb_begin; nb < nb_end; ++nb) {
            const int buf = (nb - nb_begin) & 1;
            gload(nb + 1);  // one step ahead; past the range: unused data or zeros
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < kBN / 32; ++c) {
                bf16x8 bw[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb) {
                    const int kr = 32 * wave + 16 * cb + l16;  // tile row k
                    const int chunk = (4 * c + q) ^ ((kr >> 3) & 7);
                    bw[cb] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sW[buf][kr * kWP + 8 * chunk]));
                }
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const bf16x8 da = as_bf16x8(
                        *reinterpret_cast<const u32x4*>(&sD[buf][(16 * tb + l16) * kWP + 32 * c + 8 * q]));
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb) acc[tb][cb] = mfma16x16x32(da, bw[cb], acc[tb][cb]);
                }
            }
            sstore(buf ^ 1);
            __syncthreads();
        }
    }

    float* dst = dxpart + size_t(blockIdx.y) * T * K;
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int cb = 0; cb < 2; ++cb) {
            const int k = k0 + 32 * wave + 16 * cb + l16;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = 16 * tb + 4 * q + e;
                if (t < T && k < K) dst[size_t(t) * K + k] = acc[tb][cb][e];
            }
        }
}

// Backward finish, two kinds of workgroups in one launch; g = sum of the pre-pass's
// partials in partial order, staged in LDS:
//  - blocks [0, dx_blocks): grid (features / 512, tokens / 8), 2 features per thread
//    with their A columns in registers: dX[t][k] = RNbf( sum_z dxpart[z][t][k] +
//    s . sum_j g[t][j] A[j][k] ), all split partials of the 8 tokens loaded first;
//  - the rest: 512 features (2 per thread) x all ranks: dA[j][k] = s . sum_t g[t][j]
//    x[t][k], every token's x loaded first, tokens added in increasing order.
template <int RB, int TB>
__global__ __launch_bounds__(kThreads) void k_skinny_bwd_finish(
    const float* __restrict__ dxpart, int splits, const float* __restrict__ gpart, int gparts,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ x, int T, int K, int r, float s, int dx_col_blocks,
    int dx_blocks, uint16_t* __restrict__ dx, float* __restrict__ dA) {
    __shared__ float sg[kSkinnyMaxT * kMaxRank];  // g [t][j] (dX role: the 8 tokens only)
    const int tid = threadIdx.x;
    const bool dx_role = int(blockIdx.x) < dx_blocks;
    const int t0 = dx_role ? (int(blockIdx.x) / dx_col_blocks) * kFinT : 0;
    const int nt = dx_role ? min(kFinT, T - t0) : T;
    // dX role: [8 tokens][r]; dA role: [16 TB][16 RB], zero-padded
    if (dx_role)
        stage_partial_sums(sg, gpart, gparts, T, r, t0, nt, r);
    else
        stage_partial_sums(sg, gpart, gparts, T, r, 0, 16 * TB, 16 * RB);
    if (dx_role) {
        const int k = (int(blockIdx.x) % dx_col_blocks) * kFinCols + 2 * tid;
        // A[j][k], A[j][k+1] (ranks j >= r and columns past K read zero)
        const auto ra = make_rsrc(A, uint32_t(r) * uint32_t(K) * 2u);
        constexpr int R = 16 * RB;  // ranks held per thread (>= r)
        float a0[R], a1[R];
#pragma unroll
        for (int j = 0; j < R; ++j) {
            const uint32_t w = buf_load_u32(ra, j < r && k < K ? (uint32_t(j) * uint32_t(K) + uint32_t(k)) * 2u : kOutOfRange);
            a0[j] = __uint_as_float(w << 16);
            a1[j] = __uint_as_float(w & 0xFFFF0000u);
        }
        __syncthreads();
        if (k >= K) return;  // K % 64 == 0: both features are in or out
        const auto rp = make_rsrc(dxpart, uint32_t(splits) * uint32_t(T) * uint32_t(K) * 4u);
        f32x2 acc[kFinT];
#pragma unroll
        for (int i = 0; i < kFinT; ++i) acc[i] = f32x2{0.f, 0.f};
        for (int z0 = 0; z0 < splits; z0 += 4) {
            u32x2 pv[4][kFinT];
#pragma unroll
            for (int zz = 0; zz < 4; ++zz)
#pragma unroll
                for (int i = 0; i < kFinT; ++i) {
                    const bool ok = z0 + zz < splits && i < nt;
                    pv[zz][i] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                        rp, int(ok ? ((uint32_t(z0 + zz) * uint32_t(T) + uint32_t(t0 + i)) * uint32_t(K) + uint32_t(k)) * 4u
                                   : kOutOfRange), 0, 0));
                }
#pragma unroll
            for (int zz = 0; zz < 4; ++zz)
                if (z0 + zz < splits)
#pragma unroll
                    for (int i = 0; i < kFinT; ++i) acc[i] += __builtin_bit_cast(f32x2, pv[zz][i]);
        }
#pragma unroll
        for (int i = 0; i < kFinT; ++i) {
            if (i >= nt) break;
            float l0 = 0.0f, l1 = 0.0f;
#pragma unroll
            for (int j = 0; j < R; ++j)
                if (j < r) {
                    const float gj = sg[i * r + j];
                    l0 += gj * a0[j];
                    l1 += gj * a1[j];
                }
            *reinterpret_cast<uint32_t*>(&dx[size_t(t0 + i) * K + k]) =
                pack_bf16x2(acc[i][0] + s * l0, acc[i][1] + s * l1);
        }
        return;
    }
    const int k = (int(blockIdx.x) - dx_blocks) * kFinCols + 2 * tid;
    const auto rx = make_rsrc(x, uint32_t(T) * uint32_t(K) * 2u);
    constexpr int R = 16 * RB;  // ranks held per thread (>= r)
    float c0[R], c1[R];
#pragma unroll
    for (int j = 0; j < R; ++j) c0[j] = c1[j] = 0.0f;
    // tokens in groups of 8, the next group's x loaded while the current one is added;
    // tokens past T have x = 0 and g = 0 (staged zero)
    auto load8 = [&](int t0, uint32_t (&xv)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            xv[i] = buf_load_u32(rx, t0 + i < T ? (uint32_t(t0 + i) * uint32_t(K) + uint32_t(k)) * 2u : kOutOfRange);
    };
    uint32_t xa[8], xb[8];
    load8(0, xa);
    __syncthreads();
    if (k >= K) return;
    for (int t0 = 0; t0 < 16 * TB; t0 += 8) {
        load8(t0 + 8, xb);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float x0 = __uint_as_float(xa[i] << 16), x1 = __uint_as_float(xa[i] & 0xFFFF0000u);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                const float gj = sg[(t0 + i) * R + j];
                c0[j] += gj * x0;
                c1[j] += gj * x1;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) xa[i] = xb[i];
    }
#pragma unroll
    for (int j = 0; j < R; ++j)
        if (j < r) *reinterpret_cast<f32x2*>(&dA[size_t(j) * K + k]) = f32x2{s * c0[j], s * c1[j]};
}

template <int TB>
void launch_fwd_tb(const SkinnyPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* x,
                   const uint16_t* A, int64_t T, int64_t N, int64_t K, int r, float* ypart, float* upart,
                   hipStream_t stream) {
    const dim3 grid(unsigned(p.row_blocks + (r > 0 ? kUParts : 0)), unsigned(p.splits));
    hipLaunchKernelGGL(k_skinny_fwd<TB>, grid, dim3(kThreads), 0, stream, x, codes, absmax, A, int(T), int(N), int(K),
                       r, p.steps_per_split, p.row_blocks, ypart, upart, tables());
}

template <int TB>
void launch_bwd_tb(const SkinnyPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* dy, int64_t T,
                   int64_t N, int64_t K, float* dxpart, hipStream_t stream) {
    const dim3 grid(unsigned(p.col_blocks), unsigned(p.splits));
    hipLaunchKernelGGL(k_skinny_bwd<TB>, grid, dim3(kThreads), 0, stream, dy, codes, absmax, int(T), int(N), int(K),
                       p.steps_per_split, dxpart, tables());
}

template <int RB, int TB>
void launch_bwd_finish_rt(dim3 grid, hipStream_t stream, const float* dxpart, int splits, const float* gpart,
                          int gparts, const uint16_t* A, const uint16_t* x, int T, int K, int r, float s,
                          int col_blocks, int dx_blocks, uint16_t* dx, float* dA) {
    hipLaunchKernelGGL((k_skinny_bwd_finish<RB, TB>), grid, dim3(kThreads), 0, stream, dxpart, splits, gpart, gparts,
                       A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA);
}

template <int RB>
void launch_bwd_finish_r(int tb, dim3 grid, hipStream_t stream, const float* dxpart, int splits, const float* gpart,
                         int gparts, const uint16_t* A, const uint16_t* x, int T, int K, int r, float s,
                         int col_blocks, int dx_blocks, uint16_t* dx, float* dA) {
    switch (tb) {
        case 1: launch_bwd_finish_rt<RB, 1>(grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        case 2: launch_bwd_finish_rt<RB, 2>(grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        case 3: launch_bwd_finish_rt<RB, 3>(grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        default: launch_bwd_finish_rt<RB, 4>(grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
    }
}

void launch_bwd_finish(int rb, int tb, dim3 grid, hipStream_t stream, const float* dxpart, int splits,
                       const float* gpart, int gparts, const uint16_t* A, const uint16_t* x, int T, int K, int r,
                       float s, int col_blocks, int dx_blocks, uint16_t* dx, float* dA) {
    switch (rb) {
        case 1: launch_bwd_finish_r<1>(tb, grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        case 2: launch_bwd_finish_r<2>(tb, grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        case 3: launch_bwd_finish_r<3>(tb, grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
        default: launch_bwd_finish_r<4>(tb, grid, stream, dxpart, splits, gpart, gparts, A, x, T, K, r, s, col_blocks, dx_blocks, dx, dA); break;
    }
}

// Workgroups of a streaming kernel: 2 per CU, each running several steps so that its
// loads stay in steady state.
constexpr int64_t kStreamWGs = 512;
constexpr int64_t kMinSteps = 4;

}  // namespace

SkinnyPlan plan_skinny_fwd(int64_t T, int64_t N, int64_t K, int r) {
    SkinnyPlan p{};
    p.row_blocks = int(cdiv(N, kRows));
    const int64_t steps = cdiv(K, kDK);
    // split K until about kStreamWGs workgroups, >= 2 steps each; the fp32 partials,
    // written and read back (8 x splits x T x N bytes), stay within about a quarter of
    // the codes (N x K / 2 bytes)
    int64_t s = std::max<int64_t>(1, kStreamWGs / (p.row_blocks + 1));
    s = std::min<int64_t>(s, std::max<int64_t>(1, steps / kMinSteps));
    s = std::min<int64_t>(s, std::max<int64_t>(1, K / (64 * T)));
    p.steps_per_split = int(cdiv(steps, s));
    p.splits = int(cdiv(steps, p.steps_per_split));
    p.off_part = 0;
    size_t off = align256(size_t(p.splits) * size_t(T) * size_t(N) * 4);
    p.off_upart = off;
    off += align256(size_t(p.splits) * kUParts * size_t(T) * size_t(std::max(r, 1)) * 4);
    p.ws_bytes = off;
    return p;
}

SkinnyPlan plan_skinny_bwd(int64_t T, int64_t N, int64_t K) {
    SkinnyPlan p{};
    p.col_blocks = int(cdiv(K, kCols));
    const int64_t steps = cdiv(N, kBN);
    int64_t s = std::max<int64_t>(1, kStreamWGs / p.col_blocks);
    s = std::min<int64_t>(s, std::max<int64_t>(1, steps / kMinSteps));
    s = std::min<int64_t>(s, std::max<int64_t>(1, N / (64 * T)));
    p.steps_per_split = int(cdiv(steps, s));
    p.splits = int(cdiv(steps, p.steps_per_split));
    p.off_part = 0;
    p.ws_bytes = align256(size_t(p.splits) * size_t(T) * size_t(K) * 4);
    return p;
}

hipError_t launch_skinny_fwd(const SkinnyPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* x,
                             const uint16_t* A, const uint16_t* B, int64_t T, int64_t N, int64_t K, int r, float s,
                             uint16_t* y, float* u_save, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    float* ypart = reinterpret_cast<float*>(w + p.off_part);
    float* upart = reinterpret_cast<float*>(w + p.off_upart);
    prof_gemm_begin(stream);
    switch ((T + 15) / 16) {
        case 1: launch_fwd_tb<1>(p, codes, absmax, x, A, T, N, K, r, ypart, upart, stream); break;
        case 2: launch_fwd_tb<2>(p, codes, absmax, x, A, T, N, K, r, ypart, upart, stream); break;
        case 3: launch_fwd_tb<3>(p, codes, absmax, x, A, T, N, K, r, ypart, upart, stream); break;
        default: launch_fwd_tb<4>(p, codes, absmax, x, A, T, N, K, r, ypart, upart, stream); break;
    }
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 fgrid(unsigned(cdiv(N, kFinCols)), unsigned(cdiv(T, kFinT)));
    const int uparts = p.splits * kUParts;
    switch (std::max(1, (r + 15) / 16)) {
        case 1: hipLaunchKernelGGL(k_skinny_fwd_finish<1>, fgrid, dim3(kThreads), 0, stream, ypart, upart, uparts, p.splits, B,
                                   int(T), int(N), r, s, y, u_save); break;
        case 2: hipLaunchKernelGGL(k_skinny_fwd_finish<2>, fgrid, dim3(kThreads), 0, stream, ypart, upart, uparts, p.splits, B,
                                   int(T), int(N), r, s, y, u_save); break;
        case 3: hipLaunchKernelGGL(k_skinny_fwd_finish<3>, fgrid, dim3(kThreads), 0, stream, ypart, upart, uparts, p.splits, B,
                                   int(T), int(N), r, s, y, u_save); break;
        default: hipLaunchKernelGGL(k_skinny_fwd_finish<4>, fgrid, dim3(kThreads), 0, stream, ypart, upart, uparts, p.splits, B,
                                    int(T), int(N), r, s, y, u_save); break;
    }
    return hipGetLastError();
}

hipError_t launch_skinny_bwd(const SkinnyPlan& p, const BwdPlan& bp, const uint8_t* codes, const float* absmax,
                             const uint16_t* dy, const uint16_t* x, const uint16_t* A, int64_t T, int64_t N,
                             int64_t K, int r, float s, uint16_t* dx, float* dA, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    float* dxpart = reinterpret_cast<float*>(w + bp.off_dx);
    if (dx) {
        prof_gemm_begin(stream);
        switch ((T + 15) / 16) {
            case 1: launch_bwd_tb<1>(p, codes, absmax, dy, T, N, K, dxpart, stream); break;
            case 2: launch_bwd_tb<2>(p, codes, absmax, dy, T, N, K, dxpart, stream); break;
            case 3: launch_bwd_tb<3>(p, codes, absmax, dy, T, N, K, dxpart, stream); break;
            default: launch_bwd_tb<4>(p, codes, absmax, dy, T, N, K, dxpart, stream); break;
        }
        prof_gemm_end(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int col_blocks = int(cdiv(K, kFinCols));
    const int dx_blocks = dx ? col_blocks * int(cdiv(T, kFinT)) : 0;
    const int da_blocks = r > 0 ? col_blocks : 0;
    if (dx_blocks + da_blocks == 0) return hipSuccess;
    launch_bwd_finish(std::max(1, (r + 15) / 16), int((T + 15) / 16), dim3(unsigned(dx_blocks + da_blocks)), stream,
                      dxpart, p.splits, reinterpret_cast<const float*>(w + bp.off_gpart), bp.gparts, A, x, int(T),
                      int(K), r, s, col_blocks, dx_blocks, dx, dA);
    return hipGetLastError();
}

}  // namespace nf4
