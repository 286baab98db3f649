// NF4-LoRA linear for few tokens (forward T <= 32, or T <= 64 for long, narrow weights;
// backward T <= 32): the same operations
// as the 128-token GEMMs, organised for the HBM-bound regime, where every weight byte
// should be read once and streamed at full rate while MFMA work is cheap.
//
//   forward:  y  = RNbf( x . W^T + s . u . B^T ),  u = x . A^T (saved)
//   backward: dX = RNbf( dY . W + s . g . A ),     dA = s . g^T . x
//             (g and dB from the pre-pass roles of lora_pre.h, run as extra
//             workgroups of the backward launch)
//
// The frozen NF4 base is only read (HN comment thread on streaming the frozen base,
// main comment); LoRA rank r and alpha as in the Poros API reference
// ("PorosTrainer.from_pretrained"). Tokens are padded to blocks of 16 for
// v_mfma_f32_16x16x32_bf16 (the forward's TB template counts such blocks, one to four,
// and each dequantised weight fragment feeds all of them; the backward takes one or two);
// both GEMM kernels split their contraction over the grid's y dimension
// and write fp32 partials, which the finish kernels add in split order, together with
// the LoRA terms, and round once.
#include <type_traits>

#include "common.h"
#include "device.h"
#include "lora_pre.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRank = 16 * NF4_MAX_RANK_BLOCKS;
constexpr int kSkinnyMaxT = int(kSkinnyBwdT);  // the backward finish kernel's g rows
constexpr int kRows = 128;    // forward: weight rows per workgroup (4 waves x 2 blocks of 16)
constexpr int kDK = 256;      // forward: K per main-loop step (four NF4 blocks)
constexpr int kXP = kDK + 8;  // LDS pitch of the x tile (bf16)

// ------------------------------------------------------------------ forward
// Weight workgroups: 128 weight rows (wave w: rows 32w .. 32w+31, two 16-row blocks) x
// one K range of 256-wide steps. Within a step the contraction order is permuted
// identically for both operands: lane quarter q (lane / 16) supplies k = 64q + 8c ..
// 64q + 8c + 7 at MFMA chunk c (0..7), so a lane's 32 bytes of codes per row block are
// one whole NF4 block (one scale). Codes and scales are loaded kFRing - 1 steps ahead
// into a ring of kFRing register sets (two, measured: a ring of three, or twice the
// workgroups, gave nothing), x kFRing steps ahead into a ring of its own; the x tile of
// the current step is in double-buffered LDS, and the table reads of MFMA chunk c + 1 are
// issued before the multiplies of chunk c. Output: fp32 partials ypart[split][T][N].
//
// u workgroups (blockIdx.x >= row_blocks, kUParts per split): the rows of A (bf16, wave
// w: ranks 16w .. 16w+15) against the same x for u = x.A^T, each over a quarter of the
// split's steps with plain loads (few registers, so the weight workgroups keep their
// occupancy) -> upart[split * kUParts + part][T][r].
constexpr int kUParts = 4;
constexpr int kFRing = 2;       // forward weight workgroups: register sets (loads kFRing - 1 steps ahead)
static_assert(kFRing == 2 || kFRing == 3, "ring of two or three register sets");

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
    };
    constexpr int R = kFRing;
    Set ring[R];
    // x of a step, loaded R steps ahead into its own ring of R sets (the set of the step
    // being computed is in LDS already), so that the tile stored at the end of a step was
    // loaded a step before that step's codes and storing it never waits for code loads
    // still in flight; only the threads of real tokens load (the padded rows stay zero)
    u32x4 xr[R][XCH];
#pragma unroll
    for (int c = 0; c < R; ++c)
#pragma unroll
        for (int i = 0; i < XCH; ++i) xr[c][i] = u32x4{0u, 0u, 0u, 0u};
    auto gload_x = [&](int kb, u32x4 (&xv)[XCH]) {
        const uint32_t k0 = uint32_t(kb) * kDK;
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;  // token c / 32, columns 8 (c % 32)
            const int t = c / (kDK / 8), k8 = 8 * (c % (kDK / 8));
            if (t < T) {
                const bool ok = int(k0) + k8 < K;
                xv[i] = buf_load16(rx, ok ? (uint32_t(t) * uint32_t(K) + k0 + uint32_t(k8)) * 2u : kOutOfRange);
            }
        }
    };
    auto gload = [&](int kb, Set& st) {
        const uint32_t k0 = uint32_t(kb) * kDK;
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
            for (int p = 0; p < 2; ++p) st.cw[nb][p] = buf_load16(rcd, c_off[nb] + k0 / 2u + uint32_t(p) * 16u);
            st.sc[nb] = buf_load_f32(rsc, s_off[nb] + (k0 / 64u) * 4u);
        }
    };
    typedef uint16_t XTile[TP * kXP];
    XTile* sX = reinterpret_cast<XTile*>(sXflat);
    auto store_x = [&](const u32x4 (&xv)[XCH], int buf) {
#pragma unroll
        for (int i = 0; i < XCH; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(&sX[buf][(c / (kDK / 8)) * kXP + 8 * (c % (kDK / 8))]) = xv[i];
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);

    f32x4 acc[TB][2];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[tb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (kb_begin < kb_end) {
#pragma unroll
        for (int c = 0; c < R; ++c) gload_x(kb_begin + c, xr[c]);
#pragma unroll
        for (int c = 0; c < R - 1; ++c) gload(kb_begin + c, ring[c]);
        store_x(xr[0], 0);
        __syncthreads();  // sLut and x tile 0
        // one step on ring slot C (compile-time: the loop is unrolled by R)
        auto step = [&](int kb, auto c_) {
            constexpr int C = decltype(c_)::value;
            const int buf = (kb - kb_begin) & 1;
            // x R steps ahead into the set whose tile is in LDS already, codes R - 1 steps
            // ahead; past the range: unused or zeros
            gload_x(kb + R, xr[C % R]);
            gload(kb + R - 1, ring[(C + R - 1) % R]);
            __builtin_amdgcn_sched_barrier(0);
            const Set& cur = ring[C % R];
            // table reads of chunk c + 1 are issued before the arithmetic of chunk c
            float2 lv[2][2][4];
            auto table = [&](int c, float2 (&v)[2][4]) {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const uint32_t w = cur.cw[nb][c >> 2][c & 3];
#pragma unroll
                    for (int b = 0; b < 4; ++b)
                        v[nb][b] = *reinterpret_cast<const float2*>(lut + (((w >> (8 * b)) & 0xFFu) << 3));
                }
            };
            table(0, lv[0]);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (c + 1 < 8) table(c + 1, lv[(c + 1) & 1]);
                bf16x8 bw[2];
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    u32x4 o;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const float2 v = lv[c & 1][nb][b];
                        // level * absmax in fp32, then RNbf: the format's two roundings
                        o[b] = pack_bf16x2(v.x * cur.sc[nb], v.y * cur.sc[nb]);
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
            store_x(xr[(C + 1) % R], buf ^ 1);  // the next step's x (loaded a step before its codes)
            __syncthreads();
        };
        int kb = kb_begin;
        if constexpr (R == 3) {
            for (; kb + 2 < kb_end; kb += 3) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
                step(kb + 2, std::integral_constant<int, 2>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < kb_end) step(kb + 1, std::integral_constant<int, 1>{});
        } else {
            for (; kb + 1 < kb_end; kb += 2) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
        }
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

// Finish kernels: 64 features (one per lane) x 4 tokens (one per wave) per workgroup,
// with short loops and few unrolled bodies - they run once per call, so their code is
// fetched cold - and every independent load issued before the first wait.
constexpr int kFinF = 64;
constexpr int kFinTk = 4;
constexpr int kMaxSplits = 16;  // split partials a finish thread loads at once (32: a larger finish kernel, slower)

// Split partials of one output element: v[z] = src[base + z * zstride] for z < splits,
// 0 for the rest: rp spans exactly `splits` partials, so the offsets of z >= splits lie
// past it and read as zero with no test of their own (a dead lane starts from
// kOutOfRange, which stays past any buffer and below 2^32 for every z); sum_splits adds
// all kMaxSplits in split order (the zeros past `splits` leave the sum unchanged).
__device__ __forceinline__ void load_splits(float (&v)[kMaxSplits], __amdgpu_buffer_rsrc_t rp, int splits,
                                            uint32_t base, uint32_t zstride, bool live) {
    (void)splits;
    const uint32_t b = live ? base : kOutOfRange;
#pragma unroll
    for (int z = 0; z < kMaxSplits; ++z) v[z] = buf_load_f32(rp, b + uint32_t(z) * zstride);
}

__device__ __forceinline__ float sum_splits(const float (&v)[kMaxSplits]) {
    float acc = v[0];
#pragma unroll
    for (int z = 1; z < kMaxSplits; ++z) acc += v[z];
    return acc;
}

// Stage rows [t0, t0 + rows) and columns [j0, j0 + pitch) of an fp32 [T][r] tensor
// given as `parts` partials (src[p * T * r + t * r + j]) into dst[t - t0][j - j0];
// entries with t >= T or j >= r are 0. With few items the parts are split into G
// interleaved groups (G threads per item, G = 2 .. 16): each thread issues all of its
// loads (8 at a time) before adding, and the group sums are added in group order
// through `tmp` (kThreads floats of LDS). With many items (G = 1) each thread adds the
// parts of its items in part order, 32 loads at a time. Ends with a barrier.
__device__ __forceinline__ void stage_partial_sums(float* dst, float* tmp, const float* src, int parts, int T, int r,
                                                   int t0, int rows, int j0, int pitch) {
    const uint32_t stride = uint32_t(T) * uint32_t(r);
    const auto rs = make_rsrc(src, uint32_t(parts) * stride * 4u);
    const int tid = int(threadIdx.x);
    const int count = rows * pitch;
    int G = 1;
    while (G < 16 && 2 * G * count <= kThreads) G *= 2;
    if (G == 1) {
        for (int o = tid; o < count; o += kThreads) {
            const int t = t0 + o / pitch, j = j0 + o % pitch;
            const bool ok = t < T && j < r;
            float v = 0.0f;
            for (int p0 = 0; p0 < parts; p0 += 32) {
                float pv[32];
#pragma unroll
                for (int pp = 0; pp < 32; ++pp)  // parts past the last read past rs: zero
                    pv[pp] = buf_load_f32(rs, ok ? (uint32_t(p0 + pp) * stride + uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u
                                                 : kOutOfRange);
#pragma unroll
                for (int pp = 0; pp < 32; ++pp)
                    if (p0 + pp < parts) v += pv[pp];
            }
            dst[o] = v;
        }
        __syncthreads();
        return;
    }
    const int o = tid / G, g = tid % G;
    const int t = t0 + o / pitch, j = j0 + o % pitch;
    const bool ok = o < count && t < T && j < r;
    float v = 0.0f;
    for (int p0 = g; p0 < parts; p0 += 8 * G) {
        float pv[8];
#pragma unroll
        for (int pp = 0; pp < 8; ++pp) {
            const int p = p0 + pp * G;
            // parts past the last read past rs: zero
            pv[pp] = buf_load_f32(rs, ok ? (uint32_t(p) * stride + uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u : kOutOfRange);
        }
#pragma unroll
        for (int pp = 0; pp < 8; ++pp)
            if (p0 + pp * G < parts) v += pv[pp];
    }
    tmp[tid] = v;  // tid = o * G + g
    __syncthreads();
    if (tid < count) {
        float sum = 0.0f;
        for (int gg = 0; gg < G; ++gg) sum += tmp[tid * G + gg];
        dst[tid] = sum;
    }
    __syncthreads();
}

// y[t][n] = RNbf( sum_z ypart[z][t][n] + s . sum_j u[t][j] B[n][j] ): lane = feature n,
// wave = token t; u = the sum of its partials and the B rows of the 64 features are
// staged in LDS; the column-0 workgroups store u_save.
__global__ __launch_bounds__(kThreads) void k_skinny_fwd_finish(const float* __restrict__ ypart,
                                                                 const float* __restrict__ upart, int uparts,
                                                                 int splits, const uint16_t* __restrict__ B, int T,
                                                                 int N, int r, float s, uint16_t* __restrict__ y,
                                                                 float* __restrict__ u_save) {
    __shared__ float su[kFinTk * kMaxRank];  // u [t - t0][j]
    __shared__ float sB[kMaxRank * kFinF];   // B^T [j][n - n0]
    __shared__ float stmp[kThreads];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = int(blockIdx.x) * kFinF, t0 = int(blockIdx.y) * kFinTk;
    const int n = n0 + lane, t = t0 + wave;
    const bool live = n < N && t < T;
    // every load is issued before the first is waited for (one memory round trip): B[n][j]
    // for j = wave + 4i (rows past N and ranks past r read 0), the split partials, then
    // the u partials inside stage_partial_sums
    const auto rb = make_rsrc(B, uint32_t(N) * uint32_t(r) * 2u);
    constexpr int BV = kMaxRank / kFinTk;
    uint32_t bv[BV];
#pragma unroll
    for (int i = 0; i < BV; ++i) {
        const int j = wave + kFinTk * i;
        bv[i] = __builtin_amdgcn_raw_buffer_load_b16(
            rb, int(j < r ? (uint32_t(n) * uint32_t(r) + uint32_t(j)) * 2u : kOutOfRange), 0, 0);
    }
    float pv[kMaxSplits];
    load_splits(pv, make_rsrc(ypart, uint32_t(splits) * uint32_t(T) * uint32_t(N) * 4u), splits,
                (uint32_t(t) * uint32_t(N) + uint32_t(n)) * 4u, uint32_t(T) * uint32_t(N) * 4u, live);
    stage_partial_sums(su, stmp, upart, uparts, T, r, t0, kFinTk, 0, r);  // ends with a barrier
#pragma unroll
    for (int i = 0; i < BV; ++i) sB[(wave + kFinTk * i) * kFinF + lane] = bf16_to_f32(uint16_t(bv[i]));
    __syncthreads();
    if (blockIdx.x == 0)
        for (int o = tid; o < min(kFinTk, T - t0) * r; o += kThreads) u_save[size_t(t0) * r + o] = su[o];
    if (!live) return;
    const float acc = sum_splits(pv);
    float l = 0.0f;
#pragma unroll 8
    for (int j = 0; j < r; ++j) l += su[wave * r + j] * sB[j * kFinF + lane];
    y[size_t(t) * N + n] = bf16_bits(acc + s * l);
}

// ------------------------------------------------------------------ backward dX
// dX = dY . W contracts over the weight rows n, so a lane that dequantises 8
// consecutive rows of one weight column already holds a B operand of
// v_mfma_f32_16x16x32_bf16 (8 contraction elements of one output column): no
// transpose through LDS. Workgroup = 256 features x one range of 32-row steps; lane
// (l16, q) reads 8 bytes of codes (16 features, inside one NF4 block) of rows
// 8q .. 8q+7 of a step, and MFMA j (0..15) takes feature 16 l16 + j from every lane,
// so its output column l16 is feature 16 l16 + j. The four waves take interleaved
// steps of the workgroup's range and add their sums through LDS in a fixed order.
// Scales: two dwords per lane and step ([row][block] in memory), exchanged through the
// wave's own LDS slice as [block][row]. Codes, scales and dY are loaded kBRing - 1 steps
// ahead into a ring of kBRing register sets (two, measured: three workgroups per CU then
// fit in the registers). TB 16-token MFMA blocks (T <= 16 TB; TB = 1 or 2): each dequantised
// fragment feeds TB MFMAs, and the accumulators grow to TB x 16.
// Output: fp32 partials dxpart[split][T][K].
constexpr int kBCols = 256;  // features per workgroup
constexpr int kBRows = 32;   // weight rows per wave step
constexpr int kBRing = 2;    // register sets: loads run kBRing - 1 steps ahead
// waves per SIMD the register budget must allow: three with one token block, two with two
template <int TB>
constexpr int kBOccupancy = TB == 1 ? 3 : 2;
static_assert(kBRing == 2 || kBRing == 3, "ring of two or three register sets");

template <int TB>
struct BwdSmem {
    float lut[512];
    float sc[4][4 * kBRows];    // per wave: scales [block][row]
    float red[2][16 * TB][kBCols];  // cross-wave sums [token][feature]
};

template <int TB>
__device__ __forceinline__ void skinny_bwd_dx(const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes,
                                              const float* __restrict__ absmax, int T, int N, int K,
                                              int steps_per_split, int col, int split, float* __restrict__ dxpart,
                                              const Tables& tab, BwdSmem<TB>& sm) {
    float* sLut = sm.lut;
    auto& sSc = sm.sc;
    auto& sRed = sm.red;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, q = lane >> 4;
    const int k0 = col * kBCols;
    const int nsteps = (N + kBRows - 1) / kBRows;
    const int s_begin = split * steps_per_split;
    const int s_end = min(s_begin + steps_per_split, nsteps);
    const int nw = max(0, (s_end - s_begin - wave + 3) / 4);  // this wave's steps
    sLut[2 * tid] = tab.level[tid & 15];
    sLut[2 * tid + 1] = tab.level[tid >> 4];

    const auto rdy = make_rsrc(dy, uint32_t(T) * uint32_t(N) * 2u);
    const auto rcd = make_rsrc(codes, uint32_t(N) * uint32_t(K / 2));
    const auto rsc = make_rsrc(absmax, uint32_t(N) * uint32_t(K / 64) * 4u);
    // rows past N lie beyond the code and scale buffers (zero weights) and their dY is
    // not loaded; features past K read other rows' data and only reach dX columns that
    // are never stored
    const uint32_t c_lane = uint32_t(8 * q) * uint32_t(K / 2) + uint32_t(k0 + 16 * l16) / 2u;
    const uint32_t s_lane = (uint32_t(lane >> 2) * uint32_t(K / 64) + uint32_t(k0 / 64 + (lane & 3))) * 4u;
    struct Set {
        u32x2 cw[8];  // codes of rows 8q + i, 16 features
        float sc[2];  // scales: row 16h + lane / 4, block lane % 4
        u32x4 dv[TB];  // dY[t = 16 tb + l16][8q .. 8q + 7]
    };
    constexpr int R = kBRing;
    Set ring[R];
#pragma unroll
    for (int c = 0; c < R; ++c)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) ring[c].dv[tb] = u32x4{0u, 0u, 0u, 0u};
    auto gload = [&](int i, Set& st) {
        const uint32_t n0 = uint32_t(s_begin + wave + 4 * i) * kBRows;
#pragma unroll
        // non-temporal: each code byte is read once, and one load instruction covers whole
        // 128-byte lines (measured: 72B gate 46.8 -> 45.5 us at one token; the forward's
        // two interleaved 16-byte loads per line got slower with it)
        for (int r8 = 0; r8 < 8; ++r8) st.cw[r8] = buf_load8_nt(rcd, (n0 + uint32_t(r8)) * uint32_t(K / 2) + c_lane);
#pragma unroll
        for (int h = 0; h < 2; ++h) st.sc[h] = buf_load_f32(rsc, (n0 + 16u * h) * uint32_t(K / 64) * 4u + s_lane);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            const int t = 16 * tb + l16;
            const bool ok = t < T && int(n0) + 8 * q < N;
            st.dv[tb] = buf_load16(rdy, ok ? (uint32_t(t) * uint32_t(N) + n0 + uint32_t(8 * q)) * 2u : kOutOfRange);
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    float* ssc = sSc[wave];

    f32x4 acc[TB][16];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[tb][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    __syncthreads();  // sLut

    if (nw > 0) {
#pragma unroll
        for (int c = 0; c < R - 1; ++c) gload(c, ring[c]);
        // one step on ring slot C (compile-time: the loop is unrolled by R)
        auto step = [&](int i, auto c_) {
            constexpr int C = decltype(c_)::value;
            gload(i + R - 1, ring[(C + R - 1) % R]);  // R - 1 steps ahead; past the range: unused or zeros
            __builtin_amdgcn_sched_barrier(0);
            const Set& cur = ring[C % R];
            // the wave's LDS slice: written and read by this wave only, in program order
            ssc[(lane & 3) * kBRows + (lane >> 2)] = cur.sc[0];
            ssc[(lane & 3) * kBRows + 16 + (lane >> 2)] = cur.sc[1];
            __builtin_amdgcn_wave_barrier();
            const f32x4 sa = *reinterpret_cast<const f32x4*>(&ssc[(l16 >> 2) * kBRows + 8 * q]);
            const f32x4 sb = *reinterpret_cast<const f32x4*>(&ssc[(l16 >> 2) * kBRows + 8 * q + 4]);
            __builtin_amdgcn_wave_barrier();
            const float sc[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
#pragma unroll
            for (int p = 0; p < 8; ++p) {  // features 2p, 2p + 1 of the lane's 16
                // the eight table reads of the pair are issued together, ahead of their
                // multiplies (left to the scheduler, each read was waited for before the
                // next one was issued)
                float2 lv[8];
#pragma unroll
                for (int r8 = 0; r8 < 8; ++r8) {
                    const uint32_t byte = (cur.cw[r8][p >> 2] >> (8 * (p & 3))) & 0xFFu;
                    lv[r8] = *reinterpret_cast<const float2*>(lut + (byte << 3));
                }
                __builtin_amdgcn_sched_barrier(0);
                float v0[8], v1[8];
#pragma unroll
                for (int r8 = 0; r8 < 8; ++r8) {
                    v0[r8] = lv[r8].x * sc[r8];  // level * absmax in fp32, RNbf below
                    v1[r8] = lv[r8].y * sc[r8];
                }
                const u32x4 f0 = {pack_bf16x2(v0[0], v0[1]), pack_bf16x2(v0[2], v0[3]), pack_bf16x2(v0[4], v0[5]),
                                  pack_bf16x2(v0[6], v0[7])};
                const u32x4 f1 = {pack_bf16x2(v1[0], v1[1]), pack_bf16x2(v1[2], v1[3]), pack_bf16x2(v1[4], v1[5]),
                                  pack_bf16x2(v1[6], v1[7])};
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const bf16x8 da = as_bf16x8(cur.dv[tb]);
                    acc[tb][2 * p] = mfma16x16x32(da, as_bf16x8(f0), acc[tb][2 * p]);
                    acc[tb][2 * p + 1] = mfma16x16x32(da, as_bf16x8(f1), acc[tb][2 * p + 1]);
                }
            }
        };
        int i = 0;
        if constexpr (R == 3) {
            for (; i + 2 < nw; i += 3) {
                step(i, std::integral_constant<int, 0>{});
                step(i + 1, std::integral_constant<int, 1>{});
                step(i + 2, std::integral_constant<int, 2>{});
            }
            if (i < nw) step(i, std::integral_constant<int, 0>{});
            if (i + 1 < nw) step(i + 1, std::integral_constant<int, 1>{});
        } else {
            for (; i + 1 < nw; i += 2) {
                step(i, std::integral_constant<int, 0>{});
                step(i + 1, std::integral_constant<int, 1>{});
            }
            if (i < nw) step(i, std::integral_constant<int, 0>{});
        }
    }

    // lane holds D[t = 16 tb + 4q + e][feature 16 l16 + j] in acc[tb][j][e]; sum
    // (w0 + w2) + (w1 + w3)
    if (wave >= 2)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    *reinterpret_cast<f32x4*>(&sRed[wave - 2][16 * tb + 4 * q + e][16 * l16 + 4 * m]) =
                        f32x4{acc[tb][4 * m][e], acc[tb][4 * m + 1][e], acc[tb][4 * m + 2][e], acc[tb][4 * m + 3][e]};
    __syncthreads();
    if (wave < 2)
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    f32x4* o = reinterpret_cast<f32x4*>(&sRed[wave][16 * tb + 4 * q + e][16 * l16 + 4 * m]);
                    *o = *o + f32x4{acc[tb][4 * m][e], acc[tb][4 * m + 1][e], acc[tb][4 * m + 2][e],
                                    acc[tb][4 * m + 3][e]};
                }
    __syncthreads();
    const int k = k0 + tid;
    if (k < K) {
        float* dst = dxpart + size_t(split) * T * K + k;
        for (int t = 0; t < T; ++t) dst[size_t(t) * K] = sRed[0][t][tid] + sRed[1][t][tid];
    }
}

// The backward launch: a 1-D grid of dx_total = dx_cols x splits dX workgroups (one
// column block and split each), then the LoRA pre-pass roles, numbered from dx_total:
// g workgroups [0, gblocks), dB workgroups [gblocks, gblocks + dblocks). The roles share
// no data inside the launch (g is summed by the finish kernel, dB is final).
template <int RB, int TB>
__global__ __launch_bounds__(kThreads, kBOccupancy<TB>) void k_skinny_bwd(
    const uint16_t* __restrict__ dy, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const uint16_t* __restrict__ B, const float* __restrict__ u, int T, int N, int K, int r, float s,
    int steps_per_split, int dx_cols, int dx_total, int gsteps, int gblocks, int dblocks, float* __restrict__ dxpart,
    float* __restrict__ gpart, float* __restrict__ dB, Tables tab) {
    __shared__ __align__(16) union {
        BwdSmem<TB> dx;
        pre::PreSmem<RB, pre::kTC> pre;
    } sm;
    // dX workgroups in an XCD-aware order (each XCD runs a contiguous range of (column
    // block, split) pairs, column block fastest): the eight column blocks whose scales
    // share one 128-byte line of a row then read it through one L2
    if (int(blockIdx.x) < dx_total) {
        const int t = int(xcd_tile_order(blockIdx.x, uint32_t(dx_total)));
        skinny_bwd_dx<TB>(dy, codes, absmax, T, N, K, steps_per_split, t % dx_cols, t / dx_cols, dxpart, tab, sm.dx);
        return;
    }
    const int blk = int(blockIdx.x) - dx_total;
    if (blk < gblocks)
        pre::g_role<RB, 1>(dy, B, T, N, r, gsteps, blk, gpart, sm.pre.g);
    else if (blk < gblocks + dblocks)
        pre::db_role<RB, pre::kTC>(dy, u, T, N, r, s, blk - gblocks, 0, T, dB, sm.pre.d);
}

// Backward finish, two kinds of workgroups in one launch (64 features each, lane =
// feature k); g = the sum of the pre-pass's partials, staged in LDS:
//  - blocks [0, dx_blocks): wave = token t: dX[t][k] = RNbf( sum_z dxpart[z][t][k] +
//    s . sum_j g[t][j] A[j][k] ), A[:, k0 .. k0 + 63] staged in LDS;
//  - the rest: wave w takes ranks j = w, w + 4, ...: dA[j][k] = s . sum_t g[t][j] x[t][k],
//    x[:, k0 .. k0 + 63] staged in LDS, tokens added in increasing order.
__global__ __launch_bounds__(kThreads) void k_skinny_bwd_finish(
    const float* __restrict__ dxpart, int splits, const float* __restrict__ gpart, int gparts,
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ x, int T, int K, int r, float s, int col_blocks,
    int dx_blocks, uint16_t* __restrict__ dx, float* __restrict__ dA) {
    __shared__ float sg[kSkinnyMaxT * kMaxRank];   // g [t - t0][j]
    __shared__ float sw[kMaxRank * kFinF];  // A [j][k - k0] or x [t][k - k0]
    __shared__ float stmp[kThreads];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool dx_role = int(blockIdx.x) < dx_blocks;
    const int b = dx_role ? int(blockIdx.x) : int(blockIdx.x) - dx_blocks;
    const int k0 = (b % col_blocks) * kFinF, k = k0 + lane;
    // A rows (dX role) or x rows (dA role), columns k0 .. k0 + 63; every load of a role is
    // issued before the first is waited for (one memory round trip)
    const int wrows = dx_role ? r : T;
    const auto rw = dx_role ? make_rsrc(A, uint32_t(r) * uint32_t(K) * 2u) : make_rsrc(x, uint32_t(T) * uint32_t(K) * 2u);
    constexpr int WV = kMaxRank / kFinTk;  // rows wave + 4i
    uint32_t wv[WV];
#pragma unroll
    for (int i = 0; i < WV; ++i) {
        const int row = wave + kFinTk * i;
        wv[i] = __builtin_amdgcn_raw_buffer_load_b16(
            rw, int(row < wrows && k < K ? (uint32_t(row) * uint32_t(K) + uint32_t(k)) * 2u : kOutOfRange), 0, 0);
    }
    if (dx_role) {
        const int t = (b / col_blocks) * kFinTk + wave;
        const bool live = t < T && k < K;
        float pv[kMaxSplits];
        load_splits(pv, make_rsrc(dxpart, uint32_t(splits) * uint32_t(T) * uint32_t(K) * 4u), splits,
                    (uint32_t(t) * uint32_t(K) + uint32_t(k)) * 4u, uint32_t(T) * uint32_t(K) * 4u, live);
        const int tb0 = (b / col_blocks) * kFinTk;
        // the g partials' loads join the ones above before any is waited for
        stage_partial_sums(sg, stmp, gpart, gparts, T, r, tb0, kFinTk, 0, r);  // ends with a barrier
#pragma unroll
        for (int i = 0; i < WV; ++i) sw[(wave + kFinTk * i) * kFinF + lane] = bf16_to_f32(uint16_t(wv[i]));
        __syncthreads();
        if (!live) return;
        const float acc = sum_splits(pv);
        float l = 0.0f;
#pragma unroll 8
        for (int j = 0; j < r; ++j) l += sg[wave * r + j] * sw[j * kFinF + lane];
        dx[size_t(t) * K + k] = bf16_bits(acc + s * l);
        return;
    }
    stage_partial_sums(sg, stmp, gpart, gparts, T, r, 0, T, 0, r);  // ends with a barrier
#pragma unroll
    for (int i = 0; i < WV; ++i) sw[(wave + kFinTk * i) * kFinF + lane] = bf16_to_f32(uint16_t(wv[i]));
    __syncthreads();
    if (k >= K) return;
    for (int j = wave; j < r; j += 4) {
        float c = 0.0f;
#pragma unroll 4
        for (int t = 0; t < T; ++t) c += sg[t * r + j] * sw[t * kFinF + lane];
        dA[size_t(j) * K + k] = s * c;
    }
}

template <int TB>
void launch_fwd_tb(const SkinnyPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* x,
                   const uint16_t* A, int64_t T, int64_t N, int64_t K, int r, float* ypart, float* upart,
                   hipStream_t stream) {
    const dim3 grid(unsigned(p.row_blocks + (r > 0 ? kUParts : 0)), unsigned(p.splits));
    hipLaunchKernelGGL(k_skinny_fwd<TB>, grid, dim3(kThreads), 0, stream, x, codes, absmax, A, int(T), int(N), int(K),
                       r, p.steps_per_split, p.row_blocks, ypart, upart, tables());
}

// Split policy of the streaming kernels (measured on the 7B and 72B projection shapes
// at T = 1..32): about kWGs workgroups of at least kMinSteps main-loop steps each -
// longer-running workgroups stream better than more of them - unless that leaves
// fewer than kFillWGs workgroups, then down to one step each; the fp32 partials
// (written once and read back once, mostly in the last-level cache) at most
// 1/kPartialDiv of the code bytes; at most kMaxSplits splits (the finish kernels load
// them all at once).
constexpr int64_t kFillWGs = 256;
constexpr int64_t kFwdWGs = 512;
constexpr int64_t kFwdMinSteps = 4;
constexpr int64_t kFwdPartialDiv = 1;  // 2 was 20% slower on the 7B q forward at T = 32
constexpr int64_t kBwdWGs = 256;  // one per CU: 512 was 4-17% slower, 384 (1.5 per CU) slower still
constexpr int64_t kBwdMinSteps = 4;  // one per wave
constexpr int64_t kBwdPartialDiv = 1;

int64_t pick_skinny_splits(int64_t blocks, int64_t steps, int64_t wgs, int64_t min_steps, int64_t partial_cap) {
    int64_t by_steps = std::max<int64_t>(1, steps / min_steps);
    if (blocks * by_steps < kFillWGs) by_steps = std::min<int64_t>(steps, cdiv(kFillWGs, blocks));
    int64_t s = std::max<int64_t>(1, wgs / blocks);
    s = std::min<int64_t>(s, by_steps);
    s = std::min<int64_t>(s, std::max<int64_t>(1, partial_cap));
    return std::min<int64_t>(s, kMaxSplits);
}

}  // namespace

SkinnyPlan plan_skinny_fwd(int64_t T, int64_t N, int64_t K, int r) {
    SkinnyPlan p{};
    p.row_blocks = int(cdiv(N, kRows));
    const int64_t steps = cdiv(K, kDK);
    // partial bytes 8 s T N <= N K / (2 kPartialDiv); one u workgroup set per split
    const int64_t s = pick_skinny_splits(p.row_blocks + 1, steps, kFwdWGs, kFwdMinSteps, K / (16 * kFwdPartialDiv * T));
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
    p.col_blocks = int(cdiv(K, kBCols));
    const int64_t steps = cdiv(N, kBRows);
    // partial bytes 8 s T K <= N K / (2 kPartialDiv)
    const int64_t s = pick_skinny_splits(p.col_blocks, steps, kBwdWGs, kBwdMinSteps, N / (16 * kBwdPartialDiv * T));
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
    if (T > kSkinnyFwdLongT) return hipErrorInvalidValue;  // at most four 16-token MFMA blocks
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
    const dim3 fgrid(unsigned(cdiv(N, kFinF)), unsigned(cdiv(T, kFinTk)));
    hipLaunchKernelGGL(k_skinny_fwd_finish, fgrid, dim3(kThreads), 0, stream, ypart, upart, p.splits * kUParts,
                       p.splits, B, int(T), int(N), r, s, y, u_save);
    return hipGetLastError();
}

template <int TB>
void launch_bwd_rb(int rb, dim3 grid, const uint16_t* dy, const uint8_t* codes, const float* absmax,
                   const uint16_t* B, const float* u, int64_t T, int64_t N, int64_t K, int r, float s,
                   int steps_per_split, int dx_cols, int dx_total, int gsteps, int gblocks, int dblocks, float* dxpart,
                   float* gpart, float* dB, hipStream_t stream) {
    switch (rb) {
        case 1: hipLaunchKernelGGL((k_skinny_bwd<1, TB>), grid, dim3(kThreads), 0, stream, dy, codes, absmax, B, u,
                                   int(T), int(N), int(K), r, s, steps_per_split, dx_cols, dx_total, gsteps, gblocks,
                                   dblocks, dxpart, gpart, dB, tables()); break;
        case 2: hipLaunchKernelGGL((k_skinny_bwd<2, TB>), grid, dim3(kThreads), 0, stream, dy, codes, absmax, B, u,
                                   int(T), int(N), int(K), r, s, steps_per_split, dx_cols, dx_total, gsteps, gblocks,
                                   dblocks, dxpart, gpart, dB, tables()); break;
        case 3: hipLaunchKernelGGL((k_skinny_bwd<3, TB>), grid, dim3(kThreads), 0, stream, dy, codes, absmax, B, u,
                                   int(T), int(N), int(K), r, s, steps_per_split, dx_cols, dx_total, gsteps, gblocks,
                                   dblocks, dxpart, gpart, dB, tables()); break;
        default: hipLaunchKernelGGL((k_skinny_bwd<4, TB>), grid, dim3(kThreads), 0, stream, dy, codes, absmax, B, u,
                                    int(T), int(N), int(K), r, s, steps_per_split, dx_cols, dx_total, gsteps, gblocks,
                                    dblocks, dxpart, gpart, dB, tables()); break;
    }
}

hipError_t launch_skinny_bwd(const SkinnyPlan& p, const BwdPlan& bp, const uint8_t* codes, const float* absmax,
                             const uint16_t* dy, const uint16_t* x, const uint16_t* A, const uint16_t* B,
                             const float* u, int64_t T, int64_t N, int64_t K, int r, float s, uint16_t* dx, float* dA,
                             float* dB, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    float* dxpart = reinterpret_cast<float*>(w + bp.off_dx);
    float* gpart = reinterpret_cast<float*>(w + bp.off_gpart);
    if (T > kSkinnyBwdT) return hipErrorInvalidValue;  // at most two 16-token MFMA blocks
    static_assert(kSkinnyBwdT <= 32, "one or two token blocks are instantiated");
    const int dx_cols = dx ? p.col_blocks : 0;
    const int splits = dx ? p.splits : 1;
    const int gblocks = r > 0 ? int(cdiv(T, pre::kTC)) * bp.gparts : 0;
    const int dblocks = r > 0 ? int(cdiv(N, 64)) : 0;
    const int dx_total = dx_cols * splits;
    if (dx_total + gblocks + dblocks > 0) {
        const dim3 grid(unsigned(dx_total + gblocks + dblocks));
        if (dx) prof_gemm_begin(stream);
        const int rb = std::max(1, (r + 15) / 16);
        if (T <= 16)
            launch_bwd_rb<1>(rb, grid, dy, codes, absmax, B, u, T, N, K, r, s, p.steps_per_split, dx_cols, dx_total,
                             bp.gsteps, gblocks, dblocks, dxpart, gpart, dB, stream);
        else
            launch_bwd_rb<2>(rb, grid, dy, codes, absmax, B, u, T, N, K, r, s, p.steps_per_split, dx_cols, dx_total,
                             bp.gsteps, gblocks, dblocks, dxpart, gpart, dB, stream);
        if (dx) prof_gemm_end(stream);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int col_blocks = int(cdiv(K, kFinF));
    const int dx_blocks = dx ? col_blocks * int(cdiv(T, kFinTk)) : 0;
    const int da_blocks = r > 0 ? col_blocks : 0;
    if (dx_blocks + da_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_skinny_bwd_finish, dim3(unsigned(dx_blocks + da_blocks)), dim3(kThreads), 0, stream, dxpart,
                       p.splits, gpart, bp.gparts, A, x, int(T), int(K), r, s, col_blocks, dx_blocks, dx, dA);
    return hipGetLastError();
}

}  // namespace nf4
