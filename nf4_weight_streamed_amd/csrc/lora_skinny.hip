// Skinny rank-r GEMMs of the LoRA side path (Poros API reference,
// "PorosTrainer.from_pretrained": lora_rank 16, lora_alpha 32; adapters are the
// only trainable parameters, "patch_hf_model" Behavior 3).
//
//   forward:  u  = x . A^T        [T, r] fp32, as partials over K ranges
//   backward: g  = dY . B         [T, r] fp32, as partials over N ranges
//             dB = s . dY^T . u   [N, r] fp32, complete
//
// The partials are summed, in partial order, by the GEMM kernel that consumes them
// (which also writes u_save in the forward); dA = s . g^T . x is formed there too,
// as one share per token tile. All products run on v_mfma_f32_16x16x32_bf16; the fp32
// operand u of dB is fed as bf16 hi + lo (two MFMAs, about 2^-17 relative). Every
// reduction has a fixed order: results do not depend on scheduling.
#include "common.h"
#include "device.h"
#include "lora_pre.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------- u partials
// grid (ceil(T/16), P): 16 tokens x one K range (in 32-wide steps) per workgroup; the
// 4 waves take interleaved steps, four at a time with all loads issued first, then
// add up in wave order through LDS. RB = rank blocks of 16.
template <int RB>
__global__ __launch_bounds__(kThreads) void k_lora_down(const uint16_t* __restrict__ x, const uint16_t* __restrict__ A,
                                                        int T, int K, int r, int steps_per_part,
                                                        float* __restrict__ upart) {
    __shared__ float red[4][RB][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16;
    const int kb = blockIdx.y * steps_per_part;
    const int ke = min(kb + steps_per_part, K / 32);
    const int kof = 8 * (lane >> 4);
    const auto rx = make_rsrc(x + size_t(t0) * K, uint32_t(min(16, T - t0)) * uint32_t(K) * 2u);
    const auto ra = make_rsrc(A, uint32_t(r) * uint32_t(K) * 2u);  // rows j >= r read as zero
    const uint32_t xrow = uint32_t(lane & 15) * uint32_t(K) * 2u;

    f32x4 acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int ks0 = kb + wave; ks0 < ke; ks0 += 16) {
        u32x4 xv[4], av[4][RB];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int ks = ks0 + 4 * q;
            const uint32_t kbyte = uint32_t(ks * 32 + kof) * 2u;
            xv[q] = buf_load16(rx, ks < ke ? xrow + kbyte : kOutOfRange);
#pragma unroll
            for (int b = 0; b < RB; ++b)
                av[q][b] = buf_load16(ra, ks < ke ? uint32_t(16 * b + (lane & 15)) * uint32_t(K) * 2u + kbyte
                                                  : kOutOfRange);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int b = 0; b < RB; ++b) acc[b] = mfma16x16x32(as_bf16x8(xv[q]), as_bf16x8(av[q][b]), acc[b]);
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][b][lane][e] = acc[b][e];
    __syncthreads();
    float* dst = upart + size_t(blockIdx.y) * T * r;
    for (int o = threadIdx.x; o < 16 * r; o += kThreads) {
        const int t = o / r, j = o % r;
        const int b = j >> 4, l = 16 * (t >> 2) + (j & 15), e = t & 3;
        const float v = ((red[0][b][l][e] + red[1][b][l][e]) + red[2][b][l][e]) + red[3][b][l][e];
        if (t0 + t < T) dst[size_t(t0 + t) * r + j] = v;
    }
}

// ---------------------------------------------------------------- backward pre-pass
// One launch, the two roles of lora_pre.h: g workgroups [0, gblocks), dB workgroups
// the rest (feature block fastest, then token range; with one range dB is written
// directly, else each range's share goes to dbpart [range][N][r]).
using pre::db_role;
using pre::g_role;
using pre::kGChunk;
using pre::kTC;
using pre::PreSmem;

template <int RB>
__global__ __launch_bounds__(kThreads) void k_lora_bwd_pre(const uint16_t* __restrict__ dy,
                                                           const uint16_t* __restrict__ B,
                                                           const float* __restrict__ u, int T, int N, int r, float s,
                                                           int gsteps, int gblocks, int dbtokens, float* __restrict__ gpart,
                                                           float* __restrict__ dB, float* __restrict__ dbpart) {
    __shared__ __align__(16) PreSmem<RB, pre::kDbTLong> sm;
    if (int(blockIdx.x) < gblocks) {
        g_role<RB, (RB <= 2 ? 2 : 1)>(dy, B, T, N, r, gsteps, blockIdx.x, gpart, sm.g);  // two chunks in flight where the registers allow
        return;
    }
    const int nblocks = (N + 63) / 64, d = int(blockIdx.x) - gblocks;
    const int chunk = d / nblocks, t_begin = chunk * dbtokens;
    float* dst = dbtokens >= T ? dB : dbpart + size_t(chunk) * N * r;
    db_role<RB, pre::kDbTLong>(dy, u, T, N, r, s, d % nblocks, t_begin, min(T, t_begin + dbtokens), dst, sm.d);
}

template <int RB>
void launch_down_rb(const FwdPlan& p, const uint16_t* x, const uint16_t* A, int64_t T, int64_t K, int r,
                    float* upart, hipStream_t stream) {
    hipLaunchKernelGGL(k_lora_down<RB>, dim3(unsigned(cdiv(T, 16)), unsigned(p.down_parts)), dim3(kThreads), 0,
                       stream, x, A, int(T), int(K), r, p.down_steps, upart);
}

template <int RB>
void launch_pre_rb(const BwdPlan& p, const uint16_t* dy, const uint16_t* B, const float* u, int64_t T, int64_t N,
                   int r, float s, float* gpart, float* dB, float* dbpart, hipStream_t stream) {
    const int gblocks = int(cdiv(T, kTC)) * p.gparts;
    const int dblocks = int(cdiv(N, 64)) * p.dbchunks;
    hipLaunchKernelGGL(k_lora_bwd_pre<RB>, dim3(unsigned(gblocks + dblocks)), dim3(kThreads), 0, stream, dy, B, u,
                       int(T), int(N), r, s, p.gsteps, gblocks, p.dbtokens, gpart, dB, dbpart);
}

}  // namespace

void plan_lora_down(FwdPlan& p, int64_t K) {
    // up to 4 K ranges of 32-wide steps (fewer for short K): enough workgroups for the
    // skinny product, few enough partials for the GEMM to add up per tile
    const int64_t ks32 = K / 32;
    const int64_t parts = std::max<int64_t>(1, std::min<int64_t>(kMaxDownParts, ks32 / 8));
    p.down_steps = int(cdiv(ks32, parts));
    p.down_parts = int(cdiv(ks32, p.down_steps));
}

void plan_lora_bwd_pre(BwdPlan& p, int64_t T, int64_t N, int max_parts) {
    const int64_t chunks = cdiv(N, kGChunk);
    const int64_t parts = std::max<int64_t>(1, std::min<int64_t>(max_parts, chunks / 2));
    p.gsteps = int(cdiv(chunks, parts));
    p.gparts = int(cdiv(chunks, p.gsteps));
    // dB over token ranges of whole 128-token sub-chunks (at most kMaxDbChunks ranges):
    // each workgroup then waits on one or a few sub-chunk loads instead of all of them
    const int64_t sub = cdiv(T, pre::kDbTLong);
    const int64_t ranges = std::min<int64_t>(kMaxDbChunks, sub);
    p.dbtokens = int(pre::kDbTLong * cdiv(sub, ranges));
    p.dbchunks = int(cdiv(T, p.dbtokens));
}

hipError_t launch_lora_down(const FwdPlan& p, const uint16_t* x, const uint16_t* A, int64_t T, int64_t K, int r,
                            float* upart, hipStream_t stream) {
    switch ((r + 15) / 16) {
        case 1: launch_down_rb<1>(p, x, A, T, K, r, upart, stream); break;
        case 2: launch_down_rb<2>(p, x, A, T, K, r, upart, stream); break;
        case 3: launch_down_rb<3>(p, x, A, T, K, r, upart, stream); break;
        default: launch_down_rb<4>(p, x, A, T, K, r, upart, stream); break;
    }
    return hipGetLastError();
}

hipError_t launch_lora_bwd_pre(const BwdPlan& p, const uint16_t* dy, const uint16_t* B, const float* u, int64_t T,
                               int64_t N, int r, float s, float* gpart, float* dB, float* dbpart, hipStream_t stream) {
    switch ((r + 15) / 16) {
        case 1: launch_pre_rb<1>(p, dy, B, u, T, N, r, s, gpart, dB, dbpart, stream); break;
        case 2: launch_pre_rb<2>(p, dy, B, u, T, N, r, s, gpart, dB, dbpart, stream); break;
        case 3: launch_pre_rb<3>(p, dy, B, u, T, N, r, s, gpart, dB, dbpart, stream); break;
        default: launch_pre_rb<4>(p, dy, B, u, T, N, r, s, gpart, dB, dbpart, stream); break;
    }
    return hipGetLastError();
}

}  // namespace nf4
