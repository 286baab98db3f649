// Skinny rank-r GEMMs of the LoRA side path (Poros API reference,
// "PorosTrainer.from_pretrained": lora_rank 16, lora_alpha 32; adapters are the
// only trainable parameters, "patch_hf_model" Behavior 3).
//
//   forward:  u  = x . A^T                 [T, r] fp32 (saved for the backward)
//   backward: g  = dY . B                  [T, r] fp32 (workspace)
//             dB = s . dY^T . u            [N, r] fp32
//             dA = s . g^T . x             [r, K] fp32
//
// All four run on v_mfma_f32_16x16x32_bf16. fp32 operands (u, g) are fed as
// bf16 hi + lo pairs (two MFMAs), so the products keep about 2^-17 relative
// accuracy. Every reduction has a fixed order (fixed wave order in LDS, fixed
// partial order in the reduce kernels): results do not depend on scheduling.
#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRB = NF4_MAX_RANK_BLOCKS;  // r <= 16 * kMaxRB

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// ---------------------------------------------------------------- u = x . A^T
// grid (ceil(T/16), S): 16 tokens x one K range of 32-wide steps per workgroup;
// the 4 waves take interleaved steps, then add up in wave order through LDS.
__global__ __launch_bounds__(kThreads) void k_lora_down_partial(const uint16_t* __restrict__ x,
                                                                const uint16_t* __restrict__ A, int T, int K,
                                                                int r, int steps_per_split,
                                                                float* __restrict__ out) {
    __shared__ float red[4][kMaxRB][64][4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * 16;
    const int ksteps = K / 32;
    const int kb = blockIdx.y * steps_per_split;
    const int ke = min(kb + steps_per_split, ksteps);
    const int rb_n = (r + 15) / 16;
    const int tr = t0 + (lane & 15);
    const int kof = 8 * (lane >> 4);

    f32x4 acc[kMaxRB];
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ks = kb + wave; ks < ke; ks += 4) {
        const int k = ks * 32 + kof;
        const bf16x8 xa = as_bf16x8(tr < T ? ld16(x + size_t(tr) * K + k) : u32x4{0u, 0u, 0u, 0u});
#pragma unroll
        for (int b = 0; b < kMaxRB; ++b) {
            if (b < rb_n) {
                const int j = 16 * b + (lane & 15);
                const bf16x8 aw = as_bf16x8(j < r ? ld16(A + size_t(j) * K + k) : u32x4{0u, 0u, 0u, 0u});
                acc[b] = mfma16x16x32(xa, aw, acc[b]);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b)
        if (b < rb_n)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[wave][b][lane][e] = acc[b][e];
    __syncthreads();
    float* dst = out + size_t(blockIdx.y) * T * r;
    for (int o = threadIdx.x; o < 16 * r; o += kThreads) {
        const int t = o / r, j = o % r;
        const int b = j >> 4, l = 16 * (t >> 2) + (j & 15), e = t & 3;
        const float v = ((red[0][b][l][e] + red[1][b][l][e]) + red[2][b][l][e]) + red[3][b][l][e];
        if (t0 + t < T) dst[size_t(t0 + t) * r + j] = v;
    }
}

// out[i] = sum over z < parts of part[z * stride + i]: 64 outputs per workgroup; thread
// group q (of 4) adds parts z = q, q+4, ... in increasing z, then the four group sums
// are added in group order. The order depends on `parts` only, never on timing.
// Two independent jobs (a, b) can share one launch: workgroups [0, blocks_a) do job a.
struct SumJob {
    const float* part;
    int parts;
    int64_t stride, count;
    float* out;
};

__device__ __forceinline__ void sum_parts_block(const SumJob& j, int64_t blk, float (*red)[64]) {
    const int o = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t i = blk * 64 + o;
    float v = 0.0f;
    if (i < j.count) {
#pragma unroll 8
        for (int z = q; z < j.parts; z += 4) v += j.part[size_t(z) * j.stride + i];
    }
    red[q][o] = v;
    __syncthreads();
    if (q == 0 && i < j.count) j.out[i] = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
}

__global__ __launch_bounds__(kThreads) void k_sum_parts(SumJob a, SumJob b, int64_t blocks_a) {
    __shared__ float red[4][64];
    if (int64_t(blockIdx.x) < blocks_a)
        sum_parts_block(a, blockIdx.x, red);
    else
        sum_parts_block(b, int64_t(blockIdx.x) - blocks_a, red);
}

// ---------------------------------------------------------------- g and dB in one pass over dY
// grid (ceil(N/64), chunks): 64 output features x `tc` tokens per workgroup, in
// sub-chunks of 32 tokens whose global loads are issued before the previous
// sub-chunk's MFMAs. g partial over the slab's features -> gpart[slab][t]; dB of
// the slab over the chunk's tokens -> dbout[chunk] (wave w owns features 16w..16w+15).
constexpr int kTC = 32;  // tokens per sub-chunk
constexpr int kUV = kTC * 16 * kMaxRB / kThreads;  // u (or g) values per thread per sub-chunk

__global__ __launch_bounds__(kThreads) void k_lora_bwd_pre(const uint16_t* __restrict__ dy,
                                                           const uint16_t* __restrict__ B,
                                                           const float* __restrict__ u, int T, int N, int r,
                                                           float s, int tc, float* __restrict__ dbout,
                                                           float* __restrict__ gpart) {
    __shared__ __align__(16) uint16_t sBt[16 * kMaxRB][64 + 8];  // B^T of the slab: [j][n]
    __shared__ __align__(16) uint16_t sdy[kTC][64 + 8];          // dY sub-chunk: [t][n]
    __shared__ __align__(16) uint16_t sdyT[64][kTC + 8];         // dY sub-chunk: [n][t]
    __shared__ __align__(16) uint16_t suh[16 * kMaxRB][kTC + 8];  // (s.u)^T hi: [j][t]
    __shared__ __align__(16) uint16_t sul[16 * kMaxRB][kTC + 8];  // (s.u)^T lo
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 64;
    const int tb0 = blockIdx.y * tc, tb1 = min(tb0 + tc, T);
    const int rb_n = (r + 15) / 16;
    const int jr = 16 * rb_n;

    for (int o = tid; o < jr * 64; o += kThreads) {
        const int j = o / 64, n = o % 64;
        sBt[j][n] = (j < r && n0 + n < N) ? B[size_t(n0 + n) * r + j] : uint16_t(0);
    }
    for (int o = tid; o < jr * kTC; o += kThreads) {
        suh[o / kTC][o % kTC] = 0;
        sul[o / kTC][o % kTC] = 0;
    }

    const int lt = tid >> 3, ln8 = (tid & 7) * 8;  // this thread's 16-byte piece of a dY sub-chunk
    u32x4 vdy;
    float uv[kUV];
    auto gload = [&](int t0) {
        const bool ok = (t0 + lt < tb1) && (n0 + ln8 < N);
        vdy = ok ? ld16(dy + size_t(t0 + lt) * N + n0 + ln8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kUV; ++i) {
            const int o = tid + kThreads * i;
            const int t = o / jr, j = o % jr;
            uv[i] = (o < kTC * jr && t0 + t < tb1 && j < r) ? s * u[size_t(t0 + t) * r + j] : 0.0f;
        }
    };
    auto sstore = [&]() {
        *reinterpret_cast<u32x4*>(&sdy[lt][ln8]) = vdy;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = vdy[e >> 1];
            sdyT[ln8 + e][lt] = uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF));
        }
#pragma unroll
        for (int i = 0; i < kUV; ++i) {
            const int o = tid + kThreads * i;
            if (o < kTC * jr) {
                const int t = o / jr, j = o % jr;
                __bf16 h, l;
                split_bf16(uv[i], h, l);
                suh[j][t] = __builtin_bit_cast(uint16_t, h);
                sul[j][t] = __builtin_bit_cast(uint16_t, l);
            }
        }
    };

    f32x4 accB[kMaxRB];
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) accB[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kof = 8 * (lane >> 4);

    if (tb0 < tb1) gload(tb0);
    for (int t0 = tb0; t0 < tb1; t0 += kTC) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (t0 + kTC < tb1) gload(t0 + kTC);
        // g partial: 2 token blocks x rb_n rank blocks, contraction over the slab's 64 features
        for (int task = wave; task < 2 * rb_n; task += 4) {
            const int tbk = task & 1, b = task >> 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sdy[16 * tbk + (lane & 15)][32 * kk + kof]));
                const bf16x8 bb = as_bf16x8(*reinterpret_cast<const u32x4*>(&sBt[16 * b + (lane & 15)][32 * kk + kof]));
                acc = mfma16x16x32(a, bb, acc);
            }
            float* dst = gpart + size_t(blockIdx.x) * T * r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * tbk + 4 * (lane >> 4) + e, j = 16 * b + (lane & 15);
                if (t < tb1 && j < r) dst[size_t(t) * r + j] = acc[e];
            }
        }
        // dB: rows = features 16*wave.., contraction over the sub-chunk's 32 tokens
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sdyT[16 * wave + (lane & 15)][kof]));
#pragma unroll
        for (int b = 0; b < kMaxRB; ++b) {
            if (b < rb_n) {
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4*>(&suh[16 * b + (lane & 15)][kof]));
                const bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4*>(&sul[16 * b + (lane & 15)][kof]));
                accB[b] = mfma16x16x32(a, bh, accB[b]);
                accB[b] = mfma16x16x32(a, bl, accB[b]);
            }
        }
    }
    float* dst = dbout + size_t(blockIdx.y) * N * r;
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) {
        if (b < rb_n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + 16 * wave + 4 * (lane >> 4) + e, j = 16 * b + (lane & 15);
                if (n < N && j < r) dst[size_t(n) * r + j] = accB[b][e];
            }
        }
    }
}

// ---------------------------------------------------------------- dA = s . g^T . x
// grid (ceil(K/64), chunks): 64 input features (wave w owns 16w..16w+15) x `tc`
// tokens per workgroup, 32-token sub-chunks prefetched one ahead; dA of the chunk
// -> daout[chunk].
__global__ __launch_bounds__(kThreads) void k_lora_da(const float* __restrict__ g, const uint16_t* __restrict__ x,
                                                      int T, int K, int r, float s, int tc,
                                                      float* __restrict__ daout) {
    __shared__ __align__(16) uint16_t sxT[64][kTC + 8];           // x sub-chunk: [k][t]
    __shared__ __align__(16) uint16_t sgh[16 * kMaxRB][kTC + 8];  // (s.g)^T hi: [j][t]
    __shared__ __align__(16) uint16_t sgl[16 * kMaxRB][kTC + 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k0 = blockIdx.x * 64;
    const int tb0 = blockIdx.y * tc, tb1 = min(tb0 + tc, T);
    const int rb_n = (r + 15) / 16;
    const int jr = 16 * rb_n;
    for (int o = tid; o < jr * kTC; o += kThreads) {
        sgh[o / kTC][o % kTC] = 0;
        sgl[o / kTC][o % kTC] = 0;
    }
    const int lt = tid >> 3, lk8 = (tid & 7) * 8;
    u32x4 vx;
    float gv[kUV];
    auto gload = [&](int t0) {
        const bool ok = (t0 + lt < tb1) && (k0 + lk8 < K);
        vx = ok ? ld16(x + size_t(t0 + lt) * K + k0 + lk8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < kUV; ++i) {
            const int o = tid + kThreads * i;
            const int t = o / jr, j = o % jr;
            gv[i] = (o < kTC * jr && t0 + t < tb1 && j < r) ? s * g[size_t(t0 + t) * r + j] : 0.0f;
        }
    };
    auto sstore = [&]() {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t w = vx[e >> 1];
            sxT[lk8 + e][lt] = uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF));
        }
#pragma unroll
        for (int i = 0; i < kUV; ++i) {
            const int o = tid + kThreads * i;
            if (o < kTC * jr) {
                const int t = o / jr, j = o % jr;
                __bf16 h, l;
                split_bf16(gv[i], h, l);
                sgh[j][t] = __builtin_bit_cast(uint16_t, h);
                sgl[j][t] = __builtin_bit_cast(uint16_t, l);
            }
        }
    };
    f32x4 acc[kMaxRB];
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kof = 8 * (lane >> 4);

    if (tb0 < tb1) gload(tb0);
    for (int t0 = tb0; t0 < tb1; t0 += kTC) {
        __syncthreads();
        sstore();
        __syncthreads();
        if (t0 + kTC < tb1) gload(t0 + kTC);
        const bf16x8 bx = as_bf16x8(*reinterpret_cast<const u32x4*>(&sxT[16 * wave + (lane & 15)][kof]));
#pragma unroll
        for (int b = 0; b < kMaxRB; ++b) {
            if (b < rb_n) {
                const bf16x8 ah = as_bf16x8(*reinterpret_cast<const u32x4*>(&sgh[16 * b + (lane & 15)][kof]));
                const bf16x8 al = as_bf16x8(*reinterpret_cast<const u32x4*>(&sgl[16 * b + (lane & 15)][kof]));
                acc[b] = mfma16x16x32(ah, bx, acc[b]);
                acc[b] = mfma16x16x32(al, bx, acc[b]);
            }
        }
    }
    float* dst = daout + size_t(blockIdx.y) * r * K;
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) {
        if (b < rb_n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * b + 4 * (lane >> 4) + e, k = k0 + 16 * wave + (lane & 15);
                if (j < r && k < K) dst[size_t(j) * K + k] = acc[b][e];
            }
        }
    }
}

}  // namespace

hipError_t launch_lora_down(const uint16_t* x, const uint16_t* A, int64_t T, int64_t K, int r, float* u,
                            float* upart, int splits, int steps_per_split, hipStream_t stream) {
    const dim3 grid(unsigned(cdiv(T, 16)), unsigned(splits));
    float* out = splits > 1 ? upart : u;
    hipLaunchKernelGGL(k_lora_down_partial, grid, dim3(kThreads), 0, stream, x, A, int(T), int(K), r,
                       steps_per_split, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || splits == 1) return e;
    const int64_t count = T * r;
    const SumJob job{upart, splits, count, count, u};
    hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(count, 64))), dim3(kThreads), 0, stream, job, job,
                       cdiv(count, 64));
    return hipGetLastError();
}

hipError_t launch_lora_bwd_pre(const BwdPlan& p, const uint16_t* dy, const uint16_t* B, const float* u, int64_t T,
                               int64_t N, int r, float s, float* dB, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    float* g = reinterpret_cast<float*>(w + p.off_g);
    float* gpart = reinterpret_cast<float*>(w + p.off_gpart);
    float* dbout = p.pre_chunks > 1 ? reinterpret_cast<float*>(w + p.off_dbpart) : dB;
    hipLaunchKernelGGL(k_lora_bwd_pre, dim3(unsigned(p.nslab), unsigned(p.pre_chunks)), dim3(kThreads), 0, stream, dy,
                       B, u, int(T), int(N), r, s, p.pre_tc, dbout, gpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t cg = T * r, cb = N * r;
    const SumJob jg{gpart, p.nslab, cg, cg, g};
    if (p.pre_chunks > 1) {
        const SumJob jb{dbout, p.pre_chunks, cb, cb, dB};
        hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(cg, 64) + cdiv(cb, 64))), dim3(kThreads), 0, stream, jg, jb,
                           cdiv(cg, 64));
    } else {
        hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(cg, 64))), dim3(kThreads), 0, stream, jg, jg, cdiv(cg, 64));
    }
    return hipGetLastError();
}

hipError_t launch_lora_da(const BwdPlan& p, const uint16_t* x, int64_t T, int64_t K, int r, float s, float* dA,
                          void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    const float* g = reinterpret_cast<const float*>(w + p.off_g);
    float* daout = p.da_chunks > 1 ? reinterpret_cast<float*>(w + p.off_dapart) : dA;
    hipLaunchKernelGGL(k_lora_da, dim3(unsigned(cdiv(K, 64)), unsigned(p.da_chunks)), dim3(kThreads), 0, stream, g, x,
                       int(T), int(K), r, s, p.da_tc, daout);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.da_chunks == 1) return e;
    const int64_t count = int64_t(r) * K;
    const SumJob job{daout, p.da_chunks, count, count, dA};
    hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(count, 64))), dim3(kThreads), 0, stream, job, job,
                       cdiv(count, 64));
    return hipGetLastError();
}

}  // namespace nf4
