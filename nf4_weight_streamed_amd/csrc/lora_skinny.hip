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
__global__ __launch_bounds__(kThreads) void k_sum_parts(const float* __restrict__ part, int parts, int64_t stride,
                                                        int64_t count, float* __restrict__ out) {
    __shared__ float red[4][64];
    const int o = threadIdx.x & 63, q = threadIdx.x >> 6;
    const int64_t i = int64_t(blockIdx.x) * 64 + o;
    float v = 0.0f;
    if (i < count)
        for (int z = q; z < parts; z += 4) v += part[size_t(z) * stride + i];
    red[q][o] = v;
    __syncthreads();
    if (q == 0 && i < count) out[i] = ((red[0][o] + red[1][o]) + red[2][o]) + red[3][o];
}

// ---------------------------------------------------------------- g and dB in one pass over dY
// grid (ceil(N/64)): a slab of 64 output features per workgroup, looping over T in
// chunks of 32 tokens. g partial (over this slab's features) -> gpart[slab]; dB of
// the slab accumulates over all tokens in registers (wave w owns features 16w..16w+15).
constexpr int kTC = 32;  // tokens per chunk
__global__ __launch_bounds__(kThreads) void k_lora_bwd_pre(const uint16_t* __restrict__ dy,
                                                           const uint16_t* __restrict__ B,
                                                           const float* __restrict__ u, int T, int N, int r,
                                                           float s, float* __restrict__ dB,
                                                           float* __restrict__ gpart) {
    __shared__ __align__(16) uint16_t sBt[16 * kMaxRB][64 + 8];  // B^T of the slab: [j][n]
    __shared__ __align__(16) uint16_t sdy[kTC][64 + 8];          // dY chunk: [t][n]
    __shared__ __align__(16) uint16_t sdyT[64][kTC + 8];         // dY chunk: [n][t]
    __shared__ __align__(16) uint16_t suh[16 * kMaxRB][kTC + 8];  // (s.u)^T hi: [j][t]
    __shared__ __align__(16) uint16_t sul[16 * kMaxRB][kTC + 8];  // (s.u)^T lo
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blockIdx.x * 64;
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

    f32x4 accB[kMaxRB];
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) accB[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kof = 8 * (lane >> 4);

    for (int t0 = 0; t0 < T; t0 += kTC) {
        __syncthreads();
        {   // dY chunk: one 16-byte load per thread (32 tokens x 64 features)
            const int t = tid >> 3, n8 = (tid & 7) * 8;
            const bool ok = (t0 + t < T) && (n0 + n8 < N);
            const u32x4 v = ok ? ld16(dy + size_t(t0 + t) * N + n0 + n8) : u32x4{0u, 0u, 0u, 0u};
            *reinterpret_cast<u32x4*>(&sdy[t][n8]) = v;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = v[e >> 1];
                sdyT[n8 + e][t] = uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF));
            }
        }
        for (int o = tid; o < kTC * r; o += kThreads) {
            const int t = o / r, j = o % r;
            const float v = (t0 + t < T) ? s * u[size_t(t0 + t) * r + j] : 0.0f;
            __bf16 h, l;
            split_bf16(v, h, l);
            suh[j][t] = __builtin_bit_cast(uint16_t, h);
            sul[j][t] = __builtin_bit_cast(uint16_t, l);
        }
        __syncthreads();
        // g partial: 2 token blocks x rb_n rank blocks, contraction over the slab's 64 features
        for (int task = wave; task < 2 * rb_n; task += 4) {
            const int tb = task & 1, b = task >> 1;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(&sdy[16 * tb + (lane & 15)][32 * kk + kof]));
                const bf16x8 bb = as_bf16x8(*reinterpret_cast<const u32x4*>(&sBt[16 * b + (lane & 15)][32 * kk + kof]));
                acc = mfma16x16x32(a, bb, acc);
            }
            float* dst = gpart + size_t(blockIdx.x) * T * r;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int t = t0 + 16 * tb + 4 * (lane >> 4) + e, j = 16 * b + (lane & 15);
                if (t < T && j < r) dst[size_t(t) * r + j] = acc[e];
            }
        }
        // dB: rows = features 16*wave.., contraction over the chunk's 32 tokens
        {
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
    }
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) {
        if (b < rb_n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int n = n0 + 16 * wave + 4 * (lane >> 4) + e, j = 16 * b + (lane & 15);
                if (n < N && j < r) dB[size_t(n) * r + j] = accB[b][e];
            }
        }
    }
}

// ---------------------------------------------------------------- dA = s . g^T . x
// grid (ceil(K/64)): 64 input features per workgroup (wave w owns 16w..16w+15),
// looping over T in chunks of 32 tokens.
__global__ __launch_bounds__(kThreads) void k_lora_da(const float* __restrict__ g, const uint16_t* __restrict__ x,
                                                      int T, int K, int r, float s, float* __restrict__ dA) {
    __shared__ __align__(16) uint16_t sxT[64][kTC + 8];           // x chunk: [k][t]
    __shared__ __align__(16) uint16_t sgh[16 * kMaxRB][kTC + 8];  // (s.g)^T hi: [j][t]
    __shared__ __align__(16) uint16_t sgl[16 * kMaxRB][kTC + 8];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int k0 = blockIdx.x * 64;
    const int rb_n = (r + 15) / 16;
    const int jr = 16 * rb_n;
    for (int o = tid; o < jr * kTC; o += kThreads) {
        sgh[o / kTC][o % kTC] = 0;
        sgl[o / kTC][o % kTC] = 0;
    }
    f32x4 acc[kMaxRB];
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kof = 8 * (lane >> 4);

    for (int t0 = 0; t0 < T; t0 += kTC) {
        __syncthreads();
        {
            const int t = tid >> 3, k8 = (tid & 7) * 8;
            const bool ok = (t0 + t < T) && (k0 + k8 < K);
            const u32x4 v = ok ? ld16(x + size_t(t0 + t) * K + k0 + k8) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = v[e >> 1];
                sxT[k8 + e][t] = uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF));
            }
        }
        for (int o = tid; o < kTC * r; o += kThreads) {
            const int t = o / r, j = o % r;
            const float v = (t0 + t < T) ? s * g[size_t(t0 + t) * r + j] : 0.0f;
            __bf16 h, l;
            split_bf16(v, h, l);
            sgh[j][t] = __builtin_bit_cast(uint16_t, h);
            sgl[j][t] = __builtin_bit_cast(uint16_t, l);
        }
        __syncthreads();
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
#pragma unroll
    for (int b = 0; b < kMaxRB; ++b) {
        if (b < rb_n) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 16 * b + 4 * (lane >> 4) + e, k = k0 + 16 * wave + (lane & 15);
                if (j < r && k < K) dA[size_t(j) * K + k] = acc[b][e];
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
    hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(count, 64))), dim3(kThreads), 0, stream, upart, splits,
                       count, count, u);
    return hipGetLastError();
}

hipError_t launch_lora_bwd_pre(const BwdPlan& p, const uint16_t* dy, const uint16_t* B, const float* u, int64_t T,
                               int64_t N, int r, float s, float* dB, void* ws, hipStream_t stream) {
    float* g = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_g);
    float* gpart = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_gpart);
    hipLaunchKernelGGL(k_lora_bwd_pre, dim3(unsigned(p.nslab)), dim3(kThreads), 0, stream, dy, B, u, int(T), int(N),
                       r, s, dB, gpart);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t count = T * r;
    hipLaunchKernelGGL(k_sum_parts, dim3(unsigned(cdiv(count, 64))), dim3(kThreads), 0, stream, gpart,
                       p.nslab, count, count, g);
    return hipGetLastError();
}

hipError_t launch_lora_da(const BwdPlan& p, const uint16_t* x, int64_t T, int64_t K, int r, float s, float* dA,
                          void* ws, hipStream_t stream) {
    const float* g = reinterpret_cast<const float*>(static_cast<char*>(ws) + p.off_g);
    hipLaunchKernelGGL(k_lora_da, dim3(unsigned(cdiv(K, 64))), dim3(kThreads), 0, stream, g, x, int(T), int(K), r,
                       s, dA);
    return hipGetLastError();
}

}  // namespace nf4
