// Fused NF4-dequantise + bf16 MFMA GEMM with the LoRA side path in its epilogue (forward).
//
//   y = RNbf( x . W^T + s . u . B^T ),  W = dequantised NF4 base [N, K], u = x . A^T [T, r]
//
// The frozen base is only read (HN comment thread on streaming the frozen base,
// main comment) and is NF4 with rank-r LoRA on top (Poros API reference,
// "PorosTrainer.from_pretrained"). Design for gfx950:
//  - workgroup tile 128 tokens x 128 out-features, 4 waves side by side along the
//    out-features (128 x 32 each) on v_mfma_f32_32x32x16_bf16 with fp32 accumulators;
//  - each K step covers one 64-element NF4 block, so every weight row has one scale;
//  - weights are dequantised by the wave that multiplies them, in registers (see the
//    kernel comment), while the x tile goes through double-buffered LDS;
//  - LoRA: (s.u) is split into bf16 hi + lo and contracted with B on the same
//    accumulators (a K-extension of r per part), so y is rounded once;
//  - split-K (for shapes with too few tiles to fill 256 CUs): fp32 partials in the
//    caller's workspace (split 0 carries the LoRA term), summed in a fixed order
//    and rounded once by k_split_sum_bf16.
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBK = 64;        // K per main-loop step (= one NF4 block)
constexpr int kLds = kBK + 8;  // LDS row pitch in bf16 (144 B: conflict-free 16 B fragment reads)
constexpr int kThreads = 256;

// ------------------------------------------------------------------------------------
// 4 waves split the BN = 128 output features (32 each); every wave dequantises its own
// weight fragments in registers, so no weight tile goes through LDS and each weight
// element is dequantised once per workgroup. Within each 64-element K block the
// contraction order is permuted identically for both operands: lane half h supplies
// k = 32h + 8kk .. 32h + 8kk + 7 at sub-step kk, so one 16-byte code load per lane
// covers the four sub-steps of a K step. A code byte indexes a 256-entry LDS table of
// (level[low nibble], level[high nibble]) pairs: one 8-byte read, two fp32 multiplies
// by the block's absmax and one bf16 pack per byte. Loads are raw buffer loads
// (hardware zero outside the tensor); x and codes are fetched two K steps ahead; the
// x tile is double-buffered in LDS with one barrier per K step.
__global__ __launch_bounds__(kThreads, 2) void k_nf4_gemm_fwd(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ codes, const float* __restrict__ absmax,
    const float* __restrict__ u, const uint16_t* __restrict__ B, int T, int N, int K, int r, float s,
    int steps_per_split, uint16_t* __restrict__ y, float* __restrict__ partial, Tables tab) {
    constexpr int BM = 128, BN = 128, FM = 4;
    constexpr int A_CHUNKS = BM * (kBK / 8) / kThreads;  // 4

    __shared__ __align__(16) uint16_t sA[2][BM * kLds];
    __shared__ __align__(16) float sLut[512];  // 256 (level[lo nibble], level[hi nibble]) pairs

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int n0 = blockIdx.x * BN;
    const int m0 = blockIdx.y * BM;
    const int ksteps = K / kBK;
    const int kb_begin = blockIdx.z * steps_per_split;
    const int kb_end = min(kb_begin + steps_per_split, ksteps);
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    sLut[2 * tid] = tab.level[tid & 15];  // entry b: the two codes of byte b
    sLut[2 * tid + 1] = tab.level[tid >> 4];

    // buffer views of this workgroup's rows (offsets stay far below 2^31)
    const uint32_t xrows = uint32_t(max(0, min(BM, T - m0)));
    const uint32_t wrows = uint32_t(max(0, min(BN, N - n0)));
    const auto rx = make_rsrc(x + size_t(m0) * K, xrows * uint32_t(K) * 2u);
    const auto rcd = make_rsrc(codes + size_t(n0) * (K / 2), wrows * uint32_t(K / 2));
    const auto rsc = make_rsrc(absmax + size_t(n0) * (K / 64), wrows * uint32_t(K / 64) * 4u);
    const int wrow = 32 * wave + frag_row;  // this lane's weight row within the tile
    const uint32_t c_off = uint32_t(wrow) * uint32_t(K / 2) + uint32_t(half) * 16u;
    const uint32_t s_off = uint32_t(wrow) * uint32_t(K / 64) * 4u;
    uint32_t x_off[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + kThreads * i;
        x_off[i] = (uint32_t(c >> 3) * uint32_t(K) + uint32_t(c & 7) * 8u) * 2u;
    }

    u32x4 ra[2][A_CHUNKS];
    u32x4 rc[2];
    float rs[2];
    auto gload = [&](int kb, u32x4 (&xa)[A_CHUNKS], u32x4& cw, float& sc) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) xa[i] = buf_load16(rx, x_off[i] + uint32_t(kb) * (kBK * 2));
        cw = buf_load16(rcd, c_off + uint32_t(kb) * 32u);
        sc = buf_load_f32(rsc, s_off + uint32_t(kb) * 4u);
    };
    auto store_x = [&](const u32x4 (&xa)[A_CHUNKS], int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + kThreads * i;
            *reinterpret_cast<u32x4*>(&sA[buf][(c >> 3) * kLds + (c & 7) * 8]) = xa[i];
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    auto dequant = [&](const u32x4& cw, float sc, bf16x8 (&wf)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w = cw[q];
            u32x4 o;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float2 lv = *reinterpret_cast<const float2*>(lut + (((w >> (8 * b)) & 0xFFu) << 3));
                // level * absmax in fp32, then RNbf: the format's two roundings
                o[b] = pack_bf16x2(lv.x * sc, lv.y * sc);
            }
            wf[q] = as_bf16x8(o);
        }
    };

    f32x16 acc[FM];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][e] = 0.0f;

    if (kb_begin < kb_end) {
        bf16x8 wf[4];
        gload(kb_begin, ra[0], rc[0], rs[0]);
        if (kb_begin + 1 < kb_end) gload(kb_begin + 1, ra[1], rc[1], rs[1]);
        store_x(ra[0], 0);
        __syncthreads();  // sLut and x tile 0 visible
        dequant(rc[0], rs[0], wf);
        // one K step; C is the compile-time register/LDS buffer of step kb (the loop is
        // unrolled by two so that no register array is indexed at run time)
        auto step = [&](int kb, auto c_) {
            constexpr int C = decltype(c_)::value;
            const bool more = kb + 1 < kb_end;
            if (kb + 2 < kb_end) gload(kb + 2, ra[C], rc[C], rs[C]);  // step kb's registers are consumed
            const uint16_t* a_base = &sA[C][0];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const bf16x8 af = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        a_base + (32 * i + frag_row) * kLds + 32 * half + 8 * kk));
                    acc[i] = mfma32x32x16(af, wf[kk], acc[i]);
                }
            }
            if (more) {
                dequant(rc[C ^ 1], rs[C ^ 1], wf);  // next step's weights, independent of the MFMAs
                store_x(ra[C ^ 1], C ^ 1);
            }
            __syncthreads();
        };
        for (int kb = kb_begin; kb < kb_end; kb += 2) {
            step(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < kb_end) step(kb + 1, std::integral_constant<int, 1>{});
        }
    }

    // LoRA as a K-extension (split 0 only when split): acc += (s.u)_hi . B^T + (s.u)_lo . B^T
    const int col = n0 + 32 * wave + frag_row;
    for (int c0 = 0; c0 < (blockIdx.z == 0 ? r : 0); c0 += 16) {
        bf16x8 bb;
        const int j0 = c0 + 8 * half;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t bv = (col < N && j0 + e < r) ? B[size_t(col) * r + j0 + e] : uint16_t(0);
            bb[e] = __builtin_bit_cast(__bf16, bv);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int row = m0 + 32 * i + frag_row;
            bf16x8 hi, lo;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float v = (row < T && j0 + e < r) ? s * u[size_t(row) * r + j0 + e] : 0.0f;
                __bf16 hh, ll;
                split_bf16(v, hh, ll);
                hi[e] = hh;
                lo[e] = ll;
            }
            acc[i] = mfma32x32x16(hi, bb, acc[i]);
            acc[i] = mfma32x32x16(lo, bb, acc[i]);
        }
    }

    float* pdst = partial ? partial + size_t(blockIdx.z) * T * N : nullptr;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int row = m0 + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
            if (row < T && col < N) {
                if (pdst)
                    pdst[size_t(row) * N + col] = acc[i][e];
                else
                    y[size_t(row) * N + col] = bf16_bits(acc[i][e]);
            }
        }
}

// y = RNbf( sum_z partial[z] ), z in increasing order (split 0 already holds the LoRA
// term); four consecutive outputs per thread, float4 loads.
__global__ __launch_bounds__(256) void k_split_sum_bf16(const float* __restrict__ partial, int splits,
                                                        int64_t total, uint16_t* __restrict__ out) {
    const int64_t idx = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (idx >= total) return;
    f32x4 acc = *reinterpret_cast<const f32x4*>(partial + idx);
    for (int z = 1; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(partial + size_t(z) * total + idx);
    u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(out + idx) = o;
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
    hipLaunchKernelGGL(k_nf4_gemm_fwd, grid, dim3(kThreads), 0, stream, x, codes, absmax, u, B, int(T), int(N), int(K),
                       r, s, p.steps_per_split, y, partial, tables());
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    const int64_t total = T * N;
    hipLaunchKernelGGL(k_split_sum_bf16, dim3(unsigned(cdiv(total / 4, 256))), dim3(256), 0, stream, partial,
                       p.splits, total, y);
    return hipGetLastError();
}

}  // namespace nf4
