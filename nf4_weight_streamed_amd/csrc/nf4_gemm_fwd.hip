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
//  - split-K, for shapes with too few tiles to fill 256 CUs (every tile) or with a
//    last, partial round of tiles (those tiles only): fp32 partial tiles in the
//    caller's workspace (piece 0 carries the LoRA term), added in piece order and
//    rounded once by k_split_sum_bf16 (a kernel boundary, not in-kernel signalling:
//    the per-XCD L2 caches are only made coherent by whole-cache maintenance).
// The same kernel, with kDense, takes a dense bf16 base instead (the experimental
// dense-bf16 streaming mode of the Poros API reference, "PorosTrainer.from_pretrained"
// quantization "bf16_bitwise"): each lane then loads its 32 weights of a K step as four
// 16-byte pieces, already in MFMA fragment order, and nothing is dequantised.
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBK = 64;        // K per main-loop step (= one NF4 block)
constexpr int kLds = kBK + 8;  // LDS row pitch in bf16 (144 B: conflict-free 16 B fragment reads)
constexpr int kFwdWaves = 4;   // waves per workgroup (each 128 tokens x 128 / kFwdWaves features)
constexpr int kFwdXAhead = 1;  // K steps x is loaded ahead of its use (register sets)
constexpr int kFwdWAhead = 2;  // K steps the weights are loaded ahead of their dequantisation
constexpr int kFwdOccupancy = 3;  // waves per SIMD the register budget must allow (3 tiles per CU)
constexpr int64_t kCUs = kChipCUs;

// ------------------------------------------------------------------------------------
// NW waves split the BN = 128 output features (128 / NW each, FN = 4 / NW fragments of
// 32); every wave dequantises its own weight fragments in registers, so no weight tile
// goes through LDS and each weight element is dequantised once per workgroup. Each x
// fragment read from LDS feeds FN MFMAs, so fewer, wider waves read less LDS per MAC.
// Within each 64-element K block the contraction order is permuted identically for
// both operands: lane half h supplies k = 32h + 8kk .. 32h + 8kk + 7 at sub-step kk, so
// one 16-byte code load per lane and fragment covers the four sub-steps of a K step.
// A code byte indexes a 256-entry LDS table of (level[low nibble], level[high nibble])
// pairs: one 8-byte read, two fp32 multiplies by the block's absmax and one bf16 pack
// per byte. Loads are raw buffer loads (hardware zero outside the tensor); codes are
// fetched two K steps ahead, x one step ahead; the x tile is double-buffered in LDS
// with one barrier per K step.
struct FwdLora {
    const float* upart;  // [parts][T][r] partials of u = x.A^T
    int parts;
    float* u_save;       // [T][r] the summed u, written by the column-0 tiles
    const uint16_t* B;   // [N][r]
    int r;
    float s;
};

// Which tile (and K range) each workgroup of the 1-D grid takes: ids 0 .. full-1 are
// whole tiles, the rest pieces of the last `tail` tiles, piece z of tile full + q at
// id full + z * tail + q. Both ranges are laid over the XCDs separately (full is 0
// or a multiple of 256), so every XCD gets the same share of whole tiles and pieces.
struct FwdTiles {
    int full, tail, pieces, steps_per_piece;
    int mtiles;  // token tiles (tile index = token tile + mtiles * column tile)
    int bal_a, bal_pa;  // balanced split of all tiles (balanced_piece), 0: off
};

template <int NW, bool kDense>
__global__ __launch_bounds__(64 * NW, kFwdOccupancy) void k_nf4_gemm_fwd(
    const uint16_t* __restrict__ x, const void* __restrict__ weights, const float* __restrict__ absmax, int T,
    int N, int K, FwdTiles tl, FwdLora lora, uint16_t* __restrict__ y, float* __restrict__ partial, Tables tab) {
    constexpr int NT = 64 * NW;
    constexpr int BM = 128, BN = 128, FM = 4, FN = 4 / NW;
    constexpr int A_CHUNKS = BM * (kBK / 8) / NT;

    __shared__ __align__(16) uint16_t sA[2][BM * kLds];
    __shared__ __align__(16) float sLut[512];  // 256 (level[lo nibble], level[hi nibble]) pairs

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    // tile order: token tile fastest, then column tile (then piece); per-XCD ranges,
    // so the token tiles sharing one weight slice run together in one L2
    const int ksteps = K / kBK;
    int tile, tz = 0, kb_begin = 0, kb_end = ksteps;
    float* ptile = nullptr;  // fp32 partial tile of a split tile
    if (int(blockIdx.x) < tl.full) {
        tile = int(xcd_tile_order(blockIdx.x, uint32_t(tl.full)));
    } else if (tl.bal_a > 0) {
        int q;
        balanced_piece(blockIdx.x - uint32_t(tl.full), uint32_t(kCUs), tl.tail, tl.bal_a, tl.bal_pa, ksteps, q, tz,
                       kb_begin, kb_end);
        tile = tl.full + q;
        ptile = partial + (size_t(tz) * tl.tail + q) * (BM * BN);
    } else {
        const int u = int(xcd_tile_order(blockIdx.x - uint32_t(tl.full), uint32_t(tl.tail * tl.pieces)));
        const int q = u % tl.tail;
        tz = u / tl.tail;
        tile = tl.full + q;
        kb_begin = tz * tl.steps_per_piece;
        kb_end = min(kb_begin + tl.steps_per_piece, ksteps);
        ptile = partial + (size_t(tz) * tl.tail + q) * (BM * BN);
    }
    const int tm = tile % tl.mtiles, tc = tile / tl.mtiles;
    const int n0 = tc * BN;
    const int m0 = tm * BM;
    const int frag_row = lane & 31;
    const int half = lane >> 5;
    for (int i = tid; i < 256; i += NT) {  // entry b: the two codes of byte b
        sLut[2 * i] = tab.level[i & 15];
        sLut[2 * i + 1] = tab.level[i >> 4];
    }

    // buffer views of this workgroup's rows (offsets stay far below 2^31)
    const uint32_t xrows = uint32_t(max(0, min(BM, T - m0)));
    const uint32_t wrows = uint32_t(max(0, min(BN, N - n0)));
    const auto rx = make_rsrc(x + size_t(m0) * K, xrows * uint32_t(K) * 2u);
    // weight operand: NF4 codes (0.5 B / weight) + scales, or dense bf16 (2 B / weight)
    constexpr uint32_t kWBytesPerStep = kDense ? kBK * 2 : kBK / 2;  // per row and K step
    const auto rcd = make_rsrc(static_cast<const uint8_t*>(weights) + size_t(n0) * kWBytesPerStep * (K / kBK),
                               wrows * uint32_t(K / kBK) * kWBytesPerStep);
    const auto rsc = make_rsrc(kDense ? nullptr : absmax + size_t(n0) * (K / 64), kDense ? 0u : wrows * uint32_t(K / 64) * 4u);
    uint32_t c_off[FN], s_off[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int wrow = 32 * (FN * wave + j) + frag_row;  // this lane's weight row of fragment j
        c_off[j] = uint32_t(wrow) * uint32_t(K / kBK) * kWBytesPerStep + uint32_t(half) * (kWBytesPerStep / 2);
        s_off[j] = uint32_t(wrow) * uint32_t(K / 64) * 4u;
    }
    uint32_t x_off[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + NT * i;
        x_off[i] = (uint32_t(c >> 3) * uint32_t(K) + uint32_t(c & 7) * 8u) * 2u;
    }

    constexpr int WP = kDense ? 4 : 1;  // 16-byte weight pieces per lane, fragment and K step
    // register rings: x of a step is loaded PX steps ahead (PX sets), the weights PW steps
    // ahead (PW sets); one tile alone on a CU is bound by these loads' latency
    constexpr int PX = kDense ? 1 : kFwdXAhead, PW = kDense ? 2 : kFwdWAhead;  // dense: 4x the weight registers
    constexpr int U = (PX > PW ? PX : PW) > 2 ? 4 : 2;  // loop unroll: a multiple of 2, PX and PW
    static_assert(U % PX == 0 && U % PW == 0, "ring sizes must divide the unroll");
    u32x4 ra[PX][A_CHUNKS];
    u32x4 rc[PW][FN][WP];
    float rs[PW][FN];
    auto gload_x = [&](int kb, u32x4 (&xa)[A_CHUNKS]) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) xa[i] = buf_load16(rx, x_off[i] + uint32_t(kb) * (kBK * 2));
    };
    auto gload_w = [&](int kb, u32x4 (&cw)[FN][WP], float (&sc)[FN]) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int q = 0; q < WP; ++q) cw[j][q] = buf_load16(rcd, c_off[j] + uint32_t(kb) * kWBytesPerStep + 16u * q);
            if constexpr (!kDense) sc[j] = buf_load_f32(rsc, s_off[j] + uint32_t(kb) * 4u);
        }
    };
    auto store_x = [&](const u32x4 (&xa)[A_CHUNKS], int buf) {
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + NT * i;
            *reinterpret_cast<u32x4*>(&sA[buf][(c >> 3) * kLds + (c & 7) * 8]) = xa[i];
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    // weight fragments of the current step; sub-step q of the next step is dequantised
    // into wf[.][q] right after the MFMAs of sub-step q have read it (only its final
    // packs wait for those MFMAs: the table reads and multiplies can run under them)
    bf16x8 wf[FN][4];
    // weight fragments of sub-step q (all FN fragments) from a register set
    auto dequant_q = [&](const u32x4 (&cw)[FN][WP], const float (&sc)[FN], int q, bf16x8 (&wo)[FN][4]) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            if constexpr (kDense) {
                wo[j][q] = as_bf16x8(cw[j][q]);
                continue;
            }
            const uint32_t w = cw[j][0][q];
            u32x4 o;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const float2 lv = *reinterpret_cast<const float2*>(lut + (((w >> (8 * b)) & 0xFFu) << 3));
                // level * absmax in fp32, then RNbf: the format's two roundings
                o[b] = pack_bf16x2(lv.x * sc[j], lv.y * sc[j]);
            }
            wo[j][q] = as_bf16x8(o);
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    if (kb_begin < kb_end) {
#pragma unroll
        for (int i = 0; i < PX; ++i) gload_x(kb_begin + i, ra[i]);
#pragma unroll
        for (int i = 0; i < PW; ++i) gload_w(kb_begin + i, rc[i], rs[i]);
        store_x(ra[0], 0);
        __syncthreads();  // sLut and x tile 0 visible
#pragma unroll
        for (int q = 0; q < 4; ++q) dequant_q(rc[0], rs[0], q, wf);
        // one K step; C = (kb - kb_begin) mod U at compile time (the loop is unrolled by U
        // so that no register array is indexed at run time): LDS buffer C mod 2, x set C mod PX, weight set C mod PW. The body has no branch, so the
        // scheduler can interleave the next step's dequantisation with the MFMAs: loads,
        // the next step's dequantisation and its x store are all unconditional (a step
        // past the end reads data that is never used, or zeros beyond the buffer, and
        // writes the idle LDS buffer); with a fixed issue pattern the compiler's wait
        // counts also stay exact and never drain later loads.
        auto step = [&](int kb, auto c_) {
            constexpr int C = decltype(c_)::value;
            gload_x(kb + PX, ra[C % PX]);               // that set was stored into LDS last step
            // x first: the x store at the end of the step waits on the in-order load
            // counter, which must not also drain the weights loaded PW steps ahead
            __builtin_amdgcn_sched_barrier(0);
            gload_w(kb + PW, rc[C % PW], rs[C % PW]);   // that set is this step's, already dequantised
            // keep the loads here, ahead of the MFMAs: sinking them next to their use
            // would expose their full latency
            __builtin_amdgcn_sched_barrier(0);
            const uint16_t* a_base = &sA[C & 1][0];
            // x fragments one sub-step ahead in two register sets (the reads of sub-step
            // kk + 1 are in the program before the MFMAs of kk: 1-3% faster than reading
            // each fragment next to its MFMA; fencing the reads off with a scheduling
            // barrier was slower)
            bf16x8 afs[2][FM];
            auto read_af = [&](int kk, bf16x8 (&af)[FM]) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    af[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(a_base + (32 * i + frag_row) * kLds + 32 * half + 8 * kk));
            };
            read_af(0, afs[0]);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                if (kk + 1 < 4) read_af(kk + 1, afs[(kk + 1) & 1]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16(afs[kk & 1][i], wf[j][kk], acc[i][j]);
                // sub-step kk of the next step's weights, independent of the MFMAs
                dequant_q(rc[(C + 1) % PW], rs[(C + 1) % PW], kk, wf);
            }
            // interleave the fragment and table reads, multiplies and MFMAs of the step
            // (the scheduler's small-GEMM strategy keeps several LDS reads in flight under
            // the MFMAs; without it each read waits for the previous one). NF4 only: the
            // dense variant's larger weight registers would spill under it.
            if constexpr (!kDense) __builtin_amdgcn_iglp_opt(0);
            store_x(ra[(C + 1) % PX], (C + 1) & 1);
            __syncthreads();
        };
        int kb = kb_begin;
        if constexpr (U == 4) {
            for (; kb + 3 < kb_end; kb += 4) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
                step(kb + 2, std::integral_constant<int, 2>{});
                step(kb + 3, std::integral_constant<int, 3>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
            if (kb + 1 < kb_end) step(kb + 1, std::integral_constant<int, 1>{});
            if (kb + 2 < kb_end) step(kb + 2, std::integral_constant<int, 2>{});
        } else {
            for (; kb + 1 < kb_end; kb += 2) {
                step(kb, std::integral_constant<int, 0>{});
                step(kb + 1, std::integral_constant<int, 1>{});
            }
            if (kb < kb_end) step(kb, std::integral_constant<int, 0>{});
        }
    }

    // LoRA as a K-extension (split 0 only when split): acc += (s.u)_hi . B^T + (s.u)_lo . B^T.
    // u = sum of the partials in partial order, staged as bf16 hi/lo [t][j] in the (now
    // free) x buffers; the column-0 tiles also store it as u_save. B rows past N and
    // entries j >= r load from beyond the buffers (zero).
    const int r = lora.r;
    if (tz == 0 && r > 0) {
        uint16_t* su_hi = &sA[0][0];
        uint16_t* su_lo = &sA[1][0];
        const int rp = (r + 15) & ~15;
        // one descriptor per partial over this tile's rows, so sizes and offsets stay
        // small for any token count; 12 bytes of slack keep the last 16-byte load (4-byte
        // aligned, lanes j >= r masked below) inside it, and inside the allocation: the
        // partials region is padded to 256 bytes
        const uint32_t ubytes = uint32_t(max(0, min(BM, T - m0))) * uint32_t(r) * 4u + 12u;
        auto upart_rsrc = [&](int p) {
            return make_rsrc(lora.upart + (size_t(min(p, lora.parts - 1)) * T + m0) * r, ubytes);
        };
        const auto rb = make_rsrc(lora.B, uint32_t(N) * uint32_t(r) * 2u);
        const bool write_u = tc == 0;
        // B values of one 16-rank slice for this lane's fragments (lane: column n, ranks
        // c0 + 8 (lane / 32) .. + 7): one 16-byte load when rows are 16-byte multiples
        auto load_b = [&](int c0, u32x4 (&bv)[FN]) {
            const int jr = c0 + 8 * half;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const uint32_t col = uint32_t(n0 + 32 * (FN * wave + j) + frag_row);
                if (r % 8 == 0) {
                    bv[j] = buf_load16(rb, jr < r ? (col * uint32_t(r) + uint32_t(jr)) * 2u : kOutOfRange);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        h[e] = __builtin_amdgcn_raw_buffer_load_b16(
                            rb, int(jr + e < r ? (col * uint32_t(r) + uint32_t(jr + e)) * 2u : kOutOfRange), 0, 0);
                    bv[j] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                }
            }
        };
        u32x4 bv[FN];
        load_b(0, bv);
        // s.u staged as bf16 hi/lo [t][j]: items of 4 ranks, every load issued first
        constexpr int UI = BM * 4 / NT;  // (t, 4-rank group) items per thread per 16 ranks
        constexpr int UR = 4;  // partials loaded per round
        for (int jb = 0; jb < rp / 16; ++jb) {
            f32x4 usum[UI];
#pragma unroll
            for (int i = 0; i < UI; ++i) usum[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int p0 = 0; p0 < lora.parts; p0 += UR) {  // partials in partial order
                f32x4 pv[UI][UR];
                __amdgpu_buffer_rsrc_t rup[UR];
#pragma unroll
                for (int pp = 0; pp < UR; ++pp) rup[pp] = upart_rsrc(p0 + pp);
#pragma unroll
                for (int i = 0; i < UI; ++i) {
                    const int o = tid + NT * i, t = o / 4, j = 16 * jb + 4 * (o % 4);
                    const bool ok = m0 + t < T && j < r;
                    const uint32_t off = (uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u;
#pragma unroll
                    for (int pp = 0; pp < UR; ++pp)
                        pv[i][pp] = __builtin_bit_cast(
                            f32x4, buf_load16(rup[pp], ok && p0 + pp < lora.parts ? off : kOutOfRange));
                }
#pragma unroll
                for (int i = 0; i < UI; ++i)
#pragma unroll
                    for (int pp = 0; pp < UR; ++pp)
                        if (p0 + pp < lora.parts) usum[i] += pv[i][pp];
            }
#pragma unroll
            for (int i = 0; i < UI; ++i) {
                const int o = tid + NT * i, t = o / 4, j = 16 * jb + 4 * (o % 4);
                const f32x4 v = usum[i];
                uint16_t hb[4], lb[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float vc = j + c < r ? v[c] : 0.0f;
                    if (write_u && m0 + t < T && j + c < r) lora.u_save[size_t(m0 + t) * r + j + c] = vc;
                    __bf16 hh, ll;
                    split_bf16(lora.s * vc, hh, ll);
                    hb[c] = __builtin_bit_cast(uint16_t, hh);
                    lb[c] = __builtin_bit_cast(uint16_t, ll);
                }
                *reinterpret_cast<u32x2*>(&su_hi[t * kLds + j]) = u32x2{hb[0] | (uint32_t(hb[1]) << 16), hb[2] | (uint32_t(hb[3]) << 16)};
                *reinterpret_cast<u32x2*>(&su_lo[t * kLds + j]) = u32x2{lb[0] | (uint32_t(lb[1]) << 16), lb[2] | (uint32_t(lb[3]) << 16)};
            }
        }
        __syncthreads();
        for (int c0 = 0; c0 < r; c0 += 16) {
            const int j0 = c0 + 8 * half;
            if (c0 > 0) load_b(c0, bv);
            bf16x8 bb[FN];
#pragma unroll
            for (int j = 0; j < FN; ++j) bb[j] = as_bf16x8(bv[j]);
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int t = 32 * i + frag_row;
                const bf16x8 hi = as_bf16x8(*reinterpret_cast<const u32x4*>(&su_hi[t * kLds + j0]));
                const bf16x8 lo = as_bf16x8(*reinterpret_cast<const u32x4*>(&su_lo[t * kLds + j0]));
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    acc[i][j] = mfma32x32x16(hi, bb[j], acc[i][j]);
                    acc[i][j] = mfma32x32x16(lo, bb[j], acc[i][j]);
                }
            }
        }
    }

    if (!ptile) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int col = n0 + 32 * (FN * wave + j) + frag_row;
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int row = m0 + 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
                    if (row < T && col < N) y[size_t(row) * N + col] = bf16_bits(acc[i][j][e]);
                }
        }
        return;
    }

    // a piece of a split tile: its fp32 tile [BM][BN], rows below T and columns below N
    // only (the rest is never read); k_split_sum_bf16 adds the pieces in order
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        const int col = 32 * (FN * wave + j) + frag_row;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = 32 * i + 8 * (e >> 2) + 4 * half + (e & 3);
                if (m0 + row < T && n0 + col < N) ptile[row * BN + col] = acc[i][j][e];
            }
    }
}

// y = RNbf(((p0 + p1) + p2) + ...) of each split tile: its pieces' fp32 tiles added in
// piece order (piece 0 holds the LoRA term), rounded once; four consecutive outputs
// per thread.
struct SplitTiles {
    const float* part;  // [pieces][tail][BM * BN]
    int full, tail, pieces, mtiles, bm, bn;
    int T, N;
    int bal_a, bal_pa;  // balanced split: tiles below bal_a have bal_pa pieces
};

__global__ __launch_bounds__(256) void k_split_sum_bf16(SplitTiles f, uint16_t* __restrict__ out) {
    const int tile_elems = f.bm * f.bn;
    const int64_t total = int64_t(f.tail) * tile_elems;
    const int64_t idx = (int64_t(blockIdx.x) * 256 + threadIdx.x) * 4;
    if (idx >= total) return;
    const int q = int(idx / tile_elems), loc = int(idx % tile_elems);
    const int tile = f.full + q;
    const int row = (tile % f.mtiles) * f.bm + loc / f.bn, col = (tile / f.mtiles) * f.bn + loc % f.bn;
    if (row >= f.T || col >= f.N) return;  // N % 16 == 0: the four columns are all in or all out
    f32x4 a = *reinterpret_cast<const f32x4*>(f.part + idx);
    const int np = q < f.bal_a ? f.bal_pa : f.pieces;
    for (int z = 1; z < np; ++z) a += *reinterpret_cast<const f32x4*>(f.part + z * total + idx);
    const u32x2 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
    *reinterpret_cast<u32x2*>(out + size_t(row) * f.N + col) = o;
}

}  // namespace

FwdPlan plan_fwd(int64_t T, int64_t N, int64_t K, int r, bool dense) {
    FwdPlan p{};
    if ((T <= kSkinnyFwdT || (T <= kSkinnyFwdLongT && K >= kSkinnyLongK && N <= kSkinnyNarrowN)) && !dense) {
        p.skinny = true;
        p.sk = plan_skinny_fwd(T, N, K, r);
        p.ws_bytes = p.sk.ws_bytes;
        return p;
    }
    p.bm = 128;
    p.bn = 128;
    p.mtiles = int(cdiv(T, p.bm));
    const int64_t tiles = int64_t(p.mtiles) * cdiv(N, p.bn);
    const int64_t ksteps = K / kBK;
    // Under 256 tiles: every tile split (about 512 workgroups in all). Many: whole rounds
    // of 256 tiles (one more per CU each) run whole, and a last round of at most 128
    // tiles is split into pieces that spread over the CUs: the time of a CU grows with
    // the tiles it holds, so 2 whole tiles + a third of one beat 3 whole tiles.
    int64_t tail = 0, pieces = 1, bal_a = 0, bal_pa = 0;
    const int64_t splits = pick_splits(tiles, ksteps, 4);
    if (pick_balanced(tiles, ksteps, 4, kCUs, bal_a, bal_pa)) {
        tail = tiles;
        pieces = bal_pa + 1;
    } else if (splits > 1) {
        tail = tiles;
        pieces = splits;
    } else if (tiles > kCUs) {
        const int64_t last = tiles % kCUs;
        const int64_t pc = pick_tail_pieces(last, ksteps / 4, kCUs);
        if (pc >= 2) {
            tail = last;
            pieces = pc;
        }
    }
    p.steps_per_piece = int(cdiv(ksteps, pieces));
    p.pieces = tail > 0 ? int(cdiv(ksteps, p.steps_per_piece)) : 1;
    p.bal_a = int(bal_a);
    p.bal_pa = int(bal_pa);
    if (bal_a > 0) {  // piece bounds come from balanced_piece; the slot count is bal_pa + 1
        p.pieces = int(pieces);
        p.steps_per_piece = 0;
    }
    p.tail = int(tail);
    p.full = int(tiles - tail);  // 0 or a multiple of kCUs (a multiple of the XCD count)
    if (r > 0) plan_lora_down(p, K);
    size_t off = 0;
    p.off_upart = off;
    off += align256(size_t(p.down_parts) * size_t(T) * size_t(r) * 4);
    p.off_ypart = off;
    off += p.tail > 0 ? align256(size_t(p.pieces) * size_t(p.tail) * size_t(p.bm) * size_t(p.bn) * 4) : 0;
    p.ws_bytes = off;
    return p;
}

hipError_t launch_gemm_fwd(const FwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* wdense,
                           const uint16_t* x, const uint16_t* B, int64_t T, int64_t N, int64_t K, int r, float s,
                           uint16_t* y, float* u_save, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    const FwdTiles tl{p.full, p.tail, p.pieces, p.steps_per_piece, p.mtiles, p.bal_a, p.bal_pa};
    const dim3 grid(unsigned(p.full + (p.bal_a > 0 ? 2 * kCUs : int64_t(p.tail) * p.pieces)));
    float* partial = p.tail > 0 ? reinterpret_cast<float*>(w + p.off_ypart) : nullptr;
    const FwdLora lora{r > 0 ? reinterpret_cast<const float*>(w + p.off_upart) : nullptr, p.down_parts, u_save, B,
                       r, s};
    prof_gemm_begin(stream);
    if (wdense)
        hipLaunchKernelGGL((k_nf4_gemm_fwd<kFwdWaves, true>), grid, dim3(64 * kFwdWaves), 0, stream, x,
                           static_cast<const void*>(wdense), nullptr, int(T), int(N), int(K), tl, lora, y, partial,
                           tables());
    else
        hipLaunchKernelGGL((k_nf4_gemm_fwd<kFwdWaves, false>), grid, dim3(64 * kFwdWaves), 0, stream, x,
                           static_cast<const void*>(codes), absmax, int(T), int(N), int(K), tl, lora, y, partial,
                           tables());
    prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.tail == 0) return e;
    const SplitTiles f{partial, p.full, p.tail, p.pieces, p.mtiles, p.bm, p.bn, int(T), int(N), p.bal_a, p.bal_pa};
    const int64_t total = int64_t(p.tail) * p.bm * p.bn;
    hipLaunchKernelGGL(k_split_sum_bf16, dim3(unsigned(cdiv(total / 4, 256))), dim3(256), 0, stream, f, y);
    return hipGetLastError();
}

}  // namespace nf4
