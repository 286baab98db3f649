// Workgroup roles of the LoRA backward pre-pass (Poros API reference,
// "PorosTrainer.from_pretrained": lora_rank, lora_alpha; adapters are the only
// trainable parameters):
//   g  = dY . B         [T, r] fp32, as partials over N ranges
//   dB = s . dY^T . u   [N, r] fp32, complete
// Device functions for 256-thread workgroups, shared by the stand-alone pre-pass
// kernel and the few-token backward kernel, which runs them beside its dX workgroups.
#pragma once
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {
namespace pre {

constexpr int kThreads = 256;

// Two kinds of workgroups:
//  - g role: 32 tokens x one N range (part p); per 128-feature
//    chunk the B rows are staged transposed in LDS ([j][n], double-buffered, loads
//    one chunk ahead) and each wave contracts 16 tokens x 64 features straight from
//    dY in registers; the two waves of a token half add up in fixed order -> gpart[p].
//  - dB role: 64 features x a token range in DBT-token sub-chunks (dY
//    transposed and (s.u) hi/lo staged in LDS, loads one sub-chunk ahead) -> dB, or
//    this range's share of dB (the shares are added in range order after the dX
//    GEMM); with many tokens the sub-chunks are long (kDbTLong) so that few of them
//    (one memory round trip each) run in sequence.
constexpr int kTC = 32;         // tokens per g workgroup; dB sub-chunk for few tokens
constexpr int kDbTLong = 128;   // dB sub-chunk for many tokens
constexpr int kGChunk = 128;    // features per g chunk

template <int RB>
struct GSmem {
    uint16_t bt[2][16 * RB][kGChunk + 8];
    float red[4][RB][64][4];
};
template <int RB, int DBT>
struct DbSmem {
    uint16_t dyt[64][DBT + 8];       // [n][t]
    uint16_t uh[16 * RB][DBT + 8];   // (s.u)^T hi [j][t]
    uint16_t ul[16 * RB][DBT + 8];   // lo
};

// GRING chunks of loads in flight (1 or 2; 2 where the registers allow it)
template <int RB, int GRING>
__device__ void g_role(const uint16_t* __restrict__ dy, const uint16_t* __restrict__ B, int T, int N, int r,
                       int steps_per_part, int blk, float* __restrict__ gpart, GSmem<RB>& sm) {
    static_assert(GRING == 1 || GRING == 2, "one or two chunks in flight");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tblocks = (T + kTC - 1) / kTC;
    const int t0 = (blk % tblocks) * kTC, part = blk / tblocks;
    const int c_begin = part * steps_per_part;
    const int c_end = min(c_begin + steps_per_part, (N + kGChunk - 1) / kGChunk);
    const int th = wave & 1, nh = wave >> 1;  // token half, feature half of a chunk
    const auto rdy = make_rsrc(dy + size_t(t0) * N, uint32_t(max(0, min(kTC, T - t0))) * uint32_t(N) * 2u);
    const auto rb = make_rsrc(B, uint32_t(N) * uint32_t(r) * 2u);  // rows n >= N read as zero
    const uint32_t dyrow = uint32_t(16 * th + (lane & 15)) * uint32_t(N) * 2u;
    const int kof = 8 * (lane >> 4);
    constexpr int BV = kGChunk * 16 * RB / kThreads;  // B values per thread per chunk

    // B values of a chunk: with r % 4 == 0 thread (f, q) = (tid % 64, tid / 64) loads
    // ranks 4 RB q .. 4 RB q + 4 RB - 1 of features 2f and 2f + 1 as 8-byte pieces and
    // stores them as 4-byte feature pairs of B^T; otherwise one bf16 per load and store.
    // Ranks past r read the next row's values or zero: they only reach g columns that
    // are never written.
    static_assert(BV == 8 * RB, "8 RB B values per thread per chunk");
    const bool vec = (r & 3) == 0;
    const int bf = tid & 63, bq = tid >> 6;
    struct Set {
        u32x2 bp[BV / 2];  // vector path: 2 RB pieces of 4 ranks; scalar path: one bf16 per dword
        u32x4 dv[2];
    };
    Set ring[GRING];
    auto gload = [&](int c, Set& st) {
        u32x2(&bp)[BV / 2] = st.bp;
        u32x4(&dv)[2] = st.dv;
        const int n0 = c * kGChunk;
        if (vec) {
#pragma unroll
            for (int i = 0; i < 2 * RB; ++i) {  // piece i: feature 2 bf + (i & 1), ranks 4 RB bq + 4 (i / 2)
                const int n = n0 + 2 * bf + (i & 1), j = 4 * RB * bq + 4 * (i >> 1);
                bp[i] = buf_load8(rb, j < r ? (uint32_t(n) * uint32_t(r) + uint32_t(j)) * 2u : kOutOfRange);
            }
        } else {
#pragma unroll
            for (int i = 0; i < BV; ++i) {
                const int o = tid + kThreads * i;  // o = n * 16 RB + j
                const int n = o / (16 * RB), j = o % (16 * RB);
                bp[i >> 1][i & 1] = __builtin_amdgcn_raw_buffer_load_b16(
                    rb, int(j < r ? (uint32_t(n0 + n) * uint32_t(r) + uint32_t(j)) * 2u : kOutOfRange), 0, 0);
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int n = n0 + 64 * nh + 32 * kk + kof;
            dv[kk] = buf_load16(rdy, n < N ? dyrow + uint32_t(n) * 2u : kOutOfRange);
        }
    };
    auto bstore = [&](int buf, const Set& st) {
        const u32x2(&bp)[BV / 2] = st.bp;
        if (vec) {
            // piece 2 i + f (rank quad i, feature 2 bf + f) holds ranks j, j + 1 in its
            // first dword and j + 2, j + 3 in its second, j = 4 RB bq + 4 i
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = bp[2 * i][e >> 1], hi = bp[2 * i + 1][e >> 1];
                    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                    *reinterpret_cast<uint32_t*>(&sm.bt[buf][4 * RB * bq + 4 * i + e][2 * bf]) =
                        __builtin_amdgcn_perm(hi, lo, sel);
                }
            return;
        }
#pragma unroll
        for (int i = 0; i < BV; ++i) {
            const int o = tid + kThreads * i;
            sm.bt[buf][o % (16 * RB)][o / (16 * RB)] = uint16_t(bp[i >> 1][i & 1]);
        }
    };

    f32x4 acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c_begin < c_end) {
#pragma unroll
        for (int i = 0; i < GRING; ++i) gload(c_begin + i, ring[i]);  // past the range: unused data or zeros
        bstore(0, ring[0]);
        __syncthreads();
        // chunk c sits in ring slot S = (c - c_begin) % GRING (compile-time: the loop is
        // unrolled by GRING); its loads are replaced by those of chunk c + GRING, and the
        // next chunk's B^T (slot (S + 1) % GRING) goes to the other LDS buffer
        auto step = [&](int c, auto s_) {
            constexpr int S = decltype(s_)::value;
            const int buf = (c - c_begin) & 1;
            const u32x4 d0 = ring[S].dv[0], d1 = ring[S].dv[1];
            gload(c + GRING, ring[S]);
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const uint16_t* row = &sm.bt[buf][16 * b + (lane & 15)][64 * nh + kof];
                acc[b] = mfma16x16x32(as_bf16x8(d0), as_bf16x8(*reinterpret_cast<const u32x4*>(row)), acc[b]);
                acc[b] = mfma16x16x32(as_bf16x8(d1), as_bf16x8(*reinterpret_cast<const u32x4*>(row + 32)), acc[b]);
            }
            bstore(buf ^ 1, ring[(S + 1) % GRING]);
            __syncthreads();
        };
        int c = c_begin;
        if constexpr (GRING == 2) {
            for (; c + 1 < c_end; c += 2) {
                step(c, std::integral_constant<int, 0>{});
                step(c + 1, std::integral_constant<int, 1>{});
            }
            if (c < c_end) step(c, std::integral_constant<int, 0>{});
        } else {
            for (; c < c_end; ++c) step(c, std::integral_constant<int, 0>{});
        }
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.red[wave][b][lane][e] = acc[b][e];
    __syncthreads();
    float* dst = gpart + size_t(part) * T * r;
    for (int o = tid; o < kTC * r; o += kThreads) {
        const int t = o / r, j = o % r;
        const int h = t >> 4, tt = t & 15;
        const int b = j >> 4, l = 16 * (tt >> 2) + (j & 15), e = tt & 3;
        // waves h (features 0-63 of each chunk) and h + 2 (64-127), in that order
        const float v = sm.red[h][b][l][e] + sm.red[h + 2][b][l][e];
        if (t0 + t < T) dst[size_t(t0 + t) * r + j] = v;
    }
}

// tokens [t_begin, t_end) of features 64 blk .. 64 blk + 63 -> dst [N][r]
template <int RB, int DBT>
__device__ void db_role(const uint16_t* __restrict__ dy, const float* __restrict__ u, int T, int N, int r, float s,
                        int blk, int t_begin, int t_end, float* __restrict__ dst, DbSmem<RB, DBT>& sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n0 = blk * 64;
    // dY: 16-byte pieces of tokens DV lt .. DV lt + DV - 1, features ln8 .. ln8 + 7 per
    // thread, transposed in registers (byte permutes pairing tokens) into [n][t] rows
    const int lt = tid >> 3, ln8 = (tid & 7) * 8;
    constexpr int DV = DBT / 32;                   // dY pieces per thread per sub-chunk
    constexpr int UV = DBT * 16 * RB / kThreads;   // u values per thread per sub-chunk
    static_assert(DV == 1 || DV % 2 == 0, "dY pieces: one, or token pairs");
    static_assert(UV % 2 == 0, "u values: token pairs");
    // u: pair q of the thread is rank (tid + kThreads q) % 16 RB of tokens 2 tp, 2 tp + 1,
    // tp = (tid + kThreads q) / 16 RB

    u32x4 vdy[DV];
    float uv[UV];
    // the descriptors cover one sub-chunk (at most DBT rows of dY and u): their byte
    // sizes and offsets stay far inside 32 bits for any token count
    auto gload = [&](int t0) {
        const uint32_t rows = uint32_t(max(0, min(DBT, t_end - t0)));
        const auto rdy = make_rsrc(dy + size_t(t0) * N, rows * uint32_t(N) * 2u);
        const auto ru = make_rsrc(u + size_t(t0) * r, rows * uint32_t(r) * 4u);
#pragma unroll
        for (int i = 0; i < DV; ++i) {
            const int t = DV * lt + i;
            const bool ok = t0 + t < t_end && n0 + ln8 < N;
            vdy[i] = buf_load16(rdy, ok ? (uint32_t(t) * uint32_t(N) + uint32_t(n0 + ln8)) * 2u : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < UV; ++i) {
            const int o = tid + kThreads * (i >> 1), j = o % (16 * RB), tp = o / (16 * RB);
            const int t = 2 * tp + (i & 1);
            uv[i] = buf_load_f32(ru, (t0 + t < t_end && j < r) ? (uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u
                                                               : kOutOfRange);
        }
    };
    auto sstore = [&]() {
        if constexpr (DV == 1) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t w = vdy[0][e >> 1];
                sm.dyt[ln8 + e][lt] = uint16_t((e & 1) ? (w >> 16) : (w & 0xFFFF));
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // element e of tokens 2p, 2p + 1: low halves (e even) or high halves (e odd)
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                uint32_t col[DV / 2];
#pragma unroll
                for (int p = 0; p < DV / 2; ++p)
                    col[p] = __builtin_amdgcn_perm(vdy[2 * p + 1][e >> 1], vdy[2 * p][e >> 1], sel);
                if constexpr (DV == 4)
                    *reinterpret_cast<u32x2*>(&sm.dyt[ln8 + e][DV * lt]) = u32x2{col[0], col[1]};
                else
#pragma unroll
                    for (int p = 0; p < DV / 2; ++p)
                        *reinterpret_cast<uint32_t*>(&sm.dyt[ln8 + e][DV * lt + 2 * p]) = col[p];
            }
        }
        // (s.u)^T hi / lo as bf16 token pairs
#pragma unroll
        for (int q = 0; q < UV / 2; ++q) {
            const int o = tid + kThreads * q, j = o % (16 * RB), tp = o / (16 * RB);
            __bf16 h0, l0, h1, l1;
            split_bf16(s * uv[2 * q], h0, l0);
            split_bf16(s * uv[2 * q + 1], h1, l1);
            *reinterpret_cast<uint32_t*>(&sm.uh[j][2 * tp]) =
                uint32_t(__builtin_bit_cast(uint16_t, h0)) | (uint32_t(__builtin_bit_cast(uint16_t, h1)) << 16);
            *reinterpret_cast<uint32_t*>(&sm.ul[j][2 * tp]) =
                uint32_t(__builtin_bit_cast(uint16_t, l0)) | (uint32_t(__builtin_bit_cast(uint16_t, l1)) << 16);
        }
    };
    f32x4 acc[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int kof = 8 * (lane >> 4);
    gload(t_begin);
    for (int t0 = t_begin; t0 < t_end; t0 += DBT) {
        __syncthreads();  // the previous sub-chunk's reads are done
        sstore();
        __syncthreads();
        gload(t0 + DBT);  // past the end: zeros
#pragma unroll
        for (int kk = 0; kk < DBT / 32; ++kk) {  // tokens in increasing order
            const bf16x8 a =
                as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.dyt[16 * wave + (lane & 15)][32 * kk + kof]));
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                const bf16x8 bh = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.uh[16 * b + (lane & 15)][32 * kk + kof]));
                const bf16x8 bl = as_bf16x8(*reinterpret_cast<const u32x4*>(&sm.ul[16 * b + (lane & 15)][32 * kk + kof]));
                acc[b] = mfma16x16x32(a, bh, acc[b]);
                acc[b] = mfma16x16x32(a, bl, acc[b]);
            }
        }
    }
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int n = n0 + 16 * wave + 4 * (lane >> 4) + e, j = 16 * b + (lane & 15);
            if (n < N && j < r) dst[size_t(n) * r + j] = acc[b][e];
        }
}

template <int RB, int DBT>
union PreSmem {
    GSmem<RB> g;
    DbSmem<RB, DBT> d;
};

}  // namespace pre
}  // namespace nf4
