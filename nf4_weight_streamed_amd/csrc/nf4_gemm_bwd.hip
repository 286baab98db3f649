// Fused NF4-dequantise + bf16 MFMA GEMM for the input gradient of the LoRA linear.
//
//   dX = RNbf( dY . W + s . g . A ),  g = dY . B  (fp32, from the LoRA pre-pass)
//
// The base is frozen: only dX flows through it and no weight gradient is formed
// (Poros API reference, "patch_hf_model" Behavior 3; HN comment thread on
// streaming the frozen base, main comment). The contraction runs over N, the
// rows of W, while the codes are contiguous along K: each thread dequantises a
// 4 (n) x 8 (k) patch and packs bf16 pairs across rows, so the tile lands in LDS
// as [k][n] and the MFMA B operand is again a contiguous 16-byte read. Its rows are
// 160 bytes apart and their 16-byte chunks XOR-swizzled by (k / 16) % 8: measured on
// the MI355X's 64-bank LDS, the fragment reads (16 aligned rows share one swizzle)
// are then conflict-free and the 8-byte transposed stores as cheap as any layout
// measured (the former 144-byte pitch with a (k / 8) % 8 swizzle cost 2.6 times the
// conflict-free time per fragment read). The dY tile keeps 144-byte rows without a
// swizzle, conflict-free for its fragment reads. With kDense the base is
// dense bf16 (the experimental "bf16_bitwise" streaming mode of the Poros API
// reference, "PorosTrainer.from_pretrained"): the patch is four 16-byte row pieces,
// paired across rows the same way, with nothing to dequantise.
#include <type_traits>

#include "common.h"
#include "device.h"

namespace nf4 {

namespace {

constexpr int kBN = 64;        // contraction (N) per main-loop step
constexpr int kLds = kBN + 8;    // LDS pitch of the dY tile in bf16 (144 bytes)
constexpr int kLdsW = kBN + 16;  // LDS pitch of the weight tile in bf16 (160 bytes)
constexpr int64_t kCUs = kChipCUs;

// Workgroup tile: BM (128 or 256) tokens x 128 input features, BM / 32 waves in a
// (BM / 64) x 2 grid (64 x 64 each, 32x32x16 MFMA), contraction steps of 64 over N.
// With 256 tokens the eight waves share one weight tile, so each weight is
// dequantised and stored to LDS once per 256 tokens instead of 128: waves 0-3
// dequantise it (the same 256-thread patch layout), waves 4-7 only stage dY and keep
// the matrix cores busy meanwhile (measured about 8% faster than spreading 4 x 4
// patches over all eight waves); the main loop is compiled once per role, so each
// keeps exact wait counts. Per step each thread loads
// (raw buffer loads, hardware zero outside the tensors) a 4 (n) x 8 (k) patch of
// codes with the 4 row scales (weight waves) and 4 16-byte chunks of the dY tile, two
// steps ahead
// into a ring of two register sets. dY and the weight tile are double-buffered in
// LDS: during the MFMAs of step s each thread dequantises its patch of step s + 1 -
// one 8-byte read of a 256-entry (level[lo], level[hi]) pair table per code byte,
// fp32 multiply by the row's absmax, bf16 pack pairing rows - and stores it
// transposed, with its dY chunks, into the other buffer; one barrier per step. The
// step has no branch, so the scheduler interleaves the dequantisation with the
// MFMAs. LDS block 78 KB with 128 tokens (shared with the LoRA epilogue): two
// workgroups per CU; 132 KB with 256 tokens: one.

// Which tile (and contraction range) each workgroup of the 1-D grid takes: ids
// 0 .. full-1 are whole tiles, the rest pieces of the last `tail` tiles, piece z of
// tile full + q at id full + z * tail + q. Both ranges are laid over the XCDs
// separately (full is a multiple of the XCD count), so every XCD gets the same share
// of whole tiles and of pieces.
struct BwdTiles {
    int full, tail, pieces, steps_per_piece;
    int mtiles;  // token tiles (tile index = token tile + mtiles * column tile)
    int bal_a, bal_pa;  // balanced split of all tiles (balanced_piece), 0: off
};

struct BwdLora {
    const float* gpart;  // [parts][T][r] partials of g = dY.B
    int parts;
    const uint16_t* A;   // [r][K]
    const uint16_t* x;   // [T][K]
    float* dapart;       // [token tiles][r][K] dA share of each token tile
    int r;
    float s;
};

template <int BM, bool kDense>
__global__ __launch_bounds__(2 * BM, BM == 128 ? 2 : 1) void k_nf4_gemm_bwd_dx(
    const uint16_t* __restrict__ dy, const void* __restrict__ weights, const float* __restrict__ absmax, int T,
    int N, int K, BwdTiles tl, BwdLora lora, uint16_t* __restrict__ dx, float* __restrict__ partial, Tables tab) {
    static_assert(BM == 128 || BM == 256, "128 or 256 tokens per tile");
    static_assert(!kDense || BM == 128, "the dense base runs 128-token tiles");
    constexpr int NT = 2 * BM;  // threads: BM / 32 waves
    constexpr int BK = 128;
    constexpr int WM = 64, WK = 64;
    constexpr int FM = WM / 32, FK = WK / 32;
    constexpr int A_CHUNKS = BM * (kBN / 8) / NT;  // 4
    static_assert(A_CHUNKS == 4, "four 16-byte dY chunks per thread and step");

    // One LDS block. Main loop: two buffers of (dY tile, weight tile) and the pair
    // table; LoRA epilogue: (s.g)^T hi/lo for up to 64 ranks and the x tile transposed
    // (one 64-column half at a time with 128 tokens, all 128 columns with 256).
    constexpr int kTP = BM + 8;  // pitch of the epilogue's [.][t] tiles
    constexpr int kXHalves = BM == 256 ? 1 : 2;
    constexpr int kXCols = BK / kXHalves;         // x columns staged at once
    constexpr int kBuf = BM * kLds + BK * kLdsW;  // one buffer: dY tile, then weight tile
    constexpr int kMain = 2 * kBuf + 2 * 512;
    constexpr int kEpi = (2 * 64 + kXCols) * kTP;
    __shared__ __align__(16) uint16_t smem[kMain > kEpi ? kMain : kEpi];
    float* const sLut = reinterpret_cast<float*>(smem + 2 * kBuf);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wk = wave & 1;
    // tile order: token tile fastest, then column tile (then piece); per-XCD ranges, so
    // the token tiles sharing one weight slice run together in one L2. Without dX
    // (dx == NULL) only the LoRA part runs: no contraction steps.
    const int nsteps = dx ? (N + kBN - 1) / kBN : 0;
    int tile, tz = 0, nb_begin = 0, nb_end = nsteps;
    float* ptile = nullptr;  // fp32 partial tile of a split tile
    if (int(blockIdx.x) < tl.full) {
        tile = int(xcd_tile_order(blockIdx.x, uint32_t(tl.full)));
    } else if (tl.bal_a > 0) {
        int q;
        balanced_piece(blockIdx.x - uint32_t(tl.full), uint32_t(kCUs), tl.tail, tl.bal_a, tl.bal_pa, nsteps, q, tz,
                       nb_begin, nb_end);
        tile = tl.full + q;
        ptile = partial + (size_t(tz) * tl.tail + q) * (BM * BK);
    } else {
        const int u = int(xcd_tile_order(blockIdx.x - uint32_t(tl.full), uint32_t(tl.tail * tl.pieces)));
        const int q = u % tl.tail;
        tz = u / tl.tail;
        tile = tl.full + q;
        nb_begin = tz * tl.steps_per_piece;
        nb_end = min(nb_begin + tl.steps_per_piece, nsteps);
        ptile = partial + (size_t(tz) * tl.tail + q) * (BM * BK);
    }
    const int tm = tile % tl.mtiles, tc = tile / tl.mtiles;
    const int k0 = tc * BK;
    const int m0 = tm * BM;
    const int frag_row = lane & 31;
    const int frag_k = (lane >> 5) * 8;
    if (tid < 256) {
        sLut[2 * tid] = tab.level[tid & 15];  // entry b: the two codes of byte b
        sLut[2 * tid + 1] = tab.level[tid >> 4];
    }

    // this thread's patch (threads 0-255, the weight waves): rows 4*pr .. 4*pr+3 of the
    // step, columns 8*pc .. 8*pc+7 of the tile
    const int pr = (tid & 255) >> 4, pc = tid & 15;
    const uint32_t trows = uint32_t(max(0, min(BM, T - m0)));
    const auto rdy = make_rsrc(dy + size_t(m0) * N, trows * uint32_t(N) * 2u);
    // codes/absmax of the whole matrix (the entry points keep N*K/2 below 2^30 bytes);
    // patches beyond N or K load from kOutOfRange and read as zero
    // dense bf16: N*K*2 bytes (the entry points keep N*K <= 2^30)
    const auto rcd = make_rsrc(weights, uint32_t(N) * uint32_t(K) * (kDense ? 2u : 1u) / (kDense ? 1u : 2u));
    const auto rsc = make_rsrc(kDense ? nullptr : absmax, kDense ? 0u : uint32_t(N) * uint32_t(K / 64) * 4u);
    const uint32_t kc = uint32_t(k0 + 8 * pc);
    uint32_t a_off[A_CHUNKS];
#pragma unroll
    for (int i = 0; i < A_CHUNKS; ++i) {
        const int c = tid + NT * i;
        a_off[i] = (uint32_t(c >> 3) * uint32_t(N) + uint32_t(c & 7) * 8u) * 2u;
    }

    struct LSet {             // one step's loads
        u32x4 ra[A_CHUNKS];   // dY chunks
        uint32_t rc[4];       // NF4: 8 codes of each patch row
        float rs[4];          //      and its scale
        u32x4 rw[4];          // dense: 8 bf16 of each patch row
    };
    // kW (compile time): this wave loads and dequantises the weight patch too
    auto gload = [&](int nb, LSet& l, auto w_) {
        constexpr bool kW = decltype(w_)::value;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            // dY columns at or beyond N (ragged last step, steps past the end) read as zero
            const bool ok = nb * kBN + 8 * ((tid + NT * i) & 7) < N;
            l.ra[i] = buf_load16(rdy, ok ? a_off[i] + uint32_t(nb) * (kBN * 2) : kOutOfRange);
        }
        if constexpr (!kW) return;
        // Rows n >= N lie past the end of both buffers and read as zero (scale 0, so
        // the dequantised row is zero). Columns k >= K of a ragged tile read the next
        // row's data: they only reach dX columns that are never stored.
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t n = uint32_t(nb * kBN + 4 * pr + i);
            if constexpr (kDense) {
                l.rw[i] = buf_load16(rcd, (n * uint32_t(K) + kc) * 2u);
            } else {
                l.rc[i] = buf_load_u32(rcd, n * uint32_t(K / 2) + kc / 2);
                l.rs[i] = buf_load_f32(rsc, n * uint32_t(K / 64) * 4u + (kc / 64) * 4u);
            }
        }
    };
    const char* lut = reinterpret_cast<const char*>(sLut);
    // one step's tiles into LDS buffer b
    auto sstore = [&](const LSet& l, int b, auto w_) {
        constexpr bool kW = decltype(w_)::value;
        uint16_t* const sA = smem + b * kBuf;
        uint16_t* const sWt = sA + BM * kLds;
#pragma unroll
        for (int i = 0; i < A_CHUNKS; ++i) {
            const int c = tid + NT * i;
            *reinterpret_cast<u32x4*>(&sA[(c >> 3) * kLds + (c & 7) * 8]) = l.ra[i];
        }
        if constexpr (!kW) return;
        // row k = 8*pc + e holds n = 4*pr .. 4*pr+3: chunk pr/2, swizzled by k / 16 = pc / 2,
        // half pr&1
        const int col = (((pr >> 1) ^ ((pc >> 1) & 7)) << 3) + 4 * (pr & 1);
        if constexpr (kDense) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int sh = 16 * (e & 1);
                auto bits = [&](int i) { return (l.rw[i][e >> 1] >> sh) & 0xFFFFu; };
                const u32x2 o = {bits(0) | (bits(1) << 16), bits(2) | (bits(3) << 16)};
                *reinterpret_cast<u32x2*>(&sWt[(8 * pc + e) * kLdsW + col]) = o;
            }
            return;
        }
        float v[4][8];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float2 lv = *reinterpret_cast<const float2*>(lut + (((l.rc[i] >> (8 * q)) & 0xFFu) << 3));
                // level * absmax in fp32, then RNbf (below): the format's two roundings
                v[i][2 * q] = lv.x * l.rs[i];
                v[i][2 * q + 1] = lv.y * l.rs[i];
            }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            u32x2 o = {pack_bf16x2(v[0][e], v[1][e]), pack_bf16x2(v[2][e], v[3][e])};
            *reinterpret_cast<u32x2*>(&sWt[(8 * pc + e) * kLdsW + col]) = o;
        }
    };

    f32x16 acc[FM][FK];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    auto main_loop = [&](auto w_) {
        LSet ld[2];
        gload(nb_begin, ld[0], w_);
        gload(nb_begin + 1, ld[1], w_);
        __syncthreads();  // sLut visible
        sstore(ld[0], 0, w_);
        __syncthreads();
        // Step nb, C = (nb - nb_begin) mod 2 at compile time (the loop is unrolled by 2,
        // so no register array is indexed at run time): MFMAs on LDS buffer C, loads of
        // step nb + 2 into register set C (stored into LDS last step), and the tiles of
        // step nb + 1 from set C ^ 1 into buffer C ^ 1, which every wave finished
        // reading before the previous step's barrier. Loads and stores are
        // unconditional (a step past the end reads zeros or data that is never used and
        // writes the idle buffer), so the body has no branch and the compiler's wait
        // counts stay exact: the store waits for set C ^ 1 only, leaving the newest
        // loads in flight.
        auto step = [&](int nb, auto c_) {
            constexpr int C = decltype(c_)::value;
            gload(nb + 2, ld[C], w_);
            __builtin_amdgcn_sched_barrier(0);  // keep the loads ahead of the MFMAs
            const uint16_t* const sA = smem + C * kBuf;
            const uint16_t* const sWt = sA + BM * kLds;
            // fragments one sub-step ahead in two register sets (the reads of kk + 1 come
            // before the MFMAs of kk in the program: gate backward 2%, down 3% faster in
            // the layer step)
            bf16x8 af[2][FM], bw[2][FK];
            auto read_frags = [&](int kk, bf16x8 (&a)[FM], bf16x8 (&b)[FK]) {
#pragma unroll
                for (int i = 0; i < FM; ++i)
                    a[i] = as_bf16x8(*reinterpret_cast<const u32x4*>(
                        &sA[(wm * WM + 32 * i + frag_row) * kLds + kk * 16 + frag_k]));
#pragma unroll
                for (int j = 0; j < FK; ++j) {
                    const int row = wk * WK + 32 * j + frag_row;
                    const int chunk = (2 * kk + (lane >> 5)) ^ ((row >> 4) & 7);
                    b[j] = as_bf16x8(*reinterpret_cast<const u32x4*>(&sWt[row * kLdsW + chunk * 8]));
                }
            };
            read_frags(0, af[0], bw[0]);
#pragma unroll
            for (int kk = 0; kk < kBN / 16; ++kk) {
                if (kk + 1 < kBN / 16) read_frags(kk + 1, af[(kk + 1) & 1], bw[(kk + 1) & 1]);
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FK; ++j) acc[i][j] = mfma32x32x16(af[kk & 1][i], bw[kk & 1][j], acc[i][j]);
            }
            sstore(ld[C ^ 1], C ^ 1, w_);  // the next step's tiles
            // interleave the table reads, multiplies and stores with the MFMAs (the
            // scheduler's small-GEMM strategy). NF4 only: the dense variant has no
            // dequantisation to hide.
            if constexpr (!kDense) __builtin_amdgcn_iglp_opt(0);
            __syncthreads();  // this step's reads and the next step's stores are done
        };
        int nb = nb_begin;
        for (; nb + 1 < nb_end; nb += 2) {
            step(nb, std::integral_constant<int, 0>{});
            step(nb + 1, std::integral_constant<int, 1>{});
        }
        if (nb < nb_end) step(nb, std::integral_constant<int, 0>{});
    };
    if (nb_begin < nb_end) {
        // both roles run the same steps, so every wave meets the same barriers
        if (BM == 128 || wave < 4)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});
    }

    // LoRA (whole tiles and piece 0 of split tiles). g = sum of the partials in partial
    // order; (s.g)^T is staged as bf16 hi/lo [j][t] and the x tile as [k][t], one
    // 64-column half at a time, in the (now free) LDS block. Then
    //   dX tile += (s.g)_hi . A + (s.g)_lo . A      (K-extension on the accumulators)
    //   dA share of this token tile = (s.g)^T . x over its tokens (k_bwd_finish adds
    //   the shares in token-tile order: dA = ((d0 + d1) + d2) + ...)
    const int r = lora.r;
    if (tz == 0 && r > 0) {
        // without contraction steps (no dX, or an empty piece) no barrier has run since
        // the pair-table fill, which shares bytes with the epilogue's tiles
        if (nb_begin >= nb_end) __syncthreads();
        uint16_t* const sg_hi = smem;             // [64][kTP]
        uint16_t* const sg_lo = smem + 64 * kTP;  // [64][kTP]
        uint16_t* const sxt = smem + 128 * kTP;   // [BK / 2][kTP]
        const int rp = (r + 15) & ~15;
        // one descriptor per partial over this tile's rows, so sizes and offsets stay
        // small for any token count; 12 bytes of slack keep the last 16-byte load (4-byte
        // aligned, lanes j >= r masked below) inside it, and inside the allocation: the
        // partials region is padded to 256 bytes
        const uint32_t gbytes = trows * uint32_t(r) * 4u + 12u;
        auto gpart_rsrc = [&](int p) {
            return make_rsrc(lora.gpart + (size_t(min(p, lora.parts - 1)) * T + m0) * r, gbytes);
        };
        const auto rx = make_rsrc(lora.x + size_t(m0) * K, trows * uint32_t(K) * 2u);
        // every load of the staging is issued before the first is consumed (one memory
        // round trip at the end of the kernel, not one per loop trip)
        constexpr int XC = BM * (BK / 8) / NT;  // 16-byte x chunks per thread
        constexpr int GI = BM * 4 / NT;         // (t, 4-rank group) items per thread per 16 ranks
        const auto ra = make_rsrc(lora.A, uint32_t(r) * uint32_t(K) * 2u);  // rows j >= r read zero
        // A values of one 16-rank slice for this lane's dX fragments: B operand of the
        // LoRA K-extension (lane: column k, ranks c0 + 8 (lane / 32) .. + 7)
        auto load_a = [&](int c0, uint32_t (&av)[FK][8]) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
#pragma unroll
                for (int j = 0; j < FK; ++j) {
                    const uint32_t col = uint32_t(k0 + wk * WK + 32 * j + frag_row);
                    av[j][e] = __builtin_amdgcn_raw_buffer_load_b16(
                        ra, int(col < uint32_t(K) ? (uint32_t(c0 + frag_k + e) * uint32_t(K) + col) * 2u : kOutOfRange),
                        0, 0);
                }
        };
        uint32_t av[FK][8];
        load_a(0, av);
        // this thread's x chunks: 8 consecutive tokens xt0 .. xt0+7 of columns xk8 .. xk8+7
        static_assert(XC == 8 && BM == 8 * (NT / 16) && BK == 16 * 8, "x tile: chunk blocks of 8 x 8, 16 across");
        const int xk8 = 8 * (tid & 15), xt0 = 8 * (tid >> 4);
        u32x4 xv[XC];
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            // rows past T read zero; columns past K only feed dA columns never stored
            xv[i] = buf_load16(rx, (uint32_t(xt0 + i) * uint32_t(K) + uint32_t(k0 + xk8)) * 2u);
        }
        constexpr int GR = 8;  // partials loaded per round (registers are free after the main loop)
        for (int jb = 0; jb < rp / 16; ++jb) {
            f32x4 gsum[GI];
#pragma unroll
            for (int i = 0; i < GI; ++i) gsum[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int p0 = 0; p0 < lora.parts; p0 += GR) {  // partials in partial order
                f32x4 pv[GI][GR];
                __amdgpu_buffer_rsrc_t rgp[GR];
#pragma unroll
                for (int pp = 0; pp < GR; ++pp) rgp[pp] = gpart_rsrc(p0 + pp);
#pragma unroll
                for (int i = 0; i < GI; ++i) {
                    const int o = tid + NT * i, t = o / 4, j = 16 * jb + 4 * (o % 4);
                    const bool ok = m0 + t < T && j < r;
                    const uint32_t off = (uint32_t(t) * uint32_t(r) + uint32_t(j)) * 4u;
#pragma unroll
                    for (int pp = 0; pp < GR; ++pp)
                        pv[i][pp] = __builtin_bit_cast(
                            f32x4, buf_load16(rgp[pp], ok && p0 + pp < lora.parts ? off : kOutOfRange));
                }
#pragma unroll
                for (int i = 0; i < GI; ++i)
#pragma unroll
                    for (int pp = 0; pp < GR; ++pp)
                        if (p0 + pp < lora.parts) gsum[i] += pv[i][pp];
            }
#pragma unroll
            for (int i = 0; i < GI; ++i) {
                const int o = tid + NT * i, t = o / 4, j = 16 * jb + 4 * (o % 4);
                const f32x4 v = gsum[i];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    __bf16 hh, ll;
                    split_bf16(j + c < r ? lora.s * v[c] : 0.0f, hh, ll);
                    sg_hi[(j + c) * kTP + t] = __builtin_bit_cast(uint16_t, hh);
                    sg_lo[(j + c) * kTP + t] = __builtin_bit_cast(uint16_t, ll);
                }
            }
        }
        // x^T of columns kXCols h .. kXCols (h + 1) - 1 (with two halves a thread's chunks
        // all sit in one, their column offset being 8 (tid % 16)); the 8 x 8 block is
        // transposed in registers (byte permutes pairing tokens) and written as one
        // 16-byte row piece per column
        auto stage_x = [&](int h) {
            if (kXHalves == 2 && ((tid & 15) >> 3) != h) return;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                // element e of chunks i and i + 1: low halves (e even) or high halves (e odd)
                const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
                u32x4 col;
#pragma unroll
                for (int p = 0; p < 4; ++p)
                    col[p] = __builtin_amdgcn_perm(xv[2 * p + 1][e >> 1], xv[2 * p][e >> 1], sel);
                *reinterpret_cast<u32x4*>(&sxt[(xk8 - kXCols * h + e) * kTP + xt0]) = col;
            }
        };
        stage_x(0);
        __syncthreads();

        if (dx) {
            for (int c0 = 0; c0 < r; c0 += 16) {
                const int j0 = c0 + frag_k;
                if (c0 > 0) load_a(c0, av);
                bf16x8 hi[FM], lo[FM], aa[FK];
#pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int t = wm * WM + 32 * i + frag_row;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        hi[i][e] = __builtin_bit_cast(__bf16, sg_hi[(j0 + e) * kTP + t]);
                        lo[i][e] = __builtin_bit_cast(__bf16, sg_lo[(j0 + e) * kTP + t]);
                    }
                }
#pragma unroll
                for (int j = 0; j < FK; ++j)
#pragma unroll
                    for (int e = 0; e < 8; ++e) aa[j][e] = __builtin_bit_cast(__bf16, uint16_t(av[j][e]));
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FK; ++j) {
                        acc[i][j] = mfma32x32x16(hi[i], aa[j], acc[i][j]);
                        acc[i][j] = mfma32x32x16(lo[i], aa[j], acc[i][j]);
                    }
            }
        }

        // dA share of this token tile: D[k][j] over t, 16x16x32 MFMAs; per staged group
        // of kXCols columns, wave w owns the K sub-block w (16 columns)
        static_assert(kXCols == 16 * (NT / 64), "one 16-column K sub-block per wave");
        const int l16 = lane & 15, t8 = 8 * (lane >> 4);
        float* dpart = lora.dapart + size_t(tm) * r * K;
        for (int h = 0; h < kXHalves; ++h) {
            if (h > 0) {
                __syncthreads();  // the first half's reads are done
                stage_x(h);
                __syncthreads();
            }
            for (int jb = 0; jb < rp / 16; ++jb) {
                f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ts = 0; ts < BM / 32; ++ts) {
                    const int tt = 32 * ts + t8;
                    const bf16x8 xa = as_bf16x8(*reinterpret_cast<const u32x4*>(&sxt[(16 * wave + l16) * kTP + tt]));
                    const bf16x8 gh = as_bf16x8(*reinterpret_cast<const u32x4*>(&sg_hi[(16 * jb + l16) * kTP + tt]));
                    const bf16x8 gl = as_bf16x8(*reinterpret_cast<const u32x4*>(&sg_lo[(16 * jb + l16) * kTP + tt]));
                    d = mfma16x16x32(xa, gh, d);
                    d = mfma16x16x32(xa, gl, d);
                }
                // lane holds D[k = 64 h + 16 wave + 4 (lane / 16) + e][j = 16 jb + lane % 16]
                const int j = 16 * jb + l16, kq = k0 + kXCols * h + 16 * wave + 4 * (lane >> 4);
                if (j < r && kq < K) *reinterpret_cast<f32x4*>(&dpart[size_t(j) * K + kq]) = d;
            }
        }
    }

    if (!dx) return;
    if (!ptile) {
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
        return;
    }

    // a piece of a split tile: its fp32 tile [BM][BK], rows below T only (few tokens
    // leave most rows empty; columns past K are written but never read); k_bwd_finish
    // adds the pieces in order
    const int rlim = T - m0;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FK; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int row = wm * WM + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int col = wk * WK + 32 * j + (lane & 31);
                if (row < rlim) ptile[row * BK + col] = acc[i][j][e];
            }
}

// The backward's reductions, in one launch: blocks [0, dx_blocks) form
// dX = RNbf(((p0 + p1) + p2) + ...) of the split tiles from their pieces' fp32 tiles;
// the next da_blocks form dA = ((d0 + d1) + d2) + ... from the token tiles' shares and
// the rest dB from its token ranges' shares, in the same way. Four outputs per thread.
struct BwdFinishDx {
    const float* part;  // [pieces][tail][BM * BK]
    int full, tail, pieces, mtiles, bm, bk;
    int T, K;
    int bal_a, bal_pa;  // balanced split: tiles below bal_a have bal_pa pieces
};
struct Shares {  // dst[i] = ((src[0][i] + src[1][i]) + src[2][i]) + ...
    const float* src;
    int count;
    int64_t total;
    float* dst;
};

__device__ __forceinline__ void sum_shares(const Shares& sh, int64_t block) {
    const int64_t idx = (block * 256 + threadIdx.x) * 4;
    if (idx >= sh.total) return;
    f32x4 a = *reinterpret_cast<const f32x4*>(sh.src + idx);
    for (int z = 1; z < sh.count; ++z) a += *reinterpret_cast<const f32x4*>(sh.src + size_t(z) * sh.total + idx);
    *reinterpret_cast<f32x4*>(sh.dst + idx) = a;
}

__global__ __launch_bounds__(256) void k_bwd_finish(BwdFinishDx f, uint16_t* __restrict__ dx, int64_t dx_blocks,
                                                    Shares da, int64_t da_blocks, Shares db) {
    const int64_t b = blockIdx.x;
    if (b < dx_blocks) {
        const int64_t tile_elems = int64_t(f.bm) * f.bk, total = int64_t(f.tail) * tile_elems;
        const int64_t idx = (b * 256 + threadIdx.x) * 4;
        if (idx >= total) return;
        const int q = int(idx / tile_elems), loc = int(idx % tile_elems);
        const int tile = f.full + q;
        const int row = (tile % f.mtiles) * f.bm + loc / f.bk, col = (tile / f.mtiles) * f.bk + loc % f.bk;
        if (row >= f.T || col >= f.K) return;  // K % 64 == 0: the four columns are all in or all out
        f32x4 a = *reinterpret_cast<const f32x4*>(f.part + idx);
        const int np = q < f.bal_a ? f.bal_pa : f.pieces;
        for (int z = 1; z < np; ++z) a += *reinterpret_cast<const f32x4*>(f.part + z * total + idx);
        const u32x2 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3])};
        *reinterpret_cast<u32x2*>(dx + size_t(row) * f.K + col) = o;
    } else if (b < dx_blocks + da_blocks) {
        sum_shares(da, b - dx_blocks);
    } else {
        sum_shares(db, b - dx_blocks - da_blocks);
    }
}

}  // namespace

int bwd_tile_tokens(int64_t T, int64_t N, int64_t K, bool dense) {
    (void)N;
    return !dense && cdiv(T, 256) * cdiv(K, 128) >= kCUs ? 256 : 128;
}

BwdPlan plan_bwd(int64_t T, int64_t N, int64_t K, int r, bool dense) {
    BwdPlan p{};
    if (T <= kSkinnyBwdT && !dense) {
        p.skinny = true;
        p.sk = plan_skinny_bwd(T, N, K);
        if (r > 0) plan_lora_bwd_pre(p, T, N, kMaxGPartsFew);
        p.off_gpart = 0;
        p.off_dx = align256(size_t(p.gparts) * size_t(T) * size_t(r) * 4);
        p.ws_bytes = p.off_dx + p.sk.ws_bytes;
        return p;
    }
    // 256-token tiles (half the dequantisation and weight stores per MFMA) when they
    // still fill a whole round of CUs without splitting the contraction (the 7B down
    // projection at 512 tokens: 296 tiles, 107-109 against 114-116 us in the layer
    // step); with fewer tiles the extra split pieces cost more than that saves (gate and
    // up: 56 tiles, 113-116 against 106-109 us), so those keep 128-token tiles
    p.bm = bwd_tile_tokens(T, N, K, dense);
    p.bn = 128;
    p.mtiles = int(cdiv(T, p.bm));
    p.ktiles = int(cdiv(K, p.bn));
    const int64_t tiles = int64_t(p.mtiles) * p.ktiles;
    const int64_t nsteps = cdiv(N, kBN);
    // Under 256 tiles: every tile split (about 512 workgroups in all). Many: whole rounds
    // of 256 tiles (one more per CU each) run whole, and a last round of at most 128
    // tiles is split into pieces that spread over the CUs: the time of a CU grows with
    // the tiles it holds, so 2 whole tiles + a third of one beat 3 whole tiles.
    int64_t tail = 0, pieces = 1, bal_a = 0, bal_pa = 0;
    const int64_t splits = pick_splits(tiles, nsteps, 4);
    if (pick_balanced(tiles, nsteps, 4, kCUs, bal_a, bal_pa)) {
        tail = tiles;
        pieces = bal_pa + 1;
    } else if (splits > 1) {
        tail = tiles;
        pieces = splits;
    } else if (tiles > kCUs) {
        const int64_t last = tiles % kCUs;
        const int64_t pc = pick_tail_pieces(last, nsteps / 4, kCUs);
        if (pc >= 2) {
            tail = last;
            pieces = pc;
        }
    }
    p.steps_per_piece = int(cdiv(nsteps, pieces));
    p.pieces = tail > 0 ? int(cdiv(nsteps, p.steps_per_piece)) : 1;
    p.bal_a = int(bal_a);
    p.bal_pa = int(bal_pa);
    if (bal_a > 0) {  // piece bounds come from balanced_piece; the slot count is bal_pa + 1
        p.pieces = int(pieces);
        p.steps_per_piece = 0;
    }
    p.tail = int(tail);
    p.full = int(tiles - tail);  // 0 or a multiple of kCUs (a multiple of the XCD count)
    if (r > 0) plan_lora_bwd_pre(p, T, N, kMaxGParts);
    size_t off = 0;
    p.off_gpart = off;
    off += align256(size_t(p.gparts) * size_t(T) * size_t(r) * 4);
    p.off_dapart = off;
    off += r > 0 ? align256(size_t(p.mtiles) * size_t(r) * size_t(K) * 4) : 0;
    p.off_dbpart = off;
    off += r > 0 && p.dbchunks > 1 ? align256(size_t(p.dbchunks) * size_t(N) * size_t(r) * 4) : 0;
    p.off_dx = off;
    off += p.tail > 0 ? align256(size_t(p.pieces) * size_t(p.tail) * size_t(p.bm) * size_t(p.bn) * 4) : 0;
    p.ws_bytes = off;
    return p;
}

hipError_t launch_gemm_bwd(const BwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* wdense,
                           const uint16_t* dy, const uint16_t* x, const uint16_t* A, int64_t T, int64_t N, int64_t K,
                           int r, float s, uint16_t* dx, float* dA, float* dB, void* ws, hipStream_t stream) {
    char* w = static_cast<char*>(ws);
    // without dx only the LoRA part runs: one workgroup per tile, no contraction steps
    BwdTiles tl{p.full, p.tail, p.pieces, p.steps_per_piece, p.mtiles, p.bal_a, p.bal_pa};
    if (!dx) tl = BwdTiles{p.mtiles * p.ktiles, 0, 1, 0, p.mtiles, 0, 0};
    const dim3 grid(unsigned(tl.full + (tl.bal_a > 0 ? 2 * kCUs : int64_t(tl.tail) * tl.pieces)));
    float* partial = tl.tail > 0 ? reinterpret_cast<float*>(w + p.off_dx) : nullptr;
    float* dapart = reinterpret_cast<float*>(w + p.off_dapart);
    const BwdLora lora{reinterpret_cast<const float*>(w + p.off_gpart), p.gparts, A, x, dapart, r, s};
    if (dx) prof_gemm_begin(stream);
    if (wdense)
        hipLaunchKernelGGL((k_nf4_gemm_bwd_dx<128, true>), grid, dim3(256), 0, stream, dy,
                           static_cast<const void*>(wdense), nullptr, int(T), int(N), int(K), tl, lora, dx, partial,
                           tables());
    else if (p.bm == 256)
        hipLaunchKernelGGL((k_nf4_gemm_bwd_dx<256, false>), grid, dim3(512), 0, stream, dy,
                           static_cast<const void*>(codes), absmax, int(T), int(N), int(K), tl, lora, dx, partial,
                           tables());
    else
        hipLaunchKernelGGL((k_nf4_gemm_bwd_dx<128, false>), grid, dim3(256), 0, stream, dy,
                           static_cast<const void*>(codes), absmax, int(T), int(N), int(K), tl, lora, dx, partial,
                           tables());
    if (dx) prof_gemm_end(stream);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const BwdFinishDx f{partial, tl.full, tl.tail, tl.pieces, p.mtiles, p.bm, p.bn, int(T), int(K), tl.bal_a, tl.bal_pa};
    const int64_t dx_total = int64_t(tl.tail) * p.bm * p.bn;
    const Shares da{dapart, p.mtiles, r > 0 ? int64_t(r) * K : 0, dA};
    // dB shares (N * r is a multiple of 4: N % 16 == 0)
    const Shares db{reinterpret_cast<const float*>(w + p.off_dbpart), p.dbchunks,
                    r > 0 && p.dbchunks > 1 ? N * r : 0, dB};
    const int64_t dx_blocks = cdiv(dx_total / 4, 256), da_blocks = cdiv(da.total / 4, 256),
                  db_blocks = cdiv(db.total / 4, 256);
    if (dx_blocks + da_blocks + db_blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bwd_finish, dim3(unsigned(dx_blocks + da_blocks + db_blocks)), dim3(256), 0, stream, f, dx,
                       dx_blocks, da, da_blocks, db);
    return hipGetLastError();
}

}  // namespace nf4
