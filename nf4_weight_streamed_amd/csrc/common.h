// Internal declarations of the NF4-LoRA library (host + device). Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cstdint>

namespace nf4 {

// Levels of the NF4 code (ascending) and the quantiser's decision thresholds:
// thresh[j] is the smallest float32 strictly above the midpoint of level[j] and
// level[j+1], so "v >= thresh[j]" is "v lies above that midpoint" for float32 v.
struct Tables {
    float level[16];
    float thresh[15];
};

const Tables& tables();  // built once per process (abi.cpp)

// Error plumbing (abi.cpp): record a message for nf4_last_error() and return code.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int check_launch(const char* what);  // NF4_OK, or NF4_E_HIP with the HIP error text

// ---- kernel launchers (each returns hipError_t of the launch) ----
hipError_t launch_quantize(const void* w, int in_dtype, int64_t rows, int64_t cols, uint8_t* codes,
                           float* absmax, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* codes, const float* absmax, int64_t rows, int64_t cols,
                             uint16_t* w, hipStream_t stream);

#define NF4_MAX_RANK_BLOCKS 4  // r <= 16 * NF4_MAX_RANK_BLOCKS (= NF4_MAX_RANK)

// Partial counts of the skinny LoRA products, summed per tile by the GEMM kernels.
constexpr int kMaxDownParts = 16; // K ranges of u = x.A^T
constexpr int kMaxGParts = 16;    // N ranges of g = dY.B (128-token path)
constexpr int kMaxGPartsFew = 16; // N ranges of g = dY.B (few-token path: summed by the finish kernel;
                                  // 64 was 3-4% slower on the gate shapes at 16 and 32 tokens)
constexpr int kMaxDbChunks = 8;   // token ranges of dB = s.dY^T.u (shares summed by the finish kernel)

// Few-token path: streaming kernels with 16-token MFMA blocks and fp32 partials over a
// split contraction, finished (split sum + LoRA + rounding) by a second kernel.
// Workspace: [partials | u partials] (forward) / [g partials | dX partials] (backward).
// Both take up to 32 tokens in one or two blocks, which share each dequantised weight
// fragment (at T = 32 the 7B q, 7B gate, 72B gate and 72B down forward take 13.4, 30.6,
// 65 and 60 us against 23.3, 35.5, 88 and 90 us on the 128-token kernels, the backward
// of the 72B gate 58 against 96 us and of the 7B k 17.3 against 17.6 us; at T = 64,
// four blocks were slower than those on the 7B shapes).
constexpr int64_t kSkinnyFwdT = 32;
// The forward also takes up to 64 tokens (four blocks) for long, narrow weights, where the
// 128-token kernels have few tiles to split: at T = 64 the 72B down, q and k forward take
// 80, 37 and 17.7 us against 97, 39 and 26 us, the 7B down 35.5 against 41 us, while the
// wide 72B gate keeps the 128-token kernels (97 against 100 us).
constexpr int64_t kSkinnyFwdLongT = 64;
constexpr int64_t kSkinnyLongK = 8192;      // K at least this
constexpr int64_t kSkinnyNarrowN = 8192;    // N at most this
constexpr int64_t kSkinnyBwdT = 32;
struct SkinnyPlan {
    int row_blocks;       // forward: 128-row workgroups
    int col_blocks;       // backward: 128-column workgroups
    int splits;           // contraction splits (grid y)
    int steps_per_split;
    size_t off_part, off_upart;  // workspace offsets (bytes)
    size_t ws_bytes;
};
SkinnyPlan plan_skinny_fwd(int64_t T, int64_t N, int64_t K, int r);
SkinnyPlan plan_skinny_bwd(int64_t T, int64_t N, int64_t K);

// Forward plan: how the kernels are split for a shape (a pure function of the shape,
// so repeated calls - streamed or resident - launch identical grids). Workspace:
// [u partials | fp32 partial tiles of the split y tiles].
// y tiles (token tile fastest) 0 .. full-1 run whole; the last `tail` tiles are split
// over K into `pieces` ranges of steps_per_piece 64-wide steps, one workgroup each
// (all tiles when there are too few to fill the CUs, else the last partial round).
struct FwdPlan {
    int bm, bn;           // GEMM workgroup tile (tokens x out features)
    int full, tail;       // whole tiles, split tiles
    int pieces, steps_per_piece;
    int bal_a, bal_pa;    // balanced split: the first bal_a split tiles in bal_pa pieces, the rest in pieces (0: off)
    int mtiles;           // token tiles
    int down_parts;       // K ranges of u = x.A^T (partials summed by the GEMM); 0 if r == 0
    int down_steps;       // 32-wide K steps per range
    size_t off_upart, off_ypart;  // workspace offsets (bytes)
    size_t ws_bytes;
    bool skinny;          // few-token path (then only sk and ws_bytes apply)
    SkinnyPlan sk;
};
FwdPlan plan_fwd(int64_t T, int64_t N, int64_t K, int r, bool dense = false);  // dense: bf16 base, 128-token kernels only
void plan_lora_down(FwdPlan& p, int64_t K);

// Backward plan. Workspace: [g partials | dA shares per token tile | fp32 partial
// tiles of the split dX tiles].
// dX tiles (token tile fastest) 0 .. full-1 run whole; the last `tail` tiles are
// split over the contraction (N) into `pieces` ranges of steps_per_piece steps, one
// workgroup each, so that the workgroups of the last round fill the chip; with few
// tiles every tile is split (full = 0).
struct BwdPlan {
    int bm, bn;            // dX tile (tokens x in features)
    int full, tail;        // whole tiles, split tiles
    int pieces, steps_per_piece;
    int bal_a, bal_pa;     // balanced split (as in FwdPlan)
    int mtiles, ktiles;    // dX tile grid
    int gparts, gsteps;    // N ranges of g = dY.B (partials summed by the GEMM), 128-feature chunks each
    int dbchunks, dbtokens;  // token ranges of dB (1: written directly), tokens each
    size_t off_dbpart;     // dB shares [dbchunks][N][r] when dbchunks > 1
    size_t off_gpart, off_dapart, off_dx;  // workspace offsets (bytes)
    size_t ws_bytes;
    bool skinny;           // few-token path: g partials and dX partials (sk) at off_gpart / off_dx
    SkinnyPlan sk;
};
BwdPlan plan_bwd(int64_t T, int64_t N, int64_t K, int r, bool dense = false);
void plan_lora_bwd_pre(BwdPlan& p, int64_t T, int64_t N, int max_parts);  // g over N ranges, dB over token ranges

hipError_t launch_lora_down(const FwdPlan& p, const uint16_t* x, const uint16_t* A, int64_t T, int64_t K, int r,
                            float* upart, hipStream_t stream);
// the base is NF4 (codes, absmax) or, when wdense is not NULL, dense bf16 [N][K]
hipError_t launch_gemm_fwd(const FwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* wdense,
                           const uint16_t* x, const uint16_t* B, int64_t T, int64_t N, int64_t K, int r, float s,
                           uint16_t* y, float* u_save, void* ws, hipStream_t stream);
hipError_t launch_lora_bwd_pre(const BwdPlan& p, const uint16_t* dy, const uint16_t* B, const float* u, int64_t T,
                               int64_t N, int r, float s, float* gpart, float* dB, float* dbpart, hipStream_t stream);
hipError_t launch_gemm_bwd(const BwdPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* wdense,
                           const uint16_t* dy, const uint16_t* x, const uint16_t* A, int64_t T, int64_t N, int64_t K,
                           int r, float s, uint16_t* dx, float* dA, float* dB, void* ws, hipStream_t stream);

hipError_t launch_skinny_fwd(const SkinnyPlan& p, const uint8_t* codes, const float* absmax, const uint16_t* x,
                             const uint16_t* A, const uint16_t* B, int64_t T, int64_t N, int64_t K, int r, float s,
                             uint16_t* y, float* u_save, void* ws, hipStream_t stream);
// dX partials and the g / dB pre-pass in one launch, then the finish kernel (dX, dA)
hipError_t launch_skinny_bwd(const SkinnyPlan& p, const BwdPlan& bp, const uint8_t* codes, const float* absmax,
                             const uint16_t* dy, const uint16_t* x, const uint16_t* A, const uint16_t* B,
                             const float* u, int64_t T, int64_t N, int64_t K, int r, float s, uint16_t* dx, float* dA,
                             float* dB, void* ws, hipStream_t stream);

hipError_t launch_probe_mfma(float* out, int workgroups, int iters, hipStream_t stream);
hipError_t launch_probe_read(const void* src, uint64_t bytes, uint32_t* out, int workgroups, hipStream_t stream);
hipError_t launch_probe_read_depth(const void* src, uint64_t bytes, uint32_t* out, int workgroups, int depth,
                                  bool nontemporal, hipStream_t stream);
hipError_t launch_merge_lora(const uint8_t* codes, const float* absmax, int64_t N, int64_t K, const uint16_t* A,
                             const uint16_t* B, int r, float s, uint16_t* w_out, hipStream_t stream);

// The forward entry point's shape/rank/pointer checks and its body after them (abi.cpp);
// ws is the workspace of ws_bytes bytes (NULL allowed when the plan needs none).
int check_linear_args(const char* fn, const uint8_t* codes, const float* absmax, int64_t N, int64_t K, int64_t T, int r,
                      float alpha);
int linear_fwd(const char* fn, const uint8_t* codes, const float* absmax, const uint16_t* wdense, int64_t N, int64_t K,
               const uint16_t* x, int64_t T, const uint16_t* A, const uint16_t* B, int r, float alpha, uint16_t* y,
               float* u_save, void* ws, size_t ws_bytes, void* stream);

// Instrumentation events around the next fused GEMM launch (abi.cpp); no-ops unless requested.
void prof_gemm_begin(hipStream_t stream);
void prof_gemm_end(hipStream_t stream);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Compute units of one MI355X (gfx950): the round size of the GEMM grids (the
// dispatcher gives linear workgroup ids L, L + 256, L + 512 the same CU).
constexpr int64_t kChipCUs = 256;

// Split count for a GEMM with `tiles` output tiles and `steps` reduction steps: the
// GEMM kernels run two workgroups per CU, so up to 2 * 256 workgroups run in one
// round; a grid just above that leaves a nearly empty second round. Split only
// shapes with at most 256 tiles, up to 512 workgroups, >= min_steps steps each
// (256 tiles unsplit would leave one workgroup per CU, which runs a K step about
// 1.6x slower than two or three sharing the CU).
inline int64_t pick_splits(int64_t tiles, int64_t steps, int64_t min_steps) {
    constexpr int64_t kSlots = 512;
    if (tiles > kSlots / 2) return 1;
    int64_t s = kSlots / tiles;
    s = std::min<int64_t>(s, std::max<int64_t>(1, steps / min_steps));
    return std::max<int64_t>(1, s);
}
inline size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Pieces per tile for the `last` tiles of a final, partial round of `cus` tiles (one
// workgroup per tile otherwise). At most half a round: one piece per CU (cus / last
// pieces each). More than half: the piece count (2..4) that puts the least work on the
// busiest CU, ceil(last * pc / cus) / pc tiles' worth, if that beats one whole tile;
// these tiles run after the earlier rounds (e.g. 924 tiles: three workgroups per CU
// fill 768 slots, and 156 tiles left whole would each run alone on a CU, at the slow
// single-workgroup rate). 1: no split.
inline int64_t pick_tail_pieces(int64_t last, int64_t max_pieces, int64_t cus) {
    if (last <= 0 || max_pieces < 2) return 1;
    if (last <= cus / 2) return std::max<int64_t>(1, std::min<int64_t>(cus / last, max_pieces));
    int64_t best = 1, best_num = 1, best_den = 1;  // busiest CU's load best_num / best_den tiles
    for (int64_t pc = 2; pc <= std::min<int64_t>(4, max_pieces); ++pc) {
        const int64_t num = cdiv(last * pc, cus);
        if (num * best_den < best_num * pc) {
            best = pc;
            best_num = num;
            best_den = pc;
        }
    }
    return best;
}

// Balanced split for fewer tiles than CUs: 2 x cus workgroups, `a` tiles cut into pa
// pieces and the other tiles - cut into pa + 1, with every piece at least min_steps
// long. The dispatcher gives linear workgroup ids L and L + cus the same CU, so with
// the a * pa longer pieces (at most cus of them) in the first round and only shorter
// ones in the second, every CU runs one longer and one shorter piece or two shorter
// ones: tiles = 112 gives at most 74 + 60 K steps per CU for 296 steps per tile,
// against 2 x 74 for four pieces each (448 workgroups, 192 CUs with two). False when
// it does not apply (then the uniform split stands).
inline bool pick_balanced(int64_t tiles, int64_t steps, int64_t min_steps, int64_t cus, int64_t& a, int64_t& pa) {
    if (tiles <= 0 || tiles >= cus) return false;
    const int64_t p = 2 * cus / tiles, b = 2 * cus - p * tiles, aa = tiles - b;
    if (b <= 0 || aa <= 0 || aa * p > cus || (p + 1) * min_steps > steps) return false;
    a = aa;
    pa = p;
    return true;
}

}  // namespace nf4
