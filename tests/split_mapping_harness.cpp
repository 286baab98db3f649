// Host-side check of the GEMM split plans' workgroup mapping (the library's own
// pick_balanced, pick_tail_pieces and balanced_piece): for every tile count below the
// CU count and every step count, the balanced split's 2 x 256 workgroups cover each
// (tile, piece) once, every piece is non-empty, the pieces of a tile tile its steps, and
// the busiest CU (linear ids L and L + 256) holds no more steps than under the uniform
// split. Prints "ok" and exits 0, or names the failing case and exits 1.
#include <cstdio>
#include <vector>

#include "common.h"
#include "device.h"

using namespace nf4;

static int fail(const char* what, long tiles, long steps, long L) {
    std::printf("FAIL %s tiles=%ld steps=%ld L=%ld\n", what, tiles, steps, L);
    return 1;
}

int main() {
    const int64_t cus = kChipCUs;
    long cases = 0;
    for (int64_t tiles = 1; tiles < cus; ++tiles) {
        for (int64_t steps = 1; steps <= 400; ++steps) {
            int64_t a = 0, pa = 0;
            if (!pick_balanced(tiles, steps, 4, cus, a, pa)) continue;
            ++cases;
            const int64_t W = 2 * cus;
            if (a * pa + (tiles - a) * (pa + 1) != W) return fail("workgroup count", tiles, steps, -1);
            std::vector<int> seen(size_t(tiles) * size_t(pa + 1), 0);
            std::vector<int> lo(seen.size(), -1), hi(seen.size(), -1);
            std::vector<int> load(size_t(cus), 0);
            for (int64_t L = 0; L < W; ++L) {
                int q, z, s0, s1;
                balanced_piece(uint32_t(L), uint32_t(cus), int(tiles), int(a), int(pa), int(steps), q, z, s0, s1);
                const int P = q < a ? int(pa) : int(pa) + 1;
                if (q < 0 || q >= tiles || z < 0 || z >= P) return fail("piece out of range", tiles, steps, L);
                if (!(0 <= s0 && s0 < s1 && s1 <= steps)) return fail("empty or out-of-range steps", tiles, steps, L);
                const size_t k = size_t(z) * size_t(tiles) + size_t(q);
                if (seen[k]++) return fail("piece twice", tiles, steps, L);
                lo[k] = s0;
                hi[k] = s1;
                load[size_t(L % cus)] += s1 - s0;
            }
            for (int64_t q = 0; q < tiles; ++q) {
                const int P = q < a ? int(pa) : int(pa) + 1;
                int at = 0;
                for (int z = 0; z < P; ++z) {
                    const size_t k = size_t(z) * size_t(tiles) + size_t(q);
                    if (!seen[k] || lo[k] != at) return fail("pieces do not tile the steps", tiles, steps, q);
                    at = hi[k];
                }
                if (at != steps) return fail("pieces do not reach the last step", tiles, steps, q);
            }
            int worst = 0;
            for (int v : load) worst = v > worst ? v : worst;
            const int64_t us = pick_splits(tiles, steps, 4), per = cdiv(steps, us);
            const int64_t uworst = cdiv(tiles * cdiv(steps, per), cus) * per;
            if (worst > uworst) return fail("busiest CU above the uniform split", tiles, steps, worst);
        }
    }
    // last partial rounds: at most half a round -> one piece per CU; more -> 1..4 pieces
    for (int64_t last = 1; last < cus; ++last)
        for (int64_t maxp = 0; maxp <= 40; ++maxp) {
            const int64_t pc = pick_tail_pieces(last, maxp, cus);
            if (pc < 1 || (maxp >= 2 && pc > maxp) || (last > cus / 2 && pc > 4)) return fail("tail pieces", last, maxp, pc);
            if (last <= cus / 2 && maxp >= 2 && last * pc > cus) return fail("tail over one round", last, maxp, pc);
        }
    std::printf("ok %ld balanced cases\n", cases);
    return 0;
}
