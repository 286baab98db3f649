// Host-side check of the block pool's state machine (the library's own PoolCore from
// pool_core.h) with a host engine in place of HIP: streams are op lists with vector
// clocks, events snapshot a stream's clock when recorded and merge it into the
// waiting stream, copies run at once into a host "device" slab. The driver reads
// each part of an acquired block on a compute stream (as the layer kernels do) and
// checks, for every op:
//   - each read of a slot range happens after the copy that last wrote it, and that
//     copy wrote the block's bytes;
//   - each copy into a slot range happens after every earlier read of that range.
// Scenarios: the stack's streamed pattern (forward ascending, backward descending,
// prefetch one ahead, per-part releases) for several block/part/slot shapes, random
// call sequences, and the error cases (miss, BUSY, double release, bad part, OOM
// message with sizes). Prints "ok" and exits 0, or names the failure and exits 1.
#include <cstdarg>
#include <cstdio>
#include <algorithm>
#include <cstring>
#include <random>
#include <string>
#include <vector>

#include "pool_core.h"

namespace nf4 {
std::string g_last;
int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last = buf;
    return code;
}
}  // namespace nf4

using namespace nf4;

static int g_fail = 0;
static bool g_quiet = false;  // a negative control expects a failure: do not print it
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            if (!g_quiet) {                               \
                std::printf("FAIL line %d: ", __LINE__);  \
                std::printf(__VA_ARGS__);                 \
                std::printf(" [%s]\n", g_last.c_str());   \
            }                                             \
            g_fail = 1;                                   \
            return 1;                                     \
        }                                                 \
    } while (0)

constexpr int kStreams = 3;  // 0: copy, 1, 2: compute
using Clock = std::vector<long>;

struct HostEngine {
    using Event = int;
    using Stream = int;
    std::vector<Clock> clock = std::vector<Clock>(kStreams, Clock(kStreams, 0));
    std::vector<Clock> ev_snap;
    struct Op {  // a copy or a read of [lo, hi) of the slab
        bool is_copy;
        int stream;
        long idx;  // the op's own clock component on its stream
        Clock at;  // the stream's clock at the op
        size_t lo, hi;
        int block;
    };
    std::vector<Op> ops;
    char* slab = nullptr;

    int create_event(Event* e) {
        ev_snap.push_back(Clock(kStreams, 0));
        *e = int(ev_snap.size()) - 1;
        return NF4_OK;
    }
    void destroy_event(Event) {}
    long tick(int s) { return ++clock[s][s]; }
    int record(Event e, Stream s) {
        tick(s);
        ev_snap[e] = clock[s];
        return NF4_OK;
    }
    int wait(Stream s, Event e) {
        for (int i = 0; i < kStreams; ++i) clock[s][i] = std::max(clock[s][i], ev_snap[e][i]);
        tick(s);
        return NF4_OK;
    }
    int acquire_wait(Stream s, Event e, int /*block*/, int /*part*/) { return wait(s, e); }
    int host_waits = 0;
    int host_wait(Event) {
        ++host_waits;
        return NF4_OK;
    }
    int copy(void* dst, const void* src, size_t bytes, Stream s, int /*block*/, int /*part*/) {
        std::memcpy(dst, src, bytes);
        const long i = tick(s);
        const size_t lo = size_t(static_cast<char*>(dst) - slab);
        ops.push_back(Op{true, s, i, clock[s], lo, lo + bytes, -1});
        return NF4_OK;
    }
    void read(Stream s, size_t lo, size_t hi, int block) {
        const long i = tick(s);
        ops.push_back(Op{false, s, i, clock[s], lo, hi, block});
    }
};

static bool happens_before(const HostEngine::Op& a, const HostEngine::Op& b) {
    return b.at[a.stream] >= a.idx;
}

// Order checks over all ops recorded so far.
static int check_order(const HostEngine& eng) {
    const auto& ops = eng.ops;
    for (size_t j = 0; j < ops.size(); ++j) {
        const auto& b = ops[j];
        for (size_t i = 0; i < j; ++i) {
            const auto& a = ops[i];
            if (a.hi <= b.lo || b.hi <= a.lo) continue;
            if (!a.is_copy && b.is_copy)
                CHECK(happens_before(a, b), "copy %zu into [%zu,%zu) not ordered after read %zu", j, b.lo, b.hi, i);
        }
        if (!b.is_copy) {  // the last copy into each byte of the read range must happen before it
            for (size_t i = j; i-- > 0;) {
                const auto& a = ops[i];
                if (!a.is_copy || a.hi <= b.lo || b.hi <= a.lo) continue;
                CHECK(happens_before(a, b), "read %zu of [%zu,%zu) not ordered after copy %zu", j, b.lo, b.hi, i);
                break;
            }
        }
    }
    return 0;
}

struct Fixture {
    int n_blocks, parts_per_block, n_slots;
    size_t part_bytes;
    std::vector<std::vector<char>> host;  // per part
    std::vector<nf4_host_block> hp;
    std::vector<int> begin;
    std::vector<char> slab;
    HostEngine eng;
    PoolCore<HostEngine> pool;
    // layers: n_layers parts, grouped parts_per_block per block (the last block may be shorter)
    Fixture(int n_layers, int ppb, int slots, size_t pb) : parts_per_block(ppb), n_slots(slots), part_bytes(pb) {
        n_blocks = (n_layers + ppb - 1) / ppb;
        for (int l = 0; l < n_layers; ++l) {
            host.emplace_back(pb);
            for (size_t i = 0; i < pb; ++i) host[l][i] = char((l * 131 + i * 7) % 251);
        }
        for (int l = 0; l < n_layers; ++l) hp.push_back(nf4_host_block{host[l].data(), pb});
        for (int b = 0; b < n_blocks; ++b) begin.push_back(b * ppb);
        begin.push_back(n_layers);
        slab.resize(size_t(slots) * ppb * pb + 256);
    }
    char* base() { return reinterpret_cast<char*>((reinterpret_cast<uintptr_t>(slab.data()) + 255) & ~uintptr_t(255)); }
    int init() {
        eng.slab = base();
        return pool.init(&eng, hp.data(), begin.data(), n_blocks, base(), size_t(parts_per_block) * part_bytes, n_slots,
                         0, true);
    }
    int nparts(int b) const { return begin[b + 1] - begin[b]; }
    // read every part of a held block on `s` (data must be the block's), releasing each;
    // after a deferred acquire, wait for each part first (unless skip_waits: a
    // negative control whose reads the order check must reject)
    int use_block(int b, const void* dev, bool descending, int s, bool deferred = false, bool skip_waits = false) {
        const size_t off = size_t(static_cast<const char*>(dev) - base());
        for (int k = 0; k < nparts(b); ++k) {
            const int i = descending ? nparts(b) - 1 - k : k;
            if (deferred && !skip_waits) CHECK(pool.wait_part(b, i, s) == NF4_OK, "wait_part(%d, %d)", b, i);
            const size_t lo = off + size_t(i) * part_bytes;
            CHECK(std::memcmp(base() + lo, host[begin[b] + i].data(), part_bytes) == 0,
                  "block %d part %d: slot bytes differ from the host part", b, i);
            eng.read(s, lo, lo + part_bytes, b);
            CHECK(pool.release_part(b, i, s) == NF4_OK, "release_part(%d, %d)", b, i);
        }
        CHECK(pool.release(b, s) == NF4_OK, "release(%d)", b);
        return 0;
    }
};

// The stack's streamed pattern for `steps` steps; deferred: acquire without the
// block wait and wait for each part before reading it; max_ahead: the host's lead
// bound (one host wait per release beyond the first max_ahead).
static int stack_pattern(int n_layers, int ppb, int slots, int steps, bool deferred = false, int max_ahead = 0) {
    Fixture f(n_layers, ppb, slots, 512);
    CHECK(f.init() == NF4_OK, "init");
    CHECK(f.pool.set_max_ahead(max_ahead) == NF4_OK, "set_max_ahead");
    const int nb = f.n_blocks;
    for (int step = 0; step < steps; ++step) {
        f.pool.descending = false;
        for (int b = 0; b < nb; ++b) {
            const void* dev = nullptr;
            CHECK(f.pool.acquire(b, 1, &dev, deferred) == NF4_OK, "fwd acquire %d", b);
            if (slots > 1 && b + 1 < nb) CHECK(f.pool.prefetch(b + 1) == NF4_OK, "fwd prefetch %d", b + 1);
            if (f.use_block(b, dev, false, 1, deferred)) return 1;
        }
        f.pool.descending = true;
        for (int b = nb - 1; b >= 0; --b) {
            const void* dev = nullptr;
            CHECK(f.pool.acquire(b, 1, &dev, deferred) == NF4_OK, "bwd acquire %d", b);
            if (slots > 1 && b > 0) CHECK(f.pool.prefetch(b - 1) == NF4_OK, "bwd prefetch %d", b - 1);
            if (f.use_block(b, dev, true, 1, deferred)) return 1;
        }
    }
    if (check_order(f.eng)) return 1;
    // misses: only block 0 of the first forward when prefetching, every block otherwise
    if (slots > 1 && nb > slots) CHECK(f.pool.stats.misses == 1, "misses %llu", (unsigned long long)f.pool.stats.misses);
    const int releases = 2 * nb * steps;
    CHECK(f.eng.host_waits == (max_ahead > 0 ? std::max(0, releases - max_ahead) : 0), "host waits %d",
          f.eng.host_waits);
    CHECK(int(f.pool.ahead.size()) == std::min(releases, max_ahead), "marks kept %zu", f.pool.ahead.size());
    f.pool.destroy_events();
    return 0;
}

// Negative control of the order check: a deferred acquire whose parts are read without
// wait_part must be rejected (reads not ordered after their copies).
static int deferred_without_waits() {
    Fixture f(4, 2, 1, 512);
    CHECK(f.init() == NF4_OK, "init");
    const void* dev = nullptr;
    CHECK(f.pool.acquire(0, 1, &dev, true) == NF4_OK, "deferred acquire");
    if (f.use_block(0, dev, false, 1, true, true)) return 1;
    g_quiet = true;
    const int bad = check_order(f.eng);
    g_quiet = false;
    g_fail = 0;  // the failure above is the expected outcome
    CHECK(bad == 1, "reads without wait_part passed the order check");
    f.pool.destroy_events();
    return 0;
}

// Random call sequences on two compute streams: every accepted call keeps the order invariants.
static int random_calls(unsigned seed) {
    std::mt19937 rng(seed);
    const int n_layers = 3 + int(rng() % 8), ppb = 1 + int(rng() % 3), slots = 1 + int(rng() % 3);
    Fixture f(n_layers, ppb, slots, 256);
    CHECK(f.init() == NF4_OK, "init");
    std::vector<int> held_stream(f.n_blocks, 0);  // compute stream of a held block, 0 = not held
    std::vector<std::vector<char>> released(f.n_blocks);
    for (int it = 0; it < 400; ++it) {
        const int b = int(rng() % f.n_blocks), op = int(rng() % 5);
        if (op == 0) {
            f.pool.descending = rng() & 1;
            const int st = f.pool.prefetch(b);
            CHECK(st == NF4_OK || st == NF4_E_BUSY, "prefetch %d -> %d", b, st);
        } else if (op == 1) {
            const int s = 1 + int(rng() % 2);
            const void* dev = nullptr;
            const int st = f.pool.acquire(b, s, &dev);
            if (held_stream[b]) {
                CHECK(st == NF4_E_STATE, "acquire of held block %d -> %d", b, st);
            } else if (st == NF4_OK) {
                held_stream[b] = s;
                released[b].assign(f.nparts(b), 0);
                const size_t off = size_t(static_cast<const char*>(dev) - f.base());
                for (int i = 0; i < f.nparts(b); ++i)
                    CHECK(std::memcmp(f.base() + off + size_t(i) * 256, f.host[f.begin[b] + i].data(), 256) == 0,
                          "acquired block %d part %d holds other bytes", b, i);
            } else {
                CHECK(st == NF4_E_BUSY, "acquire %d -> %d", b, st);
            }
        } else if (op == 2 || op == 3) {  // read one part of a held block, then maybe release it
            if (!held_stream[b]) {
                CHECK(f.pool.release_part(b, 0, 1) == NF4_E_STATE, "release_part of free block %d", b);
                continue;
            }
            const int i = int(rng() % f.nparts(b));
            const size_t off = size_t(f.pool.where[b]) * f.pool.slot_bytes + size_t(i) * 256;
            if (!released[b][i]) f.eng.read(held_stream[b], off, off + 256, b);
            if (op == 3) {
                const int st = f.pool.release_part(b, i, held_stream[b]);
                CHECK(st == (released[b][i] ? NF4_E_STATE : NF4_OK), "release_part(%d, %d) -> %d", b, i, st);
                released[b][i] = 1;
            }
        } else {
            const int s = held_stream[b] ? held_stream[b] : 1;
            const int st = f.pool.release(b, s);
            CHECK(st == (held_stream[b] ? NF4_OK : NF4_E_STATE), "release %d -> %d", b, st);
            held_stream[b] = 0;
        }
    }
    if (check_order(f.eng)) return 1;
    f.pool.destroy_events();
    return 0;
}

static int errors() {
    {  // never prefetched: a miss; all slots held: BUSY; double release: STATE; bad part: ARG
        Fixture f(6, 2, 2, 256);
        CHECK(f.init() == NF4_OK, "init");
        const void* d0 = nullptr;
        const void* d1 = nullptr;
        CHECK(f.pool.acquire(0, 1, &d0) == NF4_OK && f.pool.stats.misses == 1, "first acquire is a miss");
        CHECK(f.pool.acquire(0, 1, &d0) == NF4_E_STATE, "acquire of a held block");
        CHECK(f.pool.acquire(1, 1, &d1) == NF4_OK, "second slot");
        CHECK(f.pool.prefetch(2) == NF4_E_BUSY && g_last.find("held") != std::string::npos, "BUSY with all held");
        CHECK(f.pool.release_part(0, 2, 1) == NF4_E_ARG, "part outside the block");
        CHECK(f.pool.release_part(0, 1, 1) == NF4_OK, "release_part");
        CHECK(f.pool.release_part(0, 1, 1) == NF4_E_STATE, "double release_part");
        CHECK(f.pool.release(0, 1) == NF4_OK, "release");
        CHECK(f.pool.release(0, 1) == NF4_E_STATE, "double release");
        const int freed = f.pool.where[0];
        CHECK(f.pool.prefetch(2) == NF4_OK && f.pool.where[2] == freed && f.pool.where[0] == -1,
              "prefetch after release reuses the released block's slot");
        CHECK(f.pool.prefetch(9) == NF4_E_ARG, "block out of range");
        CHECK(f.pool.wait_part(0, 0, 1) == NF4_E_STATE, "wait_part of a block not held");
        CHECK(f.pool.wait_part(1, 2, 1) == NF4_E_ARG, "wait_part of a part outside the block");
        CHECK(f.pool.wait_part(1, 1, 1) == NF4_OK, "wait_part of a held block");
        CHECK(f.pool.set_max_ahead(-1) == NF4_E_ARG, "negative lead");
        f.pool.destroy_events();
    }
    {  // a block larger than a slot: OOM, with the sizes in the message
        Fixture f(4, 2, 2, 512);
        HostEngine eng;
        PoolCore<HostEngine> pool;
        std::vector<int> begin = {0, 3, 4};  // block 0: 3 parts = 1536 bytes > 1024
        CHECK(pool.init(&eng, f.hp.data(), begin.data(), 2, f.base(), 1024, 2, 0, true) == NF4_E_OOM, "OOM");
        CHECK(g_last.find("1536") != std::string::npos && g_last.find("1024") != std::string::npos,
              "OOM message names the sizes");
        pool.destroy_events();
    }
    {  // a part that is not a multiple of 256 bytes before a block's last part
        Fixture f(4, 2, 2, 300);
        HostEngine eng;
        PoolCore<HostEngine> pool;
        CHECK(pool.init(&eng, f.hp.data(), f.begin.data(), f.n_blocks, f.base(), 1024, 2, 0, true) == NF4_E_ARG &&
                  g_last.find("300 bytes") != std::string::npos,
              "part size");
    }
    return 0;
}

int main() {
    const int shapes[][3] = {{8, 4, 2}, {7, 4, 2}, {5, 1, 2}, {6, 2, 3}, {9, 3, 2}, {4, 4, 1}, {3, 1, 1}, {12, 4, 3}};
    for (const auto& s : shapes)
        for (int deferred = 0; deferred < 2; ++deferred)
            for (int ahead : {0, 1, 2, 5})
                if (stack_pattern(s[0], s[1], s[2], 3, deferred != 0, ahead)) return 1;
    if (deferred_without_waits()) return 1;
    for (unsigned seed = 1; seed <= 300; ++seed)
        if (random_calls(seed)) return 1;
    if (errors()) return 1;
    if (g_fail) return 1;
    std::printf("ok\n");
    return 0;
}
