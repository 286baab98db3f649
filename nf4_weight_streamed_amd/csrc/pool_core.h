// State machine of the block pool (stream_pool_* in nf4lora.h), independent of the
// runtime that moves the bytes: E is an engine giving streams, events and copies. The
// library instantiates it with HIP (stream_pool.cpp); a host engine drives it in the
// CPU tests of the slot logic.
//
// HN comment thread on streaming the frozen base (main comment): the base sits in
// host RAM and streams into a small pool of pre-allocated device buffers, prefetched
// one ahead on a dedicated stream. Poros API reference, "patch_hf_model" Behavior
// 4-6: layers regrouped into blocks of block_size; a block manager with cross-stream
// safety.
//
// A block is a list of parts (host ranges, e.g. one per layer) copied back to back
// into its slot. Ordering is carried by events on the streams:
//   ready[slot]   recorded on the copy stream after the block's last part; acquire
//                 makes the compute stream wait on it;
//   part_ready    recorded on the copy stream after each part; a deferred acquire
//                 makes no wait, and wait_part makes a stream wait for one part,
//                 so a block's first layers can run while its later parts land;
//   last uses     when part i of a held block is released (stream_pool_release_part,
//                 or every part not yet released at stream_pool_release) an event
//                 is recorded on the compute stream and kept with the slot byte
//                 range of that part; the copy of a later part into the slot waits
//                 for every kept last use whose range it overwrites (and drops it:
//                 the copy stream is ordered after it from then on), and for
//                 nothing else. A range a shorter block left untouched keeps its
//                 older last use until a copy overwrites it.
// Parts of a copy are issued in ascending order, or descending after
// set_order(true) (a backward pass uses the layers of a block last to first), so
// the first part copied overwrites the first part the previous pass released.
// A slot byte is never overwritten while a kernel enqueued before the release of its
// part may still read it. The host blocks only when a lead is set (set_max_ahead):
// each release records an event on its stream, and the host waits for the one
// recorded that many releases earlier, so the host runs at most that many blocks
// ahead of the device (a host far ahead leaves long chains of pending cross-stream
// waits behind the copies, and H2D copies were measured to slow down then).
#pragma once

#include <cstddef>
#include <cstdint>
#include <deque>
#include <vector>

#include "../../include/nf4lora.h"

namespace nf4 {

int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

template <class E>
struct PoolCore {
    using Event = typename E::Event;
    using Stream = typename E::Stream;

    struct Part {
        const void* host;
        size_t bytes;
        size_t off;  // offset in the slot
    };
    struct Block {
        int first, count;
        size_t bytes;
    };
    struct LastUse {  // a release recorded on `stream` that no copy has waited for yet
        size_t lo, hi;   // slot byte range
        Stream stream;
        Event event;
    };
    struct Slot {
        int block = -1;
        bool held = false;
        uint64_t stamp = 0;
        Event ready{};
        std::vector<Event> part_ready;  // per part of the block copied last
        std::vector<LastUse> pending;
        std::vector<char> released;  // parts released in the current hold
    };

    E* eng = nullptr;
    std::vector<Part> parts;
    std::vector<Block> blocks;
    std::vector<int> where;  // block -> slot, or -1
    std::vector<Slot> slots;
    char* slab = nullptr;
    size_t slot_bytes = 0;
    Stream copy{};
    uint64_t clock = 0;
    bool descending = false;
    int max_parts = 0;
    std::vector<Event> events;  // every last-use event created (destroyed at the end)
    std::vector<Event> spare;   // last-use events free for reuse (their waits are enqueued)
    int max_ahead = 0;          // 0: the host never waits
    std::deque<Event> ahead;    // release marks not yet waited for, oldest first
    nf4_pool_stats stats{};

    // Validate and take the layout: parts [part_begin[b], part_begin[b + 1]) form block b.
    int init(E* engine, const nf4_host_block* hp, const int* part_begin, int n_blocks, void* device_slab,
             size_t slot_bytes_, int n_slots, Stream copy_stream, bool has_copy_stream) {
        eng = engine;
        if (!hp || !part_begin || n_blocks <= 0 || n_slots <= 0 || !device_slab || !has_copy_stream)
            return fail(NF4_E_ARG, "stream_pool_create: need blocks, n_blocks > 0, n_slots > 0, a device slab and a "
                                   "copy stream (got n_blocks=%d n_slots=%d)", n_blocks, n_slots);
        if (slot_bytes_ == 0 || slot_bytes_ % 256 != 0 || reinterpret_cast<uintptr_t>(device_slab) % 256 != 0)
            return fail(NF4_E_ARG, "stream_pool_create: slot_bytes (%zu) and the slab address must be multiples of 256",
                        slot_bytes_);
        if (part_begin[0] != 0)
            return fail(NF4_E_ARG, "stream_pool_create: part_begin[0] must be 0 (got %d)", part_begin[0]);
        for (int b = 0; b < n_blocks; ++b) {
            const int first = part_begin[b], count = part_begin[b + 1] - first;
            if (count <= 0)
                return fail(NF4_E_ARG, "stream_pool_create: block %d has %d parts (part_begin must increase)", b, count);
            size_t off = 0;
            for (int i = 0; i < count; ++i) {
                const nf4_host_block& h = hp[first + i];
                if (!h.host) return fail(NF4_E_ARG, "stream_pool_create: block %d part %d has a NULL host pointer", b, i);
                if (i + 1 < count && h.bytes % 256 != 0)
                    return fail(NF4_E_ARG, "stream_pool_create: block %d part %d has %zu bytes; every part but a "
                                           "block's last must be a multiple of 256", b, i, h.bytes);
                parts.push_back(Part{h.host, h.bytes, off});
                off += h.bytes;
            }
            if (off > slot_bytes_)
                return fail(NF4_E_OOM, "stream_pool_create: block %d needs %zu bytes but a slot holds %zu (%d slots, "
                                       "%zu bytes of device slab requested)", b, off, slot_bytes_, n_slots,
                            slot_bytes_ * size_t(n_slots));
            blocks.push_back(Block{first, count, off});
            if (count > max_parts) max_parts = count;
        }
        where.assign(n_blocks, -1);
        slots.resize(n_slots);
        slab = static_cast<char*>(device_slab);
        slot_bytes = slot_bytes_;
        copy = copy_stream;
        for (auto& s : slots) {
            s.released.assign(max_parts, 0);
            int st = eng->create_event(&s.ready);
            if (st != NF4_OK) return st;
            s.part_ready.assign(max_parts, Event{});
            for (auto& e : s.part_ready) {
                st = eng->create_event(&e);
                if (st != NF4_OK) return st;
                events.push_back(e);  // destroyed with the last-use events
            }
        }
        return NF4_OK;
    }

    void destroy_events() {
        for (auto& s : slots) eng->destroy_event(s.ready);
        for (auto& e : events) eng->destroy_event(e);
        events.clear();
        spare.clear();
        ahead.clear();
    }

    int take_event(Event* e) {
        if (!spare.empty()) {
            *e = spare.back();
            spare.pop_back();
            return NF4_OK;
        }
        int st = eng->create_event(e);
        if (st == NF4_OK) events.push_back(*e);
        return st;
    }

    // Record a last use of slot bytes [lo, hi) on `compute`. A kept last use of a
    // range inside this one on the same stream is implied by this one and dropped.
    int record_last_use(Slot& s, size_t lo, size_t hi, Stream compute) {
        Event e{};
        int st = take_event(&e);
        if (st != NF4_OK) return st;
        st = eng->record(e, compute);
        if (st != NF4_OK) {
            spare.push_back(e);
            return st;
        }
        for (size_t k = 0; k < s.pending.size();) {
            const LastUse& u = s.pending[k];
            if (u.stream == compute && u.lo >= lo && u.hi <= hi) {
                spare.push_back(u.event);
                s.pending[k] = s.pending.back();
                s.pending.pop_back();
            } else {
                ++k;
            }
        }
        s.pending.push_back(LastUse{lo, hi, compute, e});
        return NF4_OK;
    }

    int check_block(int block, const char* fn) const {
        if (block < 0 || block >= int(blocks.size()))
            return fail(NF4_E_ARG, "%s: block %d outside 0..%d", fn, block, int(blocks.size()) - 1);
        return NF4_OK;
    }

    // Issue the copy of `block` into a victim slot; returns the slot or a negative status.
    int issue_copy(int block) {
        int victim = -1;
        for (int i = 0; i < int(slots.size()); ++i) {
            const auto& s = slots[i];
            if (s.held) continue;
            if (s.block < 0) {  // an empty slot is always the first choice
                victim = i;
                break;
            }
            if (victim < 0 || s.stamp < slots[victim].stamp) victim = i;
        }
        if (victim < 0)
            return fail(NF4_E_BUSY, "stream_pool: all %d slots are held; release a block before prefetching block %d",
                        int(slots.size()), block);
        auto& s = slots[victim];
        const Block& nb = blocks[block];
        char* dst = slab + size_t(victim) * slot_bytes;
        for (int k = 0; k < nb.count; ++k) {
            const int i = descending ? nb.count - 1 - k : k;
            const Part& p = parts[nb.first + i];
            // wait for every kept last use of the bytes this part overwrites
            for (size_t q = 0; q < s.pending.size();) {
                const LastUse& u = s.pending[q];
                if (u.lo >= p.off + p.bytes || p.off >= u.hi) {
                    ++q;
                    continue;
                }
                int st = eng->wait(copy, u.event);
                if (st != NF4_OK) return st;
                spare.push_back(u.event);
                s.pending[q] = s.pending.back();
                s.pending.pop_back();
            }
            int st = eng->copy(dst + p.off, p.host, p.bytes, copy, block, i);
            if (st == NF4_OK) st = eng->record(s.part_ready[i], copy);
            if (st != NF4_OK) return st;
        }
        int st = eng->record(s.ready, copy);
        if (st != NF4_OK) return st;
        if (s.block >= 0) {
            where[s.block] = -1;
            stats.evictions++;
        }
        s.block = block;
        s.stamp = ++clock;
        where[block] = victim;
        stats.copies++;
        stats.bytes_copied += nb.bytes;
        return victim;
    }

    int prefetch(int block) {
        int st = check_block(block, "stream_pool_prefetch");
        if (st != NF4_OK) return st;
        if (where[block] >= 0) return NF4_OK;  // already issued or resident
        st = issue_copy(block);
        return st < 0 ? st : NF4_OK;
    }

    // deferred: make no wait (the caller calls wait_part before it reads a part)
    int acquire(int block, Stream compute, const void** dev, bool deferred = false) {
        const char* fn = deferred ? "stream_pool_acquire_deferred" : "stream_pool_acquire";
        int st = check_block(block, fn);
        if (st != NF4_OK) return st;
        if (!dev) return fail(NF4_E_ARG, "%s: NULL dev", fn);
        int slot = where[block];
        if (slot >= 0 && slots[slot].held) return fail(NF4_E_STATE, "%s: block %d is already held", fn, block);
        if (slot < 0) {
            slot = issue_copy(block);
            if (slot < 0) return slot;
            stats.misses++;
        } else {
            stats.hits++;
        }
        auto& s = slots[slot];
        if (!deferred) {
            st = eng->acquire_wait(compute, s.ready, block, -1);
            if (st != NF4_OK) return st;
        }
        s.held = true;
        s.stamp = ++clock;
        for (auto& r : s.released) r = 0;
        *dev = slab + size_t(slot) * slot_bytes;
        return NF4_OK;
    }

    int held_slot(int block, const char* fn) {
        int st = check_block(block, fn);
        if (st != NF4_OK) return st;
        const int slot = where[block];
        if (slot < 0 || !slots[slot].held) return fail(NF4_E_STATE, "%s: block %d is not held", fn, block);
        return slot;
    }

    // make `stream` wait for the copy of one part of a held block
    int wait_part(int block, int part, Stream stream) {
        const int slot = held_slot(block, "stream_pool_wait_part");
        if (slot < 0) return slot;
        if (part < 0 || part >= blocks[block].count)
            return fail(NF4_E_ARG, "stream_pool_wait_part: part %d outside 0..%d of block %d", part,
                        blocks[block].count - 1, block);
        return eng->acquire_wait(stream, slots[slot].part_ready[part], block, part);
    }

    int release_part(int block, int part, Stream compute) {
        const int slot = held_slot(block, "stream_pool_release_part");
        if (slot < 0) return slot;
        if (part < 0 || part >= blocks[block].count)
            return fail(NF4_E_ARG, "stream_pool_release_part: part %d outside 0..%d of block %d", part,
                        blocks[block].count - 1, block);
        auto& s = slots[slot];
        if (s.released[part])
            return fail(NF4_E_STATE, "stream_pool_release_part: part %d of block %d is already released", part, block);
        const Part& p = parts[blocks[block].first + part];
        int st = record_last_use(s, p.off, p.off + p.bytes, compute);
        if (st != NF4_OK) return st;
        s.released[part] = 1;
        return NF4_OK;
    }

    int release(int block, Stream compute) {
        const int slot = held_slot(block, "stream_pool_release");
        if (slot < 0) return slot;
        auto& s = slots[slot];
        const Block& b = blocks[block];
        // one last use covering the parts not released one by one, when they are contiguous
        // (always, for a release with no part released before); else one per part
        int lo = -1, hi = -1;
        bool contiguous = true;
        for (int i = 0; i < b.count; ++i) {
            if (s.released[i]) continue;
            if (lo < 0) lo = i;
            else if (hi != i - 1) contiguous = false;
            hi = i;
        }
        if (lo >= 0 && contiguous) {
            const Part& a = parts[b.first + lo];
            const Part& z = parts[b.first + hi];
            int st = record_last_use(s, a.off, z.off + z.bytes, compute);
            if (st != NF4_OK) return st;
        } else {
            for (int i = 0; i < b.count; ++i) {
                if (s.released[i]) continue;
                const Part& p = parts[b.first + i];
                int st = record_last_use(s, p.off, p.off + p.bytes, compute);
                if (st != NF4_OK) return st;
            }
        }
        s.held = false;
        s.stamp = ++clock;
        return bound_lead(compute);
    }

    // the host's lead over the device (set_max_ahead): mark this release, then wait
    // for the mark max_ahead releases back
    int bound_lead(Stream compute) {
        if (max_ahead <= 0) return NF4_OK;
        Event e{};
        int st = take_event(&e);
        if (st != NF4_OK) return st;
        st = eng->record(e, compute);
        if (st != NF4_OK) {
            spare.push_back(e);
            return st;
        }
        ahead.push_back(e);
        while (int(ahead.size()) > max_ahead) {
            st = eng->host_wait(ahead.front());
            if (st != NF4_OK) return st;
            spare.push_back(ahead.front());
            ahead.pop_front();
        }
        return NF4_OK;
    }

    int set_max_ahead(int n) {
        if (n < 0) return fail(NF4_E_ARG, "stream_pool_set_max_ahead: n must be >= 0 (got %d)", n);
        max_ahead = n;
        while (int(ahead.size()) > (n > 0 ? n : 0)) {  // a lower bound applies at once
            int st = eng->host_wait(ahead.front());
            if (st != NF4_OK) return st;
            spare.push_back(ahead.front());
            ahead.pop_front();
        }
        return NF4_OK;
    }
};

}  // namespace nf4
