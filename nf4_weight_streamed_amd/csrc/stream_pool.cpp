// Blockwise residency of the frozen NF4 base: a pool of pre-allocated device
// slots fed from pinned host slabs on a dedicated copy stream.
//
// HN comment thread on streaming the frozen base (main comment): the base sits
// in host RAM and streams into a small pool of pre-allocated device buffers,
// prefetched one ahead on a dedicated stream. Poros API reference,
// "patch_hf_model" Behavior 5-6: layers regrouped into blocks; a block manager
// with cross-stream safety. "Poros on consumer GPUs", "What you need besides
// VRAM": the streamed base lives in pinned host memory, needed for async copies.
//
// Ordering is carried entirely by HIP events on the two streams:
//   ready[slot]    recorded on the copy stream after the block's H2D copy;
//                  acquire makes the compute stream wait on it;
//   last_use[slot] recorded on the compute stream at release; the copy that
//                  later overwrites the slot waits on it first.
// The host never blocks (except in destroy), and a slot is never overwritten
// while a kernel enqueued before its release may still read it.
#include <cstdint>
#include <vector>

#include "../../include/nf4lora.h"
#include "common.h"

struct nf4_pool {
    struct Slot {
        int block = -1;
        bool held = false;
        bool has_last_use = false;
        uint64_t stamp = 0;
        hipEvent_t ready = nullptr;
        hipEvent_t last_use = nullptr;
    };
    std::vector<nf4_host_block> blocks;
    std::vector<int> where;  // block -> slot, or -1
    std::vector<Slot> slots;
    char* slab = nullptr;
    size_t slot_bytes = 0;
    hipStream_t copy = nullptr;
    uint64_t clock = 0;
    nf4_pool_stats stats{};
};

using nf4::fail;

namespace {

int hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NF4_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return NF4_OK;
}

int check_block(const nf4_pool* p, int block, const char* fn) {
    if (!p) return fail(NF4_E_ARG, "%s: NULL pool", fn);
    if (block < 0 || block >= int(p->blocks.size()))
        return fail(NF4_E_ARG, "%s: block %d outside 0..%d", fn, block, int(p->blocks.size()) - 1);
    return NF4_OK;
}

// Issue the copy of `block` into a victim slot; returns the slot or a negative status.
int issue_copy(nf4_pool* p, int block) {
    int victim = -1;
    for (int i = 0; i < int(p->slots.size()); ++i) {
        const auto& s = p->slots[i];
        if (s.held) continue;
        if (s.block < 0) {  // an empty slot is always the first choice
            victim = i;
            break;
        }
        if (victim < 0 || s.stamp < p->slots[victim].stamp) victim = i;
    }
    if (victim < 0)
        return fail(NF4_E_BUSY, "stream_pool: all %d slots are held; release a block before prefetching block %d",
                    int(p->slots.size()), block);
    auto& s = p->slots[victim];
    if (s.has_last_use) {
        int st = hip_ok(hipStreamWaitEvent(p->copy, s.last_use, 0), "stream_pool: wait for last use");
        if (st != NF4_OK) return st;
    }
    const nf4_host_block& hb = p->blocks[block];
    int st = hip_ok(hipMemcpyAsync(p->slab + size_t(victim) * p->slot_bytes, hb.host, hb.bytes,
                                   hipMemcpyHostToDevice, p->copy),
                    "stream_pool: H2D copy");
    if (st != NF4_OK) return st;
    st = hip_ok(hipEventRecord(s.ready, p->copy), "stream_pool: record ready");
    if (st != NF4_OK) return st;
    if (s.block >= 0) {
        p->where[s.block] = -1;
        p->stats.evictions++;
    }
    s.block = block;
    s.stamp = ++p->clock;
    p->where[block] = victim;
    p->stats.copies++;
    p->stats.bytes_copied += hb.bytes;
    return victim;
}

}  // namespace

extern "C" {

int stream_pool_create(const nf4_host_block* blocks, int n_blocks, void* device_slab, size_t slot_bytes, int n_slots,
                       nf4_stream copy_stream, nf4_pool** out) {
    if (!out) return fail(NF4_E_ARG, "stream_pool_create: NULL out");
    *out = nullptr;
    if (!blocks || n_blocks <= 0 || n_slots <= 0 || !device_slab || !copy_stream)
        return fail(NF4_E_ARG, "stream_pool_create: need blocks, n_blocks > 0, n_slots > 0, a device slab and a copy "
                               "stream (got n_blocks=%d n_slots=%d)", n_blocks, n_slots);
    if (slot_bytes == 0 || slot_bytes % 256 != 0 || reinterpret_cast<uintptr_t>(device_slab) % 256 != 0)
        return fail(NF4_E_ARG, "stream_pool_create: slot_bytes (%zu) and the slab address must be multiples of 256",
                    slot_bytes);
    for (int b = 0; b < n_blocks; ++b) {
        if (!blocks[b].host) return fail(NF4_E_ARG, "stream_pool_create: block %d has a NULL host pointer", b);
        if (blocks[b].bytes > slot_bytes)
            return fail(NF4_E_OOM, "stream_pool_create: block %d needs %zu bytes but a slot holds %zu (%d slots, %zu "
                                   "bytes of device slab requested)", b, blocks[b].bytes, slot_bytes, n_slots,
                        slot_bytes * size_t(n_slots));
    }
    auto* p = new nf4_pool;
    p->blocks.assign(blocks, blocks + n_blocks);
    p->where.assign(n_blocks, -1);
    p->slots.resize(n_slots);
    p->slab = static_cast<char*>(device_slab);
    p->slot_bytes = slot_bytes;
    p->copy = static_cast<hipStream_t>(copy_stream);
    for (auto& s : p->slots) {
        if (hipEventCreateWithFlags(&s.ready, hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&s.last_use, hipEventDisableTiming) != hipSuccess) {
            stream_pool_destroy(p);
            return fail(NF4_E_HIP, "stream_pool_create: hipEventCreate failed");
        }
    }
    *out = p;
    return NF4_OK;
}

int stream_pool_prefetch(nf4_pool* p, int block) {
    int st = check_block(p, block, "stream_pool_prefetch");
    if (st != NF4_OK) return st;
    if (p->where[block] >= 0) return NF4_OK;  // already issued or resident
    st = issue_copy(p, block);
    return st < 0 ? st : NF4_OK;
}

int stream_pool_acquire(nf4_pool* p, int block, nf4_stream compute, const void** dev) {
    int st = check_block(p, block, "stream_pool_acquire");
    if (st != NF4_OK) return st;
    if (!dev) return fail(NF4_E_ARG, "stream_pool_acquire: NULL dev");
    int slot = p->where[block];
    if (slot >= 0 && p->slots[slot].held)
        return fail(NF4_E_STATE, "stream_pool_acquire: block %d is already held", block);
    if (slot < 0) {
        slot = issue_copy(p, block);
        if (slot < 0) return slot;
        p->stats.misses++;
    } else {
        p->stats.hits++;
    }
    auto& s = p->slots[slot];
    st = hip_ok(hipStreamWaitEvent(static_cast<hipStream_t>(compute), s.ready, 0), "stream_pool_acquire: wait");
    if (st != NF4_OK) return st;
    s.held = true;
    s.stamp = ++p->clock;
    *dev = p->slab + size_t(slot) * p->slot_bytes;
    return NF4_OK;
}

int stream_pool_release(nf4_pool* p, int block, nf4_stream compute) {
    int st = check_block(p, block, "stream_pool_release");
    if (st != NF4_OK) return st;
    const int slot = p->where[block];
    if (slot < 0 || !p->slots[slot].held)
        return fail(NF4_E_STATE, "stream_pool_release: block %d is not held", block);
    auto& s = p->slots[slot];
    st = hip_ok(hipEventRecord(s.last_use, static_cast<hipStream_t>(compute)), "stream_pool_release: record");
    if (st != NF4_OK) return st;
    s.held = false;
    s.has_last_use = true;
    s.stamp = ++p->clock;
    return NF4_OK;
}

int stream_pool_stats(const nf4_pool* p, nf4_pool_stats* out) {
    if (!p || !out) return fail(NF4_E_ARG, "stream_pool_stats: NULL argument");
    *out = p->stats;
    return NF4_OK;
}

int stream_pool_slot_block(const nf4_pool* p, int slot, int* block_out) {
    if (!p || !block_out) return fail(NF4_E_ARG, "stream_pool_slot_block: NULL argument");
    if (slot < 0 || slot >= int(p->slots.size()))
        return fail(NF4_E_ARG, "stream_pool_slot_block: slot %d outside 0..%d", slot, int(p->slots.size()) - 1);
    *block_out = p->slots[slot].block;
    return NF4_OK;
}

int stream_pool_destroy(nf4_pool* p) {
    if (!p) return NF4_OK;
    int st = NF4_OK;
    if (p->copy) st = hip_ok(hipStreamSynchronize(p->copy), "stream_pool_destroy: drain copy stream");
    for (auto& s : p->slots) {
        if (s.ready) (void)hipEventDestroy(s.ready);
        if (s.last_use) (void)hipEventDestroy(s.last_use);
    }
    delete p;
    return st;
}

}  // extern "C"
