// Blockwise residency of the frozen NF4 base on HIP: the pool state machine of
// pool_core.h driven by a HIP engine (hipMemcpyAsync on the dedicated copy stream,
// hipEventRecord / hipStreamWaitEvent between the copy and compute streams), plus
// optional timing spans for the copy/compute overlap. See pool_core.h for the ordering
// rules; the pages behind them: HN comment thread on streaming the frozen base (main
// comment); Poros API reference, "patch_hf_model" Behavior 4-6; "Poros on consumer
// GPUs", "What you need besides VRAM" (the streamed base lives in pinned host memory,
// needed for asynchronous copies).
#include <algorithm>
#include <chrono>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/nf4lora.h"
#include "common.h"
#include "pool_core.h"

using nf4::fail;

namespace {

int hip_ok(hipError_t e, const char* what) {
    if (e != hipSuccess) return fail(NF4_E_HIP, "%s: %s", what, hipGetErrorString(e));
    return NF4_OK;
}

struct HipEngine {
    using Event = hipEvent_t;
    using Stream = hipStream_t;
    struct Span {  // two timing events around one interval on one stream
        hipEvent_t a = nullptr, b = nullptr;
        int kind = 0, block = -1, part = -1;
        double host_at_ms = 0.0, host_call_ms = 0.0;  // host clock at the issuing call, its duration
    };
    // timing (stream_pool_timing_enable): copy spans on the copy stream, stall spans
    // around each acquire's wait on the compute stream, and recycled events
    bool timing = false;
    std::vector<Span> copy_spans, stall_spans;
    std::vector<hipEvent_t> spare;
    // host time spent inside the pool's HIP calls, whether or not the device spans are
    // recorded (a call that blocks the host shows here, not in the device spans)
    // per kind of call: 0 copy issue, 1 event record, 2 stream wait, 3 host wait for an event
    double host_ms = 0.0, host_max_ms = 0.0, host_kind_ms[4] = {0.0, 0.0, 0.0, 0.0};
    double last_call_ms = 0.0, last_call_at_ms = 0.0;
    const std::chrono::steady_clock::time_point origin = std::chrono::steady_clock::now();

    template <class F>
    hipError_t host_timed(int kind, F&& call) {
        const auto t0 = std::chrono::steady_clock::now();
        const hipError_t e = call();
        const auto t1 = std::chrono::steady_clock::now();
        const double ms = std::chrono::duration<double, std::milli>(t1 - t0).count();
        host_ms += ms;
        host_kind_ms[kind] += ms;
        if (ms > host_max_ms) host_max_ms = ms;
        last_call_ms = ms;
        last_call_at_ms = std::chrono::duration<double, std::milli>(t0 - origin).count();
        return e;
    }

    int create_event(hipEvent_t* e) {
        return hip_ok(hipEventCreateWithFlags(e, hipEventDisableTiming), "stream_pool: hipEventCreate");
    }
    void destroy_event(hipEvent_t e) {
        if (e) (void)hipEventDestroy(e);
    }
    int record(hipEvent_t e, hipStream_t s) {
        return hip_ok(host_timed(1, [&] { return hipEventRecord(e, s); }), "stream_pool: record event");
    }
    int wait(hipStream_t s, hipEvent_t e) {
        return hip_ok(host_timed(2, [&] { return hipStreamWaitEvent(s, e, 0); }), "stream_pool: wait event");
    }
    int host_wait(hipEvent_t e) {
        return hip_ok(host_timed(3, [&] { return hipEventSynchronize(e); }), "stream_pool: host wait for a release");
    }

    hipEvent_t timing_event() {
        if (!spare.empty()) {
            hipEvent_t e = spare.back();
            spare.pop_back();
            return e;
        }
        hipEvent_t e = nullptr;
        return hipEventCreate(&e) == hipSuccess ? e : nullptr;
    }
    int span_begin(Span& sp, hipStream_t stream) {
        if (!timing) return NF4_OK;
        sp.a = timing_event();
        sp.b = timing_event();
        if (!sp.a || !sp.b) return fail(NF4_E_HIP, "stream_pool: hipEventCreate failed (timing)");
        return hip_ok(hipEventRecord(sp.a, stream), "stream_pool: record timing event");
    }
    // closes the span and tags it with the call it timed (the engine's last HIP call)
    int span_end(Span& sp, hipStream_t stream, std::vector<Span>& into, int kind, int block, int part) {
        if (!timing) return NF4_OK;
        int st = hip_ok(hipEventRecord(sp.b, stream), "stream_pool: record timing event");
        sp.kind = kind;
        sp.block = block;
        sp.part = part;
        sp.host_at_ms = last_call_at_ms;
        sp.host_call_ms = last_call_ms;
        if (st == NF4_OK) into.push_back(sp);
        return st;
    }

    // one part's H2D copy (after its waits: the span is the copy alone)
    int copy(void* dst, const void* src, size_t bytes, hipStream_t s, int block, int part) {
        Span sp;
        int st = span_begin(sp, s);
        if (st == NF4_OK)
            st = hip_ok(host_timed(0, [&] { return hipMemcpyAsync(dst, src, bytes, hipMemcpyHostToDevice, s); }),
                        "stream_pool: H2D copy");
        if (st == NF4_OK) st = span_end(sp, s, copy_spans, NF4_SPAN_COPY, block, part);
        return st;
    }
    // a compute stream's wait for a block's (part = -1) or one part's copy (the span is
    // the time it stood still)
    int acquire_wait(hipStream_t compute, hipEvent_t ready, int block, int part) {
        Span sp;
        int st = span_begin(sp, compute);
        if (st == NF4_OK) st = wait(compute, ready);
        if (st == NF4_OK) st = span_end(sp, compute, stall_spans, NF4_SPAN_ACQUIRE, block, part);
        return st;
    }

    void destroy_spans() {
        for (auto* v : {&copy_spans, &stall_spans})
            for (auto& sp : *v) {
                (void)hipEventSynchronize(sp.b);  // their work is already enqueued
                (void)hipEventDestroy(sp.a);
                (void)hipEventDestroy(sp.b);
            }
        for (hipEvent_t e : spare) (void)hipEventDestroy(e);
        copy_spans.clear();
        stall_spans.clear();
        spare.clear();
    }
};

}  // namespace

struct nf4_pool {
    HipEngine eng;
    nf4::PoolCore<HipEngine> core;
};

namespace {

int create(const nf4_host_block* parts, const int* part_begin, int n_blocks, void* device_slab, size_t slot_bytes,
           int n_slots, nf4_stream copy_stream, nf4_pool** out) {
    if (!out) return fail(NF4_E_ARG, "stream_pool_create: NULL out");
    *out = nullptr;
    auto* p = new nf4_pool;
    const int st = p->core.init(&p->eng, parts, part_begin, n_blocks, device_slab, slot_bytes, n_slots,
                                static_cast<hipStream_t>(copy_stream), copy_stream != nullptr);
    if (st != NF4_OK) {
        p->core.destroy_events();
        delete p;
        return st;
    }
    *out = p;
    return NF4_OK;
}

}  // namespace

extern "C" {

int stream_pool_create(const nf4_host_block* blocks, int n_blocks, void* device_slab, size_t slot_bytes, int n_slots,
                       nf4_stream copy_stream, nf4_pool** out) {
    if (n_blocks <= 0 || !blocks) return create(blocks, nullptr, n_blocks, device_slab, slot_bytes, n_slots, copy_stream, out);
    std::vector<int> begin(size_t(n_blocks) + 1);
    for (int b = 0; b <= n_blocks; ++b) begin[b] = b;  // one part per block
    return create(blocks, begin.data(), n_blocks, device_slab, slot_bytes, n_slots, copy_stream, out);
}

int stream_pool_create_parts(const nf4_host_block* parts, const int* part_begin, int n_blocks, void* device_slab,
                             size_t slot_bytes, int n_slots, nf4_stream copy_stream, nf4_pool** out) {
    return create(parts, part_begin, n_blocks, device_slab, slot_bytes, n_slots, copy_stream, out);
}

int stream_pool_set_order(nf4_pool* p, int descending) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_set_order: NULL pool");
    p->core.descending = descending != 0;
    return NF4_OK;
}

int stream_pool_prefetch(nf4_pool* p, int block) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_prefetch: NULL pool");
    return p->core.prefetch(block);
}

int stream_pool_acquire(nf4_pool* p, int block, nf4_stream compute, const void** dev) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_acquire: NULL pool");
    return p->core.acquire(block, static_cast<hipStream_t>(compute), dev);
}

int stream_pool_acquire_deferred(nf4_pool* p, int block, nf4_stream compute, const void** dev) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_acquire_deferred: NULL pool");
    return p->core.acquire(block, static_cast<hipStream_t>(compute), dev, true);
}

int stream_pool_wait_part(nf4_pool* p, int block, int part, nf4_stream stream) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_wait_part: NULL pool");
    return p->core.wait_part(block, part, static_cast<hipStream_t>(stream));
}

int stream_pool_set_max_ahead(nf4_pool* p, int blocks) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_set_max_ahead: NULL pool");
    return p->core.set_max_ahead(blocks);
}

int stream_pool_release_part(nf4_pool* p, int block, int part, nf4_stream compute) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_release_part: NULL pool");
    return p->core.release_part(block, part, static_cast<hipStream_t>(compute));
}

int stream_pool_release(nf4_pool* p, int block, nf4_stream compute) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_release: NULL pool");
    return p->core.release(block, static_cast<hipStream_t>(compute));
}

int stream_pool_stats(const nf4_pool* p, nf4_pool_stats* out) {
    if (!p || !out) return fail(NF4_E_ARG, "stream_pool_stats: NULL argument");
    *out = p->core.stats;
    return NF4_OK;
}

int stream_pool_slot_block(const nf4_pool* p, int slot, int* block_out) {
    if (!p || !block_out) return fail(NF4_E_ARG, "stream_pool_slot_block: NULL argument");
    if (slot < 0 || slot >= int(p->core.slots.size()))
        return fail(NF4_E_ARG, "stream_pool_slot_block: slot %d outside 0..%d", slot, int(p->core.slots.size()) - 1);
    *block_out = p->core.slots[slot].block;
    return NF4_OK;
}

int stream_pool_streams(nf4_stream* compute_out, nf4_stream* copy_out) {
    if (!compute_out || !copy_out) return fail(NF4_E_ARG, "stream_pool_streams: NULL argument");
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static hipStream_t pairs[kMaxDevices][2] = {};
    int dev = 0;
    int st = hip_ok(hipGetDevice(&dev), "stream_pool_streams: hipGetDevice");
    if (st != NF4_OK) return st;
    if (dev < 0 || dev >= kMaxDevices)
        return fail(NF4_E_ARG, "stream_pool_streams: device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(mu);
    if (!pairs[dev][0]) {
        // back to back, so that HIP gives them different hardware queues
        hipStream_t c = nullptr, k = nullptr;
        st = hip_ok(hipStreamCreateWithFlags(&c, hipStreamNonBlocking), "stream_pool_streams: create compute stream");
        if (st == NF4_OK)
            st = hip_ok(hipStreamCreateWithFlags(&k, hipStreamNonBlocking), "stream_pool_streams: create copy stream");
        if (st != NF4_OK) {
            if (c) (void)hipStreamDestroy(c);
            return st;
        }
        pairs[dev][0] = c;
        pairs[dev][1] = k;
    }
    *compute_out = pairs[dev][0];
    *copy_out = pairs[dev][1];
    return NF4_OK;
}

int stream_pool_timing_enable(nf4_pool* p, int enable) {
    if (!p) return fail(NF4_E_ARG, "stream_pool_timing_enable: NULL pool");
    p->eng.timing = enable != 0;
    return NF4_OK;
}

int stream_pool_timing_collect(nf4_pool* p, nf4_pool_timing* out) {
    if (!p || !out) return fail(NF4_E_ARG, "stream_pool_timing_collect: NULL argument");
    *out = nf4_pool_timing{};
    int st = NF4_OK;
    auto sum = [&](std::vector<HipEngine::Span>& spans, double& ms, uint64_t& count) {
        for (auto& sp : spans) {
            float v = 0.0f;
            if (st == NF4_OK) st = hip_ok(hipEventSynchronize(sp.b), "stream_pool_timing_collect: wait");
            if (st == NF4_OK) st = hip_ok(hipEventElapsedTime(&v, sp.a, sp.b), "stream_pool_timing_collect: elapsed");
            ms += v;
            count++;
            p->eng.spare.push_back(sp.a);
            p->eng.spare.push_back(sp.b);
        }
        spans.clear();
    };
    sum(p->eng.copy_spans, out->copy_ms, out->copies);
    sum(p->eng.stall_spans, out->stall_ms, out->acquires);
    out->host_ms = p->eng.host_ms;
    out->host_max_ms = p->eng.host_max_ms;
    out->host_copy_ms = p->eng.host_kind_ms[0];
    out->host_record_ms = p->eng.host_kind_ms[1];
    out->host_wait_ms = p->eng.host_kind_ms[2];
    out->host_sync_ms = p->eng.host_kind_ms[3];
    p->eng.host_ms = p->eng.host_max_ms = 0.0;
    for (double& v : p->eng.host_kind_ms) v = 0.0;
    return st;
}

int stream_pool_timing_spans(nf4_pool* p, nf4_pool_span* out, int max_spans, int* n_out) {
    if (!p || !n_out || max_spans < 0 || (max_spans > 0 && !out))
        return fail(NF4_E_ARG, "stream_pool_timing_spans: need pool, n_out, max_spans >= 0 and out when max_spans > 0");
    std::vector<const HipEngine::Span*> all;
    for (auto* v : {&p->eng.copy_spans, &p->eng.stall_spans})
        for (auto& sp : *v) all.push_back(&sp);
    *n_out = int(all.size());
    if (all.empty()) return NF4_OK;
    int st = NF4_OK;
    for (const auto* sp : all)
        if (st == NF4_OK) st = hip_ok(hipEventSynchronize(sp->b), "stream_pool_timing_spans: wait");
    if (st != NF4_OK) return st;
    // origin: the earliest span start on the device; host times from the same span's call
    const HipEngine::Span* first = all[0];
    for (const auto* sp : all) {
        float d = 0.0f;
        st = hip_ok(hipEventElapsedTime(&d, first->a, sp->a), "stream_pool_timing_spans: elapsed");
        if (st != NF4_OK) return st;
        if (d < 0.0f) first = sp;
    }
    const int n = std::min(max_spans, int(all.size()));
    for (int i = 0; i < n; ++i) {
        const auto* sp = all[size_t(i)];
        float a = 0.0f, b = 0.0f;
        st = hip_ok(hipEventElapsedTime(&a, first->a, sp->a), "stream_pool_timing_spans: elapsed");
        if (st == NF4_OK) st = hip_ok(hipEventElapsedTime(&b, first->a, sp->b), "stream_pool_timing_spans: elapsed");
        if (st != NF4_OK) return st;
        out[i] = nf4_pool_span{sp->kind, sp->block, sp->part, 0, double(a), double(b),
                               sp->host_at_ms - first->host_at_ms, sp->host_call_ms};
    }
    return NF4_OK;
}

int stream_pool_destroy(nf4_pool* p) {
    if (!p) return NF4_OK;
    int st = NF4_OK;
    if (p->core.copy) st = hip_ok(hipStreamSynchronize(p->core.copy), "stream_pool_destroy: drain copy stream");
    p->core.destroy_events();
    p->eng.destroy_spans();
    delete p;
    return st;
}

}  // extern "C"

extern "C" int nf4_block_layout(const int64_t* shapes, int n_proj, int layers, int dense, size_t* offsets_out,
                                size_t* bytes_out) {
    if (!shapes || !bytes_out || n_proj <= 0 || layers <= 0)
        return fail(NF4_E_ARG, "nf4_block_layout: need shapes, bytes_out, n_proj > 0 and layers > 0 (got n_proj=%d "
                               "layers=%d)", n_proj, layers);
    for (int j = 0; j < n_proj; ++j) {
        const int64_t n = shapes[2 * j], k = shapes[2 * j + 1];
        if (n <= 0 || k <= 0 || k % NF4_BLOCK != 0 || n > (int64_t(1) << 21) || k > (int64_t(1) << 21))
            return fail(NF4_E_SHAPE, "nf4_block_layout: projection %d has N=%lld K=%lld (need N, K in 1..2^21, K %% %d "
                                     "== 0)", j, (long long)n, (long long)k, NF4_BLOCK);
    }
    auto align = [](size_t v) { return (v + 255) & ~size_t(255); };
    size_t off = 0;
    for (int l = 0; l < layers; ++l)
        for (int j = 0; j < n_proj; ++j) {
            const size_t n = size_t(shapes[2 * j]), k = size_t(shapes[2 * j + 1]);
            size_t* o = offsets_out ? offsets_out + (size_t(l) * n_proj + j) * 2 : nullptr;
            if (dense) {
                if (o) o[0] = off, o[1] = 0;
                off = align(off + n * k * 2);
            } else {
                if (o) o[0] = off;
                off = align(off + n * k / 2);
                if (o) o[1] = off;
                off = align(off + n * (k / NF4_BLOCK) * 4);
            }
        }
    *bytes_out = off;
    return NF4_OK;
}
