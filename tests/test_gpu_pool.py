"""The stream pool on the GPU: copies land intact, reuse is ordered, states are checked."""

import time

import pytest
import torch

pytestmark = pytest.mark.gpu


def _blocks(n, nbytes):
    out = []
    for b in range(n):
        h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(torch.arange(nbytes, dtype=torch.int64).add_(977 * b).remainder_(251).to(torch.uint8))
        out.append(h)
    return out


def test_pool_copies_and_states(gpu_lib):
    L = gpu_lib
    blocks = _blocks(4, 1 << 20)
    slot = 1 << 20
    slab = torch.empty(2 * slot, dtype=torch.uint8, device="cuda")
    cs = torch.cuda.Stream()
    pool = L.StreamPool(blocks, slab, slot, 2, cs)
    try:
        for b in range(4):
            ptr = pool.acquire(b)
            s = (ptr - slab.data_ptr()) // slot
            got = slab[s * slot:(s + 1) * slot].cpu()
            assert torch.equal(got, blocks[b]), b
            with pytest.raises(L.Nf4Error) as e:
                pool.acquire(b)
            assert e.value.code == L.NF4_E_STATE
            pool.release(b)
            with pytest.raises(L.Nf4Error) as e:
                pool.release(b)
            assert e.value.code == L.NF4_E_STATE
        st = pool.stats()
        assert st["copies"] == 4 and st["misses"] == 4 and st["hits"] == 0 and st["evictions"] == 2
        assert st["bytes_copied"] == 4 << 20
        # the two most recent blocks are still resident: acquiring one is a hit
        assert {pool.slot_block(0), pool.slot_block(1)} == {2, 3}
        pool.acquire(3)
        assert pool.stats()["hits"] == 1
        pool.prefetch(1)                   # evicts block 2: the only slot not held
        assert {pool.slot_block(0), pool.slot_block(1)} == {3, 1}
        pool.prefetch(3)                   # already in a slot: no copy
        assert pool.stats()["copies"] == 5
        pool.release(3)
    finally:
        pool.close()


def test_pool_busy_when_all_held(gpu_lib):
    L = gpu_lib
    blocks = _blocks(3, 4096)
    slab = torch.empty(2 * 4096, dtype=torch.uint8, device="cuda")
    pool = L.StreamPool(blocks, slab, 4096, 2, torch.cuda.Stream())
    try:
        pool.acquire(0)
        pool.acquire(1)
        with pytest.raises(L.Nf4Error) as e:
            pool.prefetch(2)
        assert e.value.code == L.NF4_E_BUSY
        with pytest.raises(L.Nf4Error) as e:
            pool.acquire(2)
        assert e.value.code == L.NF4_E_BUSY
        pool.release(0)
        ptr = pool.acquire(2)          # reuses block 0's slot after its release
        assert (ptr - slab.data_ptr()) // 4096 == 0
        assert torch.equal(slab[:4096].cpu(), blocks[2])
        with pytest.raises(L.Nf4Error) as e:
            pool.prefetch(7)
        assert e.value.code == L.NF4_E_ARG
    finally:
        pool.close()


def test_pool_reuse_waits_for_compute(gpu_lib):
    L = gpu_lib
    """A slot is overwritten only after the kernels enqueued before its release ran:
    a long chain of reads on the compute stream, then release + prefetch of another
    block into the same slot; the reads must all see the old block."""
    n = 1 << 22
    blocks = _blocks(2, n)
    slab = torch.empty(n, dtype=torch.uint8, device="cuda")
    pool = L.StreamPool(blocks, slab, n, 1, torch.cuda.Stream())
    try:
        ptr = pool.acquire(0)
        sums = []
        for _ in range(50):
            sums.append(slab.to(torch.int64).sum())          # reads on the compute stream
        pool.release(0)
        pool.prefetch(1)                                     # same (only) slot
        ptr = pool.acquire(1)
        after = slab.clone()
        pool.release(1)
        torch.cuda.synchronize()
        want = int(blocks[0].to(torch.int64).sum())
        assert all(int(s) == want for s in sums)
        assert torch.equal(after.cpu(), blocks[1])
    finally:
        pool.close()


def test_pool_parts_land_back_to_back_and_wait_per_part(gpu_lib):
    """Blocks of two parts in one slot: each part lands at its offset; the copy of a
    part waits for the release of the part it overwrites: reads of part 1 enqueued
    before its release all see the old block although part 0 was released first."""
    L = gpu_lib
    n = 1 << 22
    parts = _blocks(4, n)                       # blocks (0: parts 0, 1) and (1: parts 2, 3)
    slab = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    pool = L.StreamPool(parts, slab, 2 * n, 1, torch.cuda.Stream(), part_begin=[0, 2, 4])
    try:
        ptr = pool.acquire(0)
        assert ptr == slab.data_ptr()
        pool.release_part(0, 0)                 # part 0 done early
        sums = [slab[n:].to(torch.int64).sum() for _ in range(50)]   # long reads of part 1
        pool.release_part(0, 1)
        with pytest.raises(L.Nf4Error) as e:
            pool.release_part(0, 1)
        assert e.value.code == L.NF4_E_STATE
        pool.release(0)
        for descending in (True, False):
            pool.set_order(descending)
            pool.prefetch(1)                    # the only slot: overwrites block 0 part by part
            pool.acquire(1)
            after = slab.clone()
            pool.release(1)
            pool.prefetch(0)
            pool.acquire(0)
            back = slab.clone()
            pool.release(0)
            torch.cuda.synchronize()
            assert torch.equal(after[:n].cpu(), parts[2]) and torch.equal(after[n:].cpu(), parts[3])
            assert torch.equal(back[:n].cpu(), parts[0]) and torch.equal(back[n:].cpu(), parts[1])
        want = int(parts[1].to(torch.int64).sum())
        assert all(int(s) == want for s in sums)
    finally:
        pool.close()


def test_pinned_empty_is_exact_and_pinned(gpu_lib):
    t = gpu_lib.pinned_empty(1000)
    assert t.numel() == 1000 and t.is_pinned() and t.dtype == torch.uint8
    t.fill_(7)
    d = t.cuda(non_blocking=True)
    torch.cuda.synchronize()
    assert int(d.sum()) == 7000


def test_pool_streams_pair_overlaps_copies_with_compute(gpu_lib):
    """The library's compute/copy stream pair (stream_pool_streams): the same two
    streams on every call, and a 2-slot pass over 8 blocks on them overlaps each copy
    with the previous block's compute: its time stays near that of the copies alone,
    well below copies plus compute (which a copy stream on the compute stream's
    hardware queue would give)."""
    L = gpu_lib
    comp, copy = L.pool_streams()
    again = L.pool_streams()
    assert again[0].cuda_stream == comp.cuda_stream and again[1].cuda_stream == copy.cuda_stream
    assert comp.cuda_stream != copy.cuda_stream
    nb, nbytes = 8, 128 << 20
    host = L.pinned_empty(nb * nbytes)
    blocks = [host[i * nbytes:(i + 1) * nbytes] for i in range(nb)]
    slab = torch.empty(2 * nbytes, dtype=torch.uint8, device="cuda")
    a = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda", dtype=torch.bfloat16)
    c = torch.empty_like(a)
    pool = L.StreamPool(blocks, slab, nbytes, 2, copy)

    def work():
        for _ in range(2):
            torch.matmul(a, b, out=c)

    def one_pass(compute: bool):
        with torch.cuda.stream(comp):
            for i in range(nb):
                pool.acquire(i)
                if i + 1 < nb:
                    pool.prefetch(i + 1)
                if compute:
                    work()
                pool.release(i)

    def compute_only():
        with torch.cuda.stream(comp):
            for _ in range(nb):
                work()

    def timed(fn, *args):
        best = float("inf")
        for _ in range(3):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            fn(*args)
            torch.cuda.synchronize()
            best = min(best, time.perf_counter() - t0)
        return best

    try:
        one_pass(True)
        t_copy = timed(one_pass, False)
        t_comp = timed(compute_only)
        t_both = timed(one_pass, True)
        print(f"copies {t_copy * 1e3:.2f} ms, compute {t_comp * 1e3:.2f} ms, both {t_both * 1e3:.2f} ms", flush=True)
        assert t_comp > 0.3 * t_copy, "the compute must be long enough for the check to mean something"
        assert t_both < t_copy + 0.5 * t_comp, (t_copy, t_comp, t_both)
    finally:
        pool.close()


def test_pool_timing_spans_order_and_tags(gpu_lib):
    """stream_pool_timing_spans: one copy span per part copied (tagged with its block and
    part, in issue order, back to back on the copy stream: each starts after the previous
    one ended) and one acquire span per acquire, all completed, with the sums of
    timing_collect equal to the spans' durations."""
    L = gpu_lib
    n = 1 << 22
    parts = _blocks(6, n)                       # 3 blocks of two parts
    slab = torch.empty(2 * 2 * n, dtype=torch.uint8, device="cuda")
    comp, copy = L.pool_streams()
    pool = L.StreamPool(parts, slab, 2 * n, 2, copy, part_begin=[0, 2, 4, 6])
    try:
        assert pool.timing_spans() == []
        pool.timing_enable(True)
        with torch.cuda.stream(comp):
            for b in range(3):
                pool.acquire(b)
                if b + 1 < 3:
                    pool.prefetch(b + 1)
                pool.release(b)
        spans = pool.timing_spans()
        copies = [s for s in spans if s["kind"] == "copy"]
        acq = [s for s in spans if s["kind"] == "acquire"]
        assert [(s["block"], s["part"]) for s in copies] == [(0, 0), (0, 1), (1, 0), (1, 1), (2, 0), (2, 1)]
        assert [s["block"] for s in acq] == [0, 1, 2] and all(s["part"] == -1 for s in acq)
        assert min(s["start_ms"] for s in spans) == 0.0
        for s in spans:
            assert s["end_ms"] >= s["start_ms"] >= 0.0 and s["host_call_ms"] >= 0.0
        for a, b in zip(copies, copies[1:]):
            assert b["start_ms"] >= a["end_ms"] - 1e-3 and b["host_at_ms"] >= a["host_at_ms"]
        tm = pool.timing_collect()
        assert tm["copies"] == 6 and tm["acquires"] == 3
        assert abs(tm["copy_ms"] - sum(s["end_ms"] - s["start_ms"] for s in copies)) < 1e-2
        assert tm["host_ms"] >= tm["host_copy_ms"] > 0.0
        assert abs(tm["host_ms"] - tm["host_copy_ms"] - tm["host_record_ms"] - tm["host_wait_ms"]) < 1e-6
        assert pool.timing_spans() == []        # collect forgot them
    finally:
        comp.synchronize()
        pool.close()


def test_pool_deferred_acquire_waits_per_part_and_lead_bound(gpu_lib):
    """stream_pool_acquire_deferred + stream_pool_wait_part: each part read after its own
    wait holds that part's bytes, over passes that reuse one slot part by part in both
    orders; with a lead bound of one block the host never has more than one release
    outstanding (every release returns after the previous one completed), and the bytes
    are the same. Misuse: wait_part on a block not held, or a part outside it."""
    L = gpu_lib
    n = 1 << 22
    parts = _blocks(6, n)                       # 3 blocks of two parts
    slab = torch.empty(2 * n, dtype=torch.uint8, device="cuda")
    comp, copy = L.pool_streams()
    pool = L.StreamPool(parts, slab, 2 * n, 1, copy, part_begin=[0, 2, 4, 6])
    try:
        with pytest.raises(L.Nf4Error) as e:
            pool.wait_part(0, 0, comp)
        assert e.value.code == L.NF4_E_STATE
        with pytest.raises(L.Nf4Error) as e:
            pool.set_max_ahead(-1)
        assert e.value.code == L.NF4_E_ARG
        for ahead in (0, 1):
            pool.set_max_ahead(ahead)
            got = []
            with torch.cuda.stream(comp):
                for descending in (False, True):
                    pool.set_order(descending)
                    for b in (range(3) if not descending else range(2, -1, -1)):
                        ptr = pool.acquire_deferred(b, comp)
                        assert ptr == slab.data_ptr()
                        order = (1, 0) if descending else (0, 1)
                        for i in order:
                            pool.wait_part(b, i, comp)
                            got.append((b, i, slab[i * n:(i + 1) * n].clone()))
                            pool.release_part(b, i, comp)
                        if b == 0 and not descending:
                            with pytest.raises(L.Nf4Error) as e:
                                pool.wait_part(0, 2, comp)
                            assert e.value.code == L.NF4_E_ARG
                        pool.release(b, comp)
            comp.synchronize()
            for b, i, t in got:
                assert torch.equal(t.cpu(), parts[2 * b + i]), (ahead, b, i)
        tm = pool.timing_collect()
        assert tm["host_sync_ms"] >= 0.0
    finally:
        comp.synchronize()
        pool.close()
