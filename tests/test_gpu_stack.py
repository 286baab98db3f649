"""The streamed stack: against the fp64 oracle on a tiny stack, and streamed vs
resident bitwise ("Poros on consumer GPUs", "Use NF4": bitwise parity to a fully
resident run; "OOM playbook": block_size never affects parity; HN comment thread
on streaming the frozen base: max abs logit difference 0.0)."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, f32_of, to_dev_bf16

pytestmark = pytest.mark.gpu
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


@pytest.fixture(scope="module")
def ST(gpu_lib):
    from nf4_weight_streamed_amd import stack

    return stack


def _tiny(ST):
    return ST.StackDims(hidden=128, q=128, kv=32, inter=256, head_dim=32)


def _np_weights(dims, n_layers):
    return {(l, p): S.weight(*dims.shapes()[p], proj=p, layer=l) for l in range(n_layers) for p in PROJS}


def _np_lora(dims, n_layers, r=16):
    out = {}
    for l in range(n_layers):
        for p in PROJS:
            n, k = dims.shapes()[p]
            out[(l, p)] = (S.lora_a(r, k, proj=p, layer=l), S.lora_b(n, r, proj=p, layer=l, std=0.05))
    return out


def _tiny_stack(ST, n_layers, block_size):
    tiny = _tiny(ST)
    w = _np_weights(tiny, n_layers)
    lo = _np_lora(tiny, n_layers)
    base = ST.HostNF4Base(tiny, n_layers, block_size, lambda l, p, n, k: to_dev_bf16(w[(l, p)]))
    lora = ST.LoraParams(tiny, n_layers, 16, lambda l, p, n, k: tuple(to_dev_bf16(t) for t in lo[(l, p)]))
    return w, lo, base, lora


def test_tiny_stack_matches_oracle(ST):
    L, T, alpha = 3, 40, 32.0
    TINY = _tiny(ST)
    w, lo, base, lora = _tiny_stack(ST, L, 2)
    h0 = S.activations(T, TINY.hidden, tensor="h0")
    dh = S.activations(T, TINY.hidden, tensor="dH")
    st = ST.NF4Stack(base, lora, T, alpha, mode="streamed")
    out, dh0 = st.step(to_dev_bf16(h0), to_dev_bf16(dh))
    torch.cuda.synchronize()
    od = O.StackLayerDims(TINY.hidden, TINY.q, TINY.kv, TINY.inter, TINY.head_dim)
    layers = []
    for l in range(L):
        layer = {}
        for p in PROJS:
            codes, absmax = O.quantize(O.bf16_bits_to_f64(w[(l, p)]).astype(np.float32))
            layer[p] = (O.dequantize(codes, absmax), lo[(l, p)][0], lo[(l, p)][1])
        layers.append(layer)
    out_ref, saved = O.stack_forward(h0, layers, od, alpha)
    dh0_ref, grads = O.stack_backward(dh, layers, od, alpha, saved)
    assert O.rel_l2(O.bf16_bits_to_f64(bits_of(out)), out_ref) <= 2e-3
    assert O.rel_l2(O.bf16_bits_to_f64(bits_of(dh0)), dh0_ref) <= 2e-3
    for l in range(L):
        for p in PROJS:
            dA, dB = st.grads[l][p]
            if p in ("q", "k"):                     # identity mixing: exactly zero
                assert not torch.any(dA) and not torch.any(dB)
                assert not np.any(grads[l][p + "_dA"])
                continue
            assert O.rel_l2(f32_of(dA), grads[l][p + "_dA"]) <= 2e-3, (l, p)
            assert O.rel_l2(f32_of(dB), grads[l][p + "_dB"]) <= 2e-3, (l, p)
    st.close()


def _run(ST, base, lora, T, mode, **kw):
    """Two steps; the outputs and gradients of each are cloned as soon as it ends (the
    stack reuses its buffers), so step 1 - the one that starts from an empty pool - and
    step 2 - slots reused across steps - are both compared."""
    st = ST.NF4Stack(base, lora, T, 32.0, mode=mode, **kw)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h0 = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    res = {"steps": []}
    for _ in range(2):
        out, dh0 = st.step(h0, dh)
        res["steps"].append({"out": out.clone(), "dh0": dh0.clone(),
                             "grads": [{p: (a.clone(), b.clone()) for p, (a, b) in gl.items()} for gl in st.grads]})
    torch.cuda.synchronize()
    res["stats"] = st.pool.stats()
    res["out"], res["dh0"] = res["steps"][0]["out"], res["steps"][0]["dh0"]
    st.close()
    return res


def _same(a, b):
    """Both steps of run a equal those of run b bit for bit, and each run's two steps
    equal each other."""
    for sa, sb in zip(a["steps"], b["steps"]):
        assert torch.equal(sa["out"], sb["out"]) and torch.equal(sa["dh0"], sb["dh0"])
        for ga, gb in zip(sa["grads"], sb["grads"]):
            for p in PROJS:
                assert torch.equal(ga[p][0], gb[p][0]) and torch.equal(ga[p][1], gb[p][1])
    for run in (a, b):
        s1, s2 = run["steps"]
        assert torch.equal(s1["out"], s2["out"]) and torch.equal(s1["dh0"], s2["dh0"])


def test_stack_is_ordered_with_the_caller_stream(ST):
    """The stack runs on the library's compute stream, after the caller's stream's
    earlier work and before its later work: inputs written late on a side stream (behind
    a bounded spin) are the ones read, and outputs cloned on that stream right after the
    step are complete - the bits equal those of a step called from the default stream."""
    _, _, base, lora = _tiny_stack(ST, 5, 2)
    T = 48
    st = ST.NF4Stack(base, lora, T, 32.0, mode="streamed")
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h0_src = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh_src = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    out, dh0 = st.step(h0_src, dh_src)
    ref = (out.clone(), dh0.clone())
    h0, dh = torch.zeros_like(h0_src), torch.zeros_like(dh_src)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        torch.cuda._sleep(10_000_000)
        h0.copy_(h0_src)
        dh.copy_(dh_src)
        out, dh0 = st.step(h0, dh)
        got = (out.clone(), dh0.clone())
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])
    st.close()


@pytest.mark.parametrize("block_size", [1, 2, 3])
def test_streamed_equals_resident_tiny(ST, block_size):
    L, T = 7, 48
    _, _, base, lora = _tiny_stack(ST, L, block_size)
    ref = _run(ST, base, lora, T, "resident")
    assert ref["stats"]["copies"] == base.n_blocks and ref["stats"]["misses"] == 0
    for kw in ({"prefetch": True, "n_slots": 2}, {"prefetch": False, "n_slots": 2}, {"prefetch": True, "n_slots": 3},
               {"prefetch": False, "n_slots": 1}, {"prefetch": True, "n_slots": 2, "layer_parts": False},
               {"prefetch": True, "n_slots": 3, "layer_parts": False}, {"prefetch": False, "n_slots": 1, "layer_parts": False},
               {"prefetch": True, "n_slots": 2, "max_ahead": 0}, {"prefetch": True, "n_slots": 2, "max_ahead": 1},
               {"prefetch": True, "n_slots": 2, "layer_parts": False, "max_ahead": 0}):
        got = _run(ST, base, lora, T, "streamed", **kw)
        _same(got, ref)
        if kw["prefetch"] and base.n_blocks > 2:
            assert got["stats"]["misses"] == 1       # only block 0 of the first forward


@pytest.mark.parametrize("block_size", [1, 2, 3])
def test_remat_equals_stored_activations_tiny(ST, block_size):
    """Rematerialisation (block-boundary states kept, each block's forward recomputed in
    its backward visit) gives bitwise the results of the stored-activation run, in both
    modes, with fewer activation bytes."""
    L, T = 7, 48
    _, _, base, lora = _tiny_stack(ST, L, block_size)
    ref = _run(ST, base, lora, T, "resident")
    for mode, kw in (("resident", {}), ("streamed", {"prefetch": True}), ("streamed", {"prefetch": False})):
        got = _run(ST, base, lora, T, mode, remat=True, **kw)
        _same(got, ref)
    full = ST.NF4Stack(base, lora, T, 32.0, mode="resident")
    rem = ST.NF4Stack(base, lora, T, 32.0, mode="resident", remat=True)
    assert rem.activation_bytes() < full.activation_bytes()
    full.close()
    rem.close()


def test_block_size_never_changes_results(ST):
    L, T = 6, 32
    runs = []
    for bs in (1, 2, 4, 6):
        _, _, base, lora = _tiny_stack(ST, L, bs)
        runs.append(_run(ST, base, lora, T, "streamed"))
    for r in runs[1:]:
        _same(r, runs[0])


def test_regrouped_blocks_share_the_host_bytes(ST):
    """regroup(block_size) groups the same pinned layer buffers: block b is layers
    [b bs, (b + 1) bs), copied back to back into a slot, which then holds the slab
    nf4_block_layout gives for that many layers; results do not depend on the grouping."""
    _, _, base, lora = _tiny_stack(ST, 5, 1)
    for bs in (2, 3, 5):
        g = base.regroup(bs)
        assert [t.data_ptr() for t in g.layers] == [t.data_ptr() for t in base.layers]
        assert g.n_blocks == (5 + bs - 1) // bs and g.part_begin[-1] == 5
        assert g.block_bytes == [min(bs, 5 - b * bs) * base.layer_bytes for b in range(g.n_blocks)]
    ref = _run(ST, base, lora, 24, "resident")
    _same(_run(ST, base.regroup(2), lora, 24, "streamed"), ref)
    st = ST.NF4Stack(base.regroup(3), lora, 24, 32.0, mode="resident")
    for b in range(2):                       # each slot holds its block's layers back to back
        ptr = st.pool.acquire(b)
        off = ptr - st.slab.data_ptr()
        for i in range(min(3, 5 - 3 * b)):
            got = st.slab[off + i * base.layer_bytes: off + (i + 1) * base.layer_bytes].cpu()
            assert torch.equal(got, base.layers[3 * b + i])
        st.pool.release(b)
    st.close()


def test_qwen7b_stack_streamed_equals_resident(ST):
    """28 Qwen2.5-7B-shaped layers, block_size 4, 512 tokens: streamed (2 slots,
    prefetch one ahead), with stored and with recomputed activations, vs fully
    resident, bitwise."""
    dims, L = ST.QWEN25["7b"]
    base = ST.HostNF4Base(dims, L, 4, ST.qwen_weight_fn())
    lora = ST.LoraParams(dims, L, 16, ST.qwen_lora_fn())
    ref = _run(ST, base, lora, 512, "resident")
    got = _run(ST, base, lora, 512, "streamed")
    _same(got, ref)
    got = _run(ST, base, lora, 512, "streamed", remat=True)
    _same(got, ref)
    _same(_run(ST, base, lora, 512, "streamed", layer_parts=False), ref)   # one copy and one wait per block
    assert torch.isfinite(ref["out"].float()).all() and torch.isfinite(ref["dh0"].float()).all()
    assert got["stats"]["bytes_copied"] > 2 * base.total_bytes()


def _big_stack_parity(ST, model, cases):
    """Streamed (two slots, prefetch one ahead) vs fully resident, bitwise, on one
    host copy of the base regrouped for each block size; `cases` = [(tokens,
    [block sizes])]. The resident result does not depend on the block size either."""
    dims, L = ST.QWEN25[model]
    print(f"{model} stack: loading {L} layers", flush=True)
    base = ST.HostNF4Base(dims, L, 4, ST.qwen_weight_fn())
    lora = ST.LoraParams(dims, L, 16, ST.qwen_lora_fn())
    for T, sizes in cases:
        print(f"{model} stack T={T}: resident", flush=True)
        ref = _run(ST, base, lora, T, "resident")
        assert torch.isfinite(ref["out"].float()).all() and torch.isfinite(ref["dh0"].float()).all()
        for bs in sizes:
            print(f"{model} stack T={T}: streamed block_size {bs}", flush=True)
            b = base.regroup(bs)
            got = _run(ST, b, lora, T, "streamed", n_slots=2, prefetch=True)
            _same(got, ref)
            assert got["stats"]["misses"] == 1 and got["stats"]["copies"] >= 2 * (b.n_blocks - 2)
            del got
            if bs == 4 and T == 512:        # one copy and one wait per block
                _same(_run(ST, b, lora, T, "streamed", n_slots=2, layer_parts=False), ref)
            torch.cuda.empty_cache()
        del ref
    base.close()
    del base, lora
    torch.cuda.empty_cache()


def test_qwen32b_stack_streamed_equals_resident(ST):
    """64 Qwen2.5-32B-shaped layers, 512 tokens, block sizes 4 and 1."""
    _big_stack_parity(ST, "32b", [(512, [4, 1])])


def test_qwen72b_stack_streamed_equals_resident(ST):
    """80 Qwen2.5-72B-shaped layers: block sizes 1, 2 and 4 at 512 tokens, and 4 at 256
    ("Poros on consumer GPUs", "OOM playbook": block_size 4 -> 2 -> 1 and a shorter
    sequence never change the results)."""
    _big_stack_parity(ST, "72b", [(512, [1, 2, 4]), (256, [4])])
