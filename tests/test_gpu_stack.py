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
    st = ST.NF4Stack(base, lora, T, 32.0, mode=mode, **kw)
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    h0 = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    out, dh0 = st.step(h0, dh)
    out2, dh02 = st.step(h0, dh)                     # second step: slot reuse across steps
    torch.cuda.synchronize()
    res = {"out": out.clone(), "dh0": dh0.clone(), "out2": out2.clone(),
           "grads": [{p: (a.clone(), b.clone()) for p, (a, b) in gl.items()} for gl in st.grads],
           "stats": st.pool.stats()}
    st.close()
    return res


def _same(a, b):
    assert torch.equal(a["out"], b["out"]) and torch.equal(a["dh0"], b["dh0"])
    assert torch.equal(a["out2"], a["out"])
    for ga, gb in zip(a["grads"], b["grads"]):
        for p in PROJS:
            assert torch.equal(ga[p][0], gb[p][0]) and torch.equal(ga[p][1], gb[p][1])


@pytest.mark.parametrize("block_size", [1, 2, 3])
def test_streamed_equals_resident_tiny(ST, block_size):
    L, T = 7, 48
    _, _, base, lora = _tiny_stack(ST, L, block_size)
    ref = _run(ST, base, lora, T, "resident")
    assert ref["stats"]["copies"] == base.n_blocks and ref["stats"]["misses"] == 0
    for kw in ({"prefetch": True, "n_slots": 2}, {"prefetch": False, "n_slots": 2}, {"prefetch": True, "n_slots": 3},
               {"prefetch": False, "n_slots": 1}):
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
    assert torch.isfinite(ref["out"].float()).all() and torch.isfinite(ref["dh0"].float()).all()
    assert got["stats"]["bytes_copied"] > 2 * base.total_bytes()
