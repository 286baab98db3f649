"""Pins of the oracle's tiny identity-mixing stack (the streamed workload's layer).

Layer structure is reading R9 of the oracle (attention mixing replaced by the
identity); storage in bf16 is reading R10 (model dtype bfloat16, Poros API
reference "PorosModel.from_pretrained").
"""

import numpy as np
import pytest
import scipy.special

import oracle as O


def _dims():
    return O.StackLayerDims(hidden=32, q=32, kv=16, inter=48, head_dim=8)


def _layers(rng, dims, n_layers, r=2, zero=False):
    layers = []
    for _ in range(n_layers):
        layer = {}
        for name, (n, k) in dims.proj_shapes().items():
            w = np.zeros((n, k)) if zero else rng.normal(0, 0.3 / np.sqrt(k), size=(n, k))
            a = rng.normal(0, 1 / np.sqrt(k), size=(r, k))
            b = np.zeros((n, r)) if zero else rng.normal(0, 0.2, size=(n, r))
            layer[name] = (w, a, b)
        layers.append(layer)
    return layers


def _loss(h0, layers, dims, dh, alpha):
    out, _ = O.stack_forward(h0, layers, dims, alpha, round_storage=False)
    return float(np.sum(out * dh))


def test_stack_finite_differences():
    rng = np.random.default_rng(21)
    dims = _dims()
    layers = _layers(rng, dims, 2)
    t, alpha = 3, 4.0
    h0 = rng.normal(size=(t, dims.hidden))
    dh = rng.normal(size=(t, dims.hidden))
    _, saved = O.stack_forward(h0, layers, dims, alpha, round_storage=False)
    dh0, grads = O.stack_backward(dh, layers, dims, alpha, saved, round_storage=False)
    eps = 1e-5

    def num_grad(mutate):
        p = mutate(+eps)
        m = mutate(-eps)
        return (_loss(*p, dims, dh, alpha) - _loss(*m, dims, dh, alpha)) / (2 * eps)

    for _ in range(8):
        idx = (rng.integers(t), rng.integers(dims.hidden))

        def mut(e, idx=idx):
            h = h0.copy()
            h[idx] += e
            return h, layers
        assert abs(num_grad(mut) - dh0[idx]) < 1e-6 * max(1, abs(dh0[idx]))
    for li in range(2):
        for name in ("v", "o", "gate", "up", "down"):
            for which, gi in (("A", 1), ("B", 2)):
                arr = layers[li][name][gi]
                idx = tuple(rng.integers(0, s) for s in arr.shape)

                def mut(e, li=li, name=name, gi=gi, idx=idx):
                    new = [dict(lay) for lay in layers]
                    trip = list(new[li][name])
                    trip[gi] = trip[gi].copy()
                    trip[gi][idx] += e
                    new[li][name] = tuple(trip)
                    return h0, new
                want = grads[li][f"{name}_d{which}"][idx]
                assert abs(num_grad(mut) - want) < 1e-6 * max(1, abs(want)), (li, name, which)
        for name in ("q", "k"):                      # identity mixing: q and k do not reach the output
            assert not np.any(grads[li][f"{name}_dA"]) and not np.any(grads[li][f"{name}_dB"])


def test_zero_weight_layers_are_identity():
    rng = np.random.default_rng(22)
    dims = _dims()
    layers = _layers(rng, dims, 3, zero=True)
    h0 = O.f32_to_bf16_bits(rng.normal(size=(4, dims.hidden)))
    out, _ = O.stack_forward(h0, [{k: tuple(O.f32_to_bf16_bits(m) for m in v) for k, v in l.items()} for l in layers],
                             dims, 32.0, round_storage=True)
    assert np.array_equal(out, O.bf16_bits_to_f64(h0))


def test_rmsnorm_closed_forms():
    c, eps = 3.0, O.RMS_EPS
    y = O.rmsnorm_fwd(np.full((1, 16), c))
    assert np.allclose(y, c / np.sqrt(c * c + eps), rtol=0, atol=1e-15)
    rng = np.random.default_rng(23)
    h = rng.normal(size=(2, 16))
    dy = rng.normal(size=(2, 16))
    g = O.rmsnorm_bwd(h, dy)
    e = 1e-6
    for i in range(16):
        hp, hm = h.copy(), h.copy()
        hp[0, i] += e
        hm[0, i] -= e
        num = (np.sum(O.rmsnorm_fwd(hp) * dy) - np.sum(O.rmsnorm_fwd(hm) * dy)) / (2 * e)
        assert abs(num - g[0, i]) < 1e-7


def test_silu_against_library_sigmoid():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    e = 1e-6
    num = (O.silu(z + e) - O.silu(z - e)) / (2 * e)
    assert np.allclose(num, O.silu_grad(z), atol=1e-7)


def test_repeat_kv_head_mapping():
    dims = _dims()
    rng = np.random.default_rng(24)
    layers = _layers(rng, dims, 1)
    h0 = rng.normal(size=(2, dims.hidden))
    _, saved = O.stack_forward(h0, layers, dims, 2.0, round_storage=False)
    v, a = saved[0]["v"], saved[0]["a"]
    hd, rep = dims.head_dim, dims.q // dims.kv
    for qh in range(dims.q // hd):
        kvh = qh // rep
        assert np.array_equal(a[:, qh * hd:(qh + 1) * hd], v[:, kvh * hd:(kvh + 1) * hd])


def test_storage_rounding_is_bf16_rounding():
    rng = np.random.default_rng(25)
    z = rng.normal(size=1000) * 10.0
    assert np.array_equal(O.round_bf16(z), O.bf16_bits_to_f64(O.f32_to_bf16_bits(z.astype(np.float32))))
