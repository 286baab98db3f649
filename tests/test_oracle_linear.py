"""Pins of the oracle's LoRA linear (forward and backward) against closed forms.

The method: a frozen NF4 base whose matmul output is summed with a rank-r LoRA
path scaled by alpha/r (Poros API reference, "PorosTrainer.from_pretrained":
lora_rank 16, lora_alpha 32), trained with gradients for the adapters only
("patch_hf_model" Behavior 3; HN comment: the base is read, never written).
"""

import numpy as np
import pytest

import oracle as O


def _ints(rng, shape, lo, hi):
    return rng.integers(lo, hi + 1, size=shape).astype(np.float64)


def test_lora_scale():
    assert O.lora_scale(32, 16) == 2.0
    assert O.lora_scale(32, 0) == 0.0
    assert O.lora_scale(1.0, 3) == float(np.float32(1.0) / np.float32(3.0))


def test_integer_closed_form_bruteforce():
    """Small integers everywhere: compute y, dX, dA, dB with Python integer loops."""
    rng = np.random.default_rng(11)
    t, n, k, r = 3, 5, 64, 2
    x = _ints(rng, (t, k), -3, 3)
    # base: codes {0, 7, 15} with absmax 2 give W in {-2, 0, 2}, exactly as dequantised
    codes = rng.choice([0, 7, 15], size=(n, k)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    absmax = np.full((n, k // 64), 2.0, np.float32)
    wbits = O.dequantize(packed, absmax)
    w = O.bf16_bits_to_f64(wbits)
    assert set(np.unique(w)) <= {-2.0, 0.0, 2.0}
    a = _ints(rng, (r, k), -2, 2)
    b = _ints(rng, (n, r), -2, 2)
    dy = _ints(rng, (t, n), -3, 3)
    alpha = 4.0                                            # s = 2
    y, u = O.lora_linear_fwd(x, wbits, a, b, alpha)
    dx, da, db = O.lora_linear_bwd(x, wbits, a, b, alpha, dy)
    xi, wi, ai, bi, dyi = (m.astype(int).tolist() for m in (x, w, a, b, dy))
    for ti in range(t):
        ui = [sum(xi[ti][kk] * ai[j][kk] for kk in range(k)) for j in range(r)]
        assert ui == u[ti].astype(int).tolist()
        for ni in range(n):
            want = sum(xi[ti][kk] * wi[ni][kk] for kk in range(k)) + 2 * sum(ui[j] * bi[ni][j] for j in range(r))
            assert y[ti, ni] == want
    for ti in range(t):
        g = [sum(dyi[ti][ni] * bi[ni][j] for ni in range(n)) for j in range(r)]
        for kk in range(k):
            want = sum(dyi[ti][ni] * wi[ni][kk] for ni in range(n)) + 2 * sum(g[j] * ai[j][kk] for j in range(r))
            assert dx[ti, kk] == want
    for j in range(r):
        for kk in range(k):
            want = 2 * sum(sum(dyi[ti][ni] * bi[ni][j] for ni in range(n)) * xi[ti][kk] for ti in range(t))
            assert da[j, kk] == want
    for ni in range(n):
        for j in range(r):
            want = 2 * sum(dyi[ti][ni] * sum(xi[ti][kk] * ai[j][kk] for kk in range(k)) for ti in range(t))
            assert db[ni, j] == want


def test_b_zero_gives_base_output():
    rng = np.random.default_rng(12)
    x = rng.normal(size=(7, 128))
    w = rng.normal(size=(9, 128))
    a = rng.normal(size=(4, 128))
    y, _ = O.lora_linear_fwd(x, w, a, np.zeros((9, 4)), 32.0)
    assert np.array_equal(y, x @ w.T)


def _loss(x, w, a, b, alpha, dy):
    y, _ = O.lora_linear_fwd(x, w, a, b, alpha)
    return float(np.sum(dy * y))


def test_central_finite_differences():
    rng = np.random.default_rng(13)
    t, n, k, r = 3, 8, 64, 2
    x, w, a, b, dy = (rng.normal(size=s) for s in [(t, k), (n, k), (r, k), (n, r), (t, n)])
    alpha = 3.0
    dx, da, db = O.lora_linear_bwd(x, w, a, b, alpha, dy)
    eps = 1e-3
    for name, arr, grad in (("x", x, dx), ("A", a, da), ("B", b, db)):
        for idx in [tuple(rng.integers(0, s) for s in arr.shape) for _ in range(12)]:
            p, m = arr.copy(), arr.copy()
            p[idx] += eps
            m[idx] -= eps
            args = {"x": x, "A": a, "B": b}
            ap, am = dict(args), dict(args)
            ap[name], am[name] = p, m
            num = (_loss(ap["x"], w, ap["A"], ap["B"], alpha, dy) - _loss(am["x"], w, am["A"], am["B"], alpha, dy)) / (2 * eps)
            assert abs(num - grad[idx]) <= 1e-8 * max(1.0, abs(grad[idx])), (name, idx)


def test_adjoint_identities():
    """y is linear in x, bilinear in (A, B): <dY, y> = <dX, x>; <dY, y - y_base> = <dA, A> = <dB, B>."""
    rng = np.random.default_rng(14)
    t, n, k, r = 6, 40, 128, 4
    x, w, a, b, dy = (rng.normal(size=s) for s in [(t, k), (n, k), (r, k), (n, r), (t, n)])
    y, _ = O.lora_linear_fwd(x, w, a, b, 8.0)
    dx, da, db = O.lora_linear_bwd(x, w, a, b, 8.0, dy)
    lhs = np.sum(dy * y)
    assert np.isclose(lhs, np.sum(dx * x), rtol=1e-12)
    lora = np.sum(dy * (y - x @ w.T))
    assert np.isclose(lora, np.sum(da * a), rtol=1e-10)
    assert np.isclose(lora, np.sum(db * b), rtol=1e-10)


def test_no_base_gradient_is_produced():
    rng = np.random.default_rng(15)
    out = O.lora_linear_bwd(rng.normal(size=(2, 64)), rng.normal(size=(3, 64)),
                            rng.normal(size=(2, 64)), rng.normal(size=(3, 2)), 2.0, rng.normal(size=(2, 3)))
    assert len(out) == 3                                   # dX, dA, dB only


def test_bits_inputs_equal_float_inputs():
    rng = np.random.default_rng(16)
    bits = [O.f32_to_bf16_bits(rng.normal(size=s)) for s in [(4, 64), (5, 64), (2, 64), (5, 2), (4, 5)]]
    vals = [O.bf16_bits_to_f64(b) for b in bits]
    y1, _ = O.lora_linear_fwd(*bits[:4], 32.0)
    y2, _ = O.lora_linear_fwd(*vals[:4], 32.0)
    assert np.array_equal(y1, y2)


def test_rel_l2():
    assert O.rel_l2([1.0, 0.0], [1.0, 0.0]) == 0.0
    assert np.isclose(O.rel_l2([3.0, 4.0], [0.0, 5.0]), np.sqrt(10.0) / 5.0)


# ----------------------------------------------------------------- merge_and_unload (R12)

def test_merge_reproduces_the_adapted_forward():
    """x.(W + s.B.A)^T is the LoRA forward's y (an identity of the two definitions)."""
    rng = np.random.default_rng(21)
    x = rng.normal(size=(6, 128))
    w = rng.normal(size=(10, 128))
    a = rng.normal(size=(5, 128))
    b = rng.normal(size=(10, 5))
    wm = O.merge_lora(w, a, b, 32.0)
    y, _ = O.lora_linear_fwd(x, w, a, b, 32.0)
    assert wm.shape == w.shape
    assert np.allclose(x @ wm.T, y, rtol=1e-12, atol=1e-12)


def test_merge_with_zero_b_is_the_dequantised_base():
    rng = np.random.default_rng(22)
    w = rng.normal(size=(16, 128)).astype(np.float32)
    codes, absmax = O.quantize(w)
    wq = O.dequantize(codes, absmax)
    a = O.f32_to_bf16_bits(rng.normal(size=(4, 128)).astype(np.float32))
    b = np.zeros((16, 4), np.uint16)
    assert np.array_equal(O.f32_to_bf16_bits(O.merge_lora(wq, a, b, 32.0).astype(np.float32)), wq)


def test_merge_integer_bruteforce():
    """Small integers: every merged entry by Python integer loops."""
    rng = np.random.default_rng(23)
    n, k, r = 3, 8, 2
    w = _ints(rng, (n, k), -4, 4)
    a = _ints(rng, (r, k), -3, 3)
    b = _ints(rng, (n, r), -3, 3)
    wm = O.merge_lora(w, a, b, 4.0)          # s = 4 / 2 = 2
    wi, ai, bi = w.astype(int).tolist(), a.astype(int).tolist(), b.astype(int).tolist()
    for i in range(n):
        for kk in range(k):
            assert wm[i, kk] == wi[i][kk] + 2 * sum(bi[i][j] * ai[j][kk] for j in range(r))
