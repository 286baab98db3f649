"""The per-element tolerance of the GPU parity tests, pinned on the CPU: an fp32
evaluation of the linear (torch's float32 matmul of the bf16 inputs, a different
summation order from the oracle's fp64 one) passes it, and a single wrong element,
a wrong sign or a dropped LoRA term fails it."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import check_linear, half_ulp_bf16, linear_mags


def _f32_linear(case, alpha):
    """Forward and backward in float32 on the CPU, the bf16 outputs rounded once."""
    f = lambda bits: torch.from_numpy(S.bf16_bits_to_f32(bits))
    x, w, a, b, dy = (f(case[key]) for key in ("x", "W", "A", "B", "dY"))
    s = np.float32(alpha) / np.float32(a.shape[0])
    u = x @ a.T
    y = x @ w.T + s * (u @ b.T)
    g = dy @ b
    dx = dy @ w + s * (g @ a)
    bits = lambda t: t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return {"y": bits(y), "u": u.numpy(), "dx": bits(dx), "dA": (s * (g.T @ x)).numpy(),
            "dB": (s * (dy.T @ u)).numpy()}


def _refs(case, alpha):
    y, u = O.lora_linear_fwd(case["x"], case["W"], case["A"], case["B"], alpha)
    dx, da, db = O.lora_linear_bwd(case["x"], case["W"], case["A"], case["B"], alpha, case["dY"])
    return {"y": y, "u": u, "dx": dx, "dA": da, "dB": db}


@pytest.fixture(scope="module")
def linear():
    t, n, k, r = 96, 256, 1024, 16
    case = S.linear_case(t, n, k, r)
    return case, (t, n, k, r), _refs(case, 32.0), linear_mags(case["x"], case["W"], case["A"], case["B"], 32.0,
                                                              case["dY"])


def test_half_ulp_bf16():
    assert half_ulp_bf16(1.0) == 2.0 ** -8
    assert half_ulp_bf16(1.99) == 2.0 ** -8
    assert half_ulp_bf16(2.0) == 2.0 ** -7
    assert half_ulp_bf16(-0.75) == 2.0 ** -9


def test_fp32_evaluation_passes(linear):
    case, (t, n, k, r), refs, mags = linear
    check_linear(_f32_linear(case, 32.0), refs, mags, t, n, k, r, "fp32 CPU")


@pytest.mark.parametrize("key", ["y", "dx", "u", "dA", "dB"])
def test_one_wrong_element_fails(linear, key):
    case, (t, n, k, r), refs, mags = linear
    outs = _f32_linear(case, 32.0)
    v = outs[key]
    idx = tuple(s // 3 for s in v.shape)
    # one element moved by a tenth of the output's mean magnitude
    if v.dtype == np.uint16:
        vals = O.bf16_bits_to_f64(v)
        v[idx] = O.f32_to_bf16_bits(np.float32(vals[idx] + 0.1 * np.abs(vals).mean())).reshape(())
    else:
        v[idx] = v[idx] + np.float32(0.1 * np.abs(v).mean())
    with pytest.raises(AssertionError):
        check_linear(outs, refs, mags, t, n, k, r, f"planted {key}")


def test_sign_flip_and_dropped_lora_fail(linear):
    case, (t, n, k, r), refs, mags = linear
    outs = _f32_linear(case, 32.0)
    outs["y"] = outs["y"].copy()
    outs["y"][3, 5] ^= np.uint16(0x8000)               # one sign flipped
    with pytest.raises(AssertionError):
        check_linear(outs, refs, mags, t, n, k, r, "sign")
    no_lora = dict(case, B=np.zeros_like(case["B"]))    # LoRA term dropped from y and dX
    outs = _f32_linear(no_lora, 32.0)
    outs.pop("dA"), outs.pop("dB"), outs.pop("u")
    with pytest.raises(AssertionError):
        check_linear(dict(outs, u=_f32_linear(case, 32.0)["u"], dA=refs["dA"], dB=refs["dB"]), refs, mags, t, n, k,
                     r, "no LoRA")
