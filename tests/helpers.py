"""Shared test helpers: tensor <-> bit-pattern conversion and tolerance checks.

Two checks apply to every floating-point output of the linear:
  - whole-tensor rel-L2 against the fp64 oracle (the 2e-3 bar; bf16 outputs also
    within 3e-4 of the rounding floor), and
  - a per-element bound, so that one wrong element (a mis-summed split piece, a
    wrong ragged edge) cannot hide in a large tensor's norm. Every output is an fp32
    sum of exact bf16 x bf16 products (plus, for the LoRA terms, operands split into
    bf16 hi + lo that equal the fp32 value within 2^-16 of it), so with `mag` the same
    sum taken over absolute values and `terms` at least the number of additions on
    any path to the element, the fp32 result lies within
        delta = (terms * 2^-24 + 2^-15) * mag
    of the exact value; a bf16 output adds at most half a bf16 ulp of its fp32 value.
"""

import numpy as np
import torch

import oracle as O

REL_L2_BAR = 2e-3          # GEMM outputs and gradients vs the fp64 oracle
FLOOR_MARGIN = 3e-4        # bf16 outputs: at most this much above the rounding floor
FP32_GRAD_BAR = 1e-4       # fp32 outputs (dA, dB, u): well inside the bar
U24 = 2.0 ** -24           # fp32 unit roundoff
SPLIT_REL = 2.0 ** -15     # hi/lo bf16 split of an fp32 LoRA operand (2^-16), doubled
SUM_SLACK = 64             # additions beyond the contraction: split pieces, partials


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def _f64(a) -> np.ndarray:
    a = np.asarray(a)
    return O.bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def half_ulp_bf16(v) -> np.ndarray:
    """Half a bf16 ulp at |v| (8 significant bits): 2^(e - 9) for |v| = m 2^e, m in [0.5, 1)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    return np.where(v > 0, np.ldexp(1.0, e - 9), 2.0 ** -134)


def linear_mags(x, w, a, b, alpha, dy):
    """The linear's outputs (y, u, dX, dA, dB) recomputed by the oracle over |x|, |W|,
    |A|, |B|, |dY|: the magnitude sums that bound the rounding error of every
    summation order."""
    ax, aw, aa, ab, ady = (np.abs(_f64(v)) for v in (x, w, a, b, dy))
    y, u = O.lora_linear_fwd(ax, aw, aa, ab, abs(alpha))
    dx, da, db = O.lora_linear_bwd(ax, aw, aa, ab, abs(alpha), ady)
    return {"y": y, "u": u, "dx": dx, "dA": da, "dB": db}


def _elementwise(got, exact, what, mag, terms, rounded_bf16):
    delta = (terms * U24 + SPLIT_REL) * np.asarray(mag, dtype=np.float64)
    reach = np.abs(exact) + delta
    bound = delta + (half_ulp_bf16(reach) if rounded_bf16 else U24 * reach)
    err = np.abs(got - exact)
    bad = ~(err <= bound)
    if np.any(bad):
        i = np.unravel_index(int(np.argmax(np.where(bad, err - bound, -np.inf))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {err.size} elements outside the per-element bound; "
                             f"worst at {i}: got {got[i]!r}, exact {exact[i]!r}, bound {bound[i]:.3e}")


def check_bf16_output(gpu_bits: np.ndarray, exact: np.ndarray, what: str, mag=None, terms: int = 0) -> float:
    """rel-L2 of a bf16 GPU output against the unrounded oracle value, with the floor
    check, and (with `mag`) every element within its rounding bound."""
    got = O.bf16_bits_to_f64(gpu_bits)
    rel = O.rel_l2(got, exact)
    floor = O.rel_l2(O.round_bf16(exact), exact)
    assert rel <= REL_L2_BAR, f"{what}: rel-L2 {rel:.3e} > {REL_L2_BAR}"
    assert rel <= floor + FLOOR_MARGIN, f"{what}: rel-L2 {rel:.3e} > floor {floor:.3e} + {FLOOR_MARGIN}"
    if mag is not None:
        _elementwise(got, np.asarray(exact, dtype=np.float64), what, mag, terms + SUM_SLACK, True)
    return rel


def check_f32_output(gpu: np.ndarray, exact: np.ndarray, what: str, bar: float = FP32_GRAD_BAR, mag=None,
                     terms: int = 0) -> float:
    got = np.asarray(gpu, dtype=np.float64)
    rel = O.rel_l2(got, exact)
    assert rel <= bar, f"{what}: rel-L2 {rel:.3e} > {bar}"
    if mag is not None:
        _elementwise(got, np.asarray(exact, dtype=np.float64), what, mag, terms + SUM_SLACK, False)
    return rel


def check_linear(outs: dict, refs: dict, mags: dict, t: int, n: int, k: int, r: int, what: str) -> None:
    """All outputs of one linear call (keys y, u, dx, dA, dB; GPU arrays: bf16 bits for
    y and dx, float for the rest) against the oracle, whole-tensor and per element.
    Additions on the longest path: y K + r, u K, dX N + r, dA N + T, dB K + T."""
    if "y" in outs:
        check_bf16_output(outs["y"], refs["y"], f"y {what}", mags["y"], k + r)
    if outs.get("dx") is not None:
        check_bf16_output(outs["dx"], refs["dx"], f"dX {what}", mags["dx"], n + r)
    if r:
        if "u" in outs:
            check_f32_output(outs["u"], refs["u"], f"u {what}", mag=mags["u"], terms=k)
        check_f32_output(outs["dA"], refs["dA"], f"dA {what}", mag=mags["dA"], terms=n + t)
        check_f32_output(outs["dB"], refs["dB"], f"dB {what}", mag=mags["dB"], terms=k + t)
