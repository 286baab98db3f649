"""Pins of the oracle's NF4 codec against what the pages and the mathematics fix.

The pages name the format only as "4-bit NF4 QLoRA" (Poros API reference,
"PorosTrainer.from_pretrained") and fix its storage cost through the host-RAM
figures ("Poros on consumer GPUs", "What you need besides VRAM"). Each check
below is independent of the oracle's own arithmetic: a second library routine,
exact rational arithmetic, a closed form or an invariant.
"""

import math
import statistics
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle as O


# ------------------------------------------------------------------ codebook

def test_codebook_two_inverse_normal_routines_agree_bitwise():
    a = O.nf4_codebook(statistics.NormalDist().inv_cdf)
    b = O.nf4_codebook(scipy.special.ndtri)
    assert a.dtype == np.float32 and a.shape == (16,)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_codebook_structure():
    t = O.nf4_codebook()
    assert t[0] == -1.0 and t[15] == 1.0
    assert t[7] == 0.0 and not np.signbit(t[7])
    assert np.all(np.diff(t.astype(np.float64)) > 0)
    assert (t < 0).sum() == 7 and (t > 0).sum() == 8


def _phi(z):
    return 0.5 * (1.0 + math.erf(z / math.sqrt(2.0)))


def _phi_inv_bisect(p):
    lo, hi = -10.0, 10.0
    for _ in range(200):
        mid = 0.5 * (lo + hi)
        if _phi(mid) < p:
            lo = mid
        else:
            hi = mid
    return 0.5 * (lo + hi)


def test_codebook_levels_are_normal_quantiles_forward_cdf():
    """Map each level back through the forward CDF (math.erf, no inverse routine):
    positive levels sit on an 8-step probability grid from delta to 1/2, negative
    levels on a 7-step one (QLoRA's NormalFloat, reading R1)."""
    t = O.nf4_codebook().astype(np.float64)
    delta = 0.5 * ((1 - 1 / 30) + (1 - 1 / 32))
    ztop = _phi_inv_bisect(delta)
    for i in range(8):                      # t[15 - i] <-> grid point i of 8
        assert abs(_phi(t[15 - i] * ztop) - (delta - (delta - 0.5) * i / 8)) < 2e-7
    for i in range(7):                      # t[i] <-> grid point i of 7, mirrored
        assert abs(_phi(-t[i] * ztop) - (delta - (delta - 0.5) * i / 7)) < 2e-7


# ------------------------------------------------------------------ bf16 rounding

def _torch_bf16_bits(f32):
    return torch.from_numpy(np.asarray(f32, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_matches_torch_cast():
    rng = np.random.default_rng(7)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    edge = np.array([0x3F808000, 0x3F818000, 0x3F807FFF, 0x3F808001, 0x00008000, 0x00018000,
                     0x7F7FFFFF, 0x7F7F8000, 0xBF808000, 0x80000000, 0x00000001, 0x807FFFFF],
                    dtype=np.uint32).view(np.float32)
    f = np.concatenate([f, edge])
    assert np.array_equal(O.f32_to_bf16_bits(f), _torch_bf16_bits(f))


# ------------------------------------------------------------------ quantise: brute force

def _rn32_exact(q: Fraction) -> Fraction:
    """Round a rational to the nearest float32 (ties to even), exactly."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = m.numerator // m.denominator
    rem = m - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def _brute_block(vals):
    """Nearest level of RN32(w/s) by exhaustive search, ties to the lower code."""
    levels = [Fraction(float(t)) for t in O.nf4_codebook()]
    fr = [Fraction(float(v)) for v in vals]
    s = max(abs(f) for f in fr)
    if s == 0:
        return [O.NF4_ZERO_CODE] * len(vals), 0.0
    codes = []
    for f in fr:
        v = _rn32_exact(f / s)
        d = [abs(v - lev) for lev in levels]
        codes.append(d.index(min(d)))
    return codes, float(s)


def _tie_block():
    """A block whose values hit every float32-representable level midpoint exactly."""
    t = O.nf4_codebook().astype(np.float64)
    mids = (t[:-1] + t[1:]) / 2
    exact = [m for m in mids if float(np.float32(m)) == m]
    assert len(exact) >= 1
    vals = [1.0] + exact
    for m in mids:                                   # neighbours of every midpoint
        m32 = np.float32(m)
        vals += [float(np.nextafter(m32, np.float32(2))), float(np.nextafter(m32, np.float32(-2)))]
    vals = (vals + [0.0, -0.0] * 64)[:64]
    return np.array(vals, dtype=np.float32)


@pytest.mark.parametrize("kind", ["normal", "uniform", "heavy", "bf16", "ties", "tiny", "mixed_zero"])
def test_quantize_matches_exact_rational_brute_force(kind):
    rng = np.random.default_rng(sum(map(ord, kind)))
    if kind == "normal":
        w = rng.normal(0, 0.02, size=(4, 128))
    elif kind == "uniform":
        w = rng.uniform(-3, 3, size=(4, 128))
    elif kind == "heavy":
        w = rng.standard_cauchy(size=(4, 128))
    elif kind == "bf16":
        w = O.bf16_bits_to_f64(O.f32_to_bf16_bits(rng.normal(0, 0.02, size=(4, 128))))
    elif kind == "ties":
        w = np.stack([_tie_block(), -_tie_block()[::-1], _tie_block() * 0.25, _tie_block() * 8])
    elif kind == "tiny":
        w = rng.normal(0, 1, size=(2, 64)) * 1e-39          # subnormal float32 scales
    else:
        w = rng.normal(0, 1, size=(3, 64))
        w[1] = 0.0
        w[2, :32] = 0.0
    w = np.asarray(w, dtype=np.float32)
    packed, absmax = O.quantize(w)
    codes = O.unpack_codes(packed)
    for r in range(w.shape[0]):
        for b in range(w.shape[1] // 64):
            want, s = _brute_block(w[r, b * 64:(b + 1) * 64])
            assert list(codes[r, b * 64:(b + 1) * 64]) == want, (kind, r, b)
            assert float(absmax[r, b]) == s


def test_quantize_ties_go_to_lower_code():
    t = O.nf4_codebook().astype(np.float64)
    mids = (t[:-1] + t[1:]) / 2
    for j, m in enumerate(mids):
        if float(np.float32(m)) != m:
            continue
        blk = np.zeros(64, dtype=np.float32)
        blk[0], blk[1] = 1.0, m
        codes = O.unpack_codes(O.quantize(blk[None, :])[0])[0]
        assert codes[1] == j and codes[0] == 15


# ------------------------------------------------------------------ quantise: invariants

def test_round_trip_of_levels_times_power_of_two():
    t = O.nf4_codebook()
    for e in (-20, -3, 0, 5):
        blk = np.concatenate([t, -t, t[::-1], np.zeros(16, np.float32)]).astype(np.float32)
        blk = (blk * np.float32(2.0 ** e)).astype(np.float32)
        packed, absmax = O.quantize(blk[None, :])
        codes = O.unpack_codes(packed)[0]
        assert absmax[0, 0] == np.float32(2.0 ** e)
        assert list(codes[:16]) == list(range(16))
        assert packed[0, 0] == 0x10 and packed[0, 7] == 0xFE        # low nibble = even element
        # fp32 stage of the dequant is exact: level * 2^e
        back = (t[codes] * absmax[0, 0]).astype(np.float32)
        nonneg_idx = [i for i in range(64) if not (16 <= i < 32)]
        assert np.array_equal(back[nonneg_idx], blk[nonneg_idx])


def test_zero_block():
    packed, absmax = O.quantize(np.zeros((2, 128), np.float32))
    assert np.all(packed == 0x77) and np.all(absmax == 0)
    deq = O.dequantize(packed, absmax)
    assert np.all(deq == 0x0000)


def test_power_of_two_scale_invariance():
    rng = np.random.default_rng(3)
    w = rng.normal(0, 0.02, size=(8, 256)).astype(np.float32)
    p0, s0 = O.quantize(w)
    for e in (-10, -1, 1, 12):
        p1, s1 = O.quantize((w * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(p0, p1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** e)).astype(np.float32))


def test_idempotent_on_fp32_dequant():
    rng = np.random.default_rng(4)
    w = rng.normal(0, 0.02, size=(16, 512)).astype(np.float32)
    packed, absmax = O.quantize(w)
    codes = O.unpack_codes(packed)
    t = O.nf4_codebook()
    w2 = (t[codes] * np.repeat(absmax, 64, axis=1)).astype(np.float32)
    p2, s2 = O.quantize(w2)
    assert np.array_equal(packed, p2) and np.array_equal(absmax, s2)


def test_pieces_equal_whole_tensor_bytes():
    """A block-by-block quantise is byte-identical to a whole-tensor one (the
    streamed loader's guarantee, "Poros on consumer GPUs", "OOM playbook")."""
    rng = np.random.default_rng(5)
    w = rng.normal(0, 0.02, size=(24, 384)).astype(np.float32)
    p, s = O.quantize(w)
    rows = [O.quantize(w[i:i + 5]) for i in range(0, 24, 5)]
    assert np.array_equal(np.concatenate([r[0] for r in rows]), p)
    assert np.array_equal(np.concatenate([r[1] for r in rows]), s)
    cols = [O.quantize(w[:, j:j + 128]) for j in range(0, 384, 128)]
    assert np.array_equal(np.concatenate([c[0] for c in cols], axis=1), p)
    assert np.array_equal(np.concatenate([c[1] for c in cols], axis=1), s)


def test_rejects_bad_shapes_and_nonfinite():
    with pytest.raises(ValueError):
        O.quantize(np.zeros((2, 63), np.float32))
    w = np.zeros((1, 64), np.float32)
    w[0, 3] = np.inf
    with pytest.raises(ValueError):
        O.quantize(w)


# ------------------------------------------------------------------ dequantise

def test_dequant_matches_library_two_step_rounding():
    """fp32 product by torch, then torch's bf16 cast: the two roundings of R6."""
    rng = np.random.default_rng(6)
    w = rng.normal(0, 0.02, size=(64, 256)).astype(np.float32)
    w[3] *= 1e-37                                            # scales near the fp32 subnormal range
    w[5] *= 3e4
    packed, absmax = O.quantize(w)
    codes = O.unpack_codes(packed)
    lv = torch.from_numpy(O.nf4_codebook()[codes])
    sc = torch.from_numpy(np.repeat(absmax, 64, axis=1))
    ref = (lv * sc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.dequantize(packed, absmax), ref)


def test_dequant_two_steps_differ_from_one_rounding_somewhere():
    """The rounding path matters: RNbf(RN32(p)) != RNbf(p) for some exact products."""
    rng = np.random.default_rng(8)
    lv = O.nf4_codebook()[rng.integers(0, 16, 400_000)].astype(np.float64)
    sc = rng.normal(0, 0.05, 400_000).astype(np.float32).astype(np.float64)
    p = lv * sc
    two = O.f32_to_bf16_bits(p.astype(np.float32))
    # one direct rounding fp64 -> bf16, done with exact integer arithmetic on the fp64 bits
    b = p.view(np.uint64)
    keep = np.uint64(45)                                     # 52 - 7 fraction bits dropped
    lsb = (b >> keep) & np.uint64(1)
    one64 = ((b + (np.uint64(1) << np.uint64(44)) - np.uint64(1) + lsb) >> keep) << keep
    one = O.f32_to_bf16_bits(one64.view(np.float64).astype(np.float32))
    assert np.any(two != one)


def test_dequant_special_codes():
    s = np.float32(0.0371)
    packed = np.array([[0x07 | (0x0F << 4)] + [0x00] * 31], dtype=np.uint8)
    deq = O.dequantize(packed, np.array([[s]], dtype=np.float32))
    assert deq[0, 0] == 0x0000
    assert deq[0, 1] == O.f32_to_bf16_bits(np.float32(s))
    assert deq[0, 2] == O.f32_to_bf16_bits(np.float32(-s))
