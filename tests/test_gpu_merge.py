"""merge_and_unload (reading R12): the merged dense weight vs the fp64 oracle.

The kernel's value is RNbf(RN32(W + RN32(s . l))) with l an fp32 sum of r products,
so against the exact W + s.B.A it may differ by half a bf16 ulp (the final rounding)
plus the fp32 error before it: at most (r + 2) . 2^-24 . (|W| + s . sum_j |B_j A_j|).
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, to_dev_bf16

pytestmark = pytest.mark.gpu


def _half_ulp_bf16(v):
    """Half a bf16 ulp at |v| (normal range): 2^(floor(log2 |v|) - 8)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 8)


def _check_merge(got_bits, w_bits, a_bits, b_bits, alpha, what):
    r = a_bits.shape[0]
    exact = O.merge_lora(w_bits, a_bits, b_bits, alpha)
    got = O.bf16_bits_to_f64(got_bits)
    s = O.lora_scale(alpha, r)
    mag = np.abs(O.bf16_bits_to_f64(w_bits)) + s * (np.abs(O.bf16_bits_to_f64(b_bits)) @ np.abs(O.bf16_bits_to_f64(a_bits)))
    bound = _half_ulp_bf16(np.maximum(np.abs(got), np.abs(exact))) + (r + 2) * 2.0 ** -24 * mag
    err = np.abs(got - exact)
    assert (err <= bound).all(), f"{what}: worst excess {(err - bound).max():.3e}"
    # nearly every element is the correctly rounded value itself
    rounded = O.f32_to_bf16_bits(exact.astype(np.float32))
    assert np.mean(got_bits == rounded) > 0.99, f"{what}: {np.mean(got_bits != rounded):.4f} not correctly rounded"


def _inputs(n, k, r, seed=42):
    w = S.weight(n, k, seed=seed)
    codes, absmax = O.quantize(O.bf16_bits_to_f64(w).astype(np.float32))
    wq = O.dequantize(codes, absmax)
    a = S.lora_a(r, k, seed=seed) if r else np.zeros((0, k), np.uint16)
    b = S.lora_b(n, r, seed=seed, std=0.05) if r else np.zeros((n, 0), np.uint16)
    return codes, absmax, wq, a, b


def _merge(lib, codes, absmax, a, b, alpha):
    r = a.shape[0]
    out = lib.merge_lora(torch.from_numpy(codes).cuda(), torch.from_numpy(absmax).cuda(),
                         to_dev_bf16(a) if r else None, to_dev_bf16(b) if r else None, alpha)
    torch.cuda.synchronize()
    return bits_of(out)


@pytest.mark.parametrize("n,k,r", [
    (64, 256, 16),      # one tile
    (150, 384, 5),      # ragged rows and columns, odd rank
    (200, 1024, 64),    # the maximum rank
    (1, 64, 1),         # the smallest shape
])
def test_merge_matches_oracle(gpu_lib, n, k, r):
    codes, absmax, wq, a, b = _inputs(n, k, r)
    got = _merge(gpu_lib, codes, absmax, a, b, 32.0)
    _check_merge(got, wq, a, b, 32.0, f"merge {n}x{k} r{r}")


def test_merge_rank0_is_the_dequantised_base(gpu_lib):
    codes, absmax, wq, a, b = _inputs(96, 512, 0)
    assert np.array_equal(_merge(gpu_lib, codes, absmax, a, b, 32.0), wq)


def test_merge_zero_b_is_the_dequantised_base(gpu_lib):
    codes, absmax, wq, a, _ = _inputs(96, 512, 16)
    b = np.zeros((96, 16), np.uint16)
    assert np.array_equal(_merge(gpu_lib, codes, absmax, a, b, 32.0), wq)


def test_merge_full_size_sampled_rows(gpu_lib):
    """The 7B gate projection (18944 x 3584, r 16): sampled rows vs the oracle."""
    n, k, r = 18944, 3584, 16
    codes, absmax = S.nf4_storage(n, k, proj="gate")
    a, b = S.lora_a(r, k, proj="gate"), S.lora_b(n, r, proj="gate", std=0.05)
    got = _merge(gpu_lib, codes, absmax, a, b, 32.0)
    rows = np.unique(np.concatenate([np.random.default_rng(3).choice(n, 64, replace=False), [0, n - 1]]))
    wq = O.dequantize(codes[rows], absmax[rows])
    _check_merge(got[rows], wq, a, b[rows], 32.0, "merge 7B gate sampled")
