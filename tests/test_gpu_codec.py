"""GPU NF4 codec vs the fp64 oracle: codes, absmax and dequantised bf16 must match bit for bit."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, to_dev_bf16

pytestmark = pytest.mark.gpu


def _gpu_quant(lib, w_dev):
    codes, absmax = lib.quantize(w_dev)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), absmax.cpu().numpy()


def test_quantize_single_linear_workload_bit_exact(gpu_lib):
    """1024 x 1024 weights ~ N(0, 0.02) in bf16, NF4 blocksize 64."""
    wb = S.weight(1024, 1024)
    codes, absmax = _gpu_quant(gpu_lib, to_dev_bf16(wb))
    oc, oa = O.quantize(O.bf16_bits_to_f64(wb).astype(np.float32))
    assert np.array_equal(codes, oc)
    assert np.array_equal(absmax.view(np.uint32), oa.view(np.uint32))


def _edge_matrix():
    rng = np.random.default_rng(99)
    t = O.nf4_codebook().astype(np.float64)
    mids = (t[:-1] + t[1:]) / 2
    rows = []
    rows.append(np.zeros(128))                                       # all-zero blocks
    r = rng.normal(size=128); r[::2] = -0.0; rows.append(r)          # signed zeros
    ties = [1.0] + [m for m in mids if float(np.float32(m)) == m]
    nb = []
    for m in mids:
        m32 = np.float32(m)
        nb += [float(np.nextafter(m32, np.float32(2))), float(np.nextafter(m32, np.float32(-2))), float(m32)]
    rows.append(np.array((ties + nb + [0.0] * 128)[:128]))           # exact ties and their neighbours
    rows.append(-rows[-1])
    rows.append(rng.normal(size=128) * 1e-39)                        # subnormal scales
    rows.append(rng.standard_cauchy(size=128))                       # heavy tails
    big = rng.normal(size=128); big[5] = 3.0e38; rows.append(big)    # near float32 max
    rows.append(np.concatenate([t, -t, t * 0.5, t[::-1]] * 2)[:128])  # every level
    # quotients on and next to every multiple of 1/32 in [-1, 1] (each block holds 1.0,
    # so its absmax is 1 and the quotient is the value itself), also scaled by 2^-3
    grid = [k / 32.0 for k in range(-32, 33)]
    vals = []
    for g in grid:
        g32 = np.float32(g)
        vals += [float(g32), float(np.nextafter(g32, np.float32(2))), float(np.nextafter(g32, np.float32(-2)))]
    vals = [v for v in vals if abs(v) <= 1.0]
    blocks = [[1.0] + vals[i:i + 63] for i in range(0, len(vals), 63)]
    flat = np.concatenate([np.pad(np.array(b), (0, 64 - len(b))) for b in blocks])
    flat = np.pad(flat, (0, (-len(flat)) % 128))
    for scale in (1.0, 0.125):
        rows += list(flat.reshape(-1, 128) * scale)
    for e in (-30, -5, 0, 7):
        rows.append(rng.normal(size=128) * 2.0 ** e)
    return np.stack(rows).astype(np.float32)


def test_quantize_float32_edge_blocks_bit_exact(gpu_lib):
    w = _edge_matrix()
    codes, absmax = _gpu_quant(gpu_lib, torch.from_numpy(w).cuda())
    oc, oa = O.quantize(w)
    assert np.array_equal(codes, oc)
    assert np.array_equal(absmax.view(np.uint32), oa.view(np.uint32))


@pytest.mark.parametrize("shape", [(1, 64), (3, 192), (37, 640), (129, 1088), (16, 4096)])
def test_quantize_random_shapes_bf16_and_f32(gpu_lib, shape):
    rng = np.random.default_rng(shape[0] * 7 + shape[1])
    w32 = (rng.normal(size=shape) * rng.choice([0.02, 1.0, 300.0])).astype(np.float32)
    oc, oa = O.quantize(w32)
    codes, absmax = _gpu_quant(gpu_lib, torch.from_numpy(w32).cuda())
    assert np.array_equal(codes, oc) and np.array_equal(absmax, oa)
    wb = S.to_bf16_bits(w32)
    oc, oa = O.quantize(O.bf16_bits_to_f64(wb).astype(np.float32))
    codes, absmax = _gpu_quant(gpu_lib, to_dev_bf16(wb))
    assert np.array_equal(codes, oc) and np.array_equal(absmax, oa)


def test_dequantize_bit_exact(gpu_lib):
    w = np.concatenate([_edge_matrix(), S.bf16_bits_to_f32(S.weight(64, 128))])
    oc, oa = O.quantize(w)
    deq = gpu_lib.dequantize(torch.from_numpy(oc).cuda(), torch.from_numpy(oa).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(deq), O.dequantize(oc, oa))


def test_quantize_pieces_equal_whole_tensor(gpu_lib):
    """Quantising row blocks separately gives the same bytes as the whole tensor
    (the property the block-by-block loader relies on)."""
    w = to_dev_bf16(S.weight(300, 512))
    c_all, a_all = gpu_lib.quantize(w)
    parts = [gpu_lib.quantize(w[i:i + 64].contiguous()) for i in range(0, 300, 64)]
    torch.cuda.synchronize()
    assert torch.equal(torch.cat([p[0] for p in parts]), c_all)
    assert torch.equal(torch.cat([p[1] for p in parts]), a_all)


def test_quantize_large_projection_sampled_rows(gpu_lib):
    """A 7B-shaped gate projection (18944 x 3584): sampled rows vs the oracle."""
    n, k = 18944, 3584
    wb = S.weight(n, k, proj="gate")
    codes, absmax = _gpu_quant(gpu_lib, to_dev_bf16(wb))
    rows = np.random.default_rng(1).choice(n, 48, replace=False)
    rows = np.concatenate([rows, [0, n - 1]])
    oc, oa = O.quantize(O.bf16_bits_to_f64(wb[rows]).astype(np.float32))
    assert np.array_equal(codes[rows], oc) and np.array_equal(absmax[rows], oa)
    deq = gpu_lib.dequantize(torch.from_numpy(codes[rows]).cuda(), torch.from_numpy(absmax[rows]).cuda())
    torch.cuda.synchronize()
    assert np.array_equal(bits_of(deq), O.dequantize(oc, oa))


def test_quantize_is_deterministic(gpu_lib):
    w = to_dev_bf16(S.weight(512, 1024))
    a = gpu_lib.quantize(w)
    b = gpu_lib.quantize(w)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
