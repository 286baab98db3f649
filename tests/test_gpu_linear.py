"""GPU NF4-LoRA linear (forward and backward) vs the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, check_f32_output, check_linear, f32_of, linear_mags, to_dev_bf16

pytestmark = pytest.mark.gpu


def _prepare(lib, case, r):
    """Quantise W on the oracle side (the oracle's codes are the GEMM's input)."""
    w32 = O.bf16_bits_to_f64(case["W"]).astype(np.float32)
    codes, absmax = O.quantize(w32)
    wq = O.dequantize(codes, absmax)
    dev = {
        "codes": torch.from_numpy(codes).cuda(), "absmax": torch.from_numpy(absmax).cuda(),
        "x": to_dev_bf16(case["x"]), "dY": to_dev_bf16(case["dY"]),
        "A": to_dev_bf16(case["A"]) if r else None, "B": to_dev_bf16(case["B"]) if r else None,
    }
    return wq, dev


def _run(lib, dev, alpha, need_dx=True):
    y, u = lib.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], dev["A"], dev["B"], alpha)
    dx, da, db = lib.lora_linear_bwd(dev["codes"], dev["absmax"], dev["x"], u, dev["dY"], dev["A"], dev["B"],
                                     alpha, need_dx=need_dx)
    torch.cuda.synchronize()
    return y, u, dx, da, db


def _check_case(lib, t, n, k, r, alpha=32.0, seed=42, b_std=0.01):
    case = S.linear_case(t, n, k, r=max(r, 1), seed=seed, b_std=b_std)
    if r == 0:
        case["A"] = np.zeros((0, k), np.uint16)
        case["B"] = np.zeros((n, 0), np.uint16)
    wq, dev = _prepare(lib, case, r)
    y, u, dx, da, db = _run(lib, dev, alpha)
    y_ref, u_ref = O.lora_linear_fwd(case["x"], wq, case["A"], case["B"], alpha)
    dx_ref, da_ref, db_ref = O.lora_linear_bwd(case["x"], wq, case["A"], case["B"], alpha, case["dY"])
    refs = {"y": y_ref, "u": u_ref, "dx": dx_ref, "dA": da_ref, "dB": db_ref}
    mags = linear_mags(case["x"], wq, case["A"], case["B"], alpha, case["dY"])
    outs = {"y": bits_of(y), "dx": bits_of(dx)}
    if r:
        outs.update(u=f32_of(u), dA=f32_of(da), dB=f32_of(db))
    check_linear(outs, refs, mags, t, n, k, r, f"{t}x{n}x{k} r{r}")
    return y, dx, da, db


def _random_shapes(count=24, seed=20261203):
    """Seeded shapes over the entry points' domain, half of them in the few-token range:
    T 1..600, N a multiple of 16 up to 4096, K a multiple of 64 up to 6144, rank 0..64,
    alpha from {8, 16, 32, 64}; the product T*N*K kept small enough for the fp64 oracle."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        t = int(rng.integers(1, 65)) if len(out) % 2 == 0 else int(rng.integers(65, 601))
        n = 16 * int(rng.integers(1, 257))
        k = 64 * int(rng.integers(1, 97))
        if t * n * k > 3_000_000_000:
            continue
        r = int(rng.choice([0, 1, 3, 8, 16, 16, 16, 24, 33, 64]))
        alpha = float(rng.choice([8.0, 16.0, 32.0, 64.0]))
        out.append((t, n, k, r, alpha, int(rng.integers(1, 1 << 30))))
    return out


@pytest.mark.parametrize("t,n,k,r,alpha,seed", _random_shapes())
def test_random_shapes(gpu_lib, t, n, k, r, alpha, seed):
    """Breadth beyond the hand-picked shapes: each case through both entry points, checked
    element by element against the oracle."""
    _check_case(gpu_lib, t, n, k, r, alpha=alpha, seed=seed)


def test_single_linear_workload(gpu_lib):
    """in = out = 1024, 256 tokens, r = 16, alpha = 32: fwd + bwd (dX, dA, dB)."""
    _check_case(gpu_lib, 256, 1024, 1024, 16)


@pytest.mark.parametrize("t,n,k,r", [
    (300, 400, 640, 16),     # several tiles and ragged tails in every dimension
    (1, 128, 256, 16),       # one token
    (17, 48, 64, 8),         # rank not a multiple of 16, one K block
    (130, 272, 320, 48),     # rank 48
    (64, 256, 1024, 64),     # maximum rank
    (200, 512, 3584, 16),    # skinny N with split-K (k/v-like)
    (96, 3584, 512, 16),     # long N, short K
    (513, 160, 192, 16),     # T one past a tile boundary
    (150, 208, 384, 5),      # odd rank: partial 4-rank groups, unaligned rows of u, g, B
    (129, 3584, 640, 12),    # rank 12: B rows not a 16-byte multiple; dX split over N
    (300, 1104, 8192, 16),   # long K and N: both GEMMs split their contraction, ragged tiles
    (40, 1040, 8256, 7),     # same with an odd step count over K and an odd rank
    (300, 640, 22976, 16),   # 540 dX tiles: a whole round of 512, the last 28 (ragged) split over N
    (300, 10992, 640, 16),   # 258 y tiles: a whole round of 256, the last 2 (ragged) split over K
    (512, 3584, 3584, 16),   # q-shaped at 512 tokens: 112 tiles, balanced two-round split in both GEMMs
    (200, 7040, 1600, 16),   # balanced split with ragged tokens and K: 110 y tiles (25 K steps), 26 dX tiles
    (512, 8192, 1024, 16),   # exactly 256 y tiles: split in two over K
    (512, 1024, 8192, 16),   # exactly 256 dX tiles: split in two over N
    (512, 12800, 1536, 16),  # 400 y tiles: a whole round, the last 144 split in three over K
    (512, 1536, 12800, 16),  # 400 dX tiles: a whole round, the last 144 split in three over N
    (300, 1024, 16448, 5),   # 256-token dX tiles (ragged second tile, ragged last column tile), odd rank
    (257, 1024, 32768, 64),  # 256-token dX tiles one token past a tile, maximum rank
    (512, 2048, 18944, 16),  # 256-token dX tiles: 296 tiles, a whole round and a split tail
])
def test_shapes(gpu_lib, t, n, k, r):
    _check_case(gpu_lib, t, n, k, r)


@pytest.mark.parametrize("t,n,k,r", [
    (1, 3584, 3584, 16),     # one token, q-shaped: forward split over K, backward over N
    (7, 208, 384, 5),        # odd rank, ragged rows (208 = 128 + 80)
    (16, 512, 3584, 64),     # the largest few-token batch at the maximum rank
    (3, 144, 128, 0),        # base only
    (12, 4096, 256, 16),     # long N, short K (one K step)
])
def test_few_token_path(gpu_lib, t, n, k, r):
    """T <= 16: the streaming kernels with one 16-token MFMA block (split contraction)."""
    _check_case(gpu_lib, t, n, k, r)


@pytest.mark.parametrize("t,n,k,r", [
    (17, 208, 384, 5),       # two token blocks, the second with one token, narrow weights
    (17, 2064, 640, 5),      # both directions two blocks, odd rank
    (32, 3584, 3584, 16),    # two full blocks, q-shaped
    (25, 4096, 256, 16),     # ragged second block, one K step
    (31, 2048, 8256, 64),    # maximum rank, odd K step count
    (31, 1040, 8256, 64),    # maximum rank, narrow weights
    (33, 208, 384, 16),      # one past the few-token path: the 128-token kernels
])
def test_few_token_two_blocks(gpu_lib, t, n, k, r):
    """17 <= T <= 32: both directions run the streaming kernels with two token blocks."""
    _check_case(gpu_lib, t, n, k, r)


@pytest.mark.parametrize("t,n,k,r", [
    (33, 1040, 8256, 16),    # three token blocks (the third with one token), long K, odd step count
    (48, 208, 8192, 5),      # three full blocks, odd rank
    (57, 2048, 8192, 64),    # four blocks (ragged), maximum rank
    (64, 8192, 1024, 16),    # short K: the 128-token kernels
    (64, 8208, 8192, 16),    # wide N: the 128-token kernels
])
def test_few_token_forward_long_k(gpu_lib, t, n, k, r):
    """33 <= T <= 64 with K >= 8192 and N <= 8192: the forward runs the streaming kernel
    with three or four token blocks (the backward the 128-token kernels)."""
    _check_case(gpu_lib, t, n, k, r)


@pytest.mark.parametrize("t,n,k,r", [
    (15, 2048, 9216, 64),    # one block below its edge, maximum rank, long K
    (1, 1424, 8256, 64),     # one token, odd K step count
    (18, 176, 9216, 33),     # two blocks, three rank blocks (ragged), narrow N
    (24, 272, 9216, 1),      # rank 1
    (40, 2064, 1920, 0),     # base only, short K: both directions on the 128-token kernels
    (47, 1056, 9216, 5),     # three blocks (forward), odd rank
    (49, 2128, 8192, 33),    # four blocks (ragged), three rank blocks
    (49, 8208, 192, 1),      # wide N, short K: 128-token kernels
    (64, 480, 9216, 33),     # four full blocks at the long-K edge
    (64, 8208, 320, 64),     # short K: 128-token kernels at the maximum rank
    (65, 384, 1152, 16),     # one past the few-token forward
])
def test_few_token_edges(gpu_lib, t, n, k, r):
    """Shapes around the few-token limits (T = 16 / 32 / 64, K >= 8192, N <= 8192) with
    ragged ranks, widths and step counts, each direction on whichever kernel the shape
    selects."""
    _check_case(gpu_lib, t, n, k, r)


def test_few_token_dx_skipped(gpu_lib):
    case = S.linear_case(4, 256, 512)
    wq, dev = _prepare(gpu_lib, case, 16)
    y, u = gpu_lib.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], dev["A"], dev["B"], 32.0)
    dx, da, db = gpu_lib.lora_linear_bwd(dev["codes"], dev["absmax"], dev["x"], u, dev["dY"], dev["A"], dev["B"],
                                         32.0, need_dx=False)
    torch.cuda.synchronize()
    assert dx is None
    _, da_ref, db_ref = O.lora_linear_bwd(case["x"], wq, case["A"], case["B"], 32.0, case["dY"])
    mags = linear_mags(case["x"], wq, case["A"], case["B"], 32.0, case["dY"])
    t, n, k = case["x"].shape[0], case["W"].shape[0], case["W"].shape[1]
    check_f32_output(f32_of(da), da_ref, "dA", mag=mags["dA"], terms=n + t)
    check_f32_output(f32_of(db), db_ref, "dB", mag=mags["dB"], terms=k + t)


def test_few_token_repeat_is_bitwise_identical(gpu_lib):
    case = S.linear_case(9, 3584, 3584, proj="q")
    _, dev = _prepare(gpu_lib, case, 16)
    a = _run(gpu_lib, dev, 32.0)
    b = _run(gpu_lib, dev, 32.0)
    for p, q in zip(a, b):
        assert torch.equal(p, q)


def test_base_only_rank0(gpu_lib):
    _check_case(gpu_lib, 100, 256, 512, 0)


def test_b_zero_equals_base_only(gpu_lib):
    t, n, k = 130, 384, 512
    case = S.linear_case(t, n, k)
    case["B"] = np.zeros_like(case["B"])
    wq, dev = _prepare(gpu_lib, case, 16)
    y_lora, _ = gpu_lib.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], dev["A"], dev["B"], 32.0)
    y_base, _ = gpu_lib.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], None, None, 32.0)
    torch.cuda.synchronize()
    assert torch.equal(y_lora, y_base)


def test_integer_exact_case(gpu_lib):
    """Codes in {0, 7, 15} with absmax 2^e and small integers elsewhere: every
    partial sum is exact in fp32, so the GPU output must be exactly the oracle's
    value rounded once to bf16 (fp32 outputs must equal it exactly)."""
    rng = np.random.default_rng(5)
    t, n, k, r = 96, 160, 256, 16
    codes = rng.choice([0, 7, 15], size=(n, k)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    absmax = np.full((n, k // 64), 0.125, np.float32)
    wq = O.dequantize(packed, absmax)
    ints = lambda shape, lo, hi: S.to_bf16_bits(rng.integers(lo, hi + 1, size=shape).astype(np.float32))
    x, a, b, dy = ints((t, k), -2, 2), ints((r, k), -1, 1), ints((n, r), -1, 1), ints((t, n), -2, 2)
    alpha = 1.0 * r / 8.0                                                  # s = 0.125
    dev = {"codes": torch.from_numpy(packed).cuda(), "absmax": torch.from_numpy(absmax).cuda(),
           "x": to_dev_bf16(x), "dY": to_dev_bf16(dy), "A": to_dev_bf16(a), "B": to_dev_bf16(b)}
    y, u, dx, da, db = _run(gpu_lib, dev, alpha)
    y_ref, u_ref = O.lora_linear_fwd(x, wq, a, b, alpha)
    dx_ref, da_ref, db_ref = O.lora_linear_bwd(x, wq, a, b, alpha, dy)
    # every partial sum is exact in fp32, so the single rounding to bf16 is the only one
    for ref in (y_ref, dx_ref, u_ref, da_ref, db_ref):
        assert np.array_equal(ref.astype(np.float32).astype(np.float64), ref)
    assert np.array_equal(bits_of(y), O.f32_to_bf16_bits(y_ref.astype(np.float32)))
    assert np.array_equal(bits_of(dx), O.f32_to_bf16_bits(dx_ref.astype(np.float32)))
    assert np.array_equal(f32_of(u).astype(np.float64), u_ref)
    assert np.array_equal(f32_of(da).astype(np.float64), da_ref)
    assert np.array_equal(f32_of(db).astype(np.float64), db_ref)


def test_repeat_is_bitwise_identical(gpu_lib):
    case = S.linear_case(512, 3584, 3584, proj="q")
    _, dev = _prepare(gpu_lib, case, 16)
    a = _run(gpu_lib, dev, 32.0)
    b = _run(gpu_lib, dev, 32.0)
    for p, q in zip(a, b):
        assert torch.equal(p, q)


def test_dx_can_be_skipped(gpu_lib):
    case = S.linear_case(64, 256, 256)
    wq, dev = _prepare(gpu_lib, case, 16)
    y, u = gpu_lib.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], dev["A"], dev["B"], 32.0)
    dx, da, db = gpu_lib.lora_linear_bwd(dev["codes"], dev["absmax"], dev["x"], u, dev["dY"], dev["A"], dev["B"],
                                         32.0, need_dx=False)
    torch.cuda.synchronize()
    assert dx is None
    _, da_ref, db_ref = O.lora_linear_bwd(case["x"], wq, case["A"], case["B"], 32.0, case["dY"])
    mags = linear_mags(case["x"], wq, case["A"], case["B"], 32.0, case["dY"])
    t, n, k = case["x"].shape[0], case["W"].shape[0], case["W"].shape[1]
    check_f32_output(f32_of(da), da_ref, "dA", mag=mags["dA"], terms=n + t)
    check_f32_output(f32_of(db), db_ref, "dB", mag=mags["dB"], terms=k + t)
