"""The dense-bf16 base variant (the experimental "bf16_bitwise" mode of the Poros API
reference, "PorosTrainer.from_pretrained"): the linear vs the fp64 oracle with W the
bf16 weights themselves, and the streamed dense stack vs resident, bitwise."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, check_linear, f32_of, linear_mags, to_dev_bf16

pytestmark = pytest.mark.gpu
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


@pytest.mark.parametrize("t,n,k,r", [
    (256, 1024, 1024, 16),   # the single-linear workload
    (300, 400, 640, 16),     # ragged in every dimension
    (1, 128, 256, 16),       # one token (128-token kernels for every T)
    (17, 3584, 512, 5),      # odd rank
    (129, 512, 3584, 64),    # maximum rank, split contraction
    (64, 256, 512, 0),       # base only
    (300, 10992, 640, 16),   # 258 y tiles: the last 2 split over K
    (300, 640, 22976, 16),   # 540 dX tiles: the last 28 split over N
])
def test_dense_linear_matches_oracle(gpu_lib, t, n, k, r):
    _dense_case(gpu_lib, t, n, k, r)


def _dense_shapes(count=10, seed=20261204):
    """Seeded shapes for the dense variant: T 1..600, N a multiple of 16 up to 4096, K a
    multiple of 64 up to 4096 (dense weights: N*K*2 bytes), ranks 0..64, alpha 8..64."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        t, n, k = int(rng.integers(1, 601)), 16 * int(rng.integers(1, 257)), 64 * int(rng.integers(1, 65))
        if t * n * k > 2_000_000_000:
            continue
        out.append((t, n, k, int(rng.choice([0, 1, 7, 16, 16, 40, 64])), float(rng.choice([8.0, 32.0, 64.0])),
                    int(rng.integers(1, 1 << 30))))
    return out


@pytest.mark.parametrize("t,n,k,r,alpha,seed", _dense_shapes())
def test_dense_random_shapes(gpu_lib, t, n, k, r, alpha, seed):
    _dense_case(gpu_lib, t, n, k, r, alpha, seed)


def _dense_case(gpu_lib, t, n, k, r, alpha=32.0, seed=42):
    case = S.linear_case(t, n, k, r=max(r, 1), seed=seed)
    if r == 0:
        case["A"], case["B"] = np.zeros((0, k), np.uint16), np.zeros((n, 0), np.uint16)
    w = to_dev_bf16(case["W"])
    A = to_dev_bf16(case["A"]) if r else None
    B = to_dev_bf16(case["B"]) if r else None
    y, u = gpu_lib.lora_linear_fwd_bf16(w, to_dev_bf16(case["x"]), A, B, alpha)
    dx, da, db = gpu_lib.lora_linear_bwd_bf16(w, to_dev_bf16(case["x"]), u, to_dev_bf16(case["dY"]), A, B, alpha)
    torch.cuda.synchronize()
    y_ref, u_ref = O.lora_linear_fwd(case["x"], case["W"], case["A"], case["B"], alpha)
    dx_ref, da_ref, db_ref = O.lora_linear_bwd(case["x"], case["W"], case["A"], case["B"], alpha, case["dY"])
    refs = {"y": y_ref, "u": u_ref, "dx": dx_ref, "dA": da_ref, "dB": db_ref}
    mags = linear_mags(case["x"], case["W"], case["A"], case["B"], alpha, case["dY"])
    outs = {"y": bits_of(y), "dx": bits_of(dx)}
    if r:
        outs.update(u=f32_of(u), dA=f32_of(da), dB=f32_of(db))
    check_linear(outs, refs, mags, t, n, k, r, f"dense {t}x{n}x{k} r{r}")


def test_dense_equals_nf4_on_the_dequantised_base(gpu_lib):
    """Fed the dequantised NF4 base as dense weights, the dense kernels compute the
    NF4 kernels' results bit for bit (same tiles, same contraction order)."""
    t, n, k = 200, 768, 1024
    case = S.linear_case(t, n, k)
    codes, absmax = O.quantize(O.bf16_bits_to_f64(case["W"]).astype(np.float32))
    wq = to_dev_bf16(O.dequantize(codes, absmax))
    c, s = torch.from_numpy(codes).cuda(), torch.from_numpy(absmax).cuda()
    x, dy, A, B = (to_dev_bf16(case[key]) for key in ("x", "dY", "A", "B"))
    y1, u1 = gpu_lib.lora_linear_fwd(c, s, x, A, B, 32.0)
    y2, u2 = gpu_lib.lora_linear_fwd_bf16(wq, x, A, B, 32.0)
    d1 = gpu_lib.lora_linear_bwd(c, s, x, u1, dy, A, B, 32.0)
    d2 = gpu_lib.lora_linear_bwd_bf16(wq, x, u2, dy, A, B, 32.0)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(u1, u2)
    for a, b in zip(d1, d2):
        assert torch.equal(a, b)


@pytest.fixture(scope="module")
def ST(gpu_lib):
    from nf4_weight_streamed_amd import stack

    return stack


def _dense_stack(ST, n_layers, block_size):
    dims = ST.StackDims(hidden=128, q=128, kv=32, inter=256, head_dim=32)
    w = {(l, p): S.weight(*dims.shapes()[p], proj=p, layer=l) for l in range(n_layers) for p in PROJS}
    lo = {}
    for l in range(n_layers):
        for p in PROJS:
            n, k = dims.shapes()[p]
            lo[(l, p)] = (S.lora_a(16, k, proj=p, layer=l), S.lora_b(n, 16, proj=p, layer=l, std=0.05))
    base = ST.HostBF16Base(dims, n_layers, block_size, lambda l, p, n, k: to_dev_bf16(w[(l, p)]))
    lora = ST.LoraParams(dims, n_layers, 16, lambda l, p, n, k: tuple(to_dev_bf16(t) for t in lo[(l, p)]))
    return dims, w, lo, base, lora


def _step(ST, base, lora, T, mode, **kw):
    st = ST.NF4Stack(base, lora, T, 32.0, mode=mode, **kw)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    h0 = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh = torch.randn(T, base.dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    out, dh0 = st.step(h0, dh)
    out2, _ = st.step(h0, dh)
    torch.cuda.synchronize()
    res = (out.clone(), dh0.clone(), out2.clone(), [{p: (a.clone(), b.clone()) for p, (a, b) in gl.items()}
                                                   for gl in st.grads])
    st.close()
    return res


@pytest.mark.parametrize("block_size", [1, 2, 3])
def test_dense_stack_streamed_equals_resident(ST, block_size):
    _, _, _, base, lora = _dense_stack(ST, 5, block_size)
    ref = _step(ST, base, lora, 40, "resident")
    for kw in ({"prefetch": True}, {"prefetch": False}, {"prefetch": True, "remat": True}):
        got = _step(ST, base, lora, 40, "streamed", **kw)
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1]) and torch.equal(got[2], ref[0])
        for ga, gb in zip(got[3], ref[3]):
            for p in PROJS:
                assert torch.equal(ga[p][0], gb[p][0]) and torch.equal(ga[p][1], gb[p][1])


def test_dense_stack_matches_oracle(ST):
    L, T, alpha = 3, 40, 32.0
    dims, w, lo, base, lora = _dense_stack(ST, L, 2)
    h0 = S.activations(T, dims.hidden, tensor="h0")
    dh = S.activations(T, dims.hidden, tensor="dH")
    st = ST.NF4Stack(base, lora, T, alpha, mode="streamed")
    out, dh0 = st.step(to_dev_bf16(h0), to_dev_bf16(dh))
    torch.cuda.synchronize()
    od = O.StackLayerDims(dims.hidden, dims.q, dims.kv, dims.inter, dims.head_dim)
    layers = [{p: (w[(l, p)], lo[(l, p)][0], lo[(l, p)][1]) for p in PROJS} for l in range(L)]
    out_ref, saved = O.stack_forward(h0, layers, od, alpha)
    dh0_ref, grads = O.stack_backward(dh, layers, od, alpha, saved)
    assert O.rel_l2(O.bf16_bits_to_f64(bits_of(out)), out_ref) <= 2e-3
    assert O.rel_l2(O.bf16_bits_to_f64(bits_of(dh0)), dh0_ref) <= 2e-3
    for l in range(L):
        for p in ("v", "o", "gate", "up", "down"):
            dA, dB = st.grads[l][p]
            assert O.rel_l2(f32_of(dA), grads[l][p + "_dA"]) <= 2e-3, (l, p)
            assert O.rel_l2(f32_of(dB), grads[l][p + "_dB"]) <= 2e-3, (l, p)
    st.close()
