"""The linear at full projection sizes, in the launch configuration bench.py times,
against the fp64 oracle on sampled outputs (each computed one by one from the rows or
columns of the dequantised base it needs) and on the complete LoRA gradients.

Shapes: the 7B gate projection at 512 tokens (the layer step's largest GEMM, the
128-token kernels) and the 72B gate projection at 16 and 1 tokens (the few-token
kernels). The NF4 storage is drawn at random by the seeded generator (quantising these
weights on the CPU would take minutes); the oracle dequantises what it needs.
"""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, check_bf16_output, check_f32_output, f32_of, to_dev_bf16

pytestmark = pytest.mark.gpu

SAMPLES = 96


def _w_rows(codes, absmax, rows):
    return O.bf16_bits_to_f64(O.dequantize(codes[rows], absmax[rows]))


def _w_col(codes, absmax, k):
    blk = k // O.NF4_BLOCK
    w = O.dequantize(codes[:, blk * 32:(blk + 1) * 32], absmax[:, blk:blk + 1])
    return O.bf16_bits_to_f64(w[:, k % O.NF4_BLOCK])


@pytest.mark.parametrize("t,n,k,proj", [(512, 18944, 3584, "gate"), (512, 3584, 18944, "down"),
                                        (16, 29568, 8192, "gate"), (1, 29568, 8192, "gate")])
def test_full_size_projection_sampled(gpu_lib, t, n, k, proj):
    r, alpha = S.RANK, S.ALPHA
    print(f"full-size projection T={t} N={n} K={k}", flush=True)
    codes, absmax = S.nf4_storage(n, k, proj=proj)
    x = S.activations(t, k, proj=proj)
    dy = S.activations(t, n, proj=proj, tensor="dY")
    a = S.lora_a(r, k, proj=proj)
    b = S.lora_b(n, r, proj=proj)
    dev_c, dev_s = torch.from_numpy(codes).cuda(), torch.from_numpy(absmax).cuda()
    dx_, dy_, da_, db_ = to_dev_bf16(x), to_dev_bf16(dy), to_dev_bf16(a), to_dev_bf16(b)
    y, u = gpu_lib.lora_linear_fwd(dev_c, dev_s, dx_, da_, db_, alpha)
    dx, dA, dB = gpu_lib.lora_linear_bwd(dev_c, dev_s, dx_, u, dy_, da_, db_, alpha)
    torch.cuda.synchronize()
    y, u, dx, dA, dB = bits_of(y), f32_of(u), bits_of(dx), f32_of(dA), f32_of(dB)

    s = O.lora_scale(alpha, r)
    xf, dyf, af, bf = (O.bf16_bits_to_f64(v) for v in (x, dy, a, b))
    ax, ady, aa, ab = (np.abs(v) for v in (xf, dyf, af, bf))
    u_ref = xf @ af.T
    g_ref = dyf @ bf
    u_mag, g_mag = ax @ aa.T, ady @ ab
    check_f32_output(u, u_ref, "u", mag=u_mag, terms=k)
    check_f32_output(dA, s * (g_ref.T @ xf), "dA", mag=s * (g_mag.T @ ax), terms=n + t)
    check_f32_output(dB, s * (dyf.T @ u_ref), "dB", mag=s * (ady.T @ u_mag), terms=k + t)

    # every token of the sampled rows / columns: at least ~2000 bf16 outputs each, so that
    # the rounding floor the check compares against is itself well estimated
    samples = max(SAMPLES, 2048 // t)
    rng = np.random.default_rng(7)
    rows = np.unique(np.concatenate([rng.choice(n, samples, replace=False), [0, n - 1]]))
    wr = _w_rows(codes, absmax, rows)
    y_ref = xf @ wr.T + s * (u_ref @ bf[rows].T)
    y_mag = ax @ np.abs(wr).T + s * (u_mag @ ab[rows].T)
    check_bf16_output(y[:, rows], y_ref, f"y sampled T={t}", mag=y_mag, terms=k + r)

    cols = np.unique(np.concatenate([rng.choice(k, samples, replace=False), [0, k - 1]]))
    wc = np.stack([_w_col(codes, absmax, kk) for kk in cols], axis=1)
    dx_ref = dyf @ wc + s * (g_ref @ af[:, cols])
    dx_mag = ady @ np.abs(wc) + s * (g_mag @ aa[:, cols])
    check_bf16_output(dx[:, cols], dx_ref, f"dX sampled T={t}", mag=dx_mag, terms=n + r)
