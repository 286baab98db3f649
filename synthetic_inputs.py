"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the method: it only draws random numbers
and turns them into bfloat16 bit patterns with torch's own float32 -> bfloat16
cast. Both the fp64 oracle and the HIP path receive the same arrays.

Distributions (one linear): W ~ N(0, 0.02), x and dY ~ N(0, 1),
A ~ U(-1/sqrt(K), 1/sqrt(K)), B ~ N(0, 0.01); r = 16, alpha = 32, seed 42 (the
default seed of the Poros API reference, "PorosConfig" Fields). Every tensor
draws from its own counter-keyed numpy stream: SeedSequence([seed, layer,
projection, tensor]) so that adding a tensor never shifts another.
"""

from __future__ import annotations

import numpy as np

SEED = 42
RANK = 16
ALPHA = 32.0

PROJ_IDS = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "single": 7}
TENSOR_IDS = {"W": 0, "x": 1, "A": 2, "B": 3, "dY": 4, "h0": 5, "dH": 6, "codes": 7, "absmax": 8}

# (hidden, q, kv, intermediate, layers) of the Qwen2.5-shaped stacks
QWEN_SHAPES = {
    "7b": (3584, 3584, 512, 18944, 28),
    "32b": (5120, 5120, 1024, 27648, 64),
    "72b": (8192, 8192, 1024, 29568, 80),
}


def rng(tensor: str, proj: str = "single", layer: int = 0, seed: int = SEED) -> np.random.Generator:
    key = [seed, layer, PROJ_IDS[proj], TENSOR_IDS[tensor]]
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(key)))


def to_bf16_bits(a) -> np.ndarray:
    """float -> bfloat16 bit patterns via torch's CPU cast (round to nearest even)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(np.asarray(a, dtype=np.float32)))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(bits) -> np.ndarray:
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def weight(n: int, k: int, proj: str = "single", layer: int = 0, seed: int = SEED) -> np.ndarray:
    """Base weight W [N, K] ~ N(0, 0.02), as bf16 bits."""
    return to_bf16_bits(rng("W", proj, layer, seed).normal(0.0, 0.02, size=(n, k)))


def activations(t: int, k: int, proj: str = "single", layer: int = 0, seed: int = SEED,
                tensor: str = "x") -> np.ndarray:
    """x [T, K] (or dY with tensor='dY') ~ N(0, 1), as bf16 bits."""
    return to_bf16_bits(rng(tensor, proj, layer, seed).normal(0.0, 1.0, size=(t, k)))


def lora_a(r: int, k: int, proj: str = "single", layer: int = 0, seed: int = SEED) -> np.ndarray:
    bound = 1.0 / np.sqrt(k)
    return to_bf16_bits(rng("A", proj, layer, seed).uniform(-bound, bound, size=(r, k)))


def lora_b(n: int, r: int, proj: str = "single", layer: int = 0, seed: int = SEED,
           std: float = 0.01) -> np.ndarray:
    return to_bf16_bits(rng("B", proj, layer, seed).normal(0.0, std, size=(n, r)))


def linear_case(t: int, n: int, k: int, r: int = RANK, proj: str = "single", layer: int = 0,
                seed: int = SEED, b_std: float = 0.01) -> dict:
    """All bf16-bit inputs of one linear: W, x, A, B, dY."""
    return {
        "W": weight(n, k, proj, layer, seed),
        "x": activations(t, k, proj, layer, seed, "x"),
        "A": lora_a(r, k, proj, layer, seed),
        "B": lora_b(n, r, proj, layer, seed, b_std),
        "dY": activations(t, n, proj, layer, seed, "dY"),
    }


def stack_dims(model: str):
    h, q, kv, i, layers = QWEN_SHAPES[model]
    return h, q, kv, i, layers


def proj_shapes(hidden: int, q: int, kv: int, inter: int) -> dict:
    """(N, K) of the seven projections of one layer, in layer order."""
    return {"q": (q, hidden), "k": (kv, hidden), "v": (kv, hidden), "o": (hidden, q),
            "gate": (inter, hidden), "up": (inter, hidden), "down": (hidden, inter)}


def nf4_storage(n: int, k: int, proj: str = "single", layer: int = 0, seed: int = SEED):
    """Random NF4 storage (codes uint8 [N, K/2], absmax float32 [N, K/64]) for the
    full-size checks, where quantising a large weight on the CPU would be slow:
    uniform code bytes, and block scales spread like the largest |value| of 64 draws
    of N(0, 0.02) (0.02 x U(2.0, 2.9))."""
    codes = rng("codes", proj, layer, seed).integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    absmax = (0.02 * rng("absmax", proj, layer, seed).uniform(2.0, 2.9, size=(n, k // 64))).astype(np.float32)
    return codes, absmax
