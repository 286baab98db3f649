"""Shared test helpers: tensor <-> bit-pattern conversion and tolerance checks."""

import numpy as np
import torch

import oracle as O

REL_L2_BAR = 2e-3          # GEMM outputs and gradients vs the fp64 oracle
FLOOR_MARGIN = 3e-4        # bf16 outputs: at most this much above the rounding floor
FP32_GRAD_BAR = 1e-4       # fp32 outputs (dA, dB, u): well inside the bar


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def bits_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def check_bf16_output(gpu_bits: np.ndarray, exact: np.ndarray, what: str) -> float:
    """rel-L2 of a bf16 GPU output against the unrounded oracle value, with the floor check."""
    got = O.bf16_bits_to_f64(gpu_bits)
    rel = O.rel_l2(got, exact)
    floor = O.rel_l2(O.round_bf16(exact), exact)
    assert rel <= REL_L2_BAR, f"{what}: rel-L2 {rel:.3e} > {REL_L2_BAR}"
    assert rel <= floor + FLOOR_MARGIN, f"{what}: rel-L2 {rel:.3e} > floor {floor:.3e} + {FLOOR_MARGIN}"
    return rel


def check_f32_output(gpu: np.ndarray, exact: np.ndarray, what: str, bar: float = FP32_GRAD_BAR) -> float:
    rel = O.rel_l2(gpu, exact)
    assert rel <= bar, f"{what}: rel-L2 {rel:.3e} > {bar}"
    return rel
