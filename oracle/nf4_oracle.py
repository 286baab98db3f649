"""fp64 CPU oracle: NF4 codec, frozen-NF4-base LoRA linear (fwd + bwd) and the tiny stack.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): plain, slow numpy written
from the definitions below; nothing from the HIP path is imported or shared.

Pages cited (by title and section):
  [consumer]  "Poros on consumer GPUs": "What you need besides VRAM" (the NF4 base
              held in host RAM, its size set by the NF4 storage format), "OOM
              playbook" (block_size never affects parity).
  [api]       Poros API reference: "PorosTrainer.from_pretrained" (quantization
              "nf4" = 4-bit NF4 QLoRA, lora_rank 16, lora_alpha 32, bitwise
              resident parity), "PorosModel.from_pretrained" (torch_dtype
              bfloat16), "patch_hf_model" Behavior (frozen base; adapters are the
              only trainable parameters), "PorosConfig" Fields (seed 42).
  [hn]        HN comment thread on streaming the frozen base (item 49166984),
              main comment: the base is read, never written; it streams into a
              pool of pre-allocated device buffers one layer/block at a time.

Readings where the pages are silent:
  R1  NF4 levels are QLoRA's 4-bit NormalFloat: 8 positive and 7 negative N(0,1)
      quantiles normalised to +-1 plus an exact zero, built in fp64 with the
      conventional offset delta = ((1-1/30)+(1-1/32))/2 and rounded once to fp32.
  R2  Blocks are 64 consecutive elements of a row; one fp32 absmax per block.
  R3  v = RN32(w/absmax) by correctly rounded division; code = number of level
      midpoints strictly below v (nearest level, ties to the lower code).
  R4  All-zero block: absmax 0 and every code 7 (the level 0).
  R5  Packing: element 2i in the low nibble of byte i, 2i+1 in the high nibble.
  R6  Dequantised weight = RNbf(RN32(level * absmax)): an fp32 product, then a
      round-to-nearest-even to bf16 (two roundings, not one).
  R7  LoRA scale s = RN32(alpha / r); y = x.W^T + s.(x.A^T).B^T; no dropout.
  R8  Backward: g = dY.B, dX = dY.W + s.g.A, dA = s.g^T.x, dB = s.dY^T.u; the
      base receives no gradient ([api] patch_hf_model Behavior 3; [hn]).
  R9  Stack layer (attention mixing = identity): h_a = RMSNorm(h);
      h' = h + L_o(repeat_kv(L_v(h_a))); h_m = RMSNorm(h');
      h'' = h' + L_down(SiLU(L_gate(h_m)) * L_up(h_m)); q = L_q(h_a), k = L_k(h_a)
      are computed and receive zero gradient. RMSNorm: unit gain, eps 1e-6.
  R10 Stack storage points: activations are stored in bf16 (the model dtype,
      [api] PorosModel.from_pretrained torch_dtype) at the outputs listed in
      ``stack_forward``; the oracle rounds at the same points (``round_storage``)
      and computes everything between them in fp64.
  R12 merge_and_unload ([api] "PorosModel.merge_and_unload": the adapters are merged
      into the base and the module unloaded): the merged weight is W + s.B.A, kept
      dense in the model dtype (bf16); the pages do not re-quantise it, and a dense
      weight keeps the merged module's output equal to the adapted one's.

Pins (tests/test_oracle_*.py), one line per function:
  nf4_codebook     pinned: two independent inverse-normal routines agree bitwise;
                   forward CDF (math.erf) reproduces the quantile grid; -1/0/+1, order.
  quantize         pinned: exact-rational brute-force argmin on tiny blocks; exact
                   round trip of level*2^e; zero block; power-of-two scale
                   invariance; idempotence; per-row-block vs whole-tensor bytes.
  dequantize       pinned: library two-step rounding (torch fp32 product + bf16
                   cast); code 7 -> +0, 15 -> RNbf(s), 0 -> RNbf(-s).
  f32_to_bf16_bits pinned: torch's float32 -> bfloat16 cast (RNE) on edge cases.
  lora_linear_fwd  pinned: integer closed form; B = 0 equals the base-only GEMM;
                   central finite differences of <dY, y>.
  lora_linear_bwd  pinned: central finite differences; dot-product adjoint identity.
  merge_lora       pinned: x.W_m^T equals the (separately pinned) LoRA forward y; B = 0
                   gives the dequantised base bit for bit; integer brute force.
  stack_forward/backward  pinned: central finite differences (storage rounding
                   off); zero-weight layers are the identity; RMSNorm and SiLU
                   against textbook closed forms; storage rounding = f32_to_bf16_bits.
"""

from __future__ import annotations

import math
import statistics

import numpy as np

NF4_BLOCK = 64          # R2
NF4_ZERO_CODE = 7       # R1: sorted level 7 is the exact 0
RMS_EPS = 1e-6          # R9

__all__ = [
    "NF4_BLOCK", "NF4_ZERO_CODE", "RMS_EPS",
    "nf4_codebook", "f32_to_bf16_bits", "bf16_bits_to_f64", "round_bf16",
    "quantize", "unpack_codes", "dequantize",
    "lora_scale", "lora_linear_fwd", "lora_linear_bwd", "lora_linear_fwd_f64",
    "lora_linear_bwd_f64", "rel_l2", "merge_lora",
    "rmsnorm_fwd", "rmsnorm_bwd", "silu", "silu_grad",
    "StackLayerDims", "stack_forward", "stack_backward",
]


# --------------------------------------------------------------------------- codebook

def nf4_codebook(ppf=None) -> np.ndarray:
    """The 16 NF4 levels as float32, ascending (reading R1; [api] quantization "nf4").

    ``ppf`` is the N(0,1) inverse CDF used (stdlib NormalDist by default); the
    construction is carried out in fp64 and each level is rounded once to fp32.
    """
    if ppf is None:
        ppf = statistics.NormalDist().inv_cdf
    delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))
    top = ppf(delta)
    # 8 positive quantiles: probability grid from delta down towards 1/2 in 8 steps
    positive = [ppf(delta - (delta - 0.5) * i / 8.0) / top for i in range(8)]
    # 7 negative quantiles: the same grid in 7 steps, mirrored
    negative = [-ppf(delta - (delta - 0.5) * i / 7.0) / top for i in range(7)]
    levels = sorted(positive + negative + [0.0])
    return np.array(levels, dtype=np.float64).astype(np.float32)


# --------------------------------------------------------------------------- bf16 helpers

def f32_to_bf16_bits(f) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns the uint16 bits."""
    f = np.ascontiguousarray(np.asarray(f, dtype=np.float32))
    if not np.isfinite(f).all():
        raise ValueError("non-finite value: the oracle supports finite inputs only")
    b = f.view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    return ((b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns, as float64."""
    bits = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """RNbf of float64 values through float32 (used only at storage points, R10).

    Values reaching a storage point on the GPU are fp32 sums, so the stored value
    is RNbf(RN32(.)); the oracle applies the same two steps.
    """
    return bf16_bits_to_f64(f32_to_bf16_bits(np.asarray(x, dtype=np.float64).astype(np.float32)))


# --------------------------------------------------------------------------- quantise

def quantize(w) -> tuple[np.ndarray, np.ndarray]:
    """NF4-quantise a row-major [N, K] matrix (readings R1-R5).

    ``w`` holds float32 values (bf16 weights are passed as their exact float32
    values). Returns (codes uint8 [N, K/2], absmax float32 [N, K/64]).
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % NF4_BLOCK != 0:
        raise ValueError(f"quantize needs [N, K] with K % {NF4_BLOCK} == 0, got {w.shape}")
    if not np.isfinite(w).all():
        raise ValueError("quantize supports finite inputs only")
    levels = nf4_codebook().astype(np.float64)
    midpoints = (levels[:-1] + levels[1:]) / 2.0            # exact in fp64
    n, k = w.shape
    blocks = w.reshape(n, k // NF4_BLOCK, NF4_BLOCK).astype(np.float64)
    absmax = np.abs(blocks).max(axis=2)                      # a max of fp32 values: exact
    divisor = np.where(absmax > 0.0, absmax, 1.0)
    # RN32(w / s): fp64 quotient rounded to fp32 is the correctly rounded fp32 quotient
    v = (blocks / divisor[..., None]).astype(np.float32).astype(np.float64)
    codes = np.zeros(v.shape, dtype=np.uint8)
    for m in midpoints:                                      # count midpoints strictly below v
        codes += (v > m)
    codes[absmax == 0.0] = NF4_ZERO_CODE                     # R4
    codes = codes.reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)   # R5
    return packed, absmax.astype(np.float32)


def unpack_codes(packed) -> np.ndarray:
    """[N, K/2] packed bytes -> [N, K] codes (R5)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], packed.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


# --------------------------------------------------------------------------- dequantise

def dequantize(packed, absmax) -> np.ndarray:
    """Dequantise to bf16 bits [N, K]: RNbf(RN32(level[code] * absmax)) (reading R6)."""
    codes = unpack_codes(packed)
    absmax = np.asarray(absmax, dtype=np.float32)
    if absmax.shape != (codes.shape[0], codes.shape[1] // NF4_BLOCK):
        raise ValueError(f"absmax shape {absmax.shape} does not match codes {codes.shape}")
    levels = nf4_codebook()
    scale = np.repeat(absmax, NF4_BLOCK, axis=1).astype(np.float64)
    exact = levels[codes].astype(np.float64) * scale          # product of two fp32: exact in fp64
    return f32_to_bf16_bits(exact.astype(np.float32))         # RN32, then RNbf


# --------------------------------------------------------------------------- linear

def lora_scale(alpha: float, r: int) -> float:
    """s = RN32(alpha / r) (R7); 0 when r == 0 (base only)."""
    if r == 0:
        return 0.0
    return float(np.float32(alpha) / np.float32(r))


def _as_f64(a) -> np.ndarray:
    """uint16 arrays are bf16 bit patterns; anything else is taken as float values."""
    a = np.asarray(a)
    return bf16_bits_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def lora_linear_fwd_f64(x, w, a, b, s):
    """y = x.W^T + s.(x.A^T).B^T and u = x.A^T in fp64 (R7). Shapes [T,K],[N,K],[r,K],[N,r]."""
    u = x @ a.T
    return x @ w.T + s * (u @ b.T), u


def lora_linear_bwd_f64(x, w, a, b, s, dy):
    """(dX, dA, dB) in fp64 (R8): g = dY.B; dX = dY.W + s.g.A; dA = s.g^T.x; dB = s.dY^T.u."""
    u = x @ a.T
    g = dy @ b
    return dy @ w + s * (g @ a), s * (g.T @ x), s * (dy.T @ u)


def lora_linear_fwd(x, w, a, b, alpha):
    """Forward of the frozen-NF4-base LoRA linear (R7).

    x [T, K], dequantised base W [N, K], A [r, K], B [N, r]: bf16 bit patterns
    (uint16) or float arrays. Returns (y [T, N], u [T, r]) as float64, unrounded.
    """
    a = _as_f64(a)
    return lora_linear_fwd_f64(_as_f64(x), _as_f64(w), a, _as_f64(b), lora_scale(alpha, a.shape[0]))


def lora_linear_bwd(x, w, a, b, alpha, dy):
    """Backward (R8): returns (dx [T, K], dA [r, K], dB [N, r]) as float64; there is no dW."""
    a = _as_f64(a)
    return lora_linear_bwd_f64(_as_f64(x), _as_f64(w), a, _as_f64(b),
                               lora_scale(alpha, a.shape[0]), _as_f64(dy))


def merge_lora(w, a, b, alpha):
    """Merged dense weight W + s.B.A (R12) in float64, unrounded.

    W [N, K] is the dequantised base (bf16 bits or floats), A [r, K], B [N, r];
    s = lora_scale(alpha, r). The exported weight is this value rounded to bf16.
    """
    a = _as_f64(a)
    return _as_f64(w) + lora_scale(alpha, a.shape[0]) * (_as_f64(b) @ a)


def rel_l2(a, ref) -> float:
    """||a - ref||_2 / ||ref||_2 in fp64 over the whole tensor."""
    a = np.asarray(a, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((a - ref).ravel()))
    if den == 0.0:
        return num
    return num / den


# --------------------------------------------------------------------------- stack glue

def rmsnorm_fwd(h, eps=RMS_EPS):
    """Unit-gain RMSNorm over the last axis: h / sqrt(mean(h^2) + eps)."""
    h = np.asarray(h, dtype=np.float64)
    return h / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)


def rmsnorm_bwd(h, dy, eps=RMS_EPS):
    """Gradient of rmsnorm_fwd: rho*dy - rho^3 * h * mean(dy*h), rho = (mean(h^2)+eps)^-1/2."""
    h = np.asarray(h, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    rho = 1.0 / np.sqrt(np.mean(h * h, axis=-1, keepdims=True) + eps)
    return rho * dy - rho ** 3 * h * np.mean(dy * h, axis=-1, keepdims=True)


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z / (1.0 + np.exp(-z))


def silu_grad(z):
    z = np.asarray(z, dtype=np.float64)
    sig = 1.0 / (1.0 + np.exp(-z))
    return sig * (1.0 + z * (1.0 - sig))


class StackLayerDims:
    """Widths of one stack layer: hidden, q, kv, intermediate, head_dim (R9)."""

    def __init__(self, hidden, q, kv, inter, head_dim=128):
        if q % head_dim or kv % head_dim or q % kv:
            raise ValueError("q and kv must be multiples of head_dim, and q of kv")
        self.hidden, self.q, self.kv, self.inter, self.head_dim = hidden, q, kv, inter, head_dim

    def proj_shapes(self):
        """(N, K) of q, k, v, o, gate, up, down in that order."""
        h, q, kv, i = self.hidden, self.q, self.kv, self.inter
        return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q),
                "gate": (i, h), "up": (i, h), "down": (h, i)}


def _repeat_kv(v, dims):
    """Each head_dim-wide kv head serves q/kv consecutive query heads."""
    t = v.shape[0]
    heads = v.reshape(t, dims.kv // dims.head_dim, 1, dims.head_dim)
    rep = dims.q // dims.kv
    return np.broadcast_to(heads, (t, dims.kv // dims.head_dim, rep, dims.head_dim)).reshape(t, dims.q)


def _repeat_kv_bwd(da, dims):
    t = da.shape[0]
    rep = dims.q // dims.kv
    return da.reshape(t, dims.kv // dims.head_dim, rep, dims.head_dim).sum(axis=2).reshape(t, dims.kv)


def _lin(xv, p, alpha):
    w, a, b = p
    return lora_linear_fwd_f64(xv, w, a, b, lora_scale(alpha, a.shape[0]))


def _lin_bwd(xv, p, alpha, dy):
    w, a, b = p
    return lora_linear_bwd_f64(xv, w, a, b, lora_scale(alpha, a.shape[0]), dy)


def _layer_f64(layer):
    return {name: tuple(_as_f64(t) for t in layer[name]) for name in layer}


def stack_forward(h0_bits, layers, dims, alpha, round_storage=True):
    """Forward of the identity-mixing stack (R9, R10).

    layers: list of dicts name -> (W bits [N,K], A bits [r,K], B bits [N,r]).
    Storage points (rounded to bf16 when ``round_storage``): h_a, q, k, v, o,
    h', h_m, gate, up, m = SiLU(gate)*up, down, h''.
    Returns (h_out float64, saved) where ``saved`` feeds ``stack_backward``.
    """
    rnd = round_bf16 if round_storage else (lambda z: np.asarray(z, dtype=np.float64))
    h = _as_f64(h0_bits)
    saved = []
    for layer in layers:
        p = _layer_f64(layer)
        st = {"h": h}
        st["ha"] = rnd(rmsnorm_fwd(h))
        for name in ("q", "k", "v"):
            y, st["u_" + name] = _lin(st["ha"], p[name], alpha)
            st[name] = rnd(y)
        st["a"] = _repeat_kv(st["v"], dims)
        y, st["u_o"] = _lin(st["a"], p["o"], alpha)
        st["o"] = rnd(y)
        st["h1"] = rnd(h + st["o"])
        st["hm"] = rnd(rmsnorm_fwd(st["h1"]))
        for name in ("gate", "up"):
            y, st["u_" + name] = _lin(st["hm"], p[name], alpha)
            st[name] = rnd(y)
        st["m"] = rnd(silu(st["gate"]) * st["up"])
        y, st["u_down"] = _lin(st["m"], p["down"], alpha)
        st["down"] = rnd(y)
        h = rnd(st["h1"] + st["down"])
        saved.append(st)
    return h, saved


def stack_backward(dh_bits_or_f64, layers, dims, alpha, saved, round_storage=True):
    """Backward of ``stack_forward``: returns (dh0, grads) with grads[l][name] = (dA, dB).

    Gradient storage points (rounded when ``round_storage``): the upstream
    gradient into each linear's backward is what the forward stored; every dX
    output, d(gate), d(up), dm and each residual-stream gradient are bf16.
    dA and dB are fp32 on the GPU and are compared unrounded.
    """
    rnd = round_bf16 if round_storage else (lambda z: np.asarray(z, dtype=np.float64))
    dh = _as_f64(dh_bits_or_f64)
    grads = [None] * len(layers)
    for li in range(len(layers) - 1, -1, -1):
        p = _layer_f64(layers[li])
        st = saved[li]
        g = {}
        # h'' = h' + down(m)
        dm, g["down_dA"], g["down_dB"] = _lin_bwd(st["m"], p["down"], alpha, dh)
        dm = rnd(dm)
        sig_gate = silu(st["gate"])
        dgate = rnd(dm * st["up"] * silu_grad(st["gate"]))
        dup = rnd(dm * sig_gate)
        dhm_g, g["gate_dA"], g["gate_dB"] = _lin_bwd(st["hm"], p["gate"], alpha, dgate)
        dhm_u, g["up_dA"], g["up_dB"] = _lin_bwd(st["hm"], p["up"], alpha, dup)
        dhm = rnd(rnd(dhm_g) + rnd(dhm_u))
        dh1 = rnd(dh + rmsnorm_bwd(st["h1"], dhm))
        # h' = h + o(repeat_kv(v))
        da, g["o_dA"], g["o_dB"] = _lin_bwd(st["a"], p["o"], alpha, dh1)
        da = rnd(da)
        dv = rnd(_repeat_kv_bwd(da, dims))
        dha, g["v_dA"], g["v_dB"] = _lin_bwd(st["ha"], p["v"], alpha, dv)
        dha = rnd(dha)
        for name in ("q", "k"):                                 # zero upstream gradient (R9)
            zero = np.zeros_like(st[name])
            dq, g[name + "_dA"], g[name + "_dB"] = _lin_bwd(st["ha"], p[name], alpha, zero)
            dha = dha + rnd(dq)
        dh = rnd(dh1 + rmsnorm_bwd(st["h"], dha))
        grads[li] = g
    return dh, grads
