"""Blockwise weight-streamed stack of NF4-LoRA decoder layers on one GPU.

The frozen NF4 base lives in one pinned host buffer, layer after layer; a block
of `block_size` layers is the contiguous slab of its layers ("Poros on consumer
GPUs", "What you need besides VRAM": the streamed base is pinned host memory;
Poros API reference, "patch_hf_model" Behavior 4-6: layers regrouped into blocks
of block_size, default 4, under a block manager). In streamed mode the slabs pass
through a pool of device slots:
block b is acquired on the compute stream while block b+1 is prefetched on a
dedicated copy stream (HN comment thread on streaming the frozen base, main
comment: prefetched one ahead on a dedicated stream). In resident mode every
block has its own slot and is copied once up front. Both modes run the same
kernels on the same bytes at the same offsets, so their results are bitwise
equal ("Poros on consumer GPUs", "OOM playbook": block_size never affects parity).

HostBF16Base holds a dense bf16 base instead (the experimental "bf16_bitwise"
mode of the Poros API reference, "PorosTrainer.from_pretrained"); the stack then
calls the dense entry points, with the same pool, modes and parity.

With remat=True only the block-boundary hidden states are kept through the
forward pass; the backward visit of block b (its base is resident for that visit
anyway) first recomputes the block's forward from its boundary into one block's
worth of activation buffers ("Poros on consumer GPUs", "OOM playbook": the
activation memory held is that at the rematerialisation boundary). Every
kernel is deterministic, so the recomputed activations - and every gradient - are
bitwise those of the stored-activation run.

Every computation is a call into libnf4lora.so; this module only orders the
calls, owns buffers (torch allocations) and the two streams.

Layer (attention mixing replaced by the identity): h_a = RMSNorm(h);
q, k, v = L_q/L_k/L_v(h_a); a = repeat_kv(v); h' = h + L_o(a); h_m = RMSNorm(h');
h'' = h' + L_down(SiLU(L_gate(h_m)) * L_up(h_m)). q and k are computed and
receive a zero gradient.
"""

from __future__ import annotations

import contextlib
import time
from dataclasses import dataclass

import torch

from . import lib

PROJS = ("q", "k", "v", "o", "gate", "up", "down")
RMS_EPS = 1e-6


@dataclass(frozen=True)
class StackDims:
    hidden: int
    q: int
    kv: int
    inter: int
    head_dim: int = 128

    def shapes(self) -> dict:
        """(N, K) of each projection."""
        h, q, kv, i = self.hidden, self.q, self.kv, self.inter
        return {"q": (q, h), "k": (kv, h), "v": (kv, h), "o": (h, q), "gate": (i, h), "up": (i, h), "down": (h, i)}

    def layer_nf4_bytes(self) -> int:
        return sum(n * k // 2 + n * (k // 64) * 4 for n, k in self.shapes().values())


QWEN25 = {
    "7b": (StackDims(3584, 3584, 512, 18944), 28),
    "32b": (StackDims(5120, 5120, 1024, 27648), 64),
    "72b": (StackDims(8192, 8192, 1024, 29568), 80),
}


def block_layout(dims: StackDims, layers: int, dense: bool = False):
    """Offsets of every (layer-in-block, projection) piece of a block slab and the slab
    size, from the library's nf4_block_layout: per layer, projections in the order q, k,
    v, o, gate, up, down, each codes then absmax (dense: the bf16 weight), every piece at
    a 256-byte aligned offset. Returns ([{proj: (codes_off, absmax_off)} or
    [{proj: (w_off,)}] per layer], block bytes)."""
    shapes = [dims.shapes()[name] for name in PROJS]
    offs, total = lib.block_layout(shapes, layers, dense)
    table = []
    for li in range(layers):
        if dense:
            table.append({name: (offs[li][j][0],) for j, name in enumerate(PROJS)})
        else:
            table.append({name: tuple(offs[li][j]) for j, name in enumerate(PROJS)})
    return table, total


def block_layout_bf16(dims: StackDims, layers: int):
    """Dense-bf16 slabs: [{proj: (w_off,)}] and the slab size, pieces 256-byte aligned."""
    return block_layout(dims, layers, dense=True)


class _HostBase:
    """The frozen base of a stack in pinned host memory: one page-locked buffer of
    exactly the stack's size, layer after layer with the block layout of a one-layer
    block (every layer's bytes are a multiple of 256), or, if so large an allocation is
    refused, one buffer per layer. A block of block_size layers is its layers' slabs
    back to back - with one buffer, a contiguous host range copied in one piece - and
    the slot then holds exactly the slab that nf4_block_layout describes for that many
    layers; regroup(block_size) re-groups the same host bytes for another block size.

    Loading ("Poros on consumer GPUs", "OOM playbook": the streamed loader keeps GPU
    residency bounded at any model size and gives bytes identical to the standard
    load): weight_fn(layer, proj, n, k) returns the projection's bf16 weight [n, k],
    either host-resident (a CPU tensor: copied to the device) or already on the device.
    Each projection is converted on the device on its own (`_convert`) and copied into
    its place in the layer's pinned buffer before the next one is read, so the device
    holds at most one projection's bf16 weight plus its converted bytes; load_stats
    records the peak and the throughput. The pinned buffers live as long as a view of
    them does (this base, a regrouped view, a pool); close() drops this base's views."""

    dense = False

    def __init__(self, dims: StackDims, n_layers: int, block_size: int, weight_fn=None, _shared=None):
        if block_size < 1:
            raise ValueError("block_size must be >= 1")
        self.dims, self.n_layers, self.block_size = dims, n_layers, block_size
        self.layer_layout, self.layer_bytes = block_layout(dims, 1, self.dense)
        self.layout, self.slot_bytes = block_layout(dims, block_size, self.dense)
        for li in range(block_size):   # a block's layout is its layers' layouts, back to back
            for name, offs in self.layout[li].items():
                assert offs == tuple(o + li * self.layer_bytes for o in self.layer_layout[0][name])
        self.n_blocks = (n_layers + block_size - 1) // block_size
        self._shared = _shared if _shared is not None else self._load(weight_fn)
        self.load_stats = self._shared["stats"]
        self.layers = list(self._shared["bufs"])
        self.contiguous = self._shared["whole"] is not None
        self.part_begin = [b * block_size for b in range(self.n_blocks)] + [n_layers]
        self.block_bytes = [(self.part_begin[b + 1] - self.part_begin[b]) * self.layer_bytes
                            for b in range(self.n_blocks)]

    def pool_ranges(self, layer_parts: bool):
        """Host ranges and part_begin for stream_pool_create_parts: one part per layer,
        or (contiguous base only) one part per block."""
        if layer_parts or not self.contiguous:
            return self.layers, self.part_begin
        whole, lb = self._shared["whole"], self.layer_bytes
        ranges = [whole[self.part_begin[b] * lb:self.part_begin[b + 1] * lb] for b in range(self.n_blocks)]
        return ranges, list(range(self.n_blocks + 1))

    def regroup(self, block_size: int):
        """The same host bytes grouped in blocks of `block_size` layers."""
        return type(self)(self.dims, self.n_layers, block_size, _shared=self._shared)

    def total_bytes(self) -> int:
        return self.n_layers * self.layer_bytes

    def layer_bytes_of(self, layer: int) -> torch.Tensor:
        """The pinned bytes of one layer (its one-layer slab)."""
        return self.layers[layer]

    def close(self) -> None:
        """Drop this base's references to the pinned buffers (they are freed when no
        regrouped view or pool holds them any more)."""
        self.layers = []
        self._shared = {"bufs": [], "whole": None, "stats": self.load_stats}

    def _load(self, weight_fn):
        shapes = self.dims.shapes()
        max_w = max(n * k for n, k in shapes.values())
        try:
            whole = lib.pinned_empty(self.n_layers * self.layer_bytes)
            bufs = [whole[l * self.layer_bytes:(l + 1) * self.layer_bytes] for l in range(self.n_layers)]
        except lib.Nf4Error:
            whole = None
            bufs = [lib.pinned_empty(self.layer_bytes) for _ in range(self.n_layers)]
        base_alloc = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        staging_w = None          # device bf16 staging for host-resident weights
        staging = torch.empty(self._converted_bytes(max_w), dtype=torch.uint8, device="cuda")
        t0 = time.perf_counter()
        read = 0
        for layer in range(self.n_layers):
            dst = bufs[layer]
            for name in PROJS:
                n, k = shapes[name]
                w = weight_fn(layer, name, n, k)
                if w.dtype != torch.bfloat16 or tuple(w.shape) != (n, k):
                    raise ValueError(f"weight_fn({layer}, {name}) must give a bf16 [{n}, {k}] tensor")
                if w.device.type == "cpu":
                    if staging_w is None:
                        staging_w = torch.empty(max_w, dtype=torch.bfloat16, device="cuda")
                    wd = staging_w[:n * k].view(n, k)
                    wd.copy_(w)                          # H2D of one projection
                else:
                    wd = w
                read += n * k * 2
                self._convert(wd, name, self.layer_layout[0][name], dst, staging)
                del w, wd
        torch.cuda.synchronize()
        secs = time.perf_counter() - t0
        stats = {"seconds": secs, "bf16_gb_read": read / 1e9, "host_gb_written": self.total_bytes() / 1e9,
                 "bf16_gbs": read / secs / 1e9,
                 "peak_device_bytes": torch.cuda.max_memory_allocated() - base_alloc}
        stats["one_pinned_buffer"] = whole is not None
        del staging, staging_w
        return {"bufs": bufs, "whole": whole, "stats": stats}


class HostNF4Base(_HostBase):
    """The frozen NF4 base in pinned host memory: each projection quantised by
    nf4_quantize on the GPU and its codes and absmax copied into the pinned buffer."""

    dense = False

    @staticmethod
    def _converted_bytes(max_w: int) -> int:
        return _align(max_w // 2) + _align(max_w // 64 * 4)

    def _convert(self, wd, name, offs, dst, staging):
        n, k = wd.shape
        c_off, a_off = offs
        codes = staging[:n * k // 2].view(n, k // 2)
        a0 = _align(n * k // 2)
        absmax = staging[a0:a0 + n * (k // 64) * 4].view(torch.float32).view(n, k // 64)
        lib.quantize(wd, codes=codes, absmax=absmax)
        dst[c_off:c_off + n * k // 2].copy_(staging[:n * k // 2])      # D2H (synchronous)
        dst[a_off:a_off + n * (k // 64) * 4].copy_(staging[a0:a0 + n * (k // 64) * 4])


class HostBF16Base(_HostBase):
    """The frozen base as dense bf16 in pinned host memory (the experimental
    "bf16_bitwise" mode of the Poros API reference, "PorosTrainer.from_pretrained": a
    dense-BF16 base streamed blockwise, bitwise equal to a resident run; 2 bytes a
    weight against NF4's 0.5625)."""

    dense = True

    @staticmethod
    def _converted_bytes(max_w: int) -> int:
        return 256

    def _convert(self, wd, name, offs, dst, staging):
        n, k = wd.shape
        (w_off,) = offs
        dst[w_off:w_off + n * k * 2].copy_(wd.contiguous().view(torch.uint8).view(-1))   # D2H (synchronous)


def _align(v: int, a: int = 256) -> int:
    return (v + a - 1) // a * a


class LoraParams:
    """A [r, K] and B [N, r] (bf16, device) for every layer and projection, from
    lora_fn(layer, proj, n, k) -> (A, B)."""

    def __init__(self, dims: StackDims, n_layers: int, rank: int, lora_fn):
        self.rank = rank
        self.p = [{name: lora_fn(layer, name, *dims.shapes()[name]) for name in PROJS} for layer in range(n_layers)]


class NF4Stack:
    """Forward + backward over the stack, streamed through a slot pool or resident."""

    def __init__(self, base: HostNF4Base, lora: LoraParams, tokens: int, alpha: float = 32.0,
                 mode: str = "streamed", n_slots: int = 2, prefetch: bool = True, remat: bool = False,
                 layer_parts: bool = True, max_ahead: int = 2):
        if mode not in ("streamed", "resident"):
            raise ValueError("mode must be 'streamed' or 'resident'")
        self.base, self.lora, self.T, self.alpha = base, lora, tokens, alpha
        self.mode, self.prefetch, self.remat = mode, prefetch, remat
        # layer_parts: each layer of a block is a part of its own (copied separately,
        # released as soon as the layer is done, so a copy into the slot can start
        # before the whole block is done); else a block is one part when the base is
        # one contiguous host buffer (one copy per block)
        self.layer_parts = layer_parts or not base.contiguous
        d = base.dims
        self.dims = d
        nb = base.n_blocks
        self.n_slots = nb if mode == "resident" else max(1, n_slots)
        self.slab = torch.empty(self.n_slots * base.slot_bytes, dtype=torch.uint8, device="cuda")
        # the library's compute/copy stream pair: on different hardware queues, so the
        # pool's waits between them never serialise copies behind kernels
        self.compute_stream, self.copy_stream = lib.pool_streams()
        ranges, part_begin = base.pool_ranges(self.layer_parts)
        self.pool = lib.StreamPool(ranges, self.slab, base.slot_bytes, self.n_slots, self.copy_stream,
                                   part_begin=part_begin)
        self._views = [self._slot_views(s) for s in range(self.n_slots)]
        # streamed with one part per layer: acquire without the block wait and wait for
        # each layer's part before its first use, so a block's first layers run while
        # its later layers land (what is left to overlap at the end of a pass)
        self.part_waits = mode == "streamed" and self.layer_parts
        self._waited = set()
        # bound the host's lead over the device (a host a whole step ahead was measured
        # to slow the copies down)
        self.max_ahead = max_ahead if mode == "streamed" else 0
        self.pool.set_max_ahead(self.max_ahead)
        T, r = tokens, lora.rank
        shapes = d.shapes()
        dev = "cuda"
        bf = dict(dtype=torch.bfloat16, device=dev)
        fws = lib.fwd_bf16_workspace_bytes if base.dense else lib.fwd_workspace_bytes
        bws = lib.bwd_bf16_workspace_bytes if base.dense else lib.bwd_workspace_bytes
        self.ws_f = lib.workspace(max(fws(T, n, k, r) for n, k in shapes.values()))
        self.ws_b = lib.workspace(max(bws(T, n, k, r) for n, k in shapes.values()))
        L = base.n_layers
        # activation sets: one per layer, or (remat) one per layer of a block, plus the
        # block-boundary hidden states
        n_sets = base.block_size if remat else L
        self.acts = []
        for _ in range(n_sets + 1):
            self.acts.append({"h": torch.empty(T, d.hidden, **bf)})
        self.boundary = [torch.empty(T, d.hidden, **bf) for _ in range(base.n_blocks + 1)] if remat else None
        for li in range(n_sets):
            a = self.acts[li]
            a.update({
                "ha": torch.empty(T, d.hidden, **bf), "v": torch.empty(T, d.kv, **bf), "a": torch.empty(T, d.q, **bf),
                "h1": torch.empty(T, d.hidden, **bf), "hm": torch.empty(T, d.hidden, **bf),
                "gate": torch.empty(T, d.inter, **bf), "up": torch.empty(T, d.inter, **bf),
                "m": torch.empty(T, d.inter, **bf),
                "rs_h": torch.empty(T, dtype=torch.float32, device=dev),
                "rs_h1": torch.empty(T, dtype=torch.float32, device=dev),
                "u": {name: torch.empty(T, r, dtype=torch.float32, device=dev) for name in PROJS},
            })
        # scratch reused by every layer (stream order makes reuse safe)
        self.tmp = {
            "q": torch.empty(T, d.q, **bf), "k": torch.empty(T, d.kv, **bf), "o": torch.empty(T, d.hidden, **bf),
            "down": torch.empty(T, d.hidden, **bf),
            "dm": torch.empty(T, d.inter, **bf), "dgate": torch.empty(T, d.inter, **bf),
            "dup": torch.empty(T, d.inter, **bf), "dhm_g": torch.empty(T, d.hidden, **bf),
            "dhm_u": torch.empty(T, d.hidden, **bf), "dhm": torch.empty(T, d.hidden, **bf),
            "dh1": torch.empty(T, d.hidden, **bf), "da": torch.empty(T, d.q, **bf), "dv": torch.empty(T, d.kv, **bf),
            "dha_v": torch.empty(T, d.hidden, **bf), "dha_q": torch.empty(T, d.hidden, **bf),
            "dha_k": torch.empty(T, d.hidden, **bf), "dha": torch.empty(T, d.hidden, **bf),
            "zq": torch.zeros(T, d.q, **bf), "zkv": torch.zeros(T, d.kv, **bf),
        }
        self.dh = [torch.empty(T, d.hidden, **bf) for _ in range(2)]
        self.grads = [{name: (torch.empty(r, shapes[name][1], dtype=torch.float32, device=dev),
                              torch.empty(shapes[name][0], r, dtype=torch.float32, device=dev)) for name in PROJS}
                      for _ in range(L)]
        if mode == "resident":
            for b in range(nb):
                self.pool.prefetch(b)
            self.copy_stream.synchronize()

    # ------------------------------------------------------------------ slot views
    def _slot_views(self, slot: int):
        sb = self.base.slot_bytes
        out = []
        for entry in self.base.layout:
            v = {}
            for name, offs in entry.items():
                n, k = self.dims.shapes()[name]
                if self.base.dense:
                    (w_off,) = offs
                    v[name] = (self.slab[slot * sb + w_off: slot * sb + w_off + n * k * 2].view(torch.bfloat16).view(n, k),)
                    continue
                c_off, a_off = offs
                c = self.slab[slot * sb + c_off: slot * sb + c_off + n * k // 2].view(n, k // 2)
                a = self.slab[slot * sb + a_off: slot * sb + a_off + n * (k // 64) * 4].view(torch.float32).view(n, k // 64)
                v[name] = (c, a)
            out.append(v)
        return out

    def _acquire(self, b: int):
        if self.part_waits:
            ptr = self.pool.acquire_deferred(b)
            self._waited.clear()
        else:
            ptr = self.pool.acquire(b)
        slot = (ptr - self.slab.data_ptr()) // self.base.slot_bytes
        return self._views[slot]

    def _ready(self, b: int, li: int) -> None:
        """Order the compute stream after the copy of layer li's part (deferred acquires)."""
        if self.part_waits and li not in self._waited:
            self.pool.wait_part(b, li - b * self.base.block_size)
            self._waited.add(li)

    # ------------------------------------------------------------------ activation sets
    def _act(self, li: int) -> dict:
        """Activations of layer li (its input "h" and everything the backward reads)."""
        return self.acts[li % self.base.block_size] if self.remat else self.acts[li]

    def _h_out(self, li: int) -> torch.Tensor:
        """Where layer li writes its output hidden state."""
        if not self.remat:
            return self.acts[li + 1]["h"]
        bs = self.base.block_size
        if (li + 1) % bs == 0 or li + 1 == self.base.n_layers:
            return self.boundary[li // bs + 1]
        return self.acts[(li + 1) % bs]["h"]

    def activation_bytes(self) -> int:
        """Device bytes held for activations between the forward and the backward pass."""
        n = sum(t.numel() * t.element_size() for a in self.acts for t in a.values() if isinstance(t, torch.Tensor))
        n += sum(t.numel() * t.element_size() for a in self.acts if "u" in a for t in a["u"].values())
        if self.boundary is not None:
            n += sum(t.numel() * t.element_size() for t in self.boundary)
        return n

    # ------------------------------------------------------------------ one layer
    def _fwd(self, w, name, x, y, u):
        p = self.lora.p[self._layer][name]
        if self.base.dense:
            lib.lora_linear_fwd_bf16(w[name][0], x, p[0], p[1], self.alpha, y=y, u=u, ws=self.ws_f)
            return
        c, a = w[name]
        lib.lora_linear_fwd(c, a, x, p[0], p[1], self.alpha, y=y, u=u, ws=self.ws_f)

    def _bwd(self, w, name, x, u, dy, dx):
        p = self.lora.p[self._layer][name]
        dA, dB = self.grads[self._layer][name]
        if self.base.dense:
            lib.lora_linear_bwd_bf16(w[name][0], x, u, dy, p[0], p[1], self.alpha, dx=dx, dA=dA, dB=dB, ws=self.ws_b,
                                     need_dx=dx is not None)
            return
        c, a = w[name]
        lib.lora_linear_bwd(c, a, x, u, dy, p[0], p[1], self.alpha, dx=dx, dA=dA, dB=dB, ws=self.ws_b,
                            need_dx=dx is not None)

    def _layer_forward(self, li: int, w):
        d, A, t = self.dims, self._act(li), self.tmp
        self._layer = li
        lib.rmsnorm_fwd(A["h"], RMS_EPS, out=A["ha"], rstd=A["rs_h"])
        self._fwd(w, "q", A["ha"], t["q"], A["u"]["q"])
        self._fwd(w, "k", A["ha"], t["k"], A["u"]["k"])
        self._fwd(w, "v", A["ha"], A["v"], A["u"]["v"])
        lib.repeat_kv_fwd(A["v"], d.q, d.head_dim, out=A["a"])
        self._fwd(w, "o", A["a"], t["o"], A["u"]["o"])
        lib.add_bf16(A["h"], t["o"], out=A["h1"])
        lib.rmsnorm_fwd(A["h1"], RMS_EPS, out=A["hm"], rstd=A["rs_h1"])
        self._fwd(w, "gate", A["hm"], A["gate"], A["u"]["gate"])
        self._fwd(w, "up", A["hm"], A["up"], A["u"]["up"])
        lib.silu_mul_fwd(A["gate"], A["up"], out=A["m"])
        self._fwd(w, "down", A["m"], t["down"], A["u"]["down"])
        lib.add_bf16(A["h1"], t["down"], out=self._h_out(li))

    def _layer_backward(self, li: int, w, dh_out, dh_in):
        d, A, t = self.dims, self._act(li), self.tmp
        self._layer = li
        self._bwd(w, "down", A["m"], A["u"]["down"], dh_out, t["dm"])
        lib.silu_mul_bwd(A["gate"], A["up"], t["dm"], dgate=t["dgate"], dup=t["dup"])
        self._bwd(w, "gate", A["hm"], A["u"]["gate"], t["dgate"], t["dhm_g"])
        self._bwd(w, "up", A["hm"], A["u"]["up"], t["dup"], t["dhm_u"])
        lib.add_bf16(t["dhm_g"], t["dhm_u"], out=t["dhm"])
        lib.rmsnorm_bwd(A["h1"], A["rs_h1"], t["dhm"], dres=dh_out, out=t["dh1"])
        self._bwd(w, "o", A["a"], A["u"]["o"], t["dh1"], t["da"])
        lib.repeat_kv_bwd(t["da"], d.kv, d.head_dim, out=t["dv"])
        self._bwd(w, "v", A["ha"], A["u"]["v"], t["dv"], t["dha_v"])
        self._bwd(w, "q", A["ha"], A["u"]["q"], t["zq"], t["dha_q"])      # identity mixing: zero gradient
        self._bwd(w, "k", A["ha"], A["u"]["k"], t["zkv"], t["dha_k"])
        lib.add_bf16(t["dha_v"], t["dha_q"], t["dha_k"], out=t["dha"])
        lib.rmsnorm_bwd(A["h"], A["rs_h"], t["dha"], dres=t["dh1"], out=dh_in)

    # ------------------------------------------------------------------ stack passes
    def _layers_of(self, b: int):
        bs = self.base.block_size
        return range(b * bs, min((b + 1) * bs, self.base.n_layers))

    def _block_forward(self, b: int, w):
        if self.remat:
            self.acts[0]["h"].copy_(self.boundary[b])
        for li in self._layers_of(b):
            self._ready(b, li)
            self._layer_forward(li, w[li - b * self.base.block_size])

    @contextlib.contextmanager
    def _on_compute(self):
        """Run the enclosed work on the stack's compute stream, ordered after the
        caller's stream's earlier work and before its later work."""
        caller = torch.cuda.current_stream()
        if caller == self.compute_stream:
            yield
            return
        self.compute_stream.wait_stream(caller)
        with torch.cuda.stream(self.compute_stream):
            yield
        caller.wait_stream(self.compute_stream)

    def forward(self, h0: torch.Tensor) -> torch.Tensor:
        with self._on_compute():
            return self._forward(h0)

    def backward(self, dh: torch.Tensor) -> torch.Tensor:
        with self._on_compute():
            return self._backward(dh)

    def _forward(self, h0: torch.Tensor) -> torch.Tensor:
        (self.boundary[0] if self.remat else self.acts[0]["h"]).copy_(h0)
        nb, bs = self.base.n_blocks, self.base.block_size
        self.pool.set_order(False)            # layers of a block used first to last
        for b in range(nb):
            w = self._acquire(b)
            if self.prefetch and self.n_slots > 1 and b + 1 < nb:
                self.pool.prefetch(b + 1)
            if self.remat:
                self.acts[0]["h"].copy_(self.boundary[b])
            for li in self._layers_of(b):
                self._ready(b, li)
                self._layer_forward(li, w[li - b * bs])
                if self.layer_parts:
                    self.pool.release_part(b, li - b * bs)   # the layer's bytes may be overwritten after this
            self.pool.release(b)
        return self.boundary[nb] if self.remat else self.acts[-1]["h"]

    def _backward(self, dh: torch.Tensor) -> torch.Tensor:
        nb = self.base.n_blocks
        cur = self.dh[0]
        cur.copy_(dh)
        k = 1
        self.pool.set_order(True)             # layers of a block used last to first
        for b in range(nb - 1, -1, -1):
            w = self._acquire(b)
            if self.prefetch and self.n_slots > 1 and b - 1 >= 0:
                self.pool.prefetch(b - 1)
            if self.remat:
                # recompute the block's activations from its boundary (the block's last
                # layer rewrites boundary[b + 1] with the same bits)
                self._block_forward(b, w)
            for li in reversed(self._layers_of(b)):
                nxt = self.dh[k]
                self._ready(b, li)
                self._layer_backward(li, w[li - b * self.base.block_size], cur, nxt)
                if self.layer_parts:
                    self.pool.release_part(b, li - b * self.base.block_size)
                cur, k = nxt, 1 - k
            self.pool.release(b)
        return cur

    def step(self, h0, dh):
        out = self.forward(h0)
        dh0 = self.backward(dh)
        return out, dh0

    def close(self):
        self.compute_stream.synchronize()   # the stack's buffers may be reused once freed
        self.pool.close()


def qwen_weight_fn(seed: int = 42):
    """Synthetic base weights drawn on the GPU: W ~ N(0, 0.02), bf16."""
    def fn(layer, name, n, k):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed * 1000003 + layer * 16 + PROJS.index(name))
        return (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    return fn


def qwen_lora_fn(rank: int = 16, seed: int = 42, b_std: float = 0.01):
    """A ~ U(+-1/sqrt(K)), B ~ N(0, b_std), bf16 on the GPU."""
    def fn(layer, name, n, k):
        g = torch.Generator(device="cuda")
        g.manual_seed(seed * 7919 + layer * 16 + PROJS.index(name) + 1)
        a = ((torch.rand(rank, k, generator=g, device="cuda") * 2 - 1) / k ** 0.5).to(torch.bfloat16)
        b = (torch.randn(n, rank, generator=g, device="cuda") * b_std).to(torch.bfloat16)
        return a, b
    return fn


def timed_steps(stack: NF4Stack, h0, dh, steps: int, warmup: int = 1) -> float:
    """Seconds per step (forward + backward over the whole stack)."""
    for _ in range(warmup):
        stack.step(h0, dh)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        stack.step(h0, dh)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps
