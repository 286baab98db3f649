"""Throughput of the NF4-LoRA linear hot path on one MI355X.

A step is one forward + backward pass of every projection of one Qwen2.5-7B-
shaped layer (q 3584x3584, k/v 512x3584, o 3584x3584, gate/up 18944x3584,
down 3584x18944; N x K), 512 tokens, LoRA rank 16, alpha 32, fully resident:
per projection the fused u = x.A^T + dequant-GEMM + LoRA forward, and the
backward g/dB pre-pass + dequant-GEMM dX + dA. x is shared by q/k/v and by
gate/up as in a real layer; dY is independent per projection. Inputs are
seeded synthetic data; the NF4 base is quantised by the library before timing.

Prints ONE JSON line (metric, value in tokens/s, TFLOP/s, the roofline of the
dominant kernel measured with HIP events on its own stream, and the fp64 CPU
oracle timed on a bounded sample of the same workload).
"""

from __future__ import annotations

import argparse
import ctypes as C
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

T_TOKENS = 512
RANK = 16
ALPHA = 32.0
HIDDEN, QW, KVW, INTER = 3584, 3584, 512, 18944
PROJ = [("q", QW, HIDDEN, "x1"), ("k", KVW, HIDDEN, "x1"), ("v", KVW, HIDDEN, "x1"), ("o", HIDDEN, QW, "x2"),
        ("gate", INTER, HIDDEN, "x3"), ("up", INTER, HIDDEN, "x3"), ("down", HIDDEN, INTER, "x4")]
MFMA_BF16_PEAK_TFLOPS = 2500.0
HBM_PEAK_GBS = 8000.0
METRIC = "NF4-LoRA linear fwd+bwd tokens/s & TFLOP/s; % of MFMA/HBM/PCIe roofline"


def step_flops(t: int, r: int) -> float:
    """Algorithmic FLOPs of one step: per projection 4TNK (base fwd + dX) + 6Tr(N+K) (LoRA)."""
    return float(sum(4 * t * n * k + 6 * t * r * (n + k) for _, n, k, _ in PROJ))


class HipEvents:
    """hipEvent_t pairs through the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]
        self.hip.hipEventRecord.argtypes = [C.c_void_p, C.c_void_p]

    def create(self) -> int:
        e = C.c_void_p()
        assert self.hip.hipEventCreate(C.byref(e)) == 0
        return e.value

    def elapsed_ms(self, a: int, b: int) -> float:
        assert self.hip.hipEventSynchronize(C.c_void_p(b)) == 0
        ms = C.c_float()
        assert self.hip.hipEventElapsedTime(C.byref(ms), C.c_void_p(a), C.c_void_p(b)) == 0
        return float(ms.value)

    def record(self, e: int, stream: int) -> None:
        assert self.hip.hipEventRecord(C.c_void_p(e), C.c_void_p(stream)) == 0

    def destroy(self, e: int) -> None:
        self.hip.hipEventDestroy(C.c_void_p(e))


def build_layer(lib, torch, seed: int = 42):
    """Synthetic layer on the GPU: W ~ N(0, 0.02) bf16 -> NF4; x, dY ~ N(0, 1); A ~ U(+-1/sqrt(K)); B ~ N(0, 0.01)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev = "cuda"
    acts = {
        "x1": torch.randn(T_TOKENS, HIDDEN, generator=g, device=dev).to(torch.bfloat16),
        "x2": torch.randn(T_TOKENS, QW, generator=g, device=dev).to(torch.bfloat16),
        "x3": torch.randn(T_TOKENS, HIDDEN, generator=g, device=dev).to(torch.bfloat16),
        "x4": torch.randn(T_TOKENS, INTER, generator=g, device=dev).to(torch.bfloat16),
    }
    layer = {}
    for name, n, k, xin in PROJ:
        w = (torch.randn(n, k, generator=g, device=dev) * 0.02).to(torch.bfloat16)
        codes, absmax = lib.quantize(w)
        del w
        a = ((torch.rand(RANK, k, generator=g, device=dev) * 2 - 1) / k ** 0.5).to(torch.bfloat16)
        b = (torch.randn(n, RANK, generator=g, device=dev) * 0.01).to(torch.bfloat16)
        p = {
            "n": n, "k": k, "codes": codes, "absmax": absmax, "A": a, "B": b, "x": acts[xin],
            "dy": torch.randn(T_TOKENS, n, generator=g, device=dev).to(torch.bfloat16),
            "y": torch.empty(T_TOKENS, n, dtype=torch.bfloat16, device=dev),
            "u": torch.empty(T_TOKENS, RANK, dtype=torch.float32, device=dev),
            "dx": torch.empty(T_TOKENS, k, dtype=torch.bfloat16, device=dev),
            "dA": torch.empty(RANK, k, dtype=torch.float32, device=dev),
            "dB": torch.empty(n, RANK, dtype=torch.float32, device=dev),
            "wsf": lib.workspace(lib.fwd_workspace_bytes(T_TOKENS, n, k, RANK)),
            "wsb": lib.workspace(lib.bwd_workspace_bytes(T_TOKENS, n, k, RANK)),
        }
        layer[name] = p
    torch.cuda.synchronize()
    return layer


def run_step(lib, layer, prof=None):
    """Forward of all 7 projections, then backward in reverse order. `prof` =
    (name, start, stop) records events around that projection's forward GEMM."""
    for name, *_ in PROJ:
        p = layer[name]
        if prof is not None and prof[0] == name:
            lib.profile_next_gemm(prof[1], prof[2])
        lib.lora_linear_fwd(p["codes"], p["absmax"], p["x"], p["A"], p["B"], ALPHA, y=p["y"], u=p["u"], ws=p["wsf"])
    for name, *_ in reversed(PROJ):
        p = layer[name]
        lib.lora_linear_bwd(p["codes"], p["absmax"], p["x"], p["u"], p["dy"], p["A"], p["B"], ALPHA, dx=p["dx"],
                            dA=p["dA"], dB=p["dB"], ws=p["wsb"])


TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "k_nf4_gemm_fwd_gate_qwen7b_t512_traffic.md")
# sources whose change invalidates the HBM traffic taken with the counters
TRAFFIC_SOURCES = [os.path.join(ROOT, "nf4_weight_streamed_amd", "csrc", f)
                   for f in ("nf4_gemm_fwd.hip", "device.h", "common.h")]
COPY_CALIBRATION_BYTES = 1 << 30


def kernel_source_digest() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic() -> int | None:
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, each scaled by the copy calibration), or None when that
    summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC_PROFILE) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, val = line[2:].split(": ", 1)
            fields[key.strip("` ")] = val.strip("` ")
    if fields.get("source_sha256") != kernel_source_digest():
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch) -> None:
    """One plain streaming kernel of known traffic for the counter calibration: an
    elementwise negation of a 1 GiB fp32 tensor (reads 1 GiB, writes 1 GiB)."""
    src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def cpu_baseline(seconds_budget: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on a bounded sample of the same workload:
    the q projection (3584 x 3584) of the layer with all 512 tokens - dequantise
    + forward + backward - repeated for about `seconds_budget` seconds, scaled
    to the whole layer by the algorithmic-FLOP ratio. Quantisation (load time)
    is outside the timed region, as on the GPU."""
    import numpy as np

    import oracle as O
    import synthetic_inputs as S

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl is optional
        threads = 1
    n, k = QW, HIDDEN
    case = S.linear_case(T_TOKENS, n, k, r=RANK, proj="q")
    codes, absmax = O.quantize(S.bf16_bits_to_f32(case["W"]))
    reps = 0
    t0 = time.perf_counter()
    while reps < 3 or time.perf_counter() - t0 < seconds_budget:
        wq = O.dequantize(codes, absmax)
        O.lora_linear_fwd(case["x"], wq, case["A"], case["B"], ALPHA)
        O.lora_linear_bwd(case["x"], wq, case["A"], case["B"], ALPHA, case["dY"])
        reps += 1
    dt = (time.perf_counter() - t0) / reps
    sample_flops = 4 * T_TOKENS * n * k + 6 * T_TOKENS * RANK * (n + k)
    layer_seconds = dt * step_flops(T_TOKENS, RANK) / sample_flops
    return {
        "value": round(T_TOKENS / layer_seconds, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"q projection 3584x3584, 512 tokens, r16: dequantise + fwd + bwd in fp64 numpy, "
                   f"{dt:.2f} s per pass (mean of {reps}); "
                   f"scaled to the 7-projection layer by algorithmic FLOPs ({step_flops(T_TOKENS, RANK) / sample_flops:.2f}x)"),
        "gflops": round(sample_flops / dt / 1e9, 3),
    }


def quantize_measure(lib, torch, ev: "HipEvents", cpu: bool) -> dict:
    """Load-time quantisation (not part of the step): the library's nf4_quantize on the
    gate weight (18944 x 3584 bf16, N(0, 0.02)) in device time, against HBM bytes
    2 + 0.5625 per parameter (bf16 read, codes + absmax written); with `cpu`, the
    oracle's quantise on a bounded sample of the same weight beside it."""
    n, k = INTER, HIDDEN
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    w = (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    codes = torch.empty(n, k // 2, dtype=torch.uint8, device="cuda")
    absmax = torch.empty(n, k // 64, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        lib.quantize(w, codes, absmax)
    reps = 10
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(e0, stream)
    for _ in range(reps):
        lib.quantize(w, codes, absmax)
    ev.record(e1, stream)
    us = ev.elapsed_ms(e0, e1) * 1e3 / reps
    ev.destroy(e0)
    ev.destroy(e1)
    nbytes = n * k * (2 + 0.5625)
    res = {"shape_NxK": [n, k], "gpu_us": round(us, 2), "gpu_params_per_s": round(n * k / us * 1e6, 1),
           "hbm_gbs": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    if cpu:
        import oracle as O

        rows = 1024  # a bounded sample: the first rows of the same weight
        ws = w[:rows].float().cpu().numpy()
        t0, cnt = time.perf_counter(), 0
        while cnt < 2 or time.perf_counter() - t0 < 3.0:
            O.quantize(ws)
            cnt += 1
        dt = (time.perf_counter() - t0) / cnt
        res["cpu_oracle_params_per_s"] = round(rows * k / dt, 1)
        res["cpu_sample"] = f"oracle quantise of {rows} x {k} rows of the same weight, {dt * 1e3:.1f} ms per pass"
    del w, codes, absmax
    torch.cuda.empty_cache()
    return res


def measured_mfma_tflops(lib, torch, ev: "HipEvents") -> float:
    """bf16 MFMA issue rate with the GEMMs' instruction (v_mfma_f32_32x32x16_bf16): 512
    workgroups x 4 waves, each 8 independent MFMAs per round on registers."""
    wg, iters = 512, 4000
    out = torch.empty(4 * wg, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    lib.probe_mfma(out, wg, 100)
    e0, e1 = ev.create(), ev.create()
    ev.record(e0, stream)
    lib.probe_mfma(out, wg, iters)
    ev.record(e1, stream)
    ms = ev.elapsed_ms(e0, e1)
    ev.destroy(e0)
    ev.destroy(e1)
    return wg * 4 * iters * 8 * 32768 / (ms * 1e-3) / 1e12  # 32x32x16 MACs x 2 per MFMA


def measured_copy_gbs(torch, ev: "HipEvents", nbytes: int = 1 << 30) -> float:
    """Device-to-device copy of 1 GiB (read + write counted): the measured HBM ceiling."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = ev.create(), ev.create()
    ev.record(e0, stream)
    for _ in range(5):
        dst.copy_(src)
    ev.record(e1, stream)
    ms = ev.elapsed_ms(e0, e1) / 5
    ev.destroy(e0)
    ev.destroy(e1)
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def measured_read_gbs(lib, torch, ev: "HipEvents", nbytes: int = 2 << 30) -> float:
    """Read-only reference: the library's read probe (coalesced 16-byte loads, grid-stride)
    over 2 GiB, best over a few grid sizes and launches: the rate a plain read-bound kernel
    reaches on this device."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    for wg in (1024, 2048, 4096):
        out = torch.empty(256 * wg, dtype=torch.int32, device="cuda")
        lib.probe_read(src, out, wg)
        for _ in range(3):
            e0, e1 = ev.create(), ev.create()
            ev.record(e0, stream)
            lib.probe_read(src, out, wg)
            ev.record(e1, stream)
            best = max(best, nbytes / (ev.elapsed_ms(e0, e1) * 1e-3) / 1e9)
            ev.destroy(e0)
            ev.destroy(e1)
        del out
    del src
    torch.cuda.empty_cache()
    return best


def pinned_h2d_gbs(torch, nbytes: int = 1 << 30) -> float:
    """Pinned host -> device hipMemcpyAsync bandwidth on a side stream (best of 3)."""
    h = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    d = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    best = 0.0
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(s):
            d.copy_(h, non_blocking=True)
        s.synchronize()
        best = max(best, nbytes / (time.perf_counter() - t0) / 1e9)
    del h, d
    return best


def stream_bench(torch, model: str, block_size: int, tokens: int, steps: int, h2d_gbs: float,
                 base_kind: str = "nf4", n_slots: int = 2) -> dict:
    """Streamed vs resident step time of a Qwen2.5-shaped identity-mixing stack, with
    the bitwise check, H2D traffic and copy/compute overlap. base_kind "bf16" streams a
    dense bf16 base (the experimental bf16_bitwise mode) instead of NF4. n_slots = device
    pool slots of one block each (the streamed runs; the resident run holds every block)."""
    from nf4_weight_streamed_amd import stack as ST

    dims, n_layers = ST.QWEN25[model]
    t0 = time.perf_counter()
    host_cls = ST.HostBF16Base if base_kind == "bf16" else ST.HostNF4Base
    base = host_cls(dims, n_layers, block_size, ST.qwen_weight_fn())
    lora = ST.LoraParams(dims, n_layers, RANK, ST.qwen_lora_fn())
    build_s = time.perf_counter() - t0
    print(f"[stream_bench] {model}: host base built in {build_s:.1f} s", file=sys.stderr, flush=True)
    g = torch.Generator(device="cuda")
    g.manual_seed(42)
    h0 = torch.randn(tokens, dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh = torch.randn(tokens, dims.hidden, generator=g, device="cuda").to(torch.bfloat16)
    out = {}
    # resident, streamed, and streamed with rematerialisation (block-boundary states kept,
    # each block's forward recomputed in its backward visit)
    for mode, remat, key in (("resident", False, "resident"), ("streamed", False, "streamed"),
                             ("streamed", True, "remat")):
        st = ST.NF4Stack(base, lora, tokens, ALPHA, mode=mode, remat=remat, n_slots=n_slots)
        y, dx = st.step(h0, dh)                       # warmup (and the parity sample)
        torch.cuda.synchronize()
        out[key + "_y"], out[key + "_dx"] = y.clone(), dx.clone()
        out[key + "_act"] = st.activation_bytes()
        c0 = st.pool.stats()["bytes_copied"]
        secs = ST.timed_steps(st, h0, dh, steps, warmup=0)
        out[key + "_s"] = secs
        out[key + "_bytes"] = (st.pool.stats()["bytes_copied"] - c0) / steps
        st.close()
        del st
        torch.cuda.empty_cache()
        print(f"[stream_bench] {model}: {key} {secs * 1e3:.1f} ms per step", file=sys.stderr, flush=True)
    flops = n_layers * sum(4 * tokens * n * k + 6 * tokens * RANK * (n + k) for n, k in dims.shapes().values())
    r_s, s_s, nbytes = out["resident_s"], out["streamed_s"], out["streamed_bytes"]
    copy_s = nbytes / (h2d_gbs * 1e9)
    overlap = (r_s + copy_s - s_s) / min(r_s, copy_s) if min(r_s, copy_s) > 0 else None
    return {
        "workload": f"qwen2.5-{model}-shaped stack, {n_layers} layers, block_size {block_size}, {n_slots} pool slots, "
                    f"{tokens} tokens, "
                    f"{'dense bf16' if base_kind == 'bf16' else 'NF4'} in pinned host, identity attention mixing, fwd+bwd",
        "bitwise_equal_to_resident": bool(torch.equal(out["resident_y"], out["streamed_y"])
                                          and torch.equal(out["resident_dx"], out["streamed_dx"])),
        "resident_ms_per_step": round(r_s * 1e3, 3),
        "streamed_ms_per_step": round(s_s * 1e3, 3),
        "streamed_over_resident": round(s_s / r_s, 3),
        "streamed_tokens_per_s": round(tokens / s_s, 2),
        "streamed_tflops": round(flops / s_s / 1e12, 2),
        "resident_tflops": round(flops / r_s / 1e12, 2),
        "h2d_gb_per_step": round(nbytes / 1e9, 3),
        "h2d_gbs_achieved_over_step": round(nbytes / s_s / 1e9, 2),
        "h2d_gbs_pinned_peak_measured": round(h2d_gbs, 2),
        "pcie_frac": round(nbytes / s_s / 1e9 / h2d_gbs, 4),
        "pcie_floor_ratio": round(max(r_s, copy_s) / r_s, 3),
        "copy_compute_overlap": None if overlap is None else round(overlap, 3),
        "host_base_gb": round(base.total_bytes() / 1e9, 3),
        "build_s": round(build_s, 1),
        "remat": {
            "bitwise_equal_to_resident": bool(torch.equal(out["resident_y"], out["remat_y"])
                                              and torch.equal(out["resident_dx"], out["remat_dx"])),
            "streamed_ms_per_step": round(out["remat_s"] * 1e3, 3),
            "over_streamed": round(out["remat_s"] / s_s, 3),
            "activation_gb": round(out["remat_act"] / 1e9, 3),
            "activation_gb_stored": round(out["streamed_act"] / 1e9, 3),
            "h2d_gb_per_step": round(out["remat_bytes"] / 1e9, 3),
        },
    }


SMALL_T = (1, 8, 16, 32, 64)
SMALL_T_SHAPES = [  # (model, projection, N, K)
    ("7b", "q", 3584, 3584), ("7b", "k", 512, 3584), ("7b", "gate", 18944, 3584), ("7b", "down", 3584, 18944),
    ("72b", "q", 8192, 8192), ("72b", "k", 1024, 8192), ("72b", "gate", 29568, 8192), ("72b", "down", 8192, 29568),
]


def small_t_sweep(lib, torch, ev: "HipEvents", reps: int = 8, shapes=None, tokens=None) -> dict:
    """Device time of one projection's forward and backward at T in {1, 8, 16, 32, 64}
    against HBM bytes = 1.125NK + T(6K + 4N + 8r) + 8r(N + K) (the base is read once in
    the forward and once in the backward). Four weight sets (>= 512 MB for the large
    shapes) are cycled so that the 256 MB last-level cache cannot serve repeated reads.
    Device time comes from replaying the calls captured in one graph; the eager loop's
    time (host launches included) is reported beside it. `shapes` ("model:proj" names)
    and `tokens` restrict the sweep (e.g. for a short profiled run)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(42)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for model, proj, n, k in SMALL_T_SHAPES:
        if shapes and f"{model}:{proj}" not in shapes:
            continue
        nsets = 4 if n * k * 0.5625 * 4 >= 512e6 else max(4, int(512e6 // (n * k * 0.5625)) + 1)
        sets = []
        for _ in range(nsets):
            w = (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            sets.append(lib.quantize(w))
            del w
        a = ((torch.rand(RANK, k, generator=g, device="cuda") * 2 - 1) / k ** 0.5).to(torch.bfloat16)
        b = (torch.randn(n, RANK, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
        for t in SMALL_T:
            if tokens and t not in tokens:
                continue
            x = torch.randn(t, k, generator=g, device="cuda").to(torch.bfloat16)
            dy = torch.randn(t, n, generator=g, device="cuda").to(torch.bfloat16)
            y = torch.empty(t, n, dtype=torch.bfloat16, device="cuda")
            u = torch.empty(t, RANK, dtype=torch.float32, device="cuda")
            dx = torch.empty(t, k, dtype=torch.bfloat16, device="cuda")
            da = torch.empty(RANK, k, dtype=torch.float32, device="cuda")
            db = torch.empty(n, RANK, dtype=torch.float32, device="cuda")
            wsf = lib.workspace(lib.fwd_workspace_bytes(t, n, k, RANK))
            wsb = lib.workspace(lib.bwd_workspace_bytes(t, n, k, RANK))

            def fwd(i):
                c, s_ = sets[i % nsets]
                lib.lora_linear_fwd(c, s_, x, a, b, ALPHA, y=y, u=u, ws=wsf)

            def bwd(i):
                c, s_ = sets[i % nsets]
                lib.lora_linear_bwd(c, s_, x, u, dy, a, b, ALPHA, dx=dx, dA=da, dB=db, ws=wsb)

            res, eager = {}, {}
            calls = reps * nsets
            for name, fn in (("fwd", fwd), ("bwd", bwd)):
                for i in range(nsets):
                    fn(i)
                # eager: host launches included (the small shapes are launch-bound)
                e0, e1 = ev.create(), ev.create()
                ev.record(e0, stream)
                for i in range(calls):
                    fn(i)
                ev.record(e1, stream)
                eager[name] = ev.elapsed_ms(e0, e1) * 1e3 / calls
                # device time: the same calls captured once in a graph (the library
                # allocates nothing and issues no memset), replayed back to back
                torch.cuda.synchronize()
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph):
                    for i in range(calls):
                        fn(i)
                graph.replay()
                torch.cuda.synchronize()
                ev.record(e0, stream)
                graph.replay()
                ev.record(e1, stream)
                res[name] = ev.elapsed_ms(e0, e1) * 1e3 / calls
                ev.destroy(e0)
                ev.destroy(e1)
                del graph
            nbytes = 1.125 * n * k + t * (6 * k + 4 * n + 8 * RANK) + 8 * RANK * (n + k)
            us = res["fwd"] + res["bwd"]
            rows.append({"model": model, "proj": proj, "N": n, "K": k, "T": t, "fwd_us": round(res["fwd"], 2),
                         "bwd_us": round(res["bwd"], 2), "fwd_us_eager": round(eager["fwd"], 2),
                         "bwd_us_eager": round(eager["bwd"], 2), "hbm_gbs": round(nbytes / us / 1e3, 1),
                         "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del sets
        torch.cuda.empty_cache()
    return {"rows": rows, "bytes_formula": "1.125NK + T(6K + 4N + 8r) + 8r(N + K)", "peak_gbs": HBM_PEAK_GBS,
            "weight_sets_cycled": ">= 4, >= 512 MB", "r": RANK}


MERGE_SHAPES = [("7b", "gate", 18944, 3584), ("72b", "gate", 29568, 8192)]


def merge_measure(lib, torch, ev: "HipEvents", reps: int = 4) -> dict:
    """Device time of nf4_merge_lora (merge_and_unload: the dense bf16 W + s.B.A) on the
    gate shapes, r = 16, against HBM bytes = 0.5625 NK (codes + scales read) + 2 NK
    (merged weight written); weight sets cycled past the last-level cache."""
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    stream = torch.cuda.current_stream().cuda_stream
    rows = []
    for model, proj, n, k in MERGE_SHAPES:
        nsets = max(2, int(768e6 // (n * k * 2.5625)) + 1)
        sets = []
        for _ in range(nsets):
            w = (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            sets.append(lib.quantize(w))
            del w
        a = ((torch.rand(RANK, k, generator=g, device="cuda") * 2 - 1) / k ** 0.5).to(torch.bfloat16)
        b = (torch.randn(n, RANK, generator=g, device="cuda") * 0.01).to(torch.bfloat16)
        outs = [torch.empty(n, k, dtype=torch.bfloat16, device="cuda") for _ in range(nsets)]
        for i in range(nsets):
            lib.merge_lora(sets[i][0], sets[i][1], a, b, ALPHA, out=outs[i])
        e0, e1 = ev.create(), ev.create()
        ev.record(e0, stream)
        for i in range(reps * nsets):
            lib.merge_lora(sets[i % nsets][0], sets[i % nsets][1], a, b, ALPHA, out=outs[i % nsets])
        ev.record(e1, stream)
        us = ev.elapsed_ms(e0, e1) * 1e3 / (reps * nsets)
        ev.destroy(e0)
        ev.destroy(e1)
        nbytes = 2.5625 * n * k
        rows.append({"model": model, "proj": proj, "N": n, "K": k, "r": RANK, "us": round(us, 2),
                     "hbm_gbs": round(nbytes / us / 1e3, 1), "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)})
        del sets, outs
        torch.cuda.empty_cache()
    return {"rows": rows, "bytes_formula": "0.5625NK + 2NK", "peak_gbs": HBM_PEAK_GBS}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streamed", default="7b", help="stack for the streamed measurement: 7b, 32b, 72b or none")
    ap.add_argument("--block-size", type=int, default=4)
    ap.add_argument("--slots", type=int, default=2, help="device pool slots (blocks) of the streamed stack")
    ap.add_argument("--stream-base", default="nf4", choices=("nf4", "bf16"),
                    help="format of the streamed base: nf4, or dense bf16 (the bf16_bitwise mode)")
    ap.add_argument("--stack-tokens", type=int, default=512)
    ap.add_argument("--stack-steps", type=int, default=3)
    ap.add_argument("--small-t-sweep", action="store_true",
                    help="instead of the layer step: per-projection fwd/bwd device time at T = 1..64 vs HBM bytes")
    ap.add_argument("--sweep-shapes", default="",
                    help="comma-separated model:projection names the small-T sweep is restricted to (e.g. 72b:gate)")
    ap.add_argument("--sweep-tokens", default="", help="comma-separated token counts the small-T sweep is restricted to")
    ap.add_argument("--merge", action="store_true",
                    help="instead of the layer step: merge_and_unload (dense W + s.B.A) device time vs HBM bytes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="launch one 1 GiB read + 1 GiB write elementwise kernel first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on a single "
              "GPU; sharding across GPUs is not built)", file=sys.stderr)
        return 2

    import torch

    from nf4_weight_streamed_amd import lib

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch)
    if args.small_t_sweep:
        ev = HipEvents()
        shapes = [v for v in args.sweep_shapes.split(",") if v]
        tokens = [int(v) for v in args.sweep_tokens.split(",") if v]
        known = {f"{m}:{p}" for m, p, _, _ in SMALL_T_SHAPES}
        bad = [v for v in shapes if v not in known] + [str(t) for t in tokens if t not in SMALL_T]
        if bad:
            print(f"unknown --sweep-shapes / --sweep-tokens values {bad}; shapes: {sorted(known)}, tokens: {SMALL_T}",
                  file=sys.stderr)
            return 2
        sweep = small_t_sweep(lib, torch, ev, shapes=shapes, tokens=tokens)
        copy_meas = measured_copy_gbs(torch, ev)
        read_meas = measured_read_gbs(lib, torch, ev)
        for row in sweep["rows"]:
            row["hbm_frac_vs_measured_copy"] = round(row["hbm_gbs"] / copy_meas, 4)
        sweep["hbm_copy_gbs_measured"] = round(copy_meas, 1)
        sweep["hbm_read_gbs_measured"] = round(read_meas, 1)
        out = {"metric": "NF4-LoRA linear fwd+bwd device time at small T; % of HBM roofline", "n_gpus": 1,
               "dtype": "bf16", "data": "synthetic", "small_t": sweep}
        print(json.dumps(out), flush=True)
        return 0
    if args.merge:
        ev = HipEvents()
        res = merge_measure(lib, torch, ev)
        copy_meas = measured_copy_gbs(torch, ev)
        for row in res["rows"]:
            row["hbm_frac_vs_measured_copy"] = round(row["hbm_gbs"] / copy_meas, 4)
        res["hbm_copy_gbs_measured"] = round(copy_meas, 1)
        print(json.dumps({"metric": "merge_and_unload device time; % of HBM roofline", "n_gpus": 1, "dtype": "bf16",
                          "data": "synthetic", "merge": res}), flush=True)
        return 0
    layer = build_layer(lib, torch)
    ev = HipEvents()
    for _ in range(args.warmup):
        run_step(lib, layer)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronized on both sides; the gate forward
    # GEMM of every step is bracketed by HIP events on the stream it runs on
    starts = [ev.create() for _ in range(args.steps)]
    stops = [ev.create() for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(lib, layer, prof=("gate", starts[i], stops[i]))
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    gemm_ms = [ev.elapsed_ms(a, b) for a, b in zip(starts, stops)]
    for e in starts + stops:
        ev.destroy(e)

    mfma_meas = measured_mfma_tflops(lib, torch, ev)
    copy_meas = measured_copy_gbs(torch, ev)
    read_meas = measured_read_gbs(lib, torch, ev)
    quant = quantize_measure(lib, torch, ev, cpu=not args.no_cpu_baseline)
    ms = dt * 1000.0 / args.steps
    tokens_per_s = T_TOKENS / (dt / args.steps)
    tflops = step_flops(T_TOKENS, RANK) / (dt / args.steps) / 1e12
    n, k = INTER, HIDDEN
    gate_flops = 2.0 * T_TOKENS * n * k + 2.0 * T_TOKENS * n * RANK
    gate_bytes = n * k * 0.5 + n * (k // 64) * 4 + T_TOKENS * k * 2 + T_TOKENS * n * 2 + T_TOKENS * RANK * 4 + n * RANK * 2
    avg_gemm_s = sum(gemm_ms) / len(gemm_ms) / 1000.0
    achieved = gate_flops / avg_gemm_s / 1e12
    out = {
        "metric": METRIC,
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "qwen2.5-7b-shaped layer, 7 NF4-LoRA projections, fwd+bwd, resident",
            "tokens": T_TOKENS, "lora_rank": RANK, "lora_alpha": ALPHA, "nf4_blocksize": 64,
            "projections_NxK": {name: [n_, k_] for name, n_, k_, _ in PROJ},
        },
        "tflops": round(tflops, 2),
        "mfma_frac_step": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
        "roofline": {
            "kernel": "k_nf4_gemm_fwd (gate projection 18944x3584, 512 tokens, LoRA epilogue)",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "peak_measured": round(mfma_meas, 1),
            "frac_vs_measured": round(achieved / mfma_meas, 4),
            "traffic": measured_traffic(),
            "avg_launch_us": round(avg_gemm_s * 1e6, 2),
            "algorithmic_flops_per_launch": gate_flops,
            "algorithmic_bytes_per_launch": gate_bytes,
            "hbm_gbs_algorithmic": round(gate_bytes / avg_gemm_s / 1e9, 1),
        },
        "quantize": quant,
        "denominators": {
            "mfma_bf16_tflops_published": MFMA_BF16_PEAK_TFLOPS,
            "mfma_bf16_tflops_measured": round(mfma_meas, 1),
            "hbm_gbs_published": HBM_PEAK_GBS,
            "hbm_copy_gbs_measured": round(copy_meas, 1),
            "hbm_read_gbs_measured": round(read_meas, 1),
        },
    }
    if args.streamed != "none":
        del layer
        torch.cuda.empty_cache()
        h2d = pinned_h2d_gbs(torch)
        out["streamed"] = stream_bench(torch, args.streamed, args.block_size, args.stack_tokens, args.stack_steps, h2d,
                                       args.stream_base, args.slots)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
