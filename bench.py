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
    """Forward of all 7 projections, then backward in reverse order. `prof` maps
    ("fwd" | "bwd", projection) to a (start, stop) pair of hipEvent_t handles that the
    library records immediately around that call's fused GEMM launch, on its stream."""
    prof = prof or {}
    for name, *_ in PROJ:
        p = layer[name]
        if ("fwd", name) in prof:
            lib.profile_next_gemm(*prof[("fwd", name)])
        lib.lora_linear_fwd(p["codes"], p["absmax"], p["x"], p["A"], p["B"], ALPHA, y=p["y"], u=p["u"], ws=p["wsf"])
    for name, *_ in reversed(PROJ):
        p = layer[name]
        if ("bwd", name) in prof:
            lib.profile_next_gemm(*prof[("bwd", name)])
        lib.lora_linear_bwd(p["codes"], p["absmax"], p["x"], p["u"], p["dy"], p["A"], p["B"], ALPHA, dx=p["dx"],
                            dA=p["dA"], dB=p["dB"], ws=p["wsb"])


def gemm_flops(kind: str, t: int, n: int, k: int, r: int) -> float:
    """Algorithmic FLOPs of one fused GEMM launch: forward 2TNK + 2TNr (base + LoRA
    epilogue); backward 2TNK + 2TKr + 2TKr (dX base, dX LoRA term, dA share)."""
    return 2.0 * t * n * k + (2.0 * t * n * r if kind == "fwd" else 4.0 * t * k * r)


def gemm_bytes(kind: str, t: int, n: int, k: int, r: int) -> float:
    """Algorithmic HBM bytes of one fused GEMM launch: the NF4 base (0.5625 B a weight)
    once, each operand read once and each output written once. Forward: x, u, B in,
    y out. Backward: dY, g, A and x (for dA) in, dX and dA out."""
    w = n * k * 0.5 + n * (k // 64) * 4
    if kind == "fwd":
        return w + 2 * t * k + 4 * t * r + 2 * n * r + 2 * t * n
    return w + 2 * t * n + 4 * t * r + 2 * r * k + 2 * t * k + 2 * t * k + 4 * r * k


def gemm_only(lib, torch, layer, ev: "HipEvents", name: str, steps: int, warmup: int) -> dict:
    """One projection's forward and backward, alone, `steps` times after `warmup`: the
    fused GEMMs' device times (events around each launch) for short profiled runs."""
    p = layer[name]
    fwd_us, bwd_us = [], []
    for i in range(warmup + steps):
        pr = {("fwd", name): (ev.create(), ev.create()), ("bwd", name): (ev.create(), ev.create())}
        lib.profile_next_gemm(*pr[("fwd", name)])
        lib.lora_linear_fwd(p["codes"], p["absmax"], p["x"], p["A"], p["B"], ALPHA, y=p["y"], u=p["u"], ws=p["wsf"])
        lib.profile_next_gemm(*pr[("bwd", name)])
        lib.lora_linear_bwd(p["codes"], p["absmax"], p["x"], p["u"], p["dy"], p["A"], p["B"], ALPHA, dx=p["dx"],
                            dA=p["dA"], dB=p["dB"], ws=p["wsb"])
        torch.cuda.synchronize()
        if i >= warmup:
            fwd_us.append(ev.elapsed_ms(*pr[("fwd", name)]) * 1e3)
            bwd_us.append(ev.elapsed_ms(*pr[("bwd", name)]) * 1e3)
        for a, b in pr.values():
            ev.destroy(a)
            ev.destroy(b)
    n, k = p["n"], p["k"]
    out = {"projection": name, "N": n, "K": k, "tokens": T_TOKENS}
    for kind, us in (("fwd", fwd_us), ("bwd", bwd_us)):
        avg = sum(us) / len(us)
        out[kind] = {"us": round(avg, 2), "tflops": round(gemm_flops(kind, T_TOKENS, n, k, RANK) / avg / 1e6, 1)}
    return out


def gemm_attribution(lib, torch, layer, ev: "HipEvents", steps: int = 3) -> dict:
    """Device time of every fused GEMM launch of the step (HIP events recorded by the
    library around each launch, on its stream), averaged over `steps` untimed steps:
    which kernel holds the most device time per step."""
    names = [n for n, *_ in PROJ]
    keys = [(kind, n) for kind in ("fwd", "bwd") for n in names]
    acc = {key: 0.0 for key in keys}
    for _ in range(steps):
        prof = {key: (ev.create(), ev.create()) for key in keys}
        run_step(lib, layer, prof)
        torch.cuda.synchronize()
        for key, (a, b) in prof.items():
            acc[key] += ev.elapsed_ms(a, b) * 1e3 / steps
            ev.destroy(a)
            ev.destroy(b)
    per = {kind: {n: round(acc[(kind, n)], 2) for n in names} for kind in ("fwd", "bwd")}
    totals = {"k_nf4_gemm_fwd": round(sum(per["fwd"].values()), 1),
              "k_nf4_gemm_bwd_dx": round(sum(per["bwd"].values()), 1)}
    return {"us_per_launch": per, "us_per_step": totals,
            "dominant": max(totals, key=totals.get)}


# committed counter summaries of the fused GEMMs, and the sources whose change
# invalidates the HBM traffic they report
_CSRC = os.path.join(ROOT, "nf4_weight_streamed_amd", "csrc")
TRAFFIC = {
    "k_nf4_gemm_fwd": (os.path.join(ROOT, "profiles", "k_nf4_gemm_fwd_gate_qwen7b_t512_traffic.md"),
                       [os.path.join(_CSRC, f) for f in ("nf4_gemm_fwd.hip", "device.h", "common.h")]),
    "k_nf4_gemm_bwd_dx": (os.path.join(ROOT, "profiles", "k_nf4_gemm_bwd_dx_gate_qwen7b_t512_traffic.md"),
                          [os.path.join(_CSRC, f) for f in ("nf4_gemm_bwd.hip", "device.h", "common.h")]),
}
COPY_CALIBRATION_BYTES = 1 << 30


def kernel_source_digest(kernel: str = "k_nf4_gemm_fwd") -> str:
    import hashlib

    h = hashlib.sha256()
    for f in TRAFFIC[kernel][1]:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel: str) -> int | None:
    """HBM bytes per launch of `kernel` (gate projection) from its committed counter
    summary (FETCH_SIZE + WRITE_SIZE, each scaled by the copy calibration), or None when
    that summary is missing or was taken on different kernel sources."""
    try:
        with open(TRAFFIC[kernel][0]) as fh:
            text = fh.read()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            key, val = line[2:].split(": ", 1)
            fields[key.strip("` ")] = val.strip("` ")
    if fields.get("source_sha256") != kernel_source_digest(kernel):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def copy_calibration(torch, lib=None) -> None:
    """Plain streaming kernels of known traffic for the counter calibration: an
    elementwise negation of a 1 GiB fp32 tensor (reads 1 GiB, writes 1 GiB) and, with
    `lib`, the library's read probe over the same 1 GiB (reads 1 GiB, writes 1 MiB)."""
    src = torch.ones(COPY_CALIBRATION_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    if lib is not None:
        out = torch.empty(256 * 1024, dtype=torch.int32, device="cuda")
        lib.probe_read(src, out, 1024)
        torch.cuda.synchronize()
        del out
    del src, dst
    torch.cuda.empty_cache()


def _blas_info() -> dict:
    """numpy's BLAS build and the host cores the oracle may use."""
    import numpy as np

    info = {"cores_affinity": len(os.sched_getaffinity(0)), "numpy": np.__version__}
    try:
        blas = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        info["blas"] = f"{blas.get('name')} {blas.get('version')}"
        info["blas_config"] = blas.get("openblas configuration", "")
    except Exception as e:  # pragma: no cover - numpy builds without the dict form
        info["blas"] = f"unknown ({e})"
    return info


def _blas_threads(n: int):
    """Pin the BLAS pool to n threads for the oracle's timing; returns (context, threads in use)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    ctx = threadpool_limits(limits=n, user_api="blas")
    used = max([i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"] or [0])
    return ctx, used


def _oracle_linear_seconds(case: dict, budget: float) -> tuple[float, int]:
    """Mean seconds of one oracle pass (dequantise + fwd + bwd) over at least 3 passes
    and about `budget` seconds; the NF4 storage is made once, outside the timing."""
    import oracle as O
    import synthetic_inputs as S

    codes, absmax = O.quantize(S.bf16_bits_to_f32(case["W"]))
    reps = 0
    t0 = time.perf_counter()
    while reps < 3 or time.perf_counter() - t0 < budget:
        wq = O.dequantize(codes, absmax)
        O.lora_linear_fwd(case["x"], wq, case["A"], case["B"], ALPHA)
        O.lora_linear_bwd(case["x"], wq, case["A"], case["B"], ALPHA, case["dY"])
        reps += 1
    return (time.perf_counter() - t0) / reps, reps


def linear_flops(t: int, n: int, k: int, r: int) -> float:
    return 4.0 * t * n * k + 6.0 * t * r * (n + k)


def cpu_baseline(seconds_budget: float = 12.0) -> dict:
    """The fp64 oracle, as it stands, on the host cores of the machine that runs the
    benchmark (BLAS pinned to the cores of this process's affinity mask), on a bounded
    sample of the same workload:
    the q projection (3584 x 3584) of the layer with all 512 tokens - dequantise +
    forward + backward - repeated for about `seconds_budget` seconds, scaled to the
    whole layer by the algorithmic-FLOP ratio. Beside it: the single 1024 x 1024 linear
    at 256 tokens timed whole, and the streamed stacks' step time extrapolated from the
    sample's FLOP rate (one layer x the layer count; labelled extrapolated).
    Quantisation (load time) is outside the timed region, as on the GPU."""
    import synthetic_inputs as S
    from nf4_weight_streamed_amd import stack as ST

    info = _blas_info()
    ctx, threads = _blas_threads(info["cores_affinity"])
    with ctx:
        n, k = QW, HIDDEN
        dt, reps = _oracle_linear_seconds(S.linear_case(T_TOKENS, n, k, r=RANK, proj="q"), seconds_budget)
        c0_dt, c0_reps = _oracle_linear_seconds(S.linear_case(256, 1024, 1024, r=RANK), 2.0)
    sample_flops = linear_flops(T_TOKENS, n, k, RANK)
    rate = sample_flops / dt
    layer_seconds = step_flops(T_TOKENS, RANK) / rate
    stacks = {}
    for model, (dims, n_layers) in ST.QWEN25.items():
        f = n_layers * sum(linear_flops(T_TOKENS, n_, k_, RANK) for n_, k_ in dims.shapes().values())
        stacks[model] = {"seconds_per_step": round(f / rate, 1), "tokens_per_s": round(T_TOKENS * rate / f, 3),
                         "layers": n_layers, "kind": "extrapolated: sample FLOP rate x the stack's algorithmic FLOPs"}
    return {
        "value": round(T_TOKENS / layer_seconds, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
        "sample": (f"q projection 3584x3584, 512 tokens, r16: dequantise + fwd + bwd in fp64 numpy, "
                   f"{dt:.2f} s per pass (mean of {reps}); "
                   f"scaled to the 7-projection layer by algorithmic FLOPs ({step_flops(T_TOKENS, RANK) / sample_flops:.2f}x)"),
        "gflops": round(rate / 1e9, 3),
        "host": info,
        "single_linear_1024": {"seconds_per_fwd_bwd": round(c0_dt, 4), "passes": c0_reps,
                               "tokens_per_s": round(256 / c0_dt, 1),
                               "gflops": round(linear_flops(256, 1024, 1024, RANK) / c0_dt / 1e9, 3)},
        "stacks_t512": stacks,
    }


def config0_measure(lib, torch, ev: "HipEvents", reps: int = 200) -> dict:
    """The single NF4-LoRA linear, in = out = 1024, 256 tokens, r 16, alpha 32: forward +
    backward (dX, dA, dB) device time from a graph replay of the calls (and, beside it,
    `reps` eager back-to-back calls timed with events on the stream, host launches
    included), against its algorithmic FLOPs and bytes. The working set (about 3 MB)
    stays in the caches: the figure is latency-bound, reported for completeness."""
    import synthetic_inputs as S

    t, n, k = 256, 1024, 1024
    case = S.linear_case(t, n, k, r=RANK)
    dev = {key: torch.from_numpy(case[key].view("int16")).view(torch.bfloat16).cuda() for key in ("W", "x", "A", "B", "dY")}
    codes, absmax = lib.quantize(dev["W"])
    y = torch.empty(t, n, dtype=torch.bfloat16, device="cuda")
    u = torch.empty(t, RANK, dtype=torch.float32, device="cuda")
    dx = torch.empty(t, k, dtype=torch.bfloat16, device="cuda")
    da = torch.empty(RANK, k, dtype=torch.float32, device="cuda")
    db = torch.empty(n, RANK, dtype=torch.float32, device="cuda")
    wsf = lib.workspace(lib.fwd_workspace_bytes(t, n, k, RANK))
    wsb = lib.workspace(lib.bwd_workspace_bytes(t, n, k, RANK))

    def one():
        lib.lora_linear_fwd(codes, absmax, dev["x"], dev["A"], dev["B"], ALPHA, y=y, u=u, ws=wsf)
        lib.lora_linear_bwd(codes, absmax, dev["x"], u, dev["dY"], dev["A"], dev["B"], ALPHA, dx=dx, dA=da, dB=db,
                            ws=wsb)

    for _ in range(10):
        one()
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = ev.create(), ev.create()
    torch.cuda.synchronize()
    ev.record(e0, stream)
    for _ in range(reps):
        one()
    ev.record(e1, stream)
    us_eager = ev.elapsed_ms(e0, e1) * 1e3 / reps
    # device time: the same calls captured once in a graph and replayed (the library
    # allocates nothing and issues no memset; tests/test_gpu_graph.py checks replays
    # against eager calls bit for bit), so host launch costs drop out
    graph_reps = 50
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        one()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(graph_reps):
            one()
    graph.replay()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(3):
        ev.record(e0, stream)
        graph.replay()
        ev.record(e1, stream)
        best = min(best, ev.elapsed_ms(e0, e1) * 1e3 / graph_reps)
    del graph
    ev.destroy(e0)
    ev.destroy(e1)
    us = best
    flops = linear_flops(t, n, k, RANK)
    nbytes = 2 * (n * k * 0.5625) + t * (6 * k + 4 * n + 8 * RANK) + 8 * RANK * (n + k)
    return {"workload": "single NF4-LoRA linear 1024x1024, 256 tokens, r16, fwd+bwd", "us_per_fwd_bwd": round(us, 2),
            "us_per_fwd_bwd_eager": round(us_eager, 2), "timing": "device time of a graph replay of 50 calls "
            "(best of 3); eager back-to-back calls beside it",
            "tokens_per_s": round(t / us * 1e6, 1), "tflops": round(flops / us / 1e6, 2),
            "mfma_frac": round(flops / us / 1e6 / MFMA_BF16_PEAK_TFLOPS, 5),
            "hbm_gbs_algorithmic": round(nbytes / us / 1e3, 1), "algorithmic_flops": flops,
            "algorithmic_bytes": nbytes}


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


READ_SWEEP: list = []  # (depth, workgroups, nontemporal, GB/s) of the last measured_read_gbs


def measured_read_gbs(lib, torch, ev: "HipEvents", nbytes: int = 2 << 30) -> float:
    """Read-only reference: the library's read probe (coalesced 16-byte loads, grid-stride)
    over 2 GiB, swept over the loads in flight per thread (4 .. 32), the grid (256 .. 8192
    workgroups) and plain or non-temporal loads, best of 3 launches each; returns the best
    rate and keeps the sweep in READ_SWEEP, so that the plateau the best comes from is on
    record."""
    src = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    best = 0.0
    READ_SWEEP.clear()
    out = torch.empty(256 * 8192, dtype=torch.int32, device="cuda")
    for nt in (False, True):
        for depth in (4, 8, 16, 32):
            for wg in (256, 384, 512, 768, 1024, 2048, 4096, 8192):
                lib.probe_read_depth(src, out, wg, depth, nt)
                rate = 0.0
                for _ in range(3):
                    e0, e1 = ev.create(), ev.create()
                    ev.record(e0, stream)
                    lib.probe_read_depth(src, out, wg, depth, nt)
                    ev.record(e1, stream)
                    rate = max(rate, nbytes / (ev.elapsed_ms(e0, e1) * 1e-3) / 1e9)
                    ev.destroy(e0)
                    ev.destroy(e1)
                READ_SWEEP.append((depth, wg, int(nt), round(rate, 1)))
                best = max(best, rate)
    del out, src
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


def _stack_inputs(torch, tokens: int, hidden: int):
    g = torch.Generator(device="cuda")
    g.manual_seed(42)
    h0 = torch.randn(tokens, hidden, generator=g, device="cuda").to(torch.bfloat16)
    dh = torch.randn(tokens, hidden, generator=g, device="cuda").to(torch.bfloat16)
    return h0, dh


def _stack_run(torch, ST, base, lora, tokens, h0, dh, steps, **kw) -> dict:
    """One stack configuration: a first step (its outputs kept for the bitwise check),
    then `steps` timed steps, then one more step with the pool's copy and acquire-stall
    spans recorded (kept out of the timed steps: the timing events can slow some pool
    configurations down)."""
    st = ST.NF4Stack(base, lora, tokens, ALPHA, **kw)
    try:
        y, dx = st.step(h0, dh)
        torch.cuda.synchronize()
        res = {"y": y.clone(), "dx": dx.clone(), "act": st.activation_bytes()}
        c0 = st.pool.stats()["bytes_copied"]
        st.pool.timing_collect()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            st.step(h0, dh)
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        res["s"] = (time.perf_counter() - t0) / steps
        res["timed_issue_s"] = (t1 - t0) / steps
        tm = st.pool.timing_collect()
        res["timed_host_ms"], res["timed_host_max_ms"] = tm["host_ms"] / steps, tm["host_max_ms"]
        res["timed_host_sync_ms"] = tm["host_sync_ms"] / steps
        res["bytes"] = (st.pool.stats()["bytes_copied"] - c0) / steps
        st.pool.timing_enable(True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        st.step(h0, dh)
        t1 = time.perf_counter()
        torch.cuda.synchronize()
        res["s_instrumented"] = time.perf_counter() - t0
        res["issue_s"] = t1 - t0
        tm = st.pool.timing_collect()
        for k in ("copy_ms", "stall_ms", "host_ms", "host_max_ms"):
            res[k] = tm[k]
        return res
    finally:
        st.close()
        del st
        torch.cuda.empty_cache()


def stream_bench(torch, model: str, block_sizes, tokens_list, steps: int, h2d_gbs: float, base_kind: str = "nf4",
                 slot_counts=(2,), remat: bool = True, layer_parts: bool = True, max_ahead: int = 2) -> dict:
    """Streamed vs resident step time of a Qwen2.5-shaped identity-mixing stack for each
    (tokens, block size), with the bitwise check, H2D traffic, and the copy/compute
    overlap measured by the pool's own events: copy_ms = device time of the H2D copies
    per step, stall_ms = time the compute stream stood waiting for a copy per step;
    copy time hidden under compute = copy_ms - stall_ms. base_kind "bf16" streams a dense
    bf16 base (the experimental bf16_bitwise mode) instead of NF4. slot_counts = device
    pool sizes in blocks (the resident run holds every block); a pool of k slots copies
    about 2(nb - k) blocks a step. One pinned host copy
    of the base serves every block size (regroup). With `remat`, the first block size is
    also run with rematerialisation (block-boundary states kept, each block's forward
    recomputed in its backward visit). layer_parts: the pool copies and releases each
    layer of a block on its own instead of one copy per block, and the compute stream
    waits for each layer's copy instead of the whole block's. max_ahead: blocks the host
    may run ahead of the device (stream_pool_set_max_ahead; 0 = no bound)."""
    from nf4_weight_streamed_amd import stack as ST

    dims, n_layers = ST.QWEN25[model]
    host_cls = ST.HostBF16Base if base_kind == "bf16" else ST.HostNF4Base
    base = host_cls(dims, n_layers, block_sizes[0], ST.qwen_weight_fn())
    lora = ST.LoraParams(dims, n_layers, RANK, ST.qwen_lora_fn())
    load = {k: round(v, 3) if isinstance(v, float) else v for k, v in base.load_stats.items()}
    print(f"[stream_bench] {model}: host base loaded in {load['seconds']:.1f} s", file=sys.stderr, flush=True)
    fmt = "dense bf16" if base_kind == "bf16" else "NF4"
    rows = []
    for tokens in tokens_list:
        h0, dh = _stack_inputs(torch, tokens, dims.hidden)
        flops = n_layers * sum(4 * tokens * n * k + 6 * tokens * RANK * (n + k) for n, k in dims.shapes().values())
        res = _stack_run(torch, ST, base, lora, tokens, h0, dh, steps, mode="resident")
        print(f"[stream_bench] {model} T={tokens}: resident {res['s'] * 1e3:.1f} ms per step", file=sys.stderr,
              flush=True)
        for i, (bs, n_slots) in enumerate((bs, k) for bs in block_sizes for k in slot_counts):
            b = base.regroup(bs)
            if n_slots >= b.n_blocks:
                continue
            got = _stack_run(torch, ST, b, lora, tokens, h0, dh, steps, mode="streamed", n_slots=n_slots,
                             layer_parts=layer_parts, max_ahead=max_ahead)
            r_s, s_s, nbytes = res["s"], got["s"], got["bytes"]
            print(f"[stream_bench] {model} T={tokens} bs={bs} slots={n_slots}: streamed {s_s * 1e3:.1f} ms per step",
                  file=sys.stderr, flush=True)
            copy_s = nbytes / (h2d_gbs * 1e9)
            c_ms, st_ms = got["copy_ms"], got["stall_ms"]
            row = {
                "workload": f"qwen2.5-{model}-shaped stack, {n_layers} layers, block_size {bs}, {n_slots} pool slots, "
                            f"{tokens} tokens, {fmt} in pinned host, identity attention mixing, fwd+bwd",
                "copies": "one per layer" if (layer_parts or not b.contiguous) else "one per block",
                "compute_waits": "per layer" if (layer_parts or not b.contiguous) else "per block",
                "host_max_blocks_ahead": max_ahead,
                "tokens": tokens, "block_size": bs, "slots": n_slots,
                "device_pool_gb": round(n_slots * b.slot_bytes / 1e9, 3),
                "bitwise_equal_to_resident": bool(torch.equal(res["y"], got["y"]) and torch.equal(res["dx"], got["dx"])),
                "resident_ms_per_step": round(r_s * 1e3, 3),
                "streamed_ms_per_step": round(s_s * 1e3, 3),
                "streamed_over_resident": round(s_s / r_s, 3),
                "streamed_tokens_per_s": round(tokens / s_s, 2),
                "streamed_tflops": round(flops / s_s / 1e12, 2),
                "resident_tflops": round(flops / r_s / 1e12, 2),
                "h2d_gb_per_step": round(nbytes / 1e9, 3),
                "h2d_gbs_achieved_over_step": round(nbytes / s_s / 1e9, 2),
                "h2d_gbs_while_copying": round(nbytes / (c_ms * 1e-3) / 1e9, 2) if c_ms > 0 else None,
                "h2d_gbs_pinned_peak_measured": round(h2d_gbs, 2),
                "pcie_frac": round(nbytes / s_s / 1e9 / h2d_gbs, 4),
                "pcie_floor_ratio": round(max(r_s, copy_s) / r_s, 3),
                "copy_engine_busy_ms_per_step": round(c_ms, 3),
                "compute_stall_ms_per_step": round(st_ms, 3),
                "compute_busy_ms_per_step": round(got["s_instrumented"] * 1e3 - st_ms, 3),
                "copy_time_hidden_frac": round((c_ms - st_ms) / c_ms, 4) if c_ms > 0 else None,
                "instrumented_step_ms": round(got["s_instrumented"] * 1e3, 3),
                "instrumented_host_issue_ms": round(got["issue_s"] * 1e3, 3),
                "host_ms_in_pool_hip_calls": round(got["host_ms"], 3),
                "host_longest_pool_hip_call_ms": round(got["host_max_ms"], 3),
                "timed_host_issue_ms_per_step": round(got["timed_issue_s"] * 1e3, 3),
                "timed_host_ms_in_pool_hip_calls_per_step": round(got["timed_host_ms"], 3),
                "timed_host_longest_pool_hip_call_ms": round(got["timed_host_max_ms"], 3),
                "timed_host_ms_held_by_lead_bound_per_step": round(got["timed_host_sync_ms"], 3),
                "overlap_source": "HIP events of the pool over one extra step: copy spans on the copy stream, "
                                  "acquire-wait spans on the compute stream",
                "host_base_gb": round(base.total_bytes() / 1e9, 3),
            }
            if remat and i == 0:
                rm = _stack_run(torch, ST, b, lora, tokens, h0, dh, steps, mode="streamed", n_slots=n_slots,
                                remat=True, layer_parts=layer_parts, max_ahead=max_ahead)
                row["remat"] = {
                    "bitwise_equal_to_resident": bool(torch.equal(res["y"], rm["y"]) and torch.equal(res["dx"], rm["dx"])),
                    "streamed_ms_per_step": round(rm["s"] * 1e3, 3),
                    "over_streamed": round(rm["s"] / s_s, 3),
                    "activation_gb": round(rm["act"] / 1e9, 3),
                    "activation_gb_stored": round(got["act"] / 1e9, 3),
                    "h2d_gb_per_step": round(rm["bytes"] / 1e9, 3),
                }
                del rm
            rows.append(row)
            del got
        del res, h0, dh
    del base, lora
    release_memory(torch)
    return {"model": model, "load": load, "rows": rows}


def release_memory(torch) -> None:
    """Free cached device memory and cached pinned host blocks while the runtime is up
    (not left to interpreter-exit destructors)."""
    import gc

    gc.collect()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    host_empty = getattr(torch._C, "_host_emptyCache", None)
    if host_empty is not None:
        host_empty()


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


def small_t_layer(lib, torch, ev: "HipEvents", model: str, tokens, reps: int = 4) -> list:
    """Device time of one whole layer's projections - the forward of q, k, v, o, gate, up,
    down, then their backward in reverse order, as in a training step - at each T in
    `tokens`, against the HBM bytes of the seven projections (per projection
    1.125NK + T(6K + 4N + 8r) + 8r(N + K)). Weight sets of the whole layer are cycled
    (>= 512 MB of distinct NF4 bases) so that the last-level cache cannot serve them;
    device time from a graph replay of reps x sets layer steps."""
    from nf4_weight_streamed_amd import stack as ST

    dims, _ = ST.QWEN25[model]
    shapes = dims.shapes()
    layer_nf4 = dims.layer_nf4_bytes()
    nsets = max(2, -(-int(512e6) // layer_nf4))
    g = torch.Generator(device="cuda")
    g.manual_seed(42)
    stream = torch.cuda.current_stream().cuda_stream
    sets = []
    for _ in range(nsets):
        ws = {}
        for name in ST.PROJS:
            n, k = shapes[name]
            w = (torch.randn(n, k, generator=g, device="cuda") * 0.02).to(torch.bfloat16)
            ws[name] = lib.quantize(w)
            del w
        sets.append(ws)
    lora = {}
    for name in ST.PROJS:
        n, k = shapes[name]
        lora[name] = (((torch.rand(RANK, k, generator=g, device="cuda") * 2 - 1) / k ** 0.5).to(torch.bfloat16),
                      (torch.randn(n, RANK, generator=g, device="cuda") * 0.01).to(torch.bfloat16))
    rows = []
    for t in tokens:
        bufs = {}
        for name in ST.PROJS:
            n, k = shapes[name]
            bufs[name] = {
                "x": torch.randn(t, k, generator=g, device="cuda").to(torch.bfloat16),
                "dy": torch.randn(t, n, generator=g, device="cuda").to(torch.bfloat16),
                "y": torch.empty(t, n, dtype=torch.bfloat16, device="cuda"),
                "u": torch.empty(t, RANK, dtype=torch.float32, device="cuda"),
                "dx": torch.empty(t, k, dtype=torch.bfloat16, device="cuda"),
                "dA": torch.empty(RANK, k, dtype=torch.float32, device="cuda"),
                "dB": torch.empty(n, RANK, dtype=torch.float32, device="cuda"),
                "wsf": lib.workspace(lib.fwd_workspace_bytes(t, n, k, RANK)),
                "wsb": lib.workspace(lib.bwd_workspace_bytes(t, n, k, RANK)),
            }

        def layer_step(i):
            ws = sets[i % nsets]
            for name in ST.PROJS:
                b, (A, Bm) = bufs[name], lora[name]
                lib.lora_linear_fwd(*ws[name], b["x"], A, Bm, ALPHA, y=b["y"], u=b["u"], ws=b["wsf"])
            for name in reversed(ST.PROJS):
                b, (A, Bm) = bufs[name], lora[name]
                lib.lora_linear_bwd(*ws[name], b["x"], b["u"], b["dy"], A, Bm, ALPHA, dx=b["dx"], dA=b["dA"],
                                    dB=b["dB"], ws=b["wsb"])

        calls = reps * nsets
        for i in range(nsets):
            layer_step(i)
        e0, e1 = ev.create(), ev.create()
        ev.record(e0, stream)
        for i in range(calls):
            layer_step(i)
        ev.record(e1, stream)
        eager = ev.elapsed_ms(e0, e1) * 1e3 / calls
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(calls):
                layer_step(i)
        graph.replay()
        torch.cuda.synchronize()
        ev.record(e0, stream)
        graph.replay()
        ev.record(e1, stream)
        us = ev.elapsed_ms(e0, e1) * 1e3 / calls
        ev.destroy(e0)
        ev.destroy(e1)
        del graph, bufs
        nbytes = sum(1.125 * n * k + t * (6 * k + 4 * n + 8 * RANK) + 8 * RANK * (n + k) for n, k in shapes.values())
        rows.append({"model": model, "T": t, "layer_us": round(us, 2), "layer_us_eager": round(eager, 2),
                     "bytes": int(nbytes), "hbm_gbs": round(nbytes / us / 1e3, 1),
                     "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                     "us_at_8tbs": round(nbytes / 8e12 * 1e6, 2),
                     "weight_sets_cycled": nsets})
        print(f"[small_t_layer] {model} T={t}: {us:.1f} us per layer fwd+bwd ({nbytes / us / 1e3:.0f} GB/s)",
              file=sys.stderr, flush=True)
    del sets, lora
    torch.cuda.empty_cache()
    return rows


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
    ap.add_argument("--streamed", default="7b",
                    help="comma-separated stacks for the streamed measurement (7b, 32b, 72b) or none")
    ap.add_argument("--block-sizes", default="4", help="comma-separated block sizes of the streamed stacks")
    ap.add_argument("--slots", default="2", help="comma-separated device pool sizes (slots of one block) of the "
                                                  "streamed stacks")
    ap.add_argument("--stream-base", default="nf4", choices=("nf4", "bf16"),
                    help="format of the streamed base: nf4, or dense bf16 (the bf16_bitwise mode)")
    ap.add_argument("--stack-tokens", default="512", help="comma-separated token counts of the streamed stacks")
    ap.add_argument("--no-remat", action="store_true", help="skip the rematerialisation run of the streamed stacks")
    ap.add_argument("--block-copies", action="store_true",
                    help="streamed stacks: one copy per block and one wait for it (default: each layer of a block "
                         "copied, waited for and released on its own)")
    ap.add_argument("--max-ahead", type=int, default=2,
                    help="streamed stacks: blocks the host may run ahead of the device (0: no bound)")
    ap.add_argument("--stack-steps", type=int, default=3)
    ap.add_argument("--small-t-sweep", action="store_true",
                    help="instead of the layer step: per-projection fwd/bwd device time at T = 1..64 vs HBM bytes")
    ap.add_argument("--sweep-shapes", default="",
                    help="comma-separated model:projection names the small-T sweep is restricted to (e.g. 72b:gate)")
    ap.add_argument("--sweep-tokens", default="", help="comma-separated token counts the small-T sweep is restricted to")
    ap.add_argument("--merge", action="store_true",
                    help="instead of the layer step: merge_and_unload (dense W + s.B.A) device time vs HBM bytes")
    ap.add_argument("--gemm-only", default="", choices=["", "q", "k", "v", "o", "gate", "up", "down"],
                    help="instead of the layer step: only this projection's forward and backward, --steps times "
                         "(short runs for counters and traces of its kernels)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="launch one 1 GiB read + 1 GiB write elementwise kernel first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path runs on a single "
              "GPU; sharding across GPUs is not built)", file=sys.stderr)
        return 2
    models = [m for m in args.streamed.split(",") if m and m != "none"]
    block_sizes = [int(v) for v in args.block_sizes.split(",") if v]
    slot_counts = [int(v) for v in args.slots.split(",") if v]
    stack_tokens = [int(v) for v in args.stack_tokens.split(",") if v]
    if any(m not in ("7b", "32b", "72b") for m in models) or not block_sizes or not stack_tokens:
        print(f"--streamed takes 7b, 32b, 72b or none; --block-sizes and --stack-tokens need values", file=sys.stderr)
        return 2

    import torch

    from nf4_weight_streamed_amd import lib

    torch.cuda.set_device(0)
    if args.copy_calibration:
        copy_calibration(torch, lib)
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
        if not shapes:
            sweep["layer_rows"] = [row for m in ("7b", "72b")
                                   for row in small_t_layer(lib, torch, ev, m, tokens or SMALL_T)]
        copy_meas = measured_copy_gbs(torch, ev)
        read_meas = measured_read_gbs(lib, torch, ev)
        for row in sweep["rows"] + sweep.get("layer_rows", []):
            row["hbm_frac_vs_measured_copy"] = round(row["hbm_gbs"] / copy_meas, 4)
        sweep["hbm_copy_gbs_measured"] = round(copy_meas, 1)
        sweep["hbm_read_gbs_measured"] = round(read_meas, 1)
        sweep["read_probe_sweep"] = {"columns": ["loads_in_flight_per_thread", "workgroups", "nontemporal", "GB/s"],
                                     "rows": READ_SWEEP}
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
    if args.gemm_only:
        print(json.dumps(gemm_only(lib, torch, layer, ev, args.gemm_only, args.steps, args.warmup)), flush=True)
        del layer
        release_memory(torch)
        return 0
    for _ in range(args.warmup):
        run_step(lib, layer)
    torch.cuda.synchronize()
    attribution = gemm_attribution(lib, torch, layer, ev)

    # timed region: exactly `steps` steps, synchronized on both sides; the gate
    # projection's forward and backward GEMMs of every step are bracketed by HIP events
    # recorded by the library on the stream they run on
    prof = [{("fwd", "gate"): (ev.create(), ev.create()), ("bwd", "gate"): (ev.create(), ev.create())}
            for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run_step(lib, layer, prof=prof[i])
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    launch_s = {kind: sum(ev.elapsed_ms(*p[(kind, "gate")]) for p in prof) / len(prof) / 1e3 for kind in ("fwd", "bwd")}
    for p in prof:
        for a, b in p.values():
            ev.destroy(a)
            ev.destroy(b)

    mfma_meas = measured_mfma_tflops(lib, torch, ev)
    copy_meas = measured_copy_gbs(torch, ev)
    read_meas = measured_read_gbs(lib, torch, ev)
    quant = quantize_measure(lib, torch, ev, cpu=not args.no_cpu_baseline)
    config0 = config0_measure(lib, torch, ev)
    ms = dt * 1000.0 / args.steps
    tokens_per_s = T_TOKENS / (dt / args.steps)
    tflops = step_flops(T_TOKENS, RANK) / (dt / args.steps) / 1e12
    n, k = INTER, HIDDEN

    def roofline(kind: str) -> dict:
        kernel = "k_nf4_gemm_fwd" if kind == "fwd" else "k_nf4_gemm_bwd_dx"
        f, b, sec = gemm_flops(kind, T_TOKENS, n, k, RANK), gemm_bytes(kind, T_TOKENS, n, k, RANK), launch_s[kind]
        achieved = f / sec / 1e12
        what = "y = x.W^T + LoRA epilogue" if kind == "fwd" else "dX = dY.W + LoRA term, dA share"
        return {
            "kernel": f"{kernel} (gate projection 18944x3584, 512 tokens: {what})",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA_BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4),
            "traffic": measured_traffic(kernel),
            "peak_measured": round(mfma_meas, 1),
            "frac_vs_measured": round(achieved / mfma_meas, 4),
            "avg_launch_us": round(sec * 1e6, 2),
            "algorithmic_flops_per_launch": f,
            "algorithmic_bytes_per_launch": b,
            "hbm_gbs_algorithmic": round(b / sec / 1e9, 1),
            "device_us_per_step_all_projections": attribution["us_per_step"][kernel],
        }

    dominant = "bwd" if attribution["dominant"] == "k_nf4_gemm_bwd_dx" else "fwd"
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
        "roofline": roofline(dominant),
        "roofline_other_gemm": roofline("fwd" if dominant == "bwd" else "bwd"),
        "gemm_device_time": attribution,
        "config0": config0,
        "quantize": quant,
        "denominators": {
            "mfma_bf16_tflops_published": MFMA_BF16_PEAK_TFLOPS,
            "mfma_bf16_tflops_measured": round(mfma_meas, 1),
            "hbm_gbs_published": HBM_PEAK_GBS,
            "hbm_copy_gbs_measured": round(copy_meas, 1),
            "hbm_read_gbs_measured": round(read_meas, 1),
            "read_probe_sweep": {"columns": ["loads_in_flight_per_thread", "workgroups", "nontemporal", "GB/s"],
                                 "rows": READ_SWEEP},
        },
    }
    del layer
    release_memory(torch)
    if models:
        h2d = pinned_h2d_gbs(torch)
        out["denominators"]["h2d_pinned_gbs_measured"] = round(h2d, 2)
        runs = [stream_bench(torch, m, block_sizes, stack_tokens, args.stack_steps, h2d, args.stream_base, slot_counts,
                             remat=not args.no_remat, layer_parts=not args.block_copies,
                             max_ahead=args.max_ahead)
                for m in models]
        out["streamed"] = dict(runs[0]["rows"][0], load=runs[0]["load"])
        out["streamed_all"] = runs
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline()
    release_memory(torch)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
