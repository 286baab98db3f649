"""The linear's entry points captured in a HIP graph (what the small-token sweep and the
single-linear timing replay): every replay gives the eager call's bits. The library
allocates nothing and issues no memset inside these calls, so the captured kernels are
the whole work; each replay is preceded by eager work that scribbles over the outputs."""

import numpy as np
import pytest
import torch

import synthetic_inputs as S
from helpers import to_dev_bf16

pytestmark = pytest.mark.gpu


def _buffers(lib, t, n, k, r, seed):
    case = S.linear_case(t, n, k, r=r, seed=seed)
    w = to_dev_bf16(case["W"])
    codes, absmax = lib.quantize(w)
    d = {"codes": codes, "absmax": absmax, "x": to_dev_bf16(case["x"]), "dY": to_dev_bf16(case["dY"]),
         "A": to_dev_bf16(case["A"]), "B": to_dev_bf16(case["B"])}
    d["y"] = torch.empty(t, n, dtype=torch.bfloat16, device="cuda")
    d["u"] = torch.empty(t, r, dtype=torch.float32, device="cuda")
    d["dx"] = torch.empty(t, k, dtype=torch.bfloat16, device="cuda")
    d["dA"] = torch.empty(r, k, dtype=torch.float32, device="cuda")
    d["dB"] = torch.empty(n, r, dtype=torch.float32, device="cuda")
    d["wsf"] = lib.workspace(lib.fwd_workspace_bytes(t, n, k, r))
    d["wsb"] = lib.workspace(lib.bwd_workspace_bytes(t, n, k, r))
    return d


def _call(lib, d, alpha=32.0):
    lib.lora_linear_fwd(d["codes"], d["absmax"], d["x"], d["A"], d["B"], alpha, y=d["y"], u=d["u"], ws=d["wsf"])
    lib.lora_linear_bwd(d["codes"], d["absmax"], d["x"], d["u"], d["dY"], d["A"], d["B"], alpha, dx=d["dx"],
                        dA=d["dA"], dB=d["dB"], ws=d["wsb"])


OUTS = ("y", "u", "dx", "dA", "dB")


@pytest.mark.parametrize("t,n,k", [
    (256, 1024, 1024),    # the single-linear workload (split tiles in both GEMMs)
    (300, 1104, 8192),    # ragged tiles, contraction split in both GEMMs
    (512, 2048, 18944),   # 256-token backward tiles, a whole round plus a split tail
    (5, 3584, 3584),      # few tokens: streaming kernels with split partials
    (29, 2048, 3584),     # two token blocks in both streaming kernels
    (50, 1024, 8192),     # four token blocks in the streaming forward (long, narrow weights)
])
def test_graph_replay_equals_eager(gpu_lib, t, n, k):
    lib = gpu_lib
    d = _buffers(lib, t, n, k, 16, seed=t + n)
    _call(lib, d)
    torch.cuda.synchronize()
    ref = {key: d[key].clone() for key in OUTS}
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):   # warm-up off the default stream, as capture wants
        _call(lib, d)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _call(lib, d)
    for rep in range(3):
        for key in OUTS:            # eager work between replays: scribble over every output
            d[key].view(torch.uint8).fill_(0xA5 + rep)
        graph.replay()
        torch.cuda.synchronize()
        for key in OUTS:
            assert torch.equal(d[key].view(torch.uint8), ref[key].view(torch.uint8)), (key, rep)
    del graph
