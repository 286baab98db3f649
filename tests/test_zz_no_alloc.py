"""nf4_lora_linear_fwd_noalloc (the forward with the library's own device scratch as
workspace, for callers that cannot allocate), called through the C ABI: its outputs
equal nf4_lora_linear_fwd's bit for bit and the fp64 oracle's within the parity
bounds, on consecutive calls of decreasing size; sizes beyond the scratch are refused;
calls after the first change no device memory."""

import ctypes as C

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S
from helpers import bits_of, check_linear, f32_of, linear_mags, to_dev_bf16

pytestmark = pytest.mark.gpu


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _case(t, n, k, r):
    case = S.linear_case(t, n, k, r=r)
    codes, absmax = O.quantize(O.bf16_bits_to_f64(case["W"]).astype(np.float32))
    dev = {"codes": torch.from_numpy(codes).cuda(), "absmax": torch.from_numpy(absmax).cuda(),
           "x": to_dev_bf16(case["x"]), "A": to_dev_bf16(case["A"]), "B": to_dev_bf16(case["B"])}
    return case, O.dequantize(codes, absmax), dev


def _noalloc(L, dev, t, n, k, r, y, u):
    raw = L.raw()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    return raw.nf4_lora_linear_fwd_noalloc(_ptr(dev["codes"]), _ptr(dev["absmax"]), n, k, _ptr(dev["x"]), t,
                                           _ptr(dev["A"]), _ptr(dev["B"]), r, 32.0, _ptr(y), _ptr(u), stream)


def test_noalloc_forward_matches_workspace_forward_and_oracle(gpu_lib):
    L = gpu_lib
    first_done = False
    for t, n, k, r in ((512, 18944, 3584, 16), (300, 1104, 8192, 16), (40, 208, 384, 5), (7, 256, 512, 16)):
        print(f"noalloc forward T={t} N={n} K={k} r={r}", flush=True)
        case, wq, dev = _case(t, n, k, r)
        y = torch.empty(t, n, dtype=torch.bfloat16, device="cuda")
        u = torch.empty(t, r, dtype=torch.float32, device="cuda")
        # the workspace entry point first: the runtime loads the kernels' code on their
        # first launch, which is not the call's doing
        y_ref, u_ref = L.lora_linear_fwd(dev["codes"], dev["absmax"], dev["x"], dev["A"], dev["B"], 32.0)
        torch.cuda.synchronize()
        free_before = torch.cuda.mem_get_info()[0]
        assert _noalloc(L, dev, t, n, k, r, y, u) == 0, L.last_error()
        torch.cuda.synchronize()
        if first_done:            # no device memory taken by the call (the first one maps the scratch)
            assert torch.cuda.mem_get_info()[0] == free_before
        first_done = True
        assert torch.equal(y, y_ref) and torch.equal(u, u_ref)
        if n * k <= 1104 * 8192:                   # the oracle on the smaller shapes
            yo, uo = O.lora_linear_fwd(case["x"], wq, case["A"], case["B"], 32.0)
            mags = linear_mags(case["x"], wq, case["A"], case["B"], 32.0, np.zeros((t, n), np.uint16))
            check_linear({"y": bits_of(y), "u": f32_of(u)}, {"y": yo, "u": uo}, mags, t, n, k, 0, f"noalloc {t}x{n}x{k}")
            assert O.rel_l2(f32_of(u), uo) <= 1e-4


def test_noalloc_refuses_sizes_beyond_the_scratch(gpu_lib):
    L = gpu_lib
    t, n, k, r = 32768, 1024, 8192, 64
    need = L.fwd_workspace_bytes(t, n, k, r)
    assert need > L.NF4_NOALLOC_SCRATCH_BYTES
    raw = L.raw()
    fake = C.c_void_p(0x10000)
    rc = raw.nf4_lora_linear_fwd_noalloc(fake, fake, n, k, fake, t, fake, fake, r, 32.0, fake, fake, None)
    assert rc == L.NF4_E_SHAPE and "scratch" in L.last_error() and str(need) in L.last_error()
