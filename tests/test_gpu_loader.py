"""The streamed NF4 loader ("Poros on consumer GPUs", "OOM playbook": the loader keeps
GPU memory bounded at any model size and its bytes are identical to the standard
load): host-resident bf16 weights are copied to the device one projection at a time,
quantised by nf4_quantize and copied into the pinned host buffer. Its bytes are
compared with the oracle's quantisation of each whole weight tensor, and the device
memory it held is bounded by one projection's bf16 weight plus its NF4 bytes."""

import numpy as np
import pytest
import torch

import oracle as O
import synthetic_inputs as S

pytestmark = pytest.mark.gpu
PROJS = ("q", "k", "v", "o", "gate", "up", "down")


@pytest.fixture(scope="module")
def ST(gpu_lib):
    from nf4_weight_streamed_amd import stack

    return stack


def _host_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _check_against_oracle(base, weights, layers):
    for layer in layers:
        host, start = base.layers[layer].numpy(), 0
        for name in PROJS:
            n, k = base.dims.shapes()[name]
            c_off, a_off = base.layer_layout[0][name]
            codes, absmax = O.quantize(O.bf16_bits_to_f64(weights[(layer, name)]).astype(np.float32))
            got_c = host[start + c_off:start + c_off + n * k // 2].reshape(n, k // 2)
            got_a = host[start + a_off:start + a_off + n * (k // 64) * 4].view(np.float32).reshape(n, k // 64)
            assert np.array_equal(got_c, codes), (layer, name, "codes")
            assert np.array_equal(got_a.view(np.uint32), absmax.view(np.uint32)), (layer, name, "absmax")


def test_loader_bytes_equal_whole_tensor_quantise_tiny(ST):
    dims = ST.StackDims(hidden=128, q=128, kv=32, inter=256, head_dim=32)
    L = 3
    weights = {(l, p): S.weight(*dims.shapes()[p], proj=p, layer=l) for l in range(L) for p in PROJS}
    host_fn = lambda l, p, n, k: _host_bf16(weights[(l, p)])
    base = ST.HostNF4Base(dims, L, 2, host_fn)
    _check_against_oracle(base, weights, range(L))
    # the same weights handed over on the device give the same bytes
    dev = ST.HostNF4Base(dims, L, 2, lambda l, p, n, k: host_fn(l, p, n, k).cuda())
    for l in range(L):
        for name in PROJS:
            for off, size in zip(base.layer_layout[0][name], _piece_sizes(dims, name)):
                a = base.layer_bytes_of(l)[off:off + size]
                assert torch.equal(a, dev.layer_bytes_of(l)[off:off + size]), (l, name)


def _piece_sizes(dims, name):
    n, k = dims.shapes()[name]
    return n * k // 2, n * (k // 64) * 4


def test_loader_qwen7b_layer_and_device_residency(ST):
    """One Qwen2.5-7B-shaped layer from host-resident bf16 weights: every projection's
    bytes equal the oracle's whole-tensor quantisation, and the device held at most the
    largest projection's bf16 weight plus its NF4 bytes during the load."""
    dims, _ = ST.QWEN25["7b"]
    print("7B layer: drawing host weights", flush=True)
    weights = {(0, p): S.weight(*dims.shapes()[p], proj=p) for p in PROJS}
    torch.cuda.empty_cache()
    base = ST.HostNF4Base(dims, 1, 1, lambda l, p, n, k: _host_bf16(weights[(l, p)]))
    print(f"7B layer: loaded, stats {base.load_stats}", flush=True)
    _check_against_oracle(base, weights, [0])
    base.close()
    max_w = max(n * k for n, k in dims.shapes().values())
    bound = max_w * 2 + max_w // 2 + max_w // 16 + (1 << 20)
    peak = base.load_stats["peak_device_bytes"]
    assert peak <= bound, (peak, bound)
    assert peak < 2 << 30
