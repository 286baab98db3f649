"""The measurement probes behind bench.py's denominators (instrumentation, not the
method): each is checked for doing the work it is timed on."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes,workgroups", [(16, 1), (4096 + 48, 3), ((1 << 20) + 16 * 37, 7), (1 << 22, 64)])
def test_read_probe_reads_every_word(gpu_lib, nbytes, workgroups):
    """The XOR of the probe's outputs equals the XOR of all 32-bit words of the buffer,
    so every word was loaded (ragged tails past the unrolled loop included)."""
    g = np.random.default_rng(nbytes)
    words = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    out = torch.full((256 * workgroups,), -1, dtype=torch.int32, device="cuda")
    gpu_lib.probe_read(src, out, workgroups)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))


@pytest.mark.parametrize("depth", [4, 8, 16, 32])
@pytest.mark.parametrize("nontemporal", [False, True])
@pytest.mark.parametrize("nbytes,workgroups", [(16 * 3, 2), ((1 << 20) + 16 * 37, 5), (1 << 22, 256)])
def test_read_probe_depth_reads_every_word(gpu_lib, depth, nontemporal, nbytes, workgroups):
    """Every depth and load kind of the swept probe loads every word (XOR check)."""
    g = np.random.default_rng(nbytes + depth)
    words = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    out = torch.full((256 * workgroups,), -1, dtype=torch.int32, device="cuda")
    gpu_lib.probe_read_depth(src, out, workgroups, depth, nontemporal)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert int(got) == int(np.bitwise_xor.reduce(words))


def test_read_probe_rejects_bad_arguments(gpu_lib):
    src = torch.zeros(5, dtype=torch.int32, device="cuda")  # 20 bytes: not a multiple of 16
    out = torch.zeros(256, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        gpu_lib.probe_read(src, out, 1)
    ok = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(RuntimeError):
        gpu_lib.probe_read_depth(ok, out, 1, 6)  # depth 4, 8, 16 or 32 only


def test_mfma_probe_writes_every_wave(gpu_lib):
    out = torch.full((4 * 8,), float("nan"), dtype=torch.float32, device="cuda")
    gpu_lib.probe_mfma(out, 8, 3)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
