"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments on the host before anything reaches the device."""

import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nf4lora.h")


@pytest.fixture(scope="module")
def L():
    from nf4_weight_streamed_amd import lib

    return lib


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert "nf4_lora_linear_fwd" in names and "stream_pool_acquire" in names
    raw = L.raw()
    for n in names:
        assert hasattr(raw, n), f"{n} declared in nf4lora.h but not exported"


def test_library_codebook_equals_oracle_bitwise(L):
    """Two independent derivations of the NF4 levels: the library's (C++,
    extended-precision erfc bisection) and the oracle's (fp64 inverse CDF)."""
    got = np.array(L.codebook(), dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), O.nf4_codebook().view(np.uint32))


def test_abi_version(L):
    assert L.abi_version() == 1


FAKE = C.c_void_p(0x10000)      # aligned, never dereferenced: every call below fails validation first


def _err(L, rc, code, needle=None):
    assert rc == code, (rc, L.last_error())
    if needle:
        assert needle in L.last_error()


def test_quantize_validation(L):
    raw = L.raw()
    _err(L, raw.nf4_quantize(FAKE, 7, 4, 64, FAKE, FAKE, None), L.NF4_E_ARG, "in_dtype")
    _err(L, raw.nf4_quantize(FAKE, 0, 4, 63, FAKE, FAKE, None), L.NF4_E_SHAPE, "63")
    _err(L, raw.nf4_quantize(None, 0, 4, 64, FAKE, FAKE, None), L.NF4_E_ARG, "NULL")
    _err(L, raw.nf4_quantize(C.c_void_p(0x10002), 0, 4, 64, FAKE, FAKE, None), L.NF4_E_ARG, "aligned")
    assert raw.nf4_quantize(None, 0, 0, 64, None, None, None) == 0       # rows == 0: no-op
    _err(L, raw.nf4_dequantize(FAKE, FAKE, 4, 100, FAKE, None), L.NF4_E_SHAPE)


def _fwd(raw, N=128, K=128, T=4, r=16, alpha=32.0, codes=FAKE, x=FAKE, ws=FAKE, ws_bytes=1 << 30):
    return raw.nf4_lora_linear_fwd(codes, FAKE, N, K, x, T, FAKE, FAKE, r, alpha, FAKE, FAKE, ws, ws_bytes, None)


def test_linear_fwd_validation(L):
    raw = L.raw()
    _err(L, _fwd(raw, K=100), L.NF4_E_SHAPE, "K=100")
    _err(L, _fwd(raw, N=100), L.NF4_E_SHAPE, "N=100")
    _err(L, _fwd(raw, N=1 << 22), L.NF4_E_SHAPE, "limits")                 # 32-bit tile offsets
    _err(L, _fwd(raw, N=1 << 21, K=1 << 11), L.NF4_E_SHAPE, "limits")      # N*K > 2^31
    _err(L, _fwd(raw, T=(1 << 23) + 1), L.NF4_E_SHAPE, "T <= 2^23")       # tile counts of the 1-D grids
    _err(L, _fwd(raw, N=29568, K=8192, T=1 << 23, ws_bytes=0), L.NF4_E_ARG, "workspace")  # T = 2^23 passes the shape check
    _err(L, _fwd(raw, r=65), L.NF4_E_ARG, "r=65")
    _err(L, _fwd(raw, r=-1), L.NF4_E_ARG)
    _err(L, _fwd(raw, alpha=float("inf")), L.NF4_E_ARG, "alpha")
    _err(L, _fwd(raw, codes=None), L.NF4_E_ARG)
    _err(L, _fwd(raw, x=C.c_void_p(0x10008)), L.NF4_E_ARG, "aligned")
    assert _fwd(raw, T=0) == 0                                              # T == 0: no-op
    need = L.fwd_workspace_bytes(512, 3584, 3584, 16)
    assert need > 0
    _err(L, _fwd(raw, N=3584, K=3584, T=512, ws_bytes=need - 1), L.NF4_E_ARG, str(need))


def test_merge_validation(L):
    raw = L.raw()

    def merge(N=128, K=128, r=16, alpha=32.0, codes=FAKE, A=FAKE, out=FAKE):
        return raw.nf4_merge_lora(codes, FAKE, N, K, A, FAKE, r, alpha, out, None)

    _err(L, merge(K=100), L.NF4_E_SHAPE, "K=100")
    _err(L, merge(N=0), L.NF4_E_SHAPE)
    _err(L, merge(N=1 << 21, K=1 << 11), L.NF4_E_SHAPE, "limits")
    _err(L, merge(r=65), L.NF4_E_ARG, "r=65")
    _err(L, merge(alpha=float("nan")), L.NF4_E_ARG, "alpha")
    _err(L, merge(codes=None), L.NF4_E_ARG, "NULL")
    _err(L, merge(A=None), L.NF4_E_ARG, "NULL")
    _err(L, merge(out=C.c_void_p(0x10008)), L.NF4_E_ARG, "aligned")


def test_dense_linear_validation(L):
    raw = L.raw()

    def fwd(w=FAKE, N=128, K=128, T=4, r=16):
        return raw.nf4_lora_linear_fwd_bf16(w, N, K, FAKE, T, FAKE, FAKE, r, 32.0, FAKE, FAKE, FAKE, 1 << 30, None)

    _err(L, fwd(w=None), L.NF4_E_ARG, "bf16 base")
    _err(L, fwd(w=C.c_void_p(0x10008)), L.NF4_E_ARG, "16-byte")
    _err(L, fwd(K=100), L.NF4_E_SHAPE, "K=100")
    _err(L, fwd(N=1 << 20, K=1 << 11), L.NF4_E_SHAPE, "2^30")      # N*K = 2^31: beyond the dense limit
    _err(L, fwd(N=1 << 16, K=1 << 14), L.NF4_E_SHAPE, "2^30")      # N*K = 2^30: 2^31 bytes, not below 2^31 - 16
    _err(L, fwd(r=65), L.NF4_E_ARG, "r=65")
    assert fwd(T=0) == 0
    rc = raw.nf4_lora_linear_bwd_bf16(None, 128, 128, FAKE, FAKE, FAKE, 4, FAKE, FAKE, 16, 32.0, FAKE, FAKE, FAKE,
                                      FAKE, 1 << 30, None)
    _err(L, rc, L.NF4_E_ARG, "bf16 base")
    # the dense variant never takes the few-token path: its plans differ from the NF4 ones at small T
    assert L.bwd_bf16_workspace_bytes(4, 1024, 1024, 16) != L.bwd_workspace_bytes(4, 1024, 1024, 16)


def test_linear_bwd_validation(L):
    raw = L.raw()
    need = L.bwd_workspace_bytes(256, 1024, 1024, 16)
    assert need >= 256 * 16 * 4
    rc = raw.nf4_lora_linear_bwd(FAKE, FAKE, 1024, 1024, FAKE, FAKE, FAKE, 256, FAKE, FAKE, 16, 32.0, FAKE,
                                 FAKE, FAKE, FAKE, need - 256, None)
    _err(L, rc, L.NF4_E_ARG, "workspace")
    rc = raw.nf4_lora_linear_bwd(FAKE, FAKE, 1024, 1024, None, FAKE, FAKE, 256, FAKE, FAKE, 16, 32.0, FAKE,
                                 FAKE, FAKE, FAKE, need, None)
    _err(L, rc, L.NF4_E_ARG, "needs x")


def test_workspace_sizes_are_pure_functions_of_shape(L):
    a = [L.fwd_workspace_bytes(512, n, k, 16) for n, k in ((3584, 3584), (512, 3584), (18944, 3584), (3584, 18944))]
    b = [L.fwd_workspace_bytes(512, n, k, 16) for n, k in ((3584, 3584), (512, 3584), (18944, 3584), (3584, 18944))]
    assert a == b
    assert all(v % 256 == 0 for v in a)
    assert L.fwd_workspace_bytes(512, 3584, 100, 16) == 0                   # invalid shape -> 0


def test_pool_validation(L):
    raw = L.raw()
    blocks = (L.HostBlock * 2)()
    blocks[0].host, blocks[0].bytes = 0x20000, 4096
    blocks[1].host, blocks[1].bytes = 0x30000, 9000
    h = C.c_void_p()
    rc = raw.stream_pool_create(blocks, 2, C.c_void_p(0x40000), 8192, 2, FAKE, C.byref(h))
    _err(L, rc, L.NF4_E_OOM, "9000")
    assert "8192" in L.last_error()
    rc = raw.stream_pool_create(blocks, 2, C.c_void_p(0x40000), 1000, 2, FAKE, C.byref(h))
    _err(L, rc, L.NF4_E_ARG, "256")
    rc = raw.stream_pool_create(blocks, 2, C.c_void_p(0x40000), 16384, 2, None, C.byref(h))
    _err(L, rc, L.NF4_E_ARG, "copy")
    rc = raw.stream_pool_prefetch(None, 0)
    _err(L, rc, L.NF4_E_ARG, "NULL pool")
    rc = raw.stream_pool_streams(None, None)
    _err(L, rc, L.NF4_E_ARG, "NULL")
    n = C.c_int(-1)
    rc = raw.stream_pool_timing_spans(None, None, 0, C.byref(n))
    _err(L, rc, L.NF4_E_ARG, "need pool")


def test_block_layout(L):
    """nf4_block_layout: pieces in layer, projection, codes-then-absmax order, each
    256-byte aligned and exactly as long as its tensor; L layers = L one-layer slabs."""
    shapes = [(3584, 3584), (512, 3584), (512, 3584), (3584, 3584), (18944, 3584), (18944, 3584), (3584, 18944)]
    one, one_bytes = L.block_layout(shapes, 1)
    four, four_bytes = L.block_layout(shapes, 4)
    assert one_bytes % 256 == 0 and four_bytes == 4 * one_bytes
    for li in range(4):
        assert [tuple(o - li * one_bytes for o in p) for p in four[li]] == one[0]
    end = 0
    for (n, k), (c, a) in zip(shapes, one[0]):
        assert c % 256 == 0 and a % 256 == 0 and c >= end
        assert a >= c + n * k // 2 and a - (c + n * k // 2) < 256
        end = a + n * (k // 64) * 4
    assert one_bytes - end < 256
    assert one_bytes == sum(-(-n * k // 2 // 256) * 256 + -(-n * (k // 64) * 4 // 256) * 256 for n, k in shapes)
    dense, dense_bytes = L.block_layout(shapes, 2, dense=True)
    assert dense_bytes == 2 * sum(-(-n * k * 2 // 256) * 256 for n, k in shapes)
    assert all(p[1] == 0 for layer in dense for p in layer)
    raw = L.raw()
    bad = (C.c_int64 * 2)(128, 100)
    out = C.c_size_t()
    _err(L, raw.nf4_block_layout(bad, 1, 1, 0, None, C.byref(out)), L.NF4_E_SHAPE, "K=100")
    _err(L, raw.nf4_block_layout(bad, 1, 0, 0, None, C.byref(out)), L.NF4_E_ARG, "layers")
