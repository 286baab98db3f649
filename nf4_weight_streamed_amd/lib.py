"""ctypes binding of libnf4lora.so (include/nf4lora.h): argument marshalling only.

Every computation runs in the HIP library; this module checks tensor
placement/dtype/shape, allocates outputs with torch (device memory is the only
thing torch provides here) and passes raw pointers plus the current stream.
There is no fallback: if the library is missing, importing this module raises.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnf4lora.so")

NF4_OK = 0
NF4_E_ARG, NF4_E_SHAPE, NF4_E_OOM, NF4_E_HIP, NF4_E_STATE, NF4_E_BUSY = -1, -2, -3, -4, -5, -6
NF4_BLOCK = 64
NF4_MAX_RANK = 64
NF4_DTYPE_BF16, NF4_DTYPE_F32 = 0, 1
_CODE_NAMES = {-1: "NF4_E_ARG", -2: "NF4_E_SHAPE", -3: "NF4_E_OOM", -4: "NF4_E_HIP", -5: "NF4_E_STATE",
               -6: "NF4_E_BUSY"}


class Nf4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_CODE_NAMES.get(code, code)}: {msg}")
        self.code = code


class HostBlock(C.Structure):
    _fields_ = [("host", C.c_void_p), ("bytes", C.c_size_t)]


class PoolTiming(C.Structure):
    _fields_ = [("copy_ms", C.c_double), ("stall_ms", C.c_double), ("copies", C.c_uint64),
                ("acquires", C.c_uint64), ("host_ms", C.c_double), ("host_max_ms", C.c_double),
                ("host_copy_ms", C.c_double), ("host_record_ms", C.c_double), ("host_wait_ms", C.c_double),
                ("host_sync_ms", C.c_double)]


class PoolSpan(C.Structure):
    _fields_ = [("kind", C.c_int), ("block", C.c_int), ("part", C.c_int), ("reserved", C.c_int),
                ("start_ms", C.c_double), ("end_ms", C.c_double), ("host_at_ms", C.c_double),
                ("host_call_ms", C.c_double)]


class PoolStats(C.Structure):
    _fields_ = [("bytes_copied", C.c_uint64), ("copies", C.c_uint64), ("hits", C.c_uint64),
                ("misses", C.c_uint64), ("evictions", C.c_uint64)]


def _load() -> C.CDLL:
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m nf4_weight_streamed_amd.build` "
                           "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    vp, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int, C.c_float, C.c_size_t
    sig = {
        "nf4_last_error": (C.c_char_p, []),
        "nf4_abi_version": (i32, []),
        "nf4_codebook": (i32, [C.POINTER(C.c_float)]),
        "nf4_quantize": (i32, [vp, i32, i64, i64, vp, vp, vp]),
        "nf4_dequantize": (i32, [vp, vp, i64, i64, vp, vp]),
        "nf4_merge_lora": (i32, [vp, vp, i64, i64, vp, vp, i32, f32, vp, vp]),
        "nf4_lora_linear_fwd_workspace": (sz, [i64, i64, i64, i32]),
        "nf4_lora_linear_fwd": (i32, [vp, vp, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "nf4_lora_linear_bwd_workspace": (sz, [i64, i64, i64, i32]),
        "nf4_lora_linear_fwd_noalloc": (i32, [vp, vp, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp, vp]),
        "nf4_lora_linear_fwd_bf16_workspace": (sz, [i64, i64, i64, i32]),
        "nf4_lora_linear_fwd_bf16": (i32, [vp, i64, i64, vp, i64, vp, vp, i32, f32, vp, vp, vp, sz, vp]),
        "nf4_lora_linear_bwd_bf16_workspace": (sz, [i64, i64, i64, i32]),
        "nf4_lora_linear_bwd_bf16": (i32, [vp, i64, i64, vp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "nf4_lora_linear_bwd": (i32, [vp, vp, i64, i64, vp, vp, vp, i64, vp, vp, i32, f32, vp, vp, vp, vp, sz, vp]),
        "nf4_profile_next_gemm": (i32, [vp, vp]),
        "nf4_probe_mfma": (i32, [vp, i32, i32, vp]),
        "nf4_probe_read": (i32, [vp, C.c_size_t, vp, i32, vp]),
        "nf4_probe_read_depth": (i32, [vp, C.c_size_t, vp, i32, i32, i32, vp]),
        "nf4_rmsnorm_fwd": (i32, [vp, i64, i64, f32, vp, vp, vp]),
        "nf4_rmsnorm_bwd": (i32, [vp, vp, vp, vp, i64, i64, vp, vp]),
        "nf4_add_bf16": (i32, [vp, vp, vp, i64, vp, vp]),
        "nf4_silu_mul_fwd": (i32, [vp, vp, i64, vp, vp]),
        "nf4_silu_mul_bwd": (i32, [vp, vp, vp, i64, vp, vp, vp]),
        "nf4_repeat_kv_fwd": (i32, [vp, i64, i64, i64, i64, vp, vp]),
        "nf4_repeat_kv_bwd": (i32, [vp, i64, i64, i64, i64, vp, vp]),
        "stream_pool_create": (i32, [C.POINTER(HostBlock), i32, vp, sz, i32, vp, C.POINTER(vp)]),
        "stream_pool_prefetch": (i32, [vp, i32]),
        "stream_pool_acquire": (i32, [vp, i32, vp, C.POINTER(vp)]),
        "stream_pool_release": (i32, [vp, i32, vp]),
        "stream_pool_stats": (i32, [vp, C.POINTER(PoolStats)]),
        "stream_pool_slot_block": (i32, [vp, i32, C.POINTER(i32)]),
        "stream_pool_destroy": (i32, [vp]),
        "stream_pool_create_parts": (i32, [C.POINTER(HostBlock), C.POINTER(i32), i32, vp, sz, i32, vp,
                                           C.POINTER(vp)]),
        "stream_pool_set_order": (i32, [vp, i32]),
        "stream_pool_release_part": (i32, [vp, i32, i32, vp]),
        "stream_pool_acquire_deferred": (i32, [vp, i32, vp, C.POINTER(vp)]),
        "stream_pool_wait_part": (i32, [vp, i32, i32, vp]),
        "stream_pool_set_max_ahead": (i32, [vp, i32]),
        "stream_pool_timing_enable": (i32, [vp, i32]),
        "stream_pool_streams": (i32, [C.POINTER(vp), C.POINTER(vp)]),
        "stream_pool_timing_collect": (i32, [vp, C.POINTER(PoolTiming)]),
        "stream_pool_timing_spans": (i32, [vp, C.POINTER(PoolSpan), i32, C.POINTER(i32)]),
        "nf4_block_layout": (i32, [C.POINTER(C.c_int64), i32, i32, i32, C.POINTER(C.c_size_t),
                                   C.POINTER(C.c_size_t)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def raw() -> C.CDLL:
    """The loaded CDLL (for tests that call the C ABI directly)."""
    return _lib


def last_error() -> str:
    return _lib.nf4_last_error().decode()


def _check(rc: int) -> None:
    if rc != NF4_OK:
        raise Nf4Error(rc, last_error())


def _stream(stream) -> C.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t) -> C.c_void_p | None:
    return None if t is None else C.c_void_p(t.data_ptr())


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def abi_version() -> int:
    return _lib.nf4_abi_version()


def profile_next_gemm(start_event, stop_event) -> None:
    """Record two hipEvent_t handles (ints) around the next call's fused GEMM kernel."""
    _check(_lib.nf4_profile_next_gemm(C.c_void_p(start_event), C.c_void_p(stop_event)))


def probe_mfma(out, workgroups: int, iters: int, stream=None) -> None:
    """Launch the bf16 MFMA-rate probe (32768 * 8 * iters FLOP per wave, 4 waves per
    workgroup); out: device fp32 tensor of >= 4 * workgroups entries."""
    if out.dtype != torch.float32 or not out.is_cuda or out.numel() < 4 * workgroups:
        raise ValueError("probe_mfma: out must be a device fp32 tensor of >= 4 * workgroups entries")
    _check(_lib.nf4_probe_mfma(_ptr(out), int(workgroups), int(iters), _stream(stream)))


def probe_read(src, out, workgroups: int, stream=None) -> None:
    """Launch the HBM read-rate probe over the device tensor `src` (its bytes, a multiple
    of 16); `out` = device int32 tensor of >= 256 * workgroups entries."""
    nbytes = src.numel() * src.element_size()
    if not src.is_cuda or not out.is_cuda or out.dtype != torch.int32 or out.numel() < 256 * workgroups:
        raise ValueError("probe_read: src and out must be device tensors, out int32 with >= 256 * workgroups entries")
    _check(_lib.nf4_probe_read(_ptr(src), C.c_size_t(nbytes), _ptr(out), int(workgroups), _stream(stream)))


def probe_read_depth(src, out, workgroups: int, depth: int, nontemporal: bool = False, stream=None) -> None:
    """The read probe with `depth` loads in flight per thread (nf4_probe_read_depth)."""
    nbytes = src.numel() * src.element_size()
    if not (src.is_cuda and out.is_cuda and out.dtype == torch.int32 and out.numel() >= 256 * workgroups):
        raise ValueError("probe_read_depth: src and out must be device tensors, out int32 with >= 256 * workgroups "
                         "entries")
    _check(_lib.nf4_probe_read_depth(_ptr(src), C.c_size_t(nbytes), _ptr(out), int(workgroups), int(depth),
                                     int(bool(nontemporal)), _stream(stream)))


def codebook() -> list:
    out = (C.c_float * 16)()
    _check(_lib.nf4_codebook(out))
    return list(out)


def quantize(w: torch.Tensor, codes: torch.Tensor | None = None, absmax: torch.Tensor | None = None, stream=None):
    """NF4-quantise a [N, K] bf16 or float32 device matrix -> (codes uint8 [N, K/2], absmax float32 [N, K/64])."""
    if w.dim() != 2:
        raise ValueError("w must be 2-D")
    n, k = w.shape
    dtype = {torch.bfloat16: NF4_DTYPE_BF16, torch.float32: NF4_DTYPE_F32}.get(w.dtype)
    if dtype is None:
        raise TypeError("w must be bfloat16 or float32")
    _need(w, "w", w.dtype, (n, k))
    if codes is None:
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    if absmax is None:
        absmax = torch.empty((n, k // NF4_BLOCK), dtype=torch.float32, device=w.device)
    _need(codes, "codes", torch.uint8, (n, k // 2))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    _check(_lib.nf4_quantize(_ptr(w), dtype, n, k, _ptr(codes), _ptr(absmax), _stream(stream)))
    return codes, absmax


def dequantize(codes: torch.Tensor, absmax: torch.Tensor, out: torch.Tensor | None = None, stream=None):
    n, kh = codes.shape
    k = kh * 2
    _need(codes, "codes", torch.uint8, (n, kh))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _need(out, "out", torch.bfloat16, (n, k))
    _check(_lib.nf4_dequantize(_ptr(codes), _ptr(absmax), n, k, _ptr(out), _stream(stream)))
    return out


def merge_lora(codes: torch.Tensor, absmax: torch.Tensor, A, B, alpha: float, out: torch.Tensor | None = None,
               stream=None):
    """Dense merged weight RNbf(W + RN32((alpha/r) . B.A)) [N, K] bf16 (merge_and_unload)."""
    n, kh = codes.shape
    k = kh * 2
    r = 0 if A is None else A.shape[0]
    _need(codes, "codes", torch.uint8, (n, kh))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    if r > 0:
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
    if out is None:
        out = torch.empty((n, k), dtype=torch.bfloat16, device=codes.device)
    _need(out, "out", torch.bfloat16, (n, k))
    _check(_lib.nf4_merge_lora(_ptr(codes), _ptr(absmax), n, k, _ptr(A) if r else None, _ptr(B) if r else None, r,
                               float(alpha), _ptr(out), _stream(stream)))
    return out


def fwd_workspace_bytes(T: int, N: int, K: int, r: int) -> int:
    return int(_lib.nf4_lora_linear_fwd_workspace(T, N, K, r))


def bwd_workspace_bytes(T: int, N: int, K: int, r: int) -> int:
    return int(_lib.nf4_lora_linear_bwd_workspace(T, N, K, r))


def workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """A 256-byte aligned device buffer of at least nbytes (torch's allocator aligns to 512)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def lora_linear_fwd(codes, absmax, x, A, B, alpha: float, y=None, u=None, ws=None, stream=None):
    """y = RNbf(x.W^T + (alpha/r).(x.A^T).B^T), u = x.A^T. Returns (y, u)."""
    n, kh = codes.shape
    k = kh * 2
    t = x.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(codes, "codes", torch.uint8, (n, kh))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    _need(x, "x", torch.bfloat16, (t, k))
    if r:
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
    if y is None:
        y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (t, n))
    if r and u is None:
        u = torch.empty((t, r), dtype=torch.float32, device=x.device)
    if r:
        _need(u, "u", torch.float32, (t, r))
    need = fwd_workspace_bytes(t, n, k, r)
    if ws is None and need:
        ws = workspace(need, x.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.nf4_lora_linear_fwd(_ptr(codes), _ptr(absmax), n, k, _ptr(x), t, _ptr(A), _ptr(B), r,
                                    float(alpha), _ptr(y), _ptr(u), _ptr(ws), ws_bytes, _stream(stream)))
    return y, u


NF4_NOALLOC_SCRATCH_BYTES = 64 << 20


def lora_linear_fwd_noalloc(codes, absmax, x, A, B, alpha: float, y, u=None, stream=None):
    """The forward with the library's own device scratch as workspace
    (nf4_lora_linear_fwd_noalloc): y and u are caller-provided; nothing is allocated."""
    n, kh = codes.shape
    k = kh * 2
    t = x.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(codes, "codes", torch.uint8, (n, kh))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    _need(x, "x", torch.bfloat16, (t, k))
    _need(y, "y", torch.bfloat16, (t, n))
    if r:
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
        _need(u, "u", torch.float32, (t, r))
    _check(_lib.nf4_lora_linear_fwd_noalloc(_ptr(codes), _ptr(absmax), n, k, _ptr(x), t, _ptr(A), _ptr(B), r,
                                            float(alpha), _ptr(y), _ptr(u), _stream(stream)))
    return y, u


def lora_linear_bwd(codes, absmax, x, u, dy, A, B, alpha: float, dx=None, dA=None, dB=None, ws=None,
                    need_dx: bool = True, stream=None):
    """Backward: returns (dx or None, dA, dB); no gradient of the frozen base exists."""
    n, kh = codes.shape
    k = kh * 2
    t = dy.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(codes, "codes", torch.uint8, (n, kh))
    _need(absmax, "absmax", torch.float32, (n, k // NF4_BLOCK))
    _need(dy, "dy", torch.bfloat16, (t, n))
    if r:
        _need(x, "x", torch.bfloat16, (t, k))
        _need(u, "u", torch.float32, (t, r))
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
        if dA is None:
            dA = torch.empty((r, k), dtype=torch.float32, device=dy.device)
        if dB is None:
            dB = torch.empty((n, r), dtype=torch.float32, device=dy.device)
        _need(dA, "dA", torch.float32, (r, k))
        _need(dB, "dB", torch.float32, (n, r))
    if need_dx and dx is None:
        dx = torch.empty((t, k), dtype=torch.bfloat16, device=dy.device)
    if dx is not None:
        _need(dx, "dx", torch.bfloat16, (t, k))
    need = bwd_workspace_bytes(t, n, k, r)
    if ws is None:
        ws = workspace(need, dy.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.nf4_lora_linear_bwd(_ptr(codes), _ptr(absmax), n, k, _ptr(x), _ptr(u), _ptr(dy), t, _ptr(A),
                                    _ptr(B), r, float(alpha), _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes,
                                    _stream(stream)))
    return dx, dA, dB


def lora_linear_fwd_bf16(w, x, A, B, alpha: float, y=None, u=None, ws=None, stream=None):
    """The linear forward with a dense bf16 base w [N, K] (the "bf16_bitwise" mode). Returns (y, u)."""
    n, k = w.shape
    t = x.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(w, "w", torch.bfloat16, (n, k))
    _need(x, "x", torch.bfloat16, (t, k))
    if r:
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
    if y is None:
        y = torch.empty((t, n), dtype=torch.bfloat16, device=x.device)
    _need(y, "y", torch.bfloat16, (t, n))
    if r and u is None:
        u = torch.empty((t, r), dtype=torch.float32, device=x.device)
    if r:
        _need(u, "u", torch.float32, (t, r))
    need = int(_lib.nf4_lora_linear_fwd_bf16_workspace(t, n, k, r))
    if ws is None and need:
        ws = workspace(need, x.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.nf4_lora_linear_fwd_bf16(_ptr(w), n, k, _ptr(x), t, _ptr(A), _ptr(B), r, float(alpha), _ptr(y),
                                         _ptr(u), _ptr(ws), ws_bytes, _stream(stream)))
    return y, u


def lora_linear_bwd_bf16(w, x, u, dy, A, B, alpha: float, dx=None, dA=None, dB=None, ws=None, need_dx: bool = True,
                         stream=None):
    """The linear backward with a dense bf16 base w [N, K]: returns (dx or None, dA, dB)."""
    n, k = w.shape
    t = dy.shape[0]
    r = 0 if A is None else A.shape[0]
    _need(w, "w", torch.bfloat16, (n, k))
    _need(dy, "dy", torch.bfloat16, (t, n))
    if r:
        _need(x, "x", torch.bfloat16, (t, k))
        _need(u, "u", torch.float32, (t, r))
        _need(A, "A", torch.bfloat16, (r, k))
        _need(B, "B", torch.bfloat16, (n, r))
        if dA is None:
            dA = torch.empty((r, k), dtype=torch.float32, device=dy.device)
        if dB is None:
            dB = torch.empty((n, r), dtype=torch.float32, device=dy.device)
        _need(dA, "dA", torch.float32, (r, k))
        _need(dB, "dB", torch.float32, (n, r))
    if need_dx and dx is None:
        dx = torch.empty((t, k), dtype=torch.bfloat16, device=dy.device)
    if dx is not None:
        _need(dx, "dx", torch.bfloat16, (t, k))
    if ws is None:
        ws = workspace(int(_lib.nf4_lora_linear_bwd_bf16_workspace(t, n, k, r)), dy.device)
    ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.nf4_lora_linear_bwd_bf16(_ptr(w), n, k, _ptr(x), _ptr(u), _ptr(dy), t, _ptr(A), _ptr(B), r,
                                         float(alpha), _ptr(dx), _ptr(dA), _ptr(dB), _ptr(ws), ws_bytes,
                                         _stream(stream)))
    return dx, dA, dB


def fwd_bf16_workspace_bytes(T: int, N: int, K: int, r: int) -> int:
    return int(_lib.nf4_lora_linear_fwd_bf16_workspace(T, N, K, r))


def bwd_bf16_workspace_bytes(T: int, N: int, K: int, r: int) -> int:
    return int(_lib.nf4_lora_linear_bwd_bf16_workspace(T, N, K, r))


# ---------------------------------------------------------------- stack glue (bf16 device tensors)

def _bf16_like(t, shape=None):
    return torch.empty(shape if shape is not None else t.shape, dtype=torch.bfloat16, device=t.device)


def rmsnorm_fwd(h, eps: float = 1e-6, out=None, rstd=None, stream=None):
    t, hd = h.shape
    _need(h, "h", torch.bfloat16, (t, hd))
    out = _bf16_like(h) if out is None else out
    rstd = torch.empty(t, dtype=torch.float32, device=h.device) if rstd is None else rstd
    _need(out, "out", torch.bfloat16, (t, hd))
    _need(rstd, "rstd", torch.float32, (t,))
    _check(_lib.nf4_rmsnorm_fwd(_ptr(h), t, hd, float(eps), _ptr(out), _ptr(rstd), _stream(stream)))
    return out, rstd


def rmsnorm_bwd(h, rstd, dy, dres=None, out=None, stream=None):
    t, hd = h.shape
    _need(h, "h", torch.bfloat16, (t, hd))
    _need(rstd, "rstd", torch.float32, (t,))
    _need(dy, "dy", torch.bfloat16, (t, hd))
    if dres is not None:
        _need(dres, "dres", torch.bfloat16, (t, hd))
    out = _bf16_like(h) if out is None else out
    _need(out, "out", torch.bfloat16, (t, hd))
    _check(_lib.nf4_rmsnorm_bwd(_ptr(h), _ptr(rstd), _ptr(dy), _ptr(dres), t, hd, _ptr(out), _stream(stream)))
    return out


def add_bf16(a, b, c=None, out=None, stream=None):
    for name, t in (("a", a), ("b", b)) + ((("c", c),) if c is not None else ()):
        _need(t, name, torch.bfloat16, tuple(a.shape))
    out = _bf16_like(a) if out is None else out
    _need(out, "out", torch.bfloat16, tuple(a.shape))
    _check(_lib.nf4_add_bf16(_ptr(a), _ptr(b), _ptr(c), a.numel(), _ptr(out), _stream(stream)))
    return out


def silu_mul_fwd(gate, up, out=None, stream=None):
    _need(up, "up", torch.bfloat16, tuple(gate.shape))
    _need(gate, "gate", torch.bfloat16, tuple(gate.shape))
    out = _bf16_like(gate) if out is None else out
    _need(out, "out", torch.bfloat16, tuple(gate.shape))
    _check(_lib.nf4_silu_mul_fwd(_ptr(gate), _ptr(up), gate.numel(), _ptr(out), _stream(stream)))
    return out


def silu_mul_bwd(gate, up, dm, dgate=None, dup=None, stream=None):
    for name, t in (("gate", gate), ("up", up), ("dm", dm)):
        _need(t, name, torch.bfloat16, tuple(gate.shape))
    dgate = _bf16_like(gate) if dgate is None else dgate
    dup = _bf16_like(gate) if dup is None else dup
    _check(_lib.nf4_silu_mul_bwd(_ptr(gate), _ptr(up), _ptr(dm), gate.numel(), _ptr(dgate), _ptr(dup),
                                 _stream(stream)))
    return dgate, dup


def repeat_kv_fwd(v, q: int, head_dim: int, out=None, stream=None):
    t, kv = v.shape
    _need(v, "v", torch.bfloat16, (t, kv))
    out = _bf16_like(v, (t, q)) if out is None else out
    _need(out, "out", torch.bfloat16, (t, q))
    _check(_lib.nf4_repeat_kv_fwd(_ptr(v), t, q, kv, head_dim, _ptr(out), _stream(stream)))
    return out


def repeat_kv_bwd(da, kv: int, head_dim: int, out=None, stream=None):
    t, q = da.shape
    _need(da, "da", torch.bfloat16, (t, q))
    out = _bf16_like(da, (t, kv)) if out is None else out
    _need(out, "out", torch.bfloat16, (t, kv))
    _check(_lib.nf4_repeat_kv_bwd(_ptr(da), t, q, kv, head_dim, _ptr(out), _stream(stream)))
    return out


def block_layout(shapes, layers: int, dense: bool = False):
    """nf4_block_layout: ([layer][proj] = (codes or weight offset, absmax offset)), slab bytes)
    for the projections' (N, K) `shapes` in order."""
    n_proj = len(shapes)
    arr = (C.c_int64 * (2 * n_proj))(*[int(v) for nk in shapes for v in nk])
    offs = (C.c_size_t * (2 * n_proj * layers))()
    total = C.c_size_t()
    _check(_lib.nf4_block_layout(arr, n_proj, int(layers), int(bool(dense)), offs, C.byref(total)))
    table = [[(offs[(l * n_proj + j) * 2], offs[(l * n_proj + j) * 2 + 1]) for j in range(n_proj)]
             for l in range(layers)]
    return table, total.value


_HIP = None


def _hip_runtime() -> C.CDLL:
    """The HIP runtime torch has loaded (same soname): for page-locked host memory."""
    global _HIP
    if _HIP is None:
        _HIP = C.CDLL("libamdhip64.so.7")
        _HIP.hipHostMalloc.argtypes = [C.POINTER(C.c_void_p), C.c_size_t, C.c_uint]
        _HIP.hipHostFree.argtypes = [C.c_void_p]
    return _HIP


def pinned_empty(nbytes: int) -> torch.Tensor:
    """A uint8 CPU tensor over page-locked host memory of exactly `nbytes` bytes
    (hipHostMalloc; torch's pinned allocator rounds every request up to a power of
    two). The memory belongs to the buffer object the tensor wraps and is freed
    (hipHostFree, which waits for the device) once the last view of it is gone."""
    hip = _hip_runtime()
    p = C.c_void_p()
    nbytes = max(int(nbytes), 1)
    rc = hip.hipHostMalloc(C.byref(p), C.c_size_t(nbytes), 0)
    if rc != 0 or not p.value:
        raise Nf4Error(NF4_E_OOM, f"hipHostMalloc of {nbytes} bytes of pinned host memory failed (hipError {rc})")
    addr = p.value

    class _PinnedOwner(C.c_uint8 * nbytes):
        # the free function and address are bound now: at interpreter exit the module's
        # globals may already be gone when the last view dies
        def __del__(self, _free=hip.hipHostFree, _addr=C.c_void_p(addr)):
            _free(_addr)

    return torch.frombuffer(_PinnedOwner.from_address(addr), dtype=torch.uint8)


_POOL_STREAMS: dict = {}


def pool_streams():
    """The current device's (compute, copy) stream pair for streamed passes
    (stream_pool_streams): created back to back so that they sit on different
    hardware queues, kept for the life of the process."""
    dev = torch.cuda.current_device()
    if dev not in _POOL_STREAMS:
        c, k = C.c_void_p(), C.c_void_p()
        _check(_lib.stream_pool_streams(C.byref(c), C.byref(k)))
        _POOL_STREAMS[dev] = (torch.cuda.ExternalStream(c.value), torch.cuda.ExternalStream(k.value))
    return _POOL_STREAMS[dev]


class StreamPool:
    """Thin handle over stream_pool_*: pinned host blocks -> device slots on a copy stream.

    host_blocks: one pinned uint8 tensor per block, or (with part_begin) one per part,
    block b being parts part_begin[b] .. part_begin[b + 1] - 1 (stream_pool_create_parts)."""

    def __init__(self, host_blocks, device_slab: torch.Tensor, slot_bytes: int, n_slots: int, copy_stream,
                 part_begin=None):
        arr = (HostBlock * len(host_blocks))()
        for i, hb in enumerate(host_blocks):
            if hb.device.type != "cpu" or not hb.is_pinned():
                raise ValueError(f"host range {i} must be pinned host memory")
            arr[i].host = hb.data_ptr()
            arr[i].bytes = hb.numel() * hb.element_size()
        self._blocks = list(host_blocks)     # keep the ranges alive
        self._slab = device_slab
        self._copy = copy_stream
        h = C.c_void_p()
        if part_begin is None:
            _check(_lib.stream_pool_create(arr, len(host_blocks), _ptr(device_slab), slot_bytes, n_slots,
                                           _stream(copy_stream), C.byref(h)))
        else:
            pb = (C.c_int * len(part_begin))(*[int(v) for v in part_begin])
            _check(_lib.stream_pool_create_parts(arr, pb, len(part_begin) - 1, _ptr(device_slab), slot_bytes, n_slots,
                                                 _stream(copy_stream), C.byref(h)))
        self._h = h
        self.slot_bytes = slot_bytes
        self.n_slots = n_slots

    def prefetch(self, block: int) -> None:
        _check(_lib.stream_pool_prefetch(self._h, block))

    def set_order(self, descending: bool) -> None:
        _check(_lib.stream_pool_set_order(self._h, int(bool(descending))))

    def acquire(self, block: int, stream=None) -> int:
        dev = C.c_void_p()
        _check(_lib.stream_pool_acquire(self._h, block, _stream(stream), C.byref(dev)))
        return dev.value

    def acquire_deferred(self, block: int, stream=None) -> int:
        """acquire without the wait for the copy: wait_part before reading each part."""
        dev = C.c_void_p()
        _check(_lib.stream_pool_acquire_deferred(self._h, block, _stream(stream), C.byref(dev)))
        return dev.value

    def wait_part(self, block: int, part: int, stream=None) -> None:
        _check(_lib.stream_pool_wait_part(self._h, block, part, _stream(stream)))

    def set_max_ahead(self, n: int) -> None:
        """Host blocks at release until the release n earlier has completed (0: no bound)."""
        _check(_lib.stream_pool_set_max_ahead(self._h, n))

    def release_part(self, block: int, part: int, stream=None) -> None:
        _check(_lib.stream_pool_release_part(self._h, block, part, _stream(stream)))

    def release(self, block: int, stream=None) -> None:
        _check(_lib.stream_pool_release(self._h, block, _stream(stream)))

    def stats(self) -> dict:
        s = PoolStats()
        _check(_lib.stream_pool_stats(self._h, C.byref(s)))
        return {f: getattr(s, f) for f, _ in PoolStats._fields_}

    def timing_enable(self, enable: bool = True) -> None:
        """Record copy and acquire-stall spans (stream_pool_timing_enable)."""
        _check(_lib.stream_pool_timing_enable(self._h, int(bool(enable))))

    def timing_collect(self) -> dict:
        """Sums of the spans recorded since the last collect (waits for them to complete)."""
        t = PoolTiming()
        _check(_lib.stream_pool_timing_collect(self._h, C.byref(t)))
        return {f: getattr(t, f) for f, _ in PoolTiming._fields_}

    def timing_spans(self) -> list:
        """The spans recorded since the last collect, copies then acquire waits, each a dict
        (stream_pool_timing_spans; call before timing_collect, which forgets them)."""
        n = C.c_int()
        _check(_lib.stream_pool_timing_spans(self._h, None, 0, C.byref(n)))
        arr = (PoolSpan * max(1, n.value))()
        _check(_lib.stream_pool_timing_spans(self._h, arr, n.value, C.byref(n)))
        kinds = {0: "copy", 1: "acquire"}
        return [{"kind": kinds[a.kind], "block": a.block, "part": a.part, "start_ms": a.start_ms, "end_ms": a.end_ms,
                 "host_at_ms": a.host_at_ms, "host_call_ms": a.host_call_ms} for a in arr[:n.value]]

    def slot_block(self, slot: int) -> int:
        b = C.c_int()
        _check(_lib.stream_pool_slot_block(self._h, slot, C.byref(b)))
        return b.value

    def close(self) -> None:
        if getattr(self, "_h", None):
            _check(_lib.stream_pool_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
