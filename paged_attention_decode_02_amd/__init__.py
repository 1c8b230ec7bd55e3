"""Python binding of libpa_decode.so, the gfx950 paged-attention decode library.

Argument marshalling only: every step of the decode runs in the HIP kernels
behind the C ABI (``include/pa_decode.h``). torch provides device memory and
the current stream; tensors must live on the GPU. If the shared library has
not been built the functions raise; there is no fallback.

    cache_write(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None)
    out, lse = decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len,
                      softmax_scale, k_scale=None, v_scale=None, partition_size=0)
    np_ = decode_partials(...)        # the split-K kernel alone
    splitk_reduce(workspace, np_, partition_size, seq_lens, out, lse)
    out, lse = decode_shared_prefix(q, k_cache, v_cache, prefix_table, prefix_len, block_table,
                                    seq_lens, max_seq_len, softmax_scale, ...)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

__all__ = [
    "PaError", "cache_write", "decode", "decode_partials", "splitk_reduce", "workspace_bytes",
    "choose_partition_size", "choose_partition_size_for_cus", "device_cu_count", "decode_kernel_name",
    "library_path", "load", "DTYPE_CODE", "decode_shared_prefix", "shared_prefix_workspace_bytes",
    "validate_decode_args", "validate_cache_write_args", "decode_noalloc", "NOALLOC_SCRATCH_BYTES",
    "sparse_mean_keys", "decode_sparse", "sparse_workspace_bytes", "sparse_max_selected",
    "Prepared", "prepare_cache_write", "prepare_decode_partials", "prepare_splitk_reduce", "prepare_decode",
    "read_probe",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_lib", "libpa_decode.so")
_lock = threading.Lock()
_lib = None

# FP8 caches hold OCP E4M3 codes (torch.float8_e4m3fn storage)
# NVFP4 caches: torch.float4_e2m1fn_x2 storage, [num_blocks, 16, Hkv, 9 D / 16]
# bytes whose blocks hold all code rows first, then one block-scale plane per
# kv head (the layout include/pa_decode.h describes)
DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.int8: 2, torch.float8_e4m3fn: 3, torch.float4_e2m1fn_x2: 4}

EXPORTS = (
    "pa_cache_write", "pa_decode", "pa_decode_splitk_reduce", "pa_decode_workspace_bytes",
    "pa_choose_partition_size", "pa_decode_check", "pa_cache_write_check", "pa_last_error",
    "pa_decode_shared_prefix", "pa_decode_shared_prefix_workspace_bytes", "pa_choose_partition_size_for_cus",
    "pa_device_cu_count", "pa_decode_kernel_name", "pa_decode_noalloc", "pa_sparse_mean_keys", "pa_decode_sparse",
    "pa_decode_sparse_workspace_bytes", "pa_read_probe",
)

# size of the library-owned scratch of pa_decode_noalloc (PA_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 32 << 20


class PaError(RuntimeError):
    """A non-zero return from the C ABI; ``code`` is the PA_ERR_* value."""

    def __init__(self, code: int, msg: str):
        super().__init__("pa error %d: %s" % (code, msg))
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load libpa_decode.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libpa_decode.so is not built (%s); run __graft_entry__.build()" % _LIB_PATH)
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64, F, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        lib.pa_cache_write.argtypes = [P, P, I32, P, I64, P, P, I32, P, P, I64, I32, I32, I32, P]
        lib.pa_cache_write.restype = ctypes.c_int
        lib.pa_decode.argtypes = [P, I32, I32, I32, I32, I32, I32, P, P, I32, P, P, I64, I32, P, I32, P, I32, F,
                                  I32, P, I32, P, P, SZ, ctypes.POINTER(I32), P]
        lib.pa_decode.restype = ctypes.c_int
        lib.pa_decode_splitk_reduce.argtypes = [P, I32, I32, I32, I32, I32, I32, P, P, I32, P, P]
        lib.pa_decode_splitk_reduce.restype = ctypes.c_int
        lib.pa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
        lib.pa_decode_workspace_bytes.restype = SZ
        lib.pa_choose_partition_size.argtypes = [I32, I32, I32, I32, I32, I32, I32]
        lib.pa_choose_partition_size.restype = I32
        lib.pa_decode_check.argtypes = [P, I32, P, I32, I32, I64, P, P]
        lib.pa_decode_check.restype = ctypes.c_int
        lib.pa_cache_write_check.argtypes = [P, I64, I64, I32, P, P]
        lib.pa_cache_write_check.restype = ctypes.c_int
        lib.pa_decode_shared_prefix.argtypes = [P, I32, I32, I32, I32, I32, I32, P, P, I32, P, P, I64, I32, P, I32,
                                                P, I32, P, I32, F, I32, I32, P, I32, P, P, SZ, P]
        lib.pa_decode_shared_prefix.restype = ctypes.c_int
        lib.pa_decode_shared_prefix_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, I32, I32]
        lib.pa_decode_shared_prefix_workspace_bytes.restype = SZ
        lib.pa_choose_partition_size_for_cus.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32]
        lib.pa_choose_partition_size_for_cus.restype = I32
        lib.pa_device_cu_count.argtypes = []
        lib.pa_device_cu_count.restype = I32
        lib.pa_decode_kernel_name.argtypes = [I32, I32, I32, I32]
        lib.pa_decode_kernel_name.restype = ctypes.c_char_p
        lib.pa_decode_noalloc.argtypes = [P, I32, I32, I32, I32, I32, I32, P, P, I32, P, P, I64, I32, P, I32, P, I32,
                                          F, I32, P, I32, P, P]
        lib.pa_decode_noalloc.restype = ctypes.c_int
        lib.pa_sparse_mean_keys.argtypes = [P, I32, P, I64, I32, I32, I32, P, I32, P, I32, I32, I32, I32, P, I32, P]
        lib.pa_sparse_mean_keys.restype = ctypes.c_int
        lib.pa_decode_sparse.argtypes = [P, I32, I32, I32, I32, I32, I32, P, P, I32, P, P, I64, I32, P, I32, P, I32, F,
                                         P, I32, I32, I32, I32, P, I32, P, P, P, SZ, P]
        lib.pa_decode_sparse.restype = ctypes.c_int
        lib.pa_decode_sparse_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32, I32, I32, I32]
        lib.pa_decode_sparse_workspace_bytes.restype = SZ
        lib.pa_read_probe.argtypes = [P, SZ, P, I32, P]
        lib.pa_read_probe.restype = ctypes.c_int
        lib.pa_last_error.argtypes = []
        lib.pa_last_error.restype = ctypes.c_char_p
        _lib = lib
        return lib


def _check(rc: int):
    if rc != 0:
        msg = load().pa_last_error()
        raise PaError(rc, msg.decode() if msg else "")


def _L():
    """The loaded library (the lock is taken only on the first call)."""
    return _lib if _lib is not None else load()


def _ptr(t: Optional[torch.Tensor]):
    # a plain int: ctypes converts it for the c_void_p parameter
    return None if t is None else t.data_ptr()


def _dev(t: Optional[torch.Tensor], name: str):
    if t is not None:
        if not t.is_cuda:
            raise ValueError("%s must be a GPU tensor" % name)
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t: Optional[torch.Tensor] = None) -> int:
    """hipStream_t of `stream`, or of the current stream of t's device."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_stream is not None and t is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream().cuda_stream


def _code(t: torch.Tensor) -> int:
    try:
        return DTYPE_CODE[t.dtype]
    except KeyError:
        raise ValueError("unsupported dtype %s" % t.dtype)


QUANTISED = (torch.int8, torch.float8_e4m3fn, torch.float4_e2m1fn_x2)


def _row_elems(cache_dtype: torch.dtype, D: int) -> int:
    """Last dimension of a cache tensor for head size D (NVFP4: bytes of codes
    and block scales per (token, kv head))."""
    return 9 * D // 16 if cache_dtype == torch.float4_e2m1fn_x2 else D


def _shape_err(msg: str):
    raise ValueError(msg)


def _check_cache_pair(k_cache, v_cache, k_scale, v_scale, D: int):
    """Shared checks of the paged caches and their row scales; returns (nb, Hkv)."""
    if k_cache.dim() != 4 or tuple(k_cache.shape) != tuple(v_cache.shape) or k_cache.dtype != v_cache.dtype:
        _shape_err("k_cache and v_cache must be 4-D tensors of one shape and dtype, got %s %s / %s %s" % (
            tuple(k_cache.shape), k_cache.dtype, tuple(v_cache.shape), v_cache.dtype))
    if k_cache.dtype not in DTYPE_CODE:
        _shape_err("unsupported cache dtype %s" % k_cache.dtype)
    nb, bs, Hkv, row = k_cache.shape
    if bs != 16:
        _shape_err("block_size (cache dim 1) must be 16, got %d" % bs)
    if row != _row_elems(k_cache.dtype, D):
        _shape_err("cache rows hold %d elements, head size %d needs %d" % (row, D, _row_elems(k_cache.dtype, D)))
    if k_cache.dtype in QUANTISED:
        for t, n in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            if t is None:
                _shape_err("%s caches need %s" % (k_cache.dtype, n))
            if t.dtype != torch.float32 or tuple(t.shape) != (nb, Hkv, 16):
                _shape_err("%s must be float32 [%d, %d, 16], got %s %s" % (n, nb, Hkv, t.dtype, tuple(t.shape)))
    return nb, Hkv


def validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, out=None, lse=None,
                         k_scale=None, v_scale=None) -> None:
    """Shape and dtype checks of a decode call (the C ABI sees only pointers,
    so a mismatched tensor would be read out of bounds on the device). Raises
    ValueError; looks at metadata only, so it runs on CPU tensors too."""
    if q.dim() != 4 or q.dtype not in (torch.float32, torch.bfloat16):
        _shape_err("q must be a 4-D float32 or bfloat16 tensor [B, Tq, Hq, D], got %s %s" % (
            tuple(q.shape), q.dtype))
    B, Tq, Hq, D = q.shape
    nb, Hkv = _check_cache_pair(k_cache, v_cache, k_scale, v_scale, D)
    if Hq % Hkv:
        _shape_err("Hq=%d is not a multiple of the caches' Hkv=%d" % (Hq, Hkv))
    if block_table.dim() != 2 or block_table.dtype != torch.int32 or block_table.shape[0] != B:
        _shape_err("block_table must be int32 [B=%d, max_blocks], got %s %s" % (B, block_table.dtype,
                                                                                tuple(block_table.shape)))
    if block_table.shape[1] * 16 < max_seq_len:
        _shape_err("block_table has %d blocks per sequence, max_seq_len %d needs %d" % (
            block_table.shape[1], max_seq_len, (max_seq_len + 15) // 16))
    if seq_lens.dim() != 1 or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        _shape_err("seq_lens must be int32 [B=%d], got %s %s" % (B, seq_lens.dtype, tuple(seq_lens.shape)))
    if out is not None and (tuple(out.shape) != (B, Tq, Hq, D) or out.dtype not in (torch.float32, torch.bfloat16)):
        _shape_err("out must be float32 or bfloat16 [%d, %d, %d, %d], got %s %s" % (B, Tq, Hq, D, out.dtype,
                                                                                   tuple(out.shape)))
    if lse is not None and (tuple(lse.shape) != (B, Tq, Hq) or lse.dtype != torch.float32):
        _shape_err("lse must be float32 [%d, %d, %d], got %s %s" % (B, Tq, Hq, lse.dtype, tuple(lse.shape)))


def validate_cache_write_args(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None) -> None:
    """Shape and dtype checks of a cache write (metadata only; raises ValueError)."""
    if k.dim() != 3 or tuple(k.shape) != tuple(v.shape) or k.dtype != v.dtype or k.dtype not in (
            torch.float32, torch.bfloat16):
        _shape_err("k and v must be float32 or bfloat16 [N, Hkv, D] of one shape, got %s %s / %s %s" % (
            tuple(k.shape), k.dtype, tuple(v.shape), v.dtype))
    N, Hkv, D = k.shape
    _, cHkv = _check_cache_pair(k_cache, v_cache, k_scale, v_scale, D)
    if cHkv != Hkv:
        _shape_err("source rows have Hkv=%d, the caches %d" % (Hkv, cHkv))
    if slot_mapping.dim() != 1 or slot_mapping.dtype != torch.int64 or slot_mapping.numel() != N:
        _shape_err("slot_mapping must be int64 [N=%d], got %s %s" % (N, slot_mapping.dtype,
                                                                      tuple(slot_mapping.shape)))


def cache_write(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                v_cache: torch.Tensor, k_scale: Optional[torch.Tensor] = None, v_scale: Optional[torch.Tensor] = None,
                stream=None) -> None:
    """Store rows k, v [N, Hkv, D] at slot_mapping [N] (int64) in the paged caches."""
    for t, n in ((k, "k"), (v, "v"), (slot_mapping, "slot_mapping"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, n)
    validate_cache_write_args(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale)
    nb, bs, Hkv, _ = k_cache.shape
    D = k.shape[-1]
    _check(_L().pa_cache_write(_ptr(k), _ptr(v), _code(k), _ptr(slot_mapping), slot_mapping.numel(),
                               _ptr(k_cache), _ptr(v_cache), _code(k_cache), _ptr(k_scale), _ptr(v_scale), nb, bs,
                               Hkv, D, _stream(stream, k_cache)))


def workspace_bytes(B: int, Tq: int, Hq: int, Hkv: int, D: int, kv_dtype: torch.dtype, max_seq_len: int,
                    partition_size: int = 0) -> int:
    return int(load().pa_decode_workspace_bytes(B, Tq, Hq, Hkv, D, DTYPE_CODE[kv_dtype], max_seq_len,
                                                partition_size))


def choose_partition_size(B: int, Tq: int, Hq: int, Hkv: int, D: int, kv_dtype: torch.dtype,
                          max_seq_len: int) -> int:
    P = int(load().pa_choose_partition_size(B, Tq, Hq, Hkv, D, DTYPE_CODE[kv_dtype], max_seq_len))
    if P < 0:
        _check(P)
    return P


def choose_partition_size_for_cus(B: int, Tq: int, Hq: int, Hkv: int, D: int, kv_dtype: torch.dtype,
                                  max_seq_len: int, num_cus: int) -> int:
    """The partition heuristic for a device of num_cus compute units."""
    P = int(load().pa_choose_partition_size_for_cus(B, Tq, Hq, Hkv, D, DTYPE_CODE[kv_dtype], max_seq_len,
                                                    num_cus))
    if P < 0:
        _check(P)
    return P


def device_cu_count() -> int:
    """Compute units of the current HIP device as the heuristic uses them."""
    return int(load().pa_device_cu_count())


def decode_kernel_name(Tq: int, Hq: int, Hkv: int, kv_dtype: torch.dtype) -> str:
    """Name of the decode kernel pa_decode launches for these arguments."""
    return load().pa_decode_kernel_name(Tq, Hq, Hkv, DTYPE_CODE[kv_dtype]).decode()


def decode_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, softmax_scale: float,
                    out: torch.Tensor, lse: Optional[torch.Tensor] = None, k_scale=None, v_scale=None,
                    partition_size: int = 0, workspace: Optional[torch.Tensor] = None, stream=None) -> int:
    """Launch the split-K decode kernel only; returns the partition count NP.

    NP == 1: out/lse are written. NP > 1: partials are in ``workspace`` and
    splitk_reduce must follow on the same stream.
    """
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"), (k_scale, "k_scale"), (v_scale, "v_scale"),
                 (workspace, "workspace")):
        _dev(t, n)
    validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, lse, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    np_ = ctypes.c_int32(0)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_L().pa_decode(_ptr(q), _code(q), B, Tq, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), _code(k_cache),
                          _ptr(k_scale), _ptr(v_scale), nb, bs, _ptr(block_table), block_table.shape[1],
                          _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(partition_size), _ptr(out),
                          _code(out), _ptr(lse), _ptr(workspace), ws_bytes, ctypes.byref(np_), _stream(stream, q)))
    return int(np_.value)


def splitk_reduce(workspace: torch.Tensor, num_partitions: int, partition_size: int, seq_lens: torch.Tensor,
                  out: torch.Tensor, lse: Optional[torch.Tensor] = None, stream=None) -> None:
    """Merge split-K partials (layout of include/pa_decode.h) into out/lse."""
    for t, n in ((workspace, "workspace"), (seq_lens, "seq_lens"), (out, "out"), (lse, "lse")):
        _dev(t, n)
    if out.dim() != 4 or seq_lens.dtype != torch.int32 or seq_lens.numel() != out.shape[0]:
        raise ValueError("out must be [B, Tq, Hq, D] and seq_lens int32 [B]")
    if lse is not None and tuple(lse.shape) != tuple(out.shape[:3]):
        raise ValueError("lse must be [B, Tq, Hq]")
    B, Tq, Hq, D = out.shape
    rows = B * Tq * Hq
    need = ((rows * num_partitions * D * 4 + 255) // 256 * 256) + rows * num_partitions * 4
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace holds %d bytes, %d partitions need %d" % (
            workspace.numel() * workspace.element_size(), num_partitions, need))
    _check(_L().pa_decode_splitk_reduce(_ptr(workspace), int(num_partitions), int(partition_size), B, Tq, Hq, D,
                                        _ptr(seq_lens), _ptr(out), _code(out), _ptr(lse), _stream(stream, out)))


class Prepared:
    """Library calls whose tensors were checked and whose arguments were
    marshalled once: calling the object launches the same work again on the
    current stream of the tensors' device (or on ``stream``) without per-call
    checks, as a serving loop with buffers at fixed addresses (or a captured
    graph) would. The tensors must stay alive and keep their shapes and
    dtypes while it is used; their contents may change between calls."""

    __slots__ = ("_calls", "_device", "_keep", "num_partitions")

    def __init__(self, calls, device: int, keep, num_partitions: int = 1):
        self._calls = calls  # [(library function, converted arguments before the stream)]
        self._device = device
        self._keep = keep  # the tensors behind the pointers
        self.num_partitions = num_partitions

    def __call__(self, stream=None) -> None:
        s = stream.cuda_stream if stream is not None else (
            _raw_stream(self._device) if _raw_stream is not None else torch.cuda.current_stream().cuda_stream)
        for fn, args in self._calls:
            rc = fn(*args, s)
            if rc != 0:
                _check(rc)


_CARG = type(ctypes.byref(ctypes.c_int32()))  # what ctypes.byref returns


def _marshal(fn, args):
    """Convert each argument but the trailing stream to fn's ctypes type once."""
    conv = []
    for typ, a in zip(fn.argtypes, args):
        conv.append(a if isinstance(a, (typ, _CARG)) else typ(a))
    return fn, tuple(conv)


def prepare_cache_write(k, v, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None) -> Prepared:
    """cache_write with its checks and argument marshalling done once."""
    for t, n in ((k, "k"), (v, "v"), (slot_mapping, "slot_mapping"), (k_cache, "k_cache"), (v_cache, "v_cache"),
                 (k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, n)
    validate_cache_write_args(k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale)
    nb, bs, Hkv, _ = k_cache.shape
    call = _marshal(_L().pa_cache_write, (_ptr(k), _ptr(v), _code(k), _ptr(slot_mapping), slot_mapping.numel(),
                                          _ptr(k_cache), _ptr(v_cache), _code(k_cache), _ptr(k_scale), _ptr(v_scale),
                                          nb, bs, Hkv, k.shape[-1]))
    return Prepared([call], k_cache.get_device(), (k, v, slot_mapping, k_cache, v_cache, k_scale, v_scale))


def prepare_decode_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, softmax_scale: float,
                            out: torch.Tensor, lse: Optional[torch.Tensor] = None, k_scale=None, v_scale=None,
                            partition_size: int = 0, workspace: Optional[torch.Tensor] = None) -> Prepared:
    """decode_partials with its checks and argument marshalling done once;
    ``.num_partitions`` is the NP every call produces (ceil(max_seq_len / P))."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"), (k_scale, "k_scale"), (v_scale, "v_scale"),
                 (workspace, "workspace")):
        _dev(t, n)
    validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, lse, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    P = partition_size or choose_partition_size(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len)
    NP = (int(max_seq_len) + P - 1) // P if max_seq_len > 0 else 1
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if NP > 1 and ws_bytes < workspace_bytes(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len, P):
        raise ValueError("workspace holds %d bytes, %d partitions need %d" % (
            ws_bytes, NP, workspace_bytes(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len, P)))
    np_out = ctypes.c_int32(0)
    call = _marshal(_L().pa_decode, (_ptr(q), _code(q), B, Tq, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache),
                                     _code(k_cache), _ptr(k_scale), _ptr(v_scale), nb, bs, _ptr(block_table),
                                     block_table.shape[1], _ptr(seq_lens), int(max_seq_len), float(softmax_scale),
                                     int(P), _ptr(out), _code(out), _ptr(lse), _ptr(workspace), ws_bytes,
                                     ctypes.byref(np_out)))
    prep = Prepared([call], q.get_device(), (q, k_cache, v_cache, block_table, seq_lens, out, lse, k_scale, v_scale,
                                            workspace, np_out), NP)
    return prep


def prepare_splitk_reduce(workspace: torch.Tensor, num_partitions: int, partition_size: int, seq_lens: torch.Tensor,
                          out: torch.Tensor, lse: Optional[torch.Tensor] = None) -> Prepared:
    """splitk_reduce with its checks and argument marshalling done once."""
    for t, n in ((workspace, "workspace"), (seq_lens, "seq_lens"), (out, "out"), (lse, "lse")):
        _dev(t, n)
    if out.dim() != 4 or seq_lens.dtype != torch.int32 or seq_lens.numel() != out.shape[0]:
        raise ValueError("out must be [B, Tq, Hq, D] and seq_lens int32 [B]")
    if lse is not None and tuple(lse.shape) != tuple(out.shape[:3]):
        raise ValueError("lse must be [B, Tq, Hq]")
    B, Tq, Hq, D = out.shape
    rows = B * Tq * Hq
    need = ((rows * num_partitions * D * 4 + 255) // 256 * 256) + rows * num_partitions * 4
    if workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace holds %d bytes, %d partitions need %d" % (
            workspace.numel() * workspace.element_size(), num_partitions, need))
    call = _marshal(_L().pa_decode_splitk_reduce, (_ptr(workspace), int(num_partitions), int(partition_size), B, Tq,
                                                   Hq, D, _ptr(seq_lens), _ptr(out), _code(out), _ptr(lse)))
    return Prepared([call], out.get_device(), (workspace, seq_lens, out, lse))


def prepare_decode(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, softmax_scale: float,
                   out: torch.Tensor, lse: torch.Tensor, k_scale=None, v_scale=None, partition_size: int = 0,
                   workspace: Optional[torch.Tensor] = None) -> Prepared:
    """decode (the split-K kernel, then the reduce when there is more than one
    partition) with its checks and argument marshalling done once."""
    dec = prepare_decode_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale, out, lse,
                                  k_scale, v_scale, partition_size, workspace)
    calls, keep = list(dec._calls), [dec._keep]
    if dec.num_partitions > 1:
        B, Tq, Hq, D = q.shape
        P = partition_size or choose_partition_size(B, Tq, Hq, k_cache.shape[2], D, k_cache.dtype, max_seq_len)
        red = prepare_splitk_reduce(workspace, dec.num_partitions, P, seq_lens, out, lse)
        calls += red._calls
        keep.append(red._keep)
    return Prepared(calls, q.get_device(), keep, dec.num_partitions)


def decode_check(block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, num_blocks: int,
                 status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Debug check of the block table and lengths pa_decode trusts; returns the
    device int32[2] status (violations, first flat index or -1), unsynchronised."""
    for t, n in ((block_table, "block_table"), (seq_lens, "seq_lens"), (status, "status")):
        _dev(t, n)
    if status is None:
        status = torch.empty(2, dtype=torch.int32, device=block_table.device)
    B, max_blocks = block_table.shape
    _check(load().pa_decode_check(_ptr(block_table), max_blocks, _ptr(seq_lens), B, int(max_seq_len),
                                  int(num_blocks), _ptr(status), _stream(stream, status)))
    return status


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> torch.Tensor:
    """Streaming-read ceiling probe (measurement only): reads every byte of the
    contiguous device tensor buf once with the decode kernels' loads, in
    sink.numel() workgroups; sink (uint32 or int32, device) receives per
    workgroup the wrap-around sum of the 32-bit words it read. Unsynchronised."""
    for t, n in ((buf, "buf"), (sink, "sink")):
        _dev(t, n)
    if sink.dtype not in (torch.int32, torch.uint32):
        raise ValueError("sink must be int32 or uint32")
    nbytes = buf.numel() * buf.element_size()
    _check(load().pa_read_probe(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(stream, buf)))
    return sink


def cache_write_check(slot_mapping: torch.Tensor, num_blocks: int, block_size: int = 16,
                      status: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Debug check of slot_mapping for pa_cache_write; returns the device int32[2]
    status (slots past the cache, first token index or -1), unsynchronised."""
    for t, n in ((slot_mapping, "slot_mapping"), (status, "status")):
        _dev(t, n)
    if status is None:
        status = torch.empty(2, dtype=torch.int32, device=slot_mapping.device)
    _check(load().pa_cache_write_check(_ptr(slot_mapping), slot_mapping.numel(), int(num_blocks), int(block_size),
                                       _ptr(status), _stream(stream, status)))
    return status


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, block_table: torch.Tensor,
           seq_lens: torch.Tensor, max_seq_len: int, softmax_scale: float, k_scale: Optional[torch.Tensor] = None,
           v_scale: Optional[torch.Tensor] = None, partition_size: int = 0, out: Optional[torch.Tensor] = None,
           lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
           out_dtype: torch.dtype = torch.float32, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Paged decode of q [B, Tq, Hq, D]; returns (out [B, Tq, Hq, D], lse [B, Tq, Hq]).

    Runs the split-K kernel and, when it used more than one partition, the
    log-sum-exp reduce. Missing out/lse/workspace tensors are allocated with
    torch (the C ABI itself never allocates).
    """
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    P = partition_size or choose_partition_size(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len)
    if workspace is None:
        nbytes = workspace_bytes(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len, P)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    np_ = decode_partials(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, softmax_scale, out, lse,
                          k_scale, v_scale, P, workspace, stream)
    if np_ > 1:
        splitk_reduce(workspace, np_, P, seq_lens, out, lse, stream)
    return out, lse


def decode_noalloc(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, softmax_scale: float,
                   out: torch.Tensor, lse: Optional[torch.Tensor] = None, k_scale=None, v_scale=None,
                   partition_size: int = 0, stream=None) -> None:
    """pa_decode_noalloc: decode and (when needed) the reduce, with the split-K
    partials in the library's own scratch; out/lse are written. Neither the
    library nor this function allocates: out (and lse) come from the caller."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"), (k_scale, "k_scale"), (v_scale, "v_scale")):
        _dev(t, n)
    validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, lse, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    _check(_L().pa_decode_noalloc(_ptr(q), _code(q), B, Tq, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), _code(k_cache),
                                  _ptr(k_scale), _ptr(v_scale), nb, bs, _ptr(block_table), block_table.shape[1],
                                  _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(partition_size),
                                  _ptr(out), _code(out), _ptr(lse), _stream(stream, q)))


def sparse_max_selected(max_seq_len: int, sparse_block: int, top_blocks: int) -> int:
    """S: selected sparse blocks per (sequence, kv head) at most."""
    nsb = (int(max_seq_len) + sparse_block - 1) // sparse_block
    return min(nsb, max(top_blocks, 2))


def sparse_mean_keys(k_cache, block_table, seq_lens, max_seq_len: int, sparse_block: int, num_new: int,
                     mean_k: torch.Tensor, k_scale=None, stream=None) -> None:
    """Refresh the mean keys [B, max_sparse_blocks, Hkv, D] (fp32) of the
    sparse blocks holding each sequence's newest num_new tokens."""
    for t, n in ((k_cache, "k_cache"), (block_table, "block_table"), (seq_lens, "seq_lens"), (mean_k, "mean_k"),
                 (k_scale, "k_scale")):
        _dev(t, n)
    nb, bs, Hkv, row = k_cache.shape
    D = row * 16 // 9 if k_cache.dtype == torch.float4_e2m1fn_x2 else row
    B = block_table.shape[0]
    if mean_k.dtype != torch.float32 or mean_k.dim() != 4 or mean_k.shape[0] != B or tuple(mean_k.shape[2:]) != (
            Hkv, D):
        raise ValueError("mean_k must be float32 [B=%d, max_sparse_blocks, %d, %d]" % (B, Hkv, D))
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("block_table and seq_lens must be int32 with B rows")
    _check(_L().pa_sparse_mean_keys(_ptr(k_cache), _code(k_cache), _ptr(k_scale), nb, bs, Hkv, D, _ptr(block_table),
                                    block_table.shape[1], _ptr(seq_lens), B, int(max_seq_len), int(sparse_block),
                                    int(num_new), _ptr(mean_k), mean_k.shape[1], _stream(stream, k_cache)))


def sparse_workspace_bytes(B: int, Tq: int, Hq: int, Hkv: int, D: int, kv_dtype: torch.dtype, max_seq_len: int,
                           sparse_block: int, top_blocks: int, partition_size: int = 0) -> int:
    return int(load().pa_decode_sparse_workspace_bytes(B, Tq, Hq, Hkv, D, DTYPE_CODE[kv_dtype], max_seq_len,
                                                       sparse_block, top_blocks, partition_size))


def decode_sparse(q, k_cache, v_cache, block_table, seq_lens, max_seq_len: int, softmax_scale: float,
                  mean_k: torch.Tensor, sparse_block: int, top_blocks: int, k_scale=None, v_scale=None,
                  partition_size: int = 0, out=None, lse=None, selected=None, workspace=None,
                  out_dtype: torch.dtype = torch.float32, stream=None):
    """Sparse block-selection decode; returns (out, lse). selected, when given,
    receives [B, Hkv, S] int32 block ids (increasing, -1 after the last)."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (block_table, "block_table"),
                 (seq_lens, "seq_lens"), (mean_k, "mean_k"), (out, "out"), (lse, "lse"), (k_scale, "k_scale"),
                 (v_scale, "v_scale"), (selected, "selected"), (workspace, "workspace")):
        _dev(t, n)
    validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, lse, k_scale, v_scale)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    if mean_k.dtype != torch.float32 or mean_k.dim() != 4 or (mean_k.shape[0], mean_k.shape[2], mean_k.shape[3]) != (
            B, Hkv, D):
        raise ValueError("mean_k must be float32 [B, max_sparse_blocks, Hkv, D]")
    S = sparse_max_selected(max_seq_len, sparse_block, top_blocks)
    if selected is not None and (selected.dtype != torch.int32 or tuple(selected.shape) != (B, Hkv, S)):
        raise ValueError("selected must be int32 [%d, %d, %d]" % (B, Hkv, S))
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    nbytes = sparse_workspace_bytes(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len, sparse_block, top_blocks,
                                    partition_size)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(_L().pa_decode_sparse(
        _ptr(q), _code(q), B, Tq, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), _code(k_cache), _ptr(k_scale),
        _ptr(v_scale), nb, bs, _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(max_seq_len),
        float(softmax_scale), _ptr(mean_k), mean_k.shape[1], int(sparse_block), int(top_blocks), int(partition_size),
        _ptr(out), _code(out), _ptr(lse), _ptr(selected), _ptr(workspace), ws_bytes, _stream(stream, q)))
    return out, lse


def shared_prefix_workspace_bytes(B: int, Tq: int, Hq: int, Hkv: int, D: int, kv_dtype: torch.dtype,
                                  max_seq_len: int, prefix_len: int, prefix_partition: int = 0,
                                  tail_partition: int = 0) -> int:
    return int(load().pa_decode_shared_prefix_workspace_bytes(B, Tq, Hq, Hkv, D, DTYPE_CODE[kv_dtype], max_seq_len,
                                                              prefix_len, prefix_partition, tail_partition))


def decode_shared_prefix(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                         prefix_table: Optional[torch.Tensor],
                         prefix_len: int, block_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
                         softmax_scale: float, k_scale: Optional[torch.Tensor] = None,
                         v_scale: Optional[torch.Tensor] = None, prefix_partition: int = 0, tail_partition: int = 0,
                         out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, out_dtype: torch.dtype = torch.float32,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Decode of a batch whose sequences share their first prefix_len tokens
    (blocks prefix_table [prefix_len / 16] int32, None when prefix_len is 0);
    same result as decode(). Missing out/lse/workspace tensors are allocated
    with torch."""
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache"), (prefix_table, "prefix_table"),
                 (block_table, "block_table"), (seq_lens, "seq_lens"), (out, "out"), (lse, "lse"),
                 (k_scale, "k_scale"), (v_scale, "v_scale"), (workspace, "workspace")):
        _dev(t, n)
    validate_decode_args(q, k_cache, v_cache, block_table, seq_lens, max_seq_len, out, lse, k_scale, v_scale)
    if prefix_table is not None and prefix_table.dtype != torch.int32:
        raise ValueError("prefix_table must be int32")
    if prefix_table is not None and prefix_table.numel() < prefix_len // 16:
        raise ValueError("prefix_table holds %d blocks, prefix_len %d needs %d" % (
            prefix_table.numel(), prefix_len, prefix_len // 16))
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    if out is None:
        out = torch.empty((B, Tq, Hq, D), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, Tq, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        nbytes = shared_prefix_workspace_bytes(B, Tq, Hq, Hkv, D, k_cache.dtype, max_seq_len, prefix_len,
                                               prefix_partition, tail_partition)
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_L().pa_decode_shared_prefix(
        _ptr(q), _code(q), B, Tq, Hq, Hkv, D, _ptr(k_cache), _ptr(v_cache), _code(k_cache), _ptr(k_scale),
        _ptr(v_scale), nb, bs, _ptr(prefix_table), int(prefix_len), _ptr(block_table), block_table.shape[1],
        _ptr(seq_lens), int(max_seq_len), float(softmax_scale), int(prefix_partition), int(tail_partition),
        _ptr(out), _code(out), _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream, q)))
    return out, lse
