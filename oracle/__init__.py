"""fp64 CPU oracle for paged-attention decode.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
benchmark's CPU-baseline leg use it; the product path never imports it. It
shares no code with the HIP library (``pa_oracle.c`` includes nothing from it
and is built by gcc, not hipcc).

Functions take numpy arrays in the layouts the decode problem fixes:
q [B, Tq, Hq, D]; caches [num_blocks, block_size, Hkv, D]; int8, FP8 and NVFP4
scales [num_blocks, Hkv, block_size] (one per token and kv head, a kv head's
scales of a block together); block_table [B, max_blocks] int32; seq_lens [B]
int32. bfloat16 data is passed as its uint16 bit patterns, FP8 (OCP E4M3) as
its uint8 codes.

Pins (see ``tests/test_oracle_pins.py``): Decimal brute force, closed forms
(single key, constant V, zero query), dense contiguous attention, block-table
permutation, GQA = repeated-KV MHA, causal = virtual batch, split = unsplit,
prefix sharing, linearity, torch SDPA in fp64, int8 round trip and bound; FP8:
hand-derived E4M3 values and roundings, torch's float8_e4m3fn decode and
(saturated) encode, round trip and error bound.
Every function here is pinned by at least one of them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "_pa_oracle.so")
_lock = threading.Lock()
_lib = None

DTYPE_CODE = {"f32": 0, "bf16": 1, "i8": 2, "fp8": 3, "nvfp4": 4}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain IEEE arithmetic, no fast-math)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC",
           "-shared", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB):
                build()
            lib = ctypes.CDLL(_LIB)
            P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
            lib.pa_oracle_cache_write.argtypes = [P, P, I, P, I64, P, P, I, P, P, I64, I, I, I]
            lib.pa_oracle_cache_write.restype = I
            dec = [P, I, I, I, I, I, I, P, P, I, P, P, I, P, I, P, F]
            lib.pa_oracle_decode.argtypes = dec + [P, I64, P, P, I]
            lib.pa_oracle_decode.restype = I
            lib.pa_oracle_decode_split.argtypes = dec + [I, P, I64, P, P, I]
            lib.pa_oracle_decode_split.restype = I
            lib.pa_oracle_max_threads.restype = I
            lib.pa_oracle_fp8_value.argtypes = [I]
            lib.pa_oracle_fp8_value.restype = ctypes.c_double
            lib.pa_oracle_fp8_encode.argtypes = [F]
            lib.pa_oracle_fp8_encode.restype = I
            lib.pa_oracle_e2m1_value.argtypes = [I]
            lib.pa_oracle_e2m1_value.restype = ctypes.c_double
            lib.pa_oracle_e2m1_encode.argtypes = [F]
            lib.pa_oracle_e2m1_encode.restype = I
            lib.pa_oracle_nvfp4_row_bytes.argtypes = [I]
            lib.pa_oracle_nvfp4_row_bytes.restype = I
            lib.pa_oracle_sparse_mean_keys.argtypes = [P, I, P, I, I, I, P, I, P, I, I, I, P]
            lib.pa_oracle_sparse_mean_keys.restype = I
            lib.pa_oracle_sparse_select.argtypes = [P, I, I, I, I, I, I, F, P, I, P, I, I, I, P, P, P]
            lib.pa_oracle_sparse_select.restype = I
            lib.pa_oracle_decode_subset.argtypes = dec + [P, P, I, I, P, P, I]
            lib.pa_oracle_decode_subset.restype = I
            _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


_MAX_THREADS = []


def max_threads() -> int:
    """OpenMP threads available to the oracle, read on the first call: a
    decode with an explicit thread count changes OpenMP's default for later
    parallel regions, so later reads would see that count instead."""
    if not _MAX_THREADS:
        _MAX_THREADS.append(int(_load().pa_oracle_max_threads()))
    return _MAX_THREADS[0]


NVFP4_HEAD_DIMS = (64, 128, 256)  # where the bytes per (token, head), 36, 72, 144, differ from D


def nvfp4_row_bytes(D: int) -> int:
    """NVFP4 storage bytes per (token, kv head): D/2 of codes and D/16 of block
    scales. An NVFP4 cache is a uint8 array [num_blocks, 16, Hkv, 9 D / 16]
    whose blocks hold all code rows first and then the block-scale planes
    (the layout is described in pa_oracle.c), so [b, t, h] is not row (t, h)."""
    if D not in NVFP4_HEAD_DIMS:
        raise ValueError("NVFP4 caches need D in %s" % (NVFP4_HEAD_DIMS,))
    return D // 2 + D // 16


def _cache_dtype(cache: np.ndarray, D: int) -> str:
    """Cache dtype; uint8 arrays whose last dim is nvfp4_row_bytes(D), not D, are NVFP4."""
    if cache.dtype == np.uint8 and D in NVFP4_HEAD_DIMS and cache.shape[-1] != D:
        assert cache.shape[-1] == nvfp4_row_bytes(D), cache.shape
        return "nvfp4"
    return _dtype_of(cache)


def _dtype_of(a: np.ndarray) -> str:
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.uint16:
        return "bf16"
    if a.dtype == np.int8:
        return "i8"
    if a.dtype == np.uint8:
        return "fp8"  # OCP E4M3 codes
    raise TypeError("unsupported array dtype %s" % a.dtype)


def alloc_cache(num_blocks: int, block_size: int, Hkv: int, D: int, cache_dtype: str):
    """Zeroed host cache arrays (k, v, k_scale, v_scale) in the cache layout."""
    npdt = {"f32": np.float32, "bf16": np.uint16, "i8": np.int8, "fp8": np.uint8, "nvfp4": np.uint8}[cache_dtype]
    shape = (num_blocks, block_size, Hkv, nvfp4_row_bytes(D) if cache_dtype == "nvfp4" else D)
    k = np.zeros(shape, npdt)
    v = np.zeros(shape, npdt)
    ks = vs = None
    if cache_dtype in ("i8", "fp8", "nvfp4"):
        ks = np.zeros((num_blocks, Hkv, block_size), np.float32)  # a kv head's scales of a block together
        vs = np.zeros((num_blocks, Hkv, block_size), np.float32)
    return k, v, ks, vs


def fp8_value(code: int) -> float:
    """The value an OCP E4M3 code stands for (NaN for the NaN codes)."""
    return float(_load().pa_oracle_fp8_value(int(code)))


def fp8_encode(y: float) -> int:
    """OCP E4M3 code of a binary32 value: nearest finite, ties to even, saturating."""
    return int(_load().pa_oracle_fp8_encode(ctypes.c_float(y)))


def e2m1_value(code: int) -> float:
    """The value an FP4 E2M1 code (0..15) stands for."""
    return float(_load().pa_oracle_e2m1_value(int(code)))


def e2m1_encode(y: float) -> int:
    """FP4 E2M1 code of a binary32 value: nearest, ties to even, saturating at 6."""
    return int(_load().pa_oracle_e2m1_encode(ctypes.c_float(y)))


def cache_write(k_src: np.ndarray, v_src: np.ndarray, slot_mapping: np.ndarray, k_cache: np.ndarray,
                v_cache: np.ndarray, k_scale: Optional[np.ndarray] = None,
                v_scale: Optional[np.ndarray] = None) -> None:
    """Store source rows [N, Hkv, D] into the paged caches at slot_mapping (in place)."""
    lib = _load()
    src_dt = _dtype_of(k_src)
    cache_dt = _cache_dtype(k_cache, k_src.shape[-1])
    assert k_src.dtype == v_src.dtype and k_cache.dtype == v_cache.dtype
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    nb, bs, Hkv, _ = k_cache.shape
    D = k_src.shape[-1]
    k_src = _c(k_src, k_src.dtype)
    v_src = _c(v_src, v_src.dtype)
    slots = _c(slot_mapping, np.int64)
    N = slots.shape[0]
    assert k_src.shape == (N, Hkv, D) and v_src.shape == (N, Hkv, D)
    rc = lib.pa_oracle_cache_write(_ptr(k_src), _ptr(v_src), DTYPE_CODE[src_dt], _ptr(slots), N,
                                   _ptr(k_cache), _ptr(v_cache), DTYPE_CODE[cache_dt], _ptr(k_scale),
                                   _ptr(v_scale), nb, bs, Hkv, D)
    if rc != 0:
        raise ValueError("oracle cache_write failed: %d" % rc)


def decode(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
           seq_lens: np.ndarray, softmax_scale: float, k_scale: Optional[np.ndarray] = None,
           v_scale: Optional[np.ndarray] = None, partition_size: int = 0,
           rows: Optional[Sequence[int]] = None, nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 decode. Returns (out [B, Tq, Hq, D], lse [B, Tq, Hq]).

    partition_size > 0 runs the split-K path (partials merged by log-sum-exp)
    instead of the plain definition. rows (flat ids (b*Tq + t)*Hq + h) limits
    the work to those rows; the other entries are NaN.
    """
    lib = _load()
    q = np.ascontiguousarray(q)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    assert v_cache.shape == k_cache.shape
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    assert table.shape[0] == B and lens.shape == (B,)
    kv_dt = _cache_dtype(k_cache, D)
    out = np.full((B, Tq, Hq, D), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    rows_arr = None if rows is None else _c(rows, np.int64)
    nrows = 0 if rows_arr is None else rows_arr.shape[0]
    common = [_ptr(q), DTYPE_CODE[_dtype_of(q)], B, Tq, Hq, Hkv, D, _ptr(np.ascontiguousarray(k_cache)),
              _ptr(np.ascontiguousarray(v_cache)), DTYPE_CODE[kv_dt], _ptr(k_scale), _ptr(v_scale), bs,
              _ptr(table), table.shape[1], _ptr(lens), ctypes.c_float(softmax_scale)]
    if partition_size > 0:
        rc = lib.pa_oracle_decode_split(*common, partition_size, _ptr(rows_arr), nrows, _ptr(out), _ptr(lse),
                                        nthreads)
    else:
        rc = lib.pa_oracle_decode(*common, _ptr(rows_arr), nrows, _ptr(out), _ptr(lse), nthreads)
    if rc != 0:
        raise ValueError("oracle decode failed: %d" % rc)
    return out, lse


# ---------------------------------------------------------------- sparse decode
def num_sparse_blocks(L: int, sparse_block: int) -> int:
    return (int(L) + sparse_block - 1) // sparse_block


def sparse_max_selected(max_seq_len: int, sparse_block: int, top_blocks: int) -> int:
    """Largest number of sparse blocks one (sequence, kv head) can select: the
    top_blocks, or the (at most two) blocks holding the query tokens."""
    return min(num_sparse_blocks(max_seq_len, sparse_block), max(top_blocks, 2))


def sparse_mean_keys(k_cache: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray, sparse_block: int,
                     max_sblocks: int, k_scale: Optional[np.ndarray] = None, D: Optional[int] = None) -> np.ndarray:
    """fp64 mean keys [B, max_sblocks, Hkv, D] of every sparse block below each
    sequence's length (NaN elsewhere)."""
    lib = _load()
    nb, bs, Hkv, row = k_cache.shape
    D = D or row
    kv_dt = _cache_dtype(k_cache, D)
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    B = lens.shape[0]
    out = np.full((B, max_sblocks, Hkv, D), np.nan)
    rc = lib.pa_oracle_sparse_mean_keys(_ptr(np.ascontiguousarray(k_cache)), DTYPE_CODE[kv_dt], _ptr(k_scale), bs,
                                        Hkv, D, _ptr(table), table.shape[1], _ptr(lens), B, sparse_block,
                                        max_sblocks, _ptr(out))
    if rc != 0:
        raise ValueError("oracle sparse_mean_keys failed: %d" % rc)
    return out


def sparse_select(q: np.ndarray, mean_k: np.ndarray, seq_lens: np.ndarray, softmax_scale: float, sparse_block: int,
                  top_blocks: int, max_sel: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Selected sparse blocks per (b, kv head): (selected [B, Hkv, max_sel]
    int32, increasing, -1 padded; count [B, Hkv]; candidate scores [B, Hkv,
    max_sblocks] fp64, NaN for the kept blocks and past the end). mean_k is
    [B, max_sblocks, Hkv, D] (fp64, or the GPU's fp32 widened)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    B, Tq, Hq, D = q.shape
    mk = _c(mean_k, np.float64)
    _, max_sblocks, Hkv, _ = mk.shape
    lens = _c(seq_lens, np.int32)
    sel = np.full((B, Hkv, max_sel), -1, dtype=np.int32)
    cnt = np.zeros((B, Hkv), dtype=np.int32)
    scores = np.full((B, Hkv, max_sblocks), np.nan)
    rc = lib.pa_oracle_sparse_select(_ptr(q), DTYPE_CODE[_dtype_of(q)], B, Tq, Hq, Hkv, D,
                                     ctypes.c_float(softmax_scale), _ptr(mk), max_sblocks, _ptr(lens), sparse_block,
                                     top_blocks, max_sel, _ptr(sel), _ptr(cnt), _ptr(scores))
    if rc != 0:
        raise ValueError("oracle sparse_select failed: %d" % rc)
    return sel, cnt, scores


def decode_subset(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                  seq_lens: np.ndarray, softmax_scale: float, selected: np.ndarray, count: np.ndarray,
                  sparse_block: int, k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
                  nthreads: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """fp64 decode of every row over the keys of its kv head's selected sparse
    blocks (causal rule as in decode)."""
    lib = _load()
    q = np.ascontiguousarray(q)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    table = _c(block_table, np.int32)
    lens = _c(seq_lens, np.int32)
    sel = _c(selected, np.int32)
    cnt = _c(count, np.int32)
    assert sel.shape[:2] == (B, Hkv) and cnt.shape == (B, Hkv)
    kv_dt = _cache_dtype(k_cache, D)
    out = np.full((B, Tq, Hq, D), np.nan)
    lse = np.full((B, Tq, Hq), np.nan)
    common = [_ptr(q), DTYPE_CODE[_dtype_of(q)], B, Tq, Hq, Hkv, D, _ptr(np.ascontiguousarray(k_cache)),
              _ptr(np.ascontiguousarray(v_cache)), DTYPE_CODE[kv_dt], _ptr(k_scale), _ptr(v_scale), bs,
              _ptr(table), table.shape[1], _ptr(lens), ctypes.c_float(softmax_scale)]
    rc = lib.pa_oracle_decode_subset(*common, _ptr(sel), _ptr(cnt), sel.shape[2], sparse_block, _ptr(out), _ptr(lse),
                                     nthreads)
    if rc != 0:
        raise ValueError("oracle decode_subset failed: %d" % rc)
    return out, lse


def decode_sparse(q: np.ndarray, k_cache: np.ndarray, v_cache: np.ndarray, block_table: np.ndarray,
                  seq_lens: np.ndarray, softmax_scale: float, sparse_block: int, top_blocks: int,
                  k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None):
    """The whole sparse decode: mean keys, selection, decode over the selected
    blocks. Returns (out, lse, selected, count, mean_k)."""
    B, Tq, Hq, D = q.shape
    L = int(np.max(seq_lens)) if len(seq_lens) else 0
    nsb = max(1, num_sparse_blocks(L, sparse_block))
    mk = sparse_mean_keys(k_cache, block_table, seq_lens, sparse_block, nsb, k_scale, D)
    sel, cnt, _ = sparse_select(q, mk, seq_lens, softmax_scale, sparse_block, top_blocks,
                                sparse_max_selected(L, sparse_block, top_blocks) or 1)
    out, lse = decode_subset(q, k_cache, v_cache, block_table, seq_lens, softmax_scale, sel, cnt, sparse_block,
                             k_scale, v_scale)
    return out, lse, sel, cnt, mk
