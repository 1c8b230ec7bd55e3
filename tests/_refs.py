"""Independent references that pin the oracle (test helpers only).

Nothing here is shared with the oracle's C code or with the HIP library:
  - ``brute_decode``: pure-Python ``decimal`` arithmetic at 50 significant
    digits (``Decimal.exp`` is correctly rounded), gathering each key through
    the block table with its own loops;
  - ``dense_decode``: numpy fp64 attention on keys/values first gathered into
    contiguous arrays by fancy indexing, softmax via numpy;
  - ``sdpa_decode``: torch's ``scaled_dot_product_attention`` on CPU in float64
    with an explicit causal mask and KV heads repeated per query group.
"""
from __future__ import annotations

import decimal
from decimal import Decimal
from typing import Optional

import numpy as np

from workloads import bf16_bits_to_f32


# NVFP4 caches: uint8 [num_blocks, 16, Hkv, 9 D / 16], last dim -> D
_NVFP4_D = {36: 64, 72: 128, 144: 256}


def nvfp4_split(a: np.ndarray, D: int):
    """E2M1 codes [nb, 16, Hkv, D] and E4M3 block-scale codes [nb, 16, Hkv, D/16]
    of an NVFP4 cache. A block holds the code rows of its 16 * Hkv (token, head)
    pairs first, D/2 bytes each in (token, head) order with element 2i in the
    low nibble of byte i, then one plane of D bytes per head, the scale of
    elements 16k .. 16k + 15 of token t = 4q + r at byte 16k + 4r + q."""
    nb, bs, Hkv, rb = a.shape
    assert bs == 16 and rb == D // 2 + D // 16, a.shape
    flat = a.reshape(nb, -1)
    cb = flat[:, : 16 * Hkv * D // 2].reshape(nb, 16, Hkv, D // 2).astype(np.int64)
    codes = np.stack([cb & 15, cb >> 4], axis=-1).reshape(nb, 16, Hkv, D)
    planes = flat[:, 16 * Hkv * D // 2:].reshape(nb, Hkv, D // 16, 4, 4)  # [b, h, k, r, q]
    scales = planes.transpose(0, 4, 3, 1, 2).reshape(nb, 16, Hkv, D // 16)  # [b, q, r, h, k]
    return codes, np.ascontiguousarray(scales)


def _e2m1(codes: np.ndarray) -> np.ndarray:
    """FP4 E2M1 values: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0."""
    s = np.where(codes & 8, -1.0, 1.0)
    e = (codes >> 1) & 3
    m = (codes & 1).astype(np.float64)
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.exp2(e.astype(np.float64) - 1.0))
    return s * mag


def nvfp4_token_bytes(Hkv: int, D: int, t: int) -> np.ndarray:
    """Byte offsets, within an NVFP4 block, of token t's code rows (every
    head) and block scales (the layout nvfp4_split reads)."""
    codes = t * Hkv * (D // 2) + np.arange(Hkv * (D // 2))
    h, k = np.meshgrid(np.arange(Hkv), np.arange(D // 16), indexing="ij")
    scales = 16 * Hkv * (D // 2) + h * D + 16 * k + 4 * (t % 4) + t // 4
    return np.concatenate([codes, scales.reshape(-1)])


def _nvfp4_f64(a: np.ndarray, scale: np.ndarray, D: int) -> np.ndarray:
    """Decoded NVFP4 cache [nb, 16, Hkv, D]: E2M1 codes times their E4M3 block
    scale (decoded by torch's float8_e4m3fn) times the row's fp32 scale."""
    import torch

    codes, sc = nvfp4_split(a, D)
    bsc = torch.from_numpy(sc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return _e2m1(codes) * np.repeat(bsc, 16, axis=-1) * _row_scales(scale)[..., None]


def _row_scales(scale: np.ndarray) -> np.ndarray:
    """fp32 scales [num_blocks, Hkv, 16] as float64 [num_blocks, 16, Hkv], the
    cache's (block, token, head) order."""
    assert scale.ndim == 3
    return np.swapaxes(scale, 1, 2).astype(np.float64)


def as_f64(a: np.ndarray, scale: Optional[np.ndarray] = None) -> np.ndarray:
    """Values of a cache/query array as float64 (int8 codes, or FP8 codes
    decoded by torch's float8_e4m3fn, times their row scale)."""
    if a.dtype == np.uint16:
        return bf16_bits_to_f32(a).reshape(a.shape).astype(np.float64)
    if a.dtype == np.int8:
        assert scale is not None
        return a.astype(np.float64) * _row_scales(scale)[..., None]
    if a.dtype == np.uint8 and a.shape[-1] in _NVFP4_D:
        return _nvfp4_f64(a, scale, _NVFP4_D[a.shape[-1]])
    if a.dtype == np.uint8:
        import torch

        assert scale is not None
        vals = torch.from_numpy(np.ascontiguousarray(a)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        return vals * _row_scales(scale)[..., None]
    return a.astype(np.float64)


def gather(cache64: np.ndarray, table_row: np.ndarray, n: int) -> np.ndarray:
    """Contiguous [n, Hkv, D] keys/values of one sequence (fancy indexing)."""
    bs = cache64.shape[1]
    j = np.arange(n)
    return cache64[table_row[j // bs], j % bs]


def dense_decode(q, k_cache, v_cache, table, seq_lens, scale, k_scale=None, v_scale=None):
    q64 = as_f64(q)
    K = as_f64(k_cache, k_scale)
    V = as_f64(v_cache, v_scale)
    B, Tq, Hq, D = q64.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Tq, Hq, D))
    lse = np.full((B, Tq, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        Kb = gather(K, table[b], max(L, 0))
        Vb = gather(V, table[b], max(L, 0))
        for t in range(Tq):
            n = L - Tq + t + 1
            if n <= 0:
                continue
            for h in range(Hq):
                s = float(np.float32(scale)) * (Kb[:n, h // G, :] @ q64[b, t, h])
                m = s.max()
                w = np.exp(s - m)
                out[b, t, h] = (w @ Vb[:n, h // G, :]) / w.sum()
                lse[b, t, h] = m + np.log(w.sum())
    return out, lse


def sdpa_decode(q, k_cache, v_cache, table, seq_lens, scale, k_scale=None, v_scale=None):
    import torch
    import torch.nn.functional as F

    q64 = torch.from_numpy(as_f64(q))
    K = as_f64(k_cache, k_scale)
    V = as_f64(v_cache, v_scale)
    B, Tq, Hq, D = q64.shape
    Hkv = K.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Tq, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        Kb = torch.from_numpy(gather(K, table[b], L)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Vb = torch.from_numpy(gather(V, table[b], L)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        qb = q64[b].permute(1, 0, 2)  # [Hq, Tq, D]
        pos = torch.arange(L)
        mask = pos[None, :] <= (L - Tq + torch.arange(Tq))[:, None]  # [Tq, L]
        o = F.scaled_dot_product_attention(qb[None], Kb[None].contiguous(), Vb[None].contiguous(),
                                           attn_mask=mask[None, None], scale=float(np.float32(scale)))
        out[b] = o[0].permute(1, 0, 2).numpy()
    return out


def brute_decode(q, k_cache, v_cache, table, seq_lens, scale, k_scale=None, v_scale=None, digits=50):
    """Decimal brute force. Every input value is converted exactly to Decimal."""
    ctx = decimal.Context(prec=digits)
    B, Tq, Hq, D = q.shape
    nb, bs, Hkv, _ = k_cache.shape
    G = Hq // Hkv
    qv = as_f64(q)
    kv = as_f64(k_cache, k_scale)  # exact: int8 code * fp32 scale fits a double
    vv = as_f64(v_cache, v_scale)
    sc = Decimal(float(np.float32(scale)))
    out = np.zeros((B, Tq, Hq, D))
    lse = np.full((B, Tq, Hq), -np.inf)
    for b in range(B):
        L = int(seq_lens[b])
        for t in range(Tq):
            n = L - Tq + t + 1
            if n <= 0:
                continue
            for h in range(Hq):
                g = h // G
                qd = [Decimal(float(x)) for x in qv[b, t, h]]
                logits = []
                for j in range(n):
                    blk = int(table[b][j // bs])
                    off = j % bs
                    krow = kv[blk, off, g]
                    acc = Decimal(0)
                    for d in range(D):
                        acc = ctx.add(acc, ctx.multiply(qd[d], Decimal(float(krow[d]))))
                    logits.append(ctx.multiply(sc, acc))
                M = max(logits)
                w = [ctx.exp(ctx.subtract(s, M)) for s in logits]
                Z = Decimal(0)
                for x in w:
                    Z = ctx.add(Z, x)
                for d in range(D):
                    acc = Decimal(0)
                    for j in range(n):
                        blk = int(table[b][j // bs])
                        acc = ctx.add(acc, ctx.multiply(w[j], Decimal(float(vv[blk, j % bs, g, d]))))
                    out[b, t, h, d] = float(ctx.divide(acc, Z))
                lse[b, t, h] = float(ctx.add(M, ctx.ln(Z)))
    return out, lse
