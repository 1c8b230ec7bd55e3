"""Host-side test plumbing: oracle caches for a generated workload, poisoning."""
from __future__ import annotations

import numpy as np

import oracle
from _refs import nvfp4_token_bytes
from workloads import BLOCK_SIZE, Workload

POISON_CODE = 127


def poison_host(w: Workload, k, v, ks, vs) -> None:
    """Fill every cache slot that holds no source row with poison.

    Float caches get NaN; int8, FP8 and NVFP4 caches get code 127 (an E4M3
    NaN) in every byte of the slot, with a NaN scale. A decode that reads any
    of these slots produces NaN.
    """
    slots = w.unused_slots()
    blk, off = slots // BLOCK_SIZE, slots % BLOCK_SIZE
    sp = w.spec
    for c in (k, v):
        if sp.cache_dtype == "nvfp4":  # a token's bytes are spread over its block
            idx = np.stack([nvfp4_token_bytes(sp.Hkv, sp.D, t) for t in range(BLOCK_SIZE)])
            c.reshape(c.shape[0], -1)[blk[:, None], idx[off]] = POISON_CODE
        elif c.dtype == np.float32:
            c[blk, off] = np.nan
        elif c.dtype == np.uint16:
            c[blk, off] = 0x7FC0  # bfloat16 quiet NaN
        else:
            c[blk, off] = POISON_CODE
    for s in (ks, vs):
        if s is not None:
            s[blk, :, off] = np.nan  # scales [num_blocks, Hkv, 16]


def oracle_cache(w: Workload, poison: bool = True):
    """(k, v, k_scale, v_scale) written by the oracle's cache writer."""
    sp = w.spec
    k, v, ks, vs = oracle.alloc_cache(w.num_blocks, BLOCK_SIZE, sp.Hkv, sp.D, sp.cache_dtype)
    oracle.cache_write(w.k_src, w.v_src, w.slot_mapping, k, v, ks, vs)
    if poison:
        poison_host(w, k, v, ks, vs)
    return k, v, ks, vs


def oracle_decode(w: Workload, cache, **kw):
    k, v, ks, vs = cache
    return oracle.decode(w.q_array(), k, v, w.block_table, w.seq_lens, w.softmax_scale, ks, vs, **kw)
